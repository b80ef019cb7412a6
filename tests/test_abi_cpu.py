"""The C ABI without a GPU: the library loads, exports every declared symbol, and
rejects bad arguments before any HIP call (CPU only; no kernel is launched)."""

import ctypes
import json
import os

import numpy as np
import pytest

from paged_attention_prefill_amd import inputs as gen
from paged_attention_prefill_amd import ops

pytestmark = pytest.mark.skipif(not os.path.exists(ops.LIB_PATH), reason="library not built")

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_numbers.json")))


def test_every_declared_symbol_is_exported():
    L = ops.lib()
    names = ops.header_symbols()
    assert "pa_paged_prefill" in names and "pa_split_kv_decode" in names and "pa_merge_states" in names
    for n in names:
        assert hasattr(L, n), n
    assert L.pa_version() == 3


def test_status_strings():
    L = ops.lib()
    for st in (0, -1, -2, -3, -4, -5):
        assert L.pa_status_string(st).decode() not in ("", "unknown status")
    assert L.pa_status_string(7).decode() == "unknown status"


def test_decode_workspace_matches_the_pages_record_size():
    g = GOLDEN["split_kv_workspace"]
    per_row = ops.decode_workspace_bytes(1, g["num_heads"], g["head_dim"], g["num_splits"])
    assert per_row == g["num_heads"] * g["num_splits"] * (g["head_dim"] + 2) * 4
    assert abs(per_row / 1024 / g["per_row_kib"] - 1) < g["tolerance_rel"]
    rows64 = ops.decode_workspace_bytes(64, g["num_heads"], g["head_dim"], g["num_splits"])
    assert abs(rows64 / 2 ** 20 / g["rows_64_mib"] - 1) < g["tolerance_rel"]


def test_prefill_workspace_sizes():
    assert ops.prefill_workspace_bytes(100, 8, 128, 1) == 0
    assert ops.prefill_workspace_bytes(100, 8, 128, 3) == 100 * 8 * 3 * 130 * 4
    assert ops.prefill_workspace_bytes(100, 8, 128, 0) == 100 * 8 * 16 * 130 * 4


@pytest.mark.parametrize("args,status", [
    ((ops.PA_F16, ops.PA_F16, 128, 16, 32, 8), 0),
    ((ops.PA_BF16, ops.PA_BF16, 256, 816, 24, 4), 0),
    ((ops.PA_F16, ops.PA_FP8_E5M2, 256, 816, 24, 4), 0),
    ((ops.PA_F16, ops.PA_FP8_E4M3, 256, 816, 24, 4), 0),
    ((ops.PA_F16, ops.PA_FP8_E4M3, 64, 16, 8, 2), 0),
    ((ops.PA_BF16, ops.PA_FP8_E4M3, 128, 16, 8, 8), 0),
    ((ops.PA_FP8_E4M3, ops.PA_FP8_E4M3, 128, 16, 8, 8), ops.PA_ERR_UNSUPPORTED),
    ((ops.PA_F16, 5, 128, 16, 8, 8), ops.PA_ERR_UNSUPPORTED),
    ((ops.PA_F32, ops.PA_F32, 64, 16, 4, 1), 0),
    ((ops.PA_F16, ops.PA_F16, 96, 48, 6, 2), 0),
    ((ops.PA_BF16, ops.PA_FP8_E5M2, 128, 16, 8, 8), 0),
    ((ops.PA_F32, ops.PA_FP8_E5M2, 128, 16, 8, 8), ops.PA_ERR_UNSUPPORTED),
    ((ops.PA_F16, ops.PA_BF16, 128, 16, 8, 8), ops.PA_ERR_UNSUPPORTED),
    ((ops.PA_F16, ops.PA_F16, 100, 16, 8, 8), ops.PA_ERR_UNSUPPORTED),
    ((ops.PA_F16, ops.PA_F16, 512, 16, 8, 8), ops.PA_ERR_UNSUPPORTED),
    ((ops.PA_F16, ops.PA_F16, 128, 24, 8, 8), ops.PA_ERR_UNSUPPORTED),
    ((ops.PA_F16, ops.PA_F16, 128, 16, 12, 8), ops.PA_ERR_UNSUPPORTED),
    ((ops.PA_FP8_E5M2, ops.PA_FP8_E5M2, 128, 16, 8, 8), ops.PA_ERR_UNSUPPORTED),
    ((9, ops.PA_F16, 128, 16, 8, 8), ops.PA_ERR_UNSUPPORTED),
])
def test_check_supported(args, status):
    st, reason = ops.check_supported(*args)
    assert st == status, reason


def test_validate_metadata_accepts_generated_cases_and_flags_corruption():
    c = gen.make_case("m", [3, 0, 5], [40, 7, 5], 4, 2, 32, 16, q_kind="f16", seed=1)
    args = (c.cu_seqlens_q, c.seq_lens, c.block_tables, c.total_q, 16, c.page_size, c.num_pages)
    assert ops.validate_metadata(*args)[0] == 0
    bad = c.block_tables.copy()
    bad[0, 1] = c.num_pages
    st, msg = ops.validate_metadata(c.cu_seqlens_q, c.seq_lens, bad, c.total_q, 16, c.page_size, c.num_pages)
    assert st == ops.PA_ERR_METADATA and "block_tables[0][1]" in msg
    cu = c.cu_seqlens_q.copy()
    cu[2] = 1
    assert ops.validate_metadata(cu, c.seq_lens, c.block_tables, c.total_q, 16, c.page_size, c.num_pages)[0] == -5
    assert ops.validate_metadata(c.cu_seqlens_q, c.seq_lens, c.block_tables, c.total_q, 4, c.page_size,
                                 c.num_pages)[0] == -5
    sl = c.seq_lens.copy()
    sl[0] = 10 ** 6
    assert ops.validate_metadata(c.cu_seqlens_q, sl, c.block_tables, c.total_q, 16, c.page_size,
                                 c.num_pages)[0] == -5


def _fake_kv(**over):
    # device pointers are never dereferenced: every call below is rejected first
    kv = dict(k_pages=0x10000, v_pages=0x20000, stride_page=16 * 2 * 128, stride_token=2 * 128,
              stride_head=128, num_pages=10, page_size=16, num_kv_heads=2, head_dim=128,
              dtype=ops.PA_F16, k_scale=1.0, v_scale=1.0)
    kv.update(over)
    return ops.KvCache(**kv)


def _prefill(kv, **over):
    a = dict(q=0x30000, q_dtype=ops.PA_F16, out=0x40000, lse=None, cu=0x50000, sl=0x60000, bt=0x70000,
             num_seqs=2, max_pages=4, total_q=10, max_q=8, hq=8, scale=0.1, splits=1, ws=None, ws_bytes=0)
    a.update(over)
    return ops.lib().pa_paged_prefill(a["q"], a["q_dtype"], a["out"], a["lse"], a["cu"], a["sl"], a["bt"],
                                      a["num_seqs"], a["max_pages"], a["total_q"], a["max_q"], a["hq"],
                                      ctypes.byref(kv) if kv is not None else None, a["scale"], a["splits"],
                                      a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kv_over,call_over,status", [
    ({}, {"q": None}, ops.PA_ERR_INVALID_ARGUMENT),
    ({}, {"cu": None}, ops.PA_ERR_INVALID_ARGUMENT),
    ({"page_size": 24}, {}, ops.PA_ERR_UNSUPPORTED),
    ({"head_dim": 72}, {}, ops.PA_ERR_UNSUPPORTED),
    ({"num_kv_heads": 3}, {}, ops.PA_ERR_UNSUPPORTED),
    ({"dtype": ops.PA_BF16}, {}, ops.PA_ERR_UNSUPPORTED),
    ({"stride_token": 100}, {}, ops.PA_ERR_INVALID_ARGUMENT),
    ({"k_pages": 0x10008}, {}, ops.PA_ERR_INVALID_ARGUMENT),
    ({"k_scale": 2.0}, {}, ops.PA_ERR_UNSUPPORTED),
    ({"dtype": ops.PA_FP8_E5M2, "k_scale": -1.0}, {}, ops.PA_ERR_INVALID_ARGUMENT),
    ({}, {"q": 0x30004}, ops.PA_ERR_INVALID_ARGUMENT),
    ({}, {"splits": 2}, ops.PA_ERR_WORKSPACE),
    ({}, {"splits": 2, "ws": 0x80000, "ws_bytes": 100}, ops.PA_ERR_WORKSPACE),
    ({}, {"splits": 99}, ops.PA_ERR_INVALID_ARGUMENT),
    ({}, {"scale": float("nan")}, ops.PA_ERR_INVALID_ARGUMENT),
    ({}, {"scale": 0.0}, ops.PA_ERR_INVALID_ARGUMENT),
    ({}, {"scale": -0.1}, ops.PA_ERR_INVALID_ARGUMENT),
    ({}, {"num_seqs": -1}, ops.PA_ERR_INVALID_ARGUMENT),
    ({}, {"max_pages": 0}, ops.PA_ERR_INVALID_ARGUMENT),
    ({"num_pages": 0}, {}, ops.PA_ERR_INVALID_ARGUMENT),
])
def test_prefill_rejects_bad_arguments_before_launch(kv_over, call_over, status):
    assert _prefill(_fake_kv(**kv_over), **call_over) == status
    assert ops.lib().pa_last_error().decode() != ""


def test_prefill_null_kv():
    assert _prefill(None) == ops.PA_ERR_INVALID_ARGUMENT


def test_empty_call_launches_nothing():
    assert _prefill(_fake_kv(), total_q=0, num_seqs=0) == ops.PA_OK


def test_decode_rejects_long_rows_and_small_workspace():
    L = ops.lib()
    kv = _fake_kv()

    def dec(max_q=1, splits=16, ws=None, ws_bytes=0):
        return L.pa_split_kv_decode(0x30000, ops.PA_F16, 0x40000, None, 0x50000, 0x60000, 0x70000, 4, 4, 4,
                                    max_q, 8, ctypes.byref(kv), 0.1, splits, ws, ws_bytes, None)
    assert dec(max_q=17) == ops.PA_ERR_UNSUPPORTED
    assert dec(splits=0) == ops.PA_ERR_INVALID_ARGUMENT
    assert dec() == ops.PA_ERR_WORKSPACE
    need = ops.decode_workspace_bytes(4, 8, 128, 16)
    assert dec(ws=0x80000, ws_bytes=need - 1) == ops.PA_ERR_WORKSPACE
    assert dec(ws=0x80004, ws_bytes=need) == ops.PA_ERR_WORKSPACE  # misaligned


def test_noalloc_decode_checks_before_any_device_call():
    """pa_split_kv_decode_noalloc rejects a NULL out and records past its buffer
    before it touches a device (no GPU here); the buffer size matches the header."""
    L = ops.lib()
    kv = _fake_kv()
    text = open(ops.HEADER_PATH).read()
    assert "#define PA_NOALLOC_SCRATCH_BYTES (64 * 1024 * 1024)" in text
    assert ops.NOALLOC_SCRATCH_BYTES == 64 * 1024 * 1024

    def dec(out=0x40000, total_q=4, splits=16):
        return L.pa_split_kv_decode_noalloc(0x30000, ops.PA_F16, out, None, 0x50000, 0x60000, 0x70000, 4, 4,
                                            total_q, 1, 8, ctypes.byref(kv), 0.1, splits, 0, None, None)
    assert dec(out=None) == ops.PA_ERR_INVALID_ARGUMENT
    # 4096 tokens x 8 heads x 4096 parts x 130 floats: past the 64 MiB buffer
    assert ops.decode_workspace_bytes(4096, 8, 128, 4096) > ops.NOALLOC_SCRATCH_BYTES
    assert dec(total_q=4096, splits=4096) == ops.PA_ERR_WORKSPACE
    assert "buffer" in L.pa_last_error().decode()


def test_fixed_part_decode_rejects_bad_part_sizes():
    L = ops.lib()
    kv = _fake_kv()

    def dec(part_keys, parts=8, ws=None, ws_bytes=0):
        return L.pa_split_kv_decode_fixed(0x30000, ops.PA_F16, 0x40000, None, 0x50000, 0x60000, 0x70000, 4, 4, 4,
                                          1, 8, ctypes.byref(kv), 0.1, part_keys, parts, ws, ws_bytes, None)
    for bad in (0, -32, 16, 48, 100):
        assert dec(bad) == ops.PA_ERR_INVALID_ARGUMENT, bad
    assert dec(64, parts=0) == ops.PA_ERR_INVALID_ARGUMENT
    assert dec(64) == ops.PA_ERR_WORKSPACE  # accepted up to the workspace check
    need = ops.decode_workspace_bytes(4, 8, 128, 8)
    assert dec(64, ws=0x80000, ws_bytes=need - 1) == ops.PA_ERR_WORKSPACE


def test_merge_rejects_bad_arguments():
    L = ops.lib()
    assert L.pa_merge_states(0x1000, 0, 4, 4, 64, 0x2000, ops.PA_F16, None, None) == ops.PA_ERR_INVALID_ARGUMENT
    assert L.pa_merge_states(0x1000, 4, 4, 4, 64, 0x2000, ops.PA_FP8_E5M2, None, None) == ops.PA_ERR_UNSUPPORTED
    assert L.pa_merge_states(None, 4, 4, 4, 64, 0x2000, ops.PA_F16, None, None) == ops.PA_ERR_INVALID_ARGUMENT
    assert L.pa_merge_states(0x1000, 4, 0, 4, 64, 0x2000, ops.PA_F16, None, None) == ops.PA_OK


def test_out_null_needs_split_and_no_lse():
    """out may be NULL (pass 1 only) for a split prefill without lse, and for a decode without lse."""
    kv = _fake_kv()
    assert _prefill(kv, out=None) == ops.PA_ERR_INVALID_ARGUMENT  # one split: no pass to stop after
    assert _prefill(kv, out=None, splits=0) == ops.PA_ERR_INVALID_ARGUMENT  # auto may choose one
    assert _prefill(kv, out=None, splits=2, lse=0x90000) == ops.PA_ERR_INVALID_ARGUMENT
    assert _prefill(kv, out=None, splits=2) == ops.PA_ERR_WORKSPACE  # accepted up to the workspace check
    L = ops.lib()

    def dec(out, lse):
        return L.pa_split_kv_decode(0x30000, ops.PA_F16, out, lse, 0x50000, 0x60000, 0x70000, 4, 4, 4, 1, 8,
                                    ctypes.byref(kv), 0.1, 16, None, 0, None)
    assert dec(None, 0x90000) == ops.PA_ERR_INVALID_ARGUMENT
    assert dec(None, None) == ops.PA_ERR_WORKSPACE


def test_options_are_checked_before_launch():
    L = ops.lib()
    kv = _fake_kv()
    for bad in (ops.AttnOptions(None, 10, -1.0, None), ops.AttnOptions(None, 10, float("inf"), None),
                ops.AttnOptions(None, 10, float("nan"), None), ops.AttnOptions(None, -1, 0.0, 0x1001)):
        st = L.pa_paged_prefill_ex(0x30000, ops.PA_F16, 0x40000, None, 0x50000, 0x60000, 0x70000, 2, 4, 10, 8, 8,
                                   ctypes.byref(kv), 0.1, 1, ctypes.byref(bad), None, 0, None)
        assert st == ops.PA_ERR_INVALID_ARGUMENT
    mis = ops.AttnOptions(0x1002, -1, 0.0, None)
    st = L.pa_split_kv_decode_ex(0x30000, ops.PA_F16, 0x40000, None, 0x50000, 0x60000, 0x70000, 4, 4, 4, 1, 8,
                                 ctypes.byref(kv), 0.1, 8, 0, ctypes.byref(mis), None, 0, None)
    assert st == ops.PA_ERR_INVALID_ARGUMENT
    st = L.pa_split_kv_decode_ex(0x30000, ops.PA_F16, 0x40000, None, 0x50000, 0x60000, 0x70000, 4, 4, 4, 1, 8,
                                 ctypes.byref(kv), 0.1, 8, 48, None, None, 0, None)
    assert st == ops.PA_ERR_INVALID_ARGUMENT  # part_keys not a multiple of 32
    ok = ops.AttnOptions(0x1000, 5, 30.0, 0x2000)
    st = L.pa_split_kv_decode_ex(0x30000, ops.PA_F16, 0x40000, None, 0x50000, 0x60000, 0x70000, 4, 4, 4, 1, 8,
                                 ctypes.byref(kv), 0.1, 8, 0, ctypes.byref(ok), None, 0, None)
    assert st == ops.PA_ERR_WORKSPACE  # accepted up to the workspace check


def test_mixed_step_arguments_are_checked_before_launch():
    L = ops.lib()
    kv = _fake_kv()

    # 4 rows: two small-q rows (1 and 2 tokens), a row without tokens and a chunk of 20
    ql = np.array([1, 2, 0, 20], dtype=np.int32)

    def mixed(out=0x40000, dmq=0, sd=8, pk=0, sp=1, ws=None, wsb=0, lens=ql, total_q=23):
        return L.pa_mixed_step(0x30000, ops.PA_F16, out, None, 0x50000, lens.ctypes.data, 0x60000, 0x70000, 4, 4,
                               total_q, 8, ctypes.byref(kv), 0.1, dmq, sd, pk, sp, None, ws, wsb, None)
    assert mixed(out=None) == ops.PA_ERR_INVALID_ARGUMENT
    assert mixed(dmq=17) == ops.PA_ERR_UNSUPPORTED               # past the decode kernels' 16 tokens
    assert mixed(dmq=-1) == ops.PA_ERR_UNSUPPORTED
    assert mixed(sd=0) == ops.PA_ERR_INVALID_ARGUMENT
    assert mixed(pk=48) == ops.PA_ERR_INVALID_ARGUMENT
    assert mixed(sp=65) == ops.PA_ERR_INVALID_ARGUMENT
    assert mixed(total_q=24) == ops.PA_ERR_INVALID_ARGUMENT      # host lengths must sum to total_q
    assert mixed(lens=np.array([1, -2, 0, 20], dtype=np.int32)) == ops.PA_ERR_INVALID_ARGUMENT
    assert mixed() == ops.PA_ERR_WORKSPACE                        # the route's metadata and records need room
    # the layout: 2 small-q rows with 3 tokens, 1 chunk; 4 pages per row, 8 heads, D 64, fp16, 8 decode parts
    a = lambda x: (x + 255) // 256 * 256  # noqa: E731
    nd, npre, nt = 2, 1, 3
    # metadata, block-table rows of each class, the small-q rows' gathered q, their records
    want = (a(4 * (3 * nd + 1 + 4 * npre + nt)) + a(4 * nd * 4) + a(4 * npre * 4) + a(nt * 8 * 64 * 2)
            + a(4 * nt * 8 * 8 * 66))
    need = ops.mixed_workspace_bytes(ql, 4, 8, 64, ops.PA_F16, 0, 8, 1)
    assert need == want
    need3 = ops.mixed_workspace_bytes(ql, 4, 8, 64, ops.PA_F16, 0, 8, 3)
    assert need3 == want + a(4 * 23 * 8 * 3 * 66)
    # with decode_max_q 1 the row of 2 tokens is a chunk: fewer compact small-q tokens
    assert ops.mixed_workspace_bytes(ql, 4, 8, 64, ops.PA_F16, 1, 8, 1) < need
    assert mixed(sp=3, ws=0x80000, wsb=need) == ops.PA_ERR_WORKSPACE
    assert mixed(sp=1, ws=0x80010, wsb=need) == ops.PA_ERR_WORKSPACE  # not 256-byte aligned
