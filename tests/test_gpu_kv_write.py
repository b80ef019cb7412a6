"""KV write on the GPU through the C ABI against the oracle's write (needs an
MI355X): bit for bit, the whole pool compared (untouched slots, NaN-poisoned
spare pages included); fp8_e5m2 quantisation with per-tensor scales, with
values that saturate, underflow to subnormals, ties and NaN; then attention
over the written cache against the oracle."""

import sys

import numpy as np
import pytest
import torch

import oracle
from paged_attention_prefill_amd import inputs as gen
from paged_attention_prefill_amd import ops

pytestmark = pytest.mark.gpu

_BITS = {torch.float16: torch.int16, torch.bfloat16: torch.int16, torch.float32: torch.int32, torch.uint8: torch.uint8,
         torch.float8_e4m3fn: torch.uint8}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def new_rows(case, kind, seed, specials=False):
    g = torch.Generator().manual_seed(seed)
    dt = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}[kind]
    shape = (case.total_q, case.num_kv_heads, case.head_dim)
    k = torch.randn(shape, generator=g).to(dt)
    v = torch.randn(shape, generator=g).to(dt)
    if specials and case.total_q:
        flat = k.view(-1)
        vals = [1e5, -1e5, 6e4, 57344.0, 3e-6, -3e-6, 1.125, 1.375, float("nan"), -0.0, 0.0, float("inf")]
        flat[:len(vals)] = torch.tensor(vals).to(dt)
    return k, v


def raw(t):
    t = t.contiguous() if t.device.type == "cpu" else t.cpu()
    return t.view(_BITS[t.dtype]).numpy()


def run_write(case, kn, vn):
    d = gen.to_device(case)
    say(f"  write {case.name}: seqs={case.num_seqs} total_q={case.total_q} Hkv={case.num_kv_heads} "
        f"D={case.head_dim} P={case.page_size} kv={case.kv_kind} layout={case.layout}")
    ops.write_kv(kn.cuda(), vn.cuda(), d["k"], d["v"], d["cu"], d["seq_lens"], d["bt"], max(1, case.max_seqlen_q),
                 k_scale=case.k_scale, v_scale=case.v_scale, k_head_scales=d.get("k_head_scales"),
                 v_head_scales=d.get("v_head_scales"))
    torch.cuda.synchronize()
    return d


CASE = dict(q_lens=[5, 0, 300, 1, 40], seq_lens=[40, 9, 1100, 1, 30], num_q_heads=8, num_kv_heads=2,
            head_dim=128, page_size=48)


@pytest.mark.parametrize("kind,layout", [("f16", "NHD"), ("bf16", "NHD"), ("f32", "NHD"), ("f16", "HND")])
def test_kv_write_same_dtype_is_an_exact_copy(kind, layout):
    case = gen.make_case(f"kvw_{kind}", q_kind=kind, seed=61, layout=layout, **CASE)
    kn, vn = new_rows(case, kind, 62)
    d = run_write(case, kn, vn)
    ko, vo = oracle.write_kv(raw(case.k_pool), raw(case.v_pool), raw(kn), raw(vn), case.cu_seqlens_q,
                             case.seq_lens, case.block_tables)
    assert np.array_equal(raw(d["k"]), ko) and np.array_equal(raw(d["v"]), vo)


@pytest.mark.parametrize("src", ["f16", "bf16"])
@pytest.mark.parametrize("fmt,k_scale,v_scale", [("e5m2", 1.0, 1.0), ("e5m2", 0.5, 3.0), ("e5m2", 0.0078125, 1.7),
                                                 ("e4m3", 1.0, 1.0), ("e4m3", 0.01, 250.0), ("e4m3", 0.3, 0.7)])
def test_kv_write_fp8_quantisation_is_bit_exact(fmt, k_scale, v_scale, src):
    case = gen.make_case(f"kvw_{fmt}_{src}", q_kind=src, kv_kind=fmt, seed=63, k_scale=k_scale, v_scale=v_scale,
                         **dict(CASE, head_dim=256, page_size=64))
    kn, vn = new_rows(case, src, 64, specials=True)
    d = run_write(case, kn, vn)
    ko, vo = oracle.write_kv(raw(case.k_pool), raw(case.v_pool), kn.float().numpy(), vn.float().numpy(),
                             case.cu_seqlens_q, case.seq_lens, case.block_tables, fp8=fmt, k_scale=k_scale,
                             v_scale=v_scale)
    gk, gv = raw(d["k"]), raw(d["v"])
    bad = int((gk != ko).sum() + (gv != vo).sum())
    say(f"  fp8 {fmt} write: {bad} bytes differ of {gk.size + gv.size}")
    assert bad == 0


def test_attention_over_the_written_cache():
    """The chunk's K/V written by the library, then the prefill reads them."""
    case = gen.make_case("kvw_then_prefill", q_lens=[300, 64], seq_lens=[1100, 64], num_q_heads=8, num_kv_heads=2,
                         head_dim=128, page_size=32, q_kind="bf16", seed=65)
    kn, vn = new_rows(case, "bf16", 66)
    d = run_write(case, kn, vn)
    out = ops.paged_prefill(d["q"], d["k"], d["v"], d["cu"], d["seq_lens"], d["bt"], case.max_seqlen_q,
                            case.scale, num_kv_splits=2)
    torch.cuda.synchronize()
    ko, vo = oracle.write_kv(gen.to_numpy64(case.k_pool), gen.to_numpy64(case.v_pool), kn.double().numpy(),
                             vn.double().numpy(), case.cu_seqlens_q, case.seq_lens, case.block_tables)
    ref, _ = oracle.paged_attention(gen.to_numpy64(case.q), ko, vo, case.cu_seqlens_q, case.seq_lens,
                                    case.block_tables, case.scale)
    err = float(np.abs(out.float().cpu().numpy() - ref).max())
    say(f"  prefill over the written cache: max|err| {err:.3e}")
    assert err < 2e-2


@pytest.mark.parametrize("fmt", ["e5m2", "e4m3"])
def test_kv_write_fp8_per_head_scales(fmt):
    case = gen.make_case(f"kvw_heads_{fmt}", q_kind="f16", kv_kind=fmt, seed=67, k_scale=0.5, v_scale=1.25,
                         **dict(CASE, head_dim=256, page_size=64))
    case.k_head_scales = np.array([0.1, 3.0], dtype=np.float32)
    case.v_head_scales = np.array([7.0, 0.3], dtype=np.float32)
    kn, vn = new_rows(case, "f16", 68, specials=True)
    d = run_write(case, kn, vn)
    ko, vo = oracle.write_kv(raw(case.k_pool), raw(case.v_pool), kn.float().numpy(), vn.float().numpy(),
                             case.cu_seqlens_q, case.seq_lens, case.block_tables, fp8=fmt, k_scale=0.5, v_scale=1.25,
                             k_head_scales=case.k_head_scales, v_head_scales=case.v_head_scales)
    assert np.array_equal(raw(d["k"]), ko) and np.array_equal(raw(d["v"]), vo)
