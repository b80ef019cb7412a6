"""pa_split_kv_decode_noalloc on the GPU, through the C ABI (needs an MI355X).

The entry point for callers that cannot allocate: the split-KV decode with its
FP32 records in the library's own per-GPU buffer instead of a workspace.  It
must give the bits of pa_split_kv_decode_ex with the same arguments (the same
kernels and partition), on consecutive calls that reuse the buffer (the second
smaller than the first, so stale records of the first lie past its end), and
reject a call whose records do not fit before launching anything.
"""

import numpy as np
import pytest
import torch

from paged_attention_prefill_amd import inputs as gen
from paged_attention_prefill_amd import ops
from parity_bars import say

pytestmark = pytest.mark.gpu


def bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)


def both(case, max_q, **kw):
    """(out, lse) of the workspace call and of the no-alloc call."""
    d = gen.to_device(case)
    args = (d["q"], d["k"], d["v"], d["cu"], d["seq_lens"], d["bt"], max_q, case.scale)
    ref_o, ref_l = ops.split_kv_decode(*args, return_lse=True, k_scale=case.k_scale, v_scale=case.v_scale, **kw)
    out = torch.full_like(d["q"], float("nan"))
    lse = torch.full(d["q"].shape[:2], float("nan"), dtype=torch.float32, device="cuda")
    ops.split_kv_decode_noalloc(*args, out, lse=lse, k_scale=case.k_scale, v_scale=case.v_scale, **kw)
    torch.cuda.synchronize()
    return (ref_o, ref_l), (out, lse)


def test_noalloc_decode_equals_the_workspace_call():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    # first call: the 32-row decode batch (bf16, 16 heads, D 128, 16 parts): 4.3 MB of records
    big = gen.decode_batch(kind="bf16")
    need = ops.decode_workspace_bytes(big.total_q, big.num_q_heads, big.head_dim, 16)
    say(f"  no-alloc decode: 32-row batch, {need} bytes of records")
    (ro, rl), (o, l) = both(big, 1, num_splits=16)
    assert torch.equal(bits(o), bits(ro)) and torch.equal(bits(l), bits(rl)), "32-row batch"
    # second call, smaller: a verify row and two decode rows, fp16 D 256 GQA 6, absolute parts and a window
    small = gen.make_case("noalloc_small", q_lens=[5, 1, 3], seq_lens=[3000, 40, 777], num_q_heads=12,
                          num_kv_heads=2, head_dim=256, page_size=64, q_kind="f16", seed=123)
    say("  no-alloc decode: 3 rows, fp16 D 256, absolute parts of 512 keys, window 600")
    (ro, rl), (o, l) = both(small, 5, num_splits=7, part_keys=512, window_left=600)
    assert torch.equal(bits(o), bits(ro)) and torch.equal(bits(l), bits(rl)), "small call after the big one"
    # and the proportional partition again, with fp8 KV, after the two
    f8 = gen.make_case("noalloc_fp8", q_lens=[1, 2], seq_lens=[5000, 9], num_q_heads=8, num_kv_heads=1,
                       head_dim=256, page_size=816, q_kind="f16", kv_kind="e5m2", seed=321, k_scale=0.5, v_scale=2.0)
    (ro, rl), (o, l) = both(f8, 2, num_splits=5)
    assert torch.equal(bits(o), bits(ro)) and torch.equal(bits(l), bits(rl)), "fp8 call"
    assert np.isfinite(o.float().cpu().numpy()).all()


def test_noalloc_decode_rejects_records_past_the_buffer():
    c = gen.make_case("noalloc_too_big", q_lens=[16], seq_lens=[64], num_q_heads=64, num_kv_heads=8,
                      head_dim=256, page_size=16, q_kind="f16", seed=5)
    d = gen.to_device(c)
    parts = 4096  # 16 x 64 x 4096 x 258 x 4 bytes: far more than the buffer
    assert ops.decode_workspace_bytes(c.total_q, c.num_q_heads, c.head_dim, parts) > ops.NOALLOC_SCRATCH_BYTES
    out = torch.zeros_like(d["q"])
    with pytest.raises(ops.PagedAttentionError) as e:
        ops.split_kv_decode_noalloc(d["q"], d["k"], d["v"], d["cu"], d["seq_lens"], d["bt"], 16, c.scale, out,
                                    num_splits=parts)
    assert e.value.status == ops.PA_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(out)) == 0  # nothing was launched
