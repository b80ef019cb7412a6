"""fp64 CPU oracle for paged attention over a block-table KV cache.

TEST INFRASTRUCTURE ONLY.  Nothing in the library's product path imports,
calls or links this package.  Only the test suite, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the
HIP path: it reads plain numpy arrays (upcast exactly to float64), gathers the
dense K/V of every sequence through the block table on its own, and evaluates
the definition of softmax attention in float64.

What it computes comes from the pages on this subject:

* InferMatrixLab/vllm-rlt PR #128, "Purpose" (Prefill): a varlen paged prefill
  with cu_seqlens_q, one block table per sequence and bottom-right causal
  alignment, GQA, exact IEEE products for FP32 inputs.
* same page, "Purpose" (Decode): each row's context split into NUM_SPLITS equal,
  tile-aligned parts, FP32 partial softmax states merged in a second kernel, the
  partition a function of the row's own length only.
* 1CatAI/1Cat-vLLM PR #616 (original description, "Purpose"): small-q rows
  (q=1, or an MTP verify row with q=K+1) expanded token-wise into decode rows.
* same page, "Test Result", fp8_e5m2 KV paragraph: KV stored as fp8_e5m2
  bytes and dequantized inside the attention kernels.

Modules:
  fp8        -- e5m2 byte -> value, written from the bit layout of the format.
  attention  -- the numpy fp64 oracle (dense gather, masked softmax, splits,
                merge, work counts).
  brute      -- a pure-Python triple loop for tiny cases, used to pin the
                numpy oracle.
  kv_write   -- the KV write into pages, with the E5M2 quantisation.

Every function here is pinned by ``tests/test_oracle_pins.py`` (brute force,
closed forms, a torch fp64 SDPA cross-check, invariants, planted mistakes).
Parity of results against printed values is unpinned: the pages print no
attention outputs, only timings and error magnitudes.
"""

from .attention import (  # noqa: F401
    dequantize_pool,
    gather_dense_kv,
    visible_key_count,
    window_start,
    window_base,
    add_sink,
    modified_logits,
    attention_rows,
    paged_attention,
    split_ranges,
    split_partials,
    merge_partials,
    attended_pairs,
)
from .fp8 import e4m3_to_float64, e5m2_to_float64  # noqa: F401
from .kv_write import e4m3_encode, e5m2_encode, fp8_encode, quantize_e5m2, quantize_fp8, write_kv  # noqa: F401
from .brute import brute_paged_attention  # noqa: F401
