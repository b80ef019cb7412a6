// One attention launch for a mixed step (1CatAI/1Cat-vLLM PR #1279: a step
// that carries prefill chunks next to decode and MTP verify rows; the small-q
// rows take the split-KV decode path and the chunks the prefill kernel).
//
// The grid is the prefill grid of the chunk sequences followed by the decode
// grid of the small-q rows, each planned exactly as for its own call (the
// same work items, parts and XCD mapping: the prefill block count is a
// multiple of 8, so a decode group keeps its XCD).  A work group runs the
// prefill body (prefill_w4_body.h) or the decode body (decode_body.h) on one
// LDS buffer as large as the larger of the two, so every result has the bits
// of the separate calls.  Prefill groups come first: they are long, and the
// short, HBM-bound decode groups fill the compute units that the prefill's
// last wave leaves idle.  Head dims padded to 256, where both bodies run 256
// threads with one group per compute unit.

#include "decode_body.h"
#include "prefill_w4_body.h"

namespace pa {

template <typename QT, int F8, int NST, int NSW, int VAR>
__global__ __launch_bounds__(256, 1) void attn_mixed_kernel(const AttnParams pp, const AttnParams pd,
                                                            int prefill_blocks) {
  constexpr int kPre = prefill_w4_lds_bytes<F8, 256, NST>();
  constexpr int kDec = decode_lds_bytes<F8, 256, NSW>();
  __shared__ __attribute__((aligned(1024))) char smem[kPre > kDec ? kPre : kDec];
  const int bid = blockIdx.x;
  if (bid < prefill_blocks)
    prefill_w4_body<QT, F8, 256, NST, VAR>(pp, bid, smem);
  else
    decode_body<QT, F8, 256, NSW, VAR == 2>(pd, bid - prefill_blocks, smem);
}

namespace {
// Only the default instantiation (VAR 0: no window, no score modifiers) is
// fused: with a window or modifiers both bodies' extra state in one register
// allocation spills inside the prefill tile loop, and the fused grid ran
// 15-57 % slower than the two kernels back to back.
template <typename QT, int F8, int NST, int NSW>
hipError_t launch_mixed(const AttnParams& pp, const AttnParams& pd, int prefill_blocks, int decode_blocks,
                        hipStream_t stream) {
  if (has_score_mods(pp) || pp.window_left >= 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL((attn_mixed_kernel<QT, F8, NST, NSW, 0>), dim3(prefill_blocks + decode_blocks), dim3(256), 0,
                     stream, pp, pd, prefill_blocks);
  return hipGetLastError();
}
}  // namespace

// Both segments at head dims padded to 256: fp16 / bf16 q with KV of the same
// dtype, or fp16 / bf16 q with fp8 KV (E5M2 or E4M3).  The ring depths are those of
// the separate kernels.
hipError_t launch_attn_mixed(const AttnParams& pp, const AttnParams& pd, int q_kind, int kv_kind, int dpad,
                             int prefill_blocks, int decode_blocks, hipStream_t stream) {
  if (dpad != 256 || (prefill_blocks & 7) != 0) return hipErrorInvalidValue;
  if (q_kind == KV_F16 && kv_kind == KV_E5M2)
    return launch_mixed<_Float16, KV_E5M2, 8, 2>(pp, pd, prefill_blocks, decode_blocks, stream);
  if (q_kind == KV_F16 && kv_kind == KV_E4M3)
    return launch_mixed<_Float16, KV_E4M3, 8, 2>(pp, pd, prefill_blocks, decode_blocks, stream);
  if (q_kind == KV_BF16 && kv_kind == KV_E5M2)
    return launch_mixed<__bf16, KV_E5M2, 8, 2>(pp, pd, prefill_blocks, decode_blocks, stream);
  if (q_kind == KV_BF16 && kv_kind == KV_E4M3)
    return launch_mixed<__bf16, KV_E4M3, 8, 2>(pp, pd, prefill_blocks, decode_blocks, stream);
  if (q_kind == KV_F16 && kv_kind == KV_F16)
    return launch_mixed<_Float16, 0, 4, 1>(pp, pd, prefill_blocks, decode_blocks, stream);
  if (q_kind == KV_BF16 && kv_kind == KV_BF16)
    return launch_mixed<__bf16, 0, 4, 1>(pp, pd, prefill_blocks, decode_blocks, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
