// Paged attention pass 1 for head dims padded to 256 (prefill_w4_body.h holds
// the work group's computation): the kernel around the body and its launch.

#include "prefill_w4_body.h"

namespace pa {

template <typename QT, int F8, int DPAD, int NST, int VAR>
__global__ __launch_bounds__(256, 1) void attn_prefill_w4_kernel(const AttnParams p) {
  __shared__ __attribute__((aligned(1024))) char smem[prefill_w4_lds_bytes<F8, DPAD, NST>()];
  prefill_w4_body<QT, F8, DPAD, NST, VAR>(p, blockIdx.x, smem);
}

// ---- host side -------------------------------------------------------------

namespace {
template <typename QT, int F8, int DPAD, int NST>
hipError_t launch_w4(const AttnParams& p, int nblocks, hipStream_t stream) {
  const bool cap = p.softcap_k2 != 0.0f, alibi = p.alibi_slopes != nullptr;
  if (cap && alibi)
    hipLaunchKernelGGL((attn_prefill_w4_kernel<QT, F8, DPAD, NST, 4>), dim3(nblocks), dim3(256), 0, stream, p);
  else if (alibi)
    hipLaunchKernelGGL((attn_prefill_w4_kernel<QT, F8, DPAD, NST, 3>), dim3(nblocks), dim3(256), 0, stream, p);
  else if (cap)
    hipLaunchKernelGGL((attn_prefill_w4_kernel<QT, F8, DPAD, NST, 2>), dim3(nblocks), dim3(256), 0, stream, p);
  else if (p.window_left >= 0)
    hipLaunchKernelGGL((attn_prefill_w4_kernel<QT, F8, DPAD, NST, 1>), dim3(nblocks), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((attn_prefill_w4_kernel<QT, F8, DPAD, NST, 0>), dim3(nblocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}
}  // namespace

// Prefill pass 1, head dims padded to 256, 256 query rows per work group:
// fp16 / bf16 q with KV of the same dtype (kv_kind = q_kind), or fp16 / bf16 q
// with fp8 KV (kv_kind = KV_E5M2 or KV_E4M3).
hipError_t launch_attn_prefill_w4(const AttnParams& p, int q_kind, int kv_kind, int dpad, int nblocks,
                                  hipStream_t stream) {
  if (dpad != 256) return hipErrorInvalidValue;
  if (q_kind == KV_F16 && kv_kind == KV_E5M2) return launch_w4<_Float16, KV_E5M2, 256, 8>(p, nblocks, stream);
  if (q_kind == KV_F16 && kv_kind == KV_E4M3) return launch_w4<_Float16, KV_E4M3, 256, 8>(p, nblocks, stream);
  if (q_kind == KV_BF16 && kv_kind == KV_E5M2) return launch_w4<__bf16, KV_E5M2, 256, 8>(p, nblocks, stream);
  if (q_kind == KV_BF16 && kv_kind == KV_E4M3) return launch_w4<__bf16, KV_E4M3, 256, 8>(p, nblocks, stream);
  if (q_kind == KV_F16 && kv_kind == KV_F16) return launch_w4<_Float16, 0, 256, 4>(p, nblocks, stream);
  if (q_kind == KV_BF16 && kv_kind == KV_BF16) return launch_w4<__bf16, 0, 256, 4>(p, nblocks, stream);
  return hipErrorInvalidValue;
}

hipError_t prefill_w4_occupancy(int q_kind, int dpad, int* blocks_per_cu) {
  (void)q_kind;
  if (dpad == 256)
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu,
                                                        attn_prefill_w4_kernel<_Float16, 0, 256, 4, 0>, 256, 0);
  return hipErrorInvalidValue;
}

}  // namespace pa
