// Split-KV decode pass 1 (decode_body.h holds the work group's computation):
// the kernel around the body and its launch.

#include "decode_body.h"

namespace pa {

// Head dims up to 128, and fp8 KV at 256 (query fragments in LDS, one ring
// stage per wave: 80 KB), are held to 256 registers so that two groups share a CU.
template <typename QT, int F8, int DPAD, int NSW, bool MOD>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(DPAD <= 128 || F8 != 0 ? 2 : 1)))
void attn_decode_kernel(const AttnParams p) {
  __shared__ __attribute__((aligned(1024))) char smem[decode_lds_bytes<F8, DPAD, NSW>()];
  decode_body<QT, F8, DPAD, NSW, MOD>(p, blockIdx.x, smem);
}

// ---- host side -------------------------------------------------------------

namespace {
template <typename QT, int F8, int DPAD, int NSW>
hipError_t launch_dec(const AttnParams& p, int nblocks, hipStream_t stream) {
  if (has_score_mods(p))
    hipLaunchKernelGGL((attn_decode_kernel<QT, F8, DPAD, NSW, true>), dim3(nblocks), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((attn_decode_kernel<QT, F8, DPAD, NSW, false>), dim3(nblocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}
template <typename QT>
hipError_t launch_dec_d(const AttnParams& p, int dpad, int nblocks, hipStream_t stream) {
  switch (dpad) {
    case 64: return launch_dec<QT, 0, 64, 2>(p, nblocks, stream);
    case 128: return launch_dec<QT, 0, 128, 1>(p, nblocks, stream);
    case 256: return launch_dec<QT, 0, 256, 1>(p, nblocks, stream);
    default: return hipErrorInvalidValue;
  }
}
}  // namespace

// Decode pass 1, 32 rows per group: fp16 / bf16 q with KV of the same dtype
// (kv_kind = q_kind), or fp16 / bf16 q with fp8 KV (E5M2 or E4M3) for head
// dims padded to 256.
hipError_t launch_attn_decode(const AttnParams& p, int q_kind, int kv_kind, int dpad, int nblocks,
                              hipStream_t stream) {
  if (kv_kind == KV_E5M2 || kv_kind == KV_E4M3) {
    if (dpad != 256) return hipErrorInvalidValue;
    if (q_kind == KV_F16)
      return kv_kind == KV_E5M2 ? launch_dec<_Float16, KV_E5M2, 256, 1>(p, nblocks, stream)
                                : launch_dec<_Float16, KV_E4M3, 256, 1>(p, nblocks, stream);
    if (q_kind == KV_BF16)
      return kv_kind == KV_E5M2 ? launch_dec<__bf16, KV_E5M2, 256, 1>(p, nblocks, stream)
                                : launch_dec<__bf16, KV_E4M3, 256, 1>(p, nblocks, stream);
    return hipErrorInvalidValue;
  }
  if (q_kind != kv_kind) return hipErrorInvalidValue;
  if (q_kind == KV_F16) return launch_dec_d<_Float16>(p, dpad, nblocks, stream);
  if (q_kind == KV_BF16) return launch_dec_d<__bf16>(p, dpad, nblocks, stream);
  return hipErrorInvalidValue;
}

int decode_rows_per_group() { return 32; }

}  // namespace pa
