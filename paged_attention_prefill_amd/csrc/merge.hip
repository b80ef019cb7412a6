// Merge of FP32 partial softmax states: the second pass of split-KV
// (InferMatrixLab/vllm-rlt PR #128, "Purpose", Decode; also the log-sum-exp
// merge of key-split prefill tiles, 1CatAI/1Cat-vLLM PR #1279, commit 5).
//
// One wave per (token, head).  Record s = (o_s[0..D), lse_s, pad) with o_s
// normalised.  M = max_s lse_s; w_s = exp(lse_s - M); o = sum_s w_s o_s /
// sum_s w_s, summed in ascending s for every output column, so a row's result
// depends only on its own records (batch invariance).  All parts empty ->
// o = 0, lse = -inf.

#include "pa_common.h"

namespace pa {

namespace {
constexpr int kMergeWaves = 4;
constexpr float kNegInfM = -__builtin_huge_valf();
constexpr float kLog2e = 1.4426950408889634f;

template <typename OT> __device__ __forceinline__ void put(OT* p, float v) { *p = (OT)v; }
}  // namespace

template <typename OT, int NCOL>
__global__ __launch_bounds__(64 * kMergeWaves) void merge_kernel(const float* __restrict__ partials,
                                                                 int S, int ntok, int H, int D,
                                                                 OT* __restrict__ out,
                                                                 float* __restrict__ out_lse) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kMergeWaves + (threadIdx.x >> 6);
  if (row >= (int64_t)ntok * H) return;
  const int R = D + 2;
  const float* rec = partials + row * (int64_t)S * R;

  float M = kNegInfM;
  for (int s = lane; s < S; s += 64) M = fmaxf(M, rec[(int64_t)s * R + D]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));

  float acc[NCOL];
#pragma unroll
  for (int c = 0; c < NCOL; ++c) acc[c] = 0.0f;
  float den = 0.0f;
  if (M != kNegInfM) {
    for (int s = 0; s < S; ++s) {
      const float* r = rec + (int64_t)s * R;
      const float ls = r[D];
      if (ls == kNegInfM) continue;  // empty part: contributes nothing
      const float ws = exp2f((ls - M) * kLog2e);
      den += ws;
#pragma unroll
      for (int c = 0; c < NCOL; ++c) {
        const int d = lane + 64 * c;
        if (d < D) acc[c] = fmaf(ws, r[d], acc[c]);
      }
    }
  }
  const bool empty = M == kNegInfM || !(den > 0.0f);
  const float inv = empty ? 0.0f : 1.0f / den;
  OT* orow = out + row * D;
#pragma unroll
  for (int c = 0; c < NCOL; ++c) {
    const int d = lane + 64 * c;
    if (d < D) put<OT>(orow + d, acc[c] * inv);
  }
  if (out_lse != nullptr && lane == 0) out_lse[row] = empty ? kNegInfM : M + logf(den);
}

template <typename OT>
static hipError_t launch_m(const float* partials, int S, int ntok, int H, int D, void* out,
                           float* out_lse, hipStream_t stream) {
  const int64_t rows = (int64_t)ntok * H;
  const int nblk = (int)((rows + kMergeWaves - 1) / kMergeWaves);
  if (nblk == 0) return hipSuccess;
  if (D <= 64)
    hipLaunchKernelGGL((merge_kernel<OT, 1>), dim3(nblk), dim3(64 * kMergeWaves), 0, stream, partials, S, ntok, H, D, (OT*)out, out_lse);
  else if (D <= 128)
    hipLaunchKernelGGL((merge_kernel<OT, 2>), dim3(nblk), dim3(64 * kMergeWaves), 0, stream, partials, S, ntok, H, D, (OT*)out, out_lse);
  else
    hipLaunchKernelGGL((merge_kernel<OT, 4>), dim3(nblk), dim3(64 * kMergeWaves), 0, stream, partials, S, ntok, H, D, (OT*)out, out_lse);
  return hipGetLastError();
}

hipError_t launch_merge(const float* partials, int S, int ntok, int H, int D, void* out, int out_kind,
                        float* out_lse, hipStream_t stream) {
  switch (out_kind) {
    case KV_F32: return launch_m<float>(partials, S, ntok, H, D, out, out_lse, stream);
    case KV_F16: return launch_m<_Float16>(partials, S, ntok, H, D, out, out_lse, stream);
    case KV_BF16: return launch_m<__bf16>(partials, S, ntok, H, D, out, out_lse, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
