// Merge of FP32 partial softmax states: the second pass of split-KV
// (InferMatrixLab/vllm-rlt PR #128, "Purpose", Decode; also the log-sum-exp
// merge of key-split prefill tiles, 1CatAI/1Cat-vLLM PR #1279, commit 5).
//
// Rows with 16 or more parts (a long decode row): one work group of 1024
// threads per (token, head), so that each thread reads at most a few parts and
// the pass costs about one memory round trip.  Fewer parts: one wave per row
// (merge_rows_kernel below).  Record s = (o_s[0..D),
// lse_s, pad) with o_s normalised.  M = max_s lse_s; w_s = exp(lse_s - M);
// o = sum_s w_s o_s / sum_s w_s; lse = M + log sum_s w_s.  All parts empty ->
// o = 0, lse = -inf; an empty part's o_s is never read into the sum.  With
// sinks, head h's sinks[h] joins as a logit with no value: M includes it and
// the denominator gains exp(sinks[h] - M), once per row.
//
// Thread t owns a pair of output columns (t % (D/2)) and a run of parts
// (t / (D/2)): a contiguous run, or every SG-th part for absolute parts; each
// run is summed in ascending part order and the runs are combined in
// ascending run order.  The order depends only on S and D (the
// kernel is a function of S), so a
// row's result does not depend on the other rows of the call (batch
// invariance), and the many parts of a long decode row are read in parallel.

#include "pa_common.h"

namespace pa {

namespace {
constexpr float kNegInfM = -__builtin_huge_valf();
constexpr float kLog2e = 1.4426950408889634f;

// Output row of record row `row` (token row / H, head row % H): the same row,
// or, with a token map (a routed call's compact tokens -> batch tokens), the
// mapped token's; -1 for a compact token the map leaves out.
__device__ __forceinline__ int64_t out_row(const int* tok_map, int64_t row, int H) {
  if (tok_map == nullptr) return row;
  const int g = tok_map[row / H];
  return g < 0 ? -1 : (int64_t)g * H + row % H;
}

template <typename OT> __device__ __forceinline__ void put2(OT* p, float a, float b) {
  p[0] = (OT)a;
  p[1] = (OT)b;
}
}  // namespace

// STRIDED: part s goes to run s % SG instead of to a contiguous run, so the
// association of the sums is a function of the part index and D alone; empty
// trailing parts add exact zeros, and a row cut into absolute parts gives the
// same bits whatever the part count of the call.
template <typename OT, int kMT, bool STRIDED>
__global__ __launch_bounds__(kMT) void merge_kernel(const float* __restrict__ partials, int S, int D,
                                                    OT* __restrict__ out, float* __restrict__ out_lse,
                                                    const float* __restrict__ sinks, int H,
                                                    const int* __restrict__ tok_map) {
  constexpr int NW = kMT / 64;
  __shared__ float red[NW];
  __shared__ float2 part[kMT];
  __shared__ float dpart[kMT];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int64_t row = blockIdx.x;
  const int64_t orow = out_row(tok_map, row, H);
  if (orow < 0) return;  // (uniform: one row per work group)
  const int R = D + 2;
  const float* rec = partials + row * (int64_t)S * R;

  // M = max_s lse_s
  float M = kNegInfM;
  for (int s = t; s < S; s += kMT) M = fmaxf(M, rec[(int64_t)s * R + D]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  if (lane == 0) red[wave] = M;
  __syncthreads();
  M = red[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) M = fmaxf(M, red[i]);
  // a sink is one more logit with no value, counted once per row
  const float sk = sinks ? sinks[row % H] : kNegInfM;
  M = fmaxf(M, sk);

  const int DC = D >> 1;                 // float2 column pairs
  const int SG = kMT / DC;               // runs of parts (>= 2 since D / 2 <= 128)
  const int dc = t % DC, sg = t / DC;
  const int per = STRIDED ? SG : (S + SG - 1) / SG;
  const int s0 = STRIDED ? sg : sg * per, s1 = STRIDED ? S : min(S, s0 + per), ds = STRIDED ? SG : 1;
  float ax = 0.0f, ay = 0.0f, den = 0.0f;
  if (M != kNegInfM && sg < SG) {
#pragma unroll 8
    for (int s = s0; s < s1; s += ds) {
      const float* r = rec + (int64_t)s * R;
      const float ls = r[D];
      const float2 v = *(const float2*)(r + 2 * dc);
      const bool live = ls != kNegInfM;
      const float ws = live ? exp2f((ls - M) * kLog2e) : 0.0f;
      ax = live ? fmaf(ws, v.x, ax) : ax;
      ay = live ? fmaf(ws, v.y, ay) : ay;
      den += ws;
    }
  }
  part[t] = make_float2(ax, ay);
  dpart[t] = den;
  __syncthreads();
  if (t < DC) {
    float sx = 0.0f, sy = 0.0f, sd = 0.0f;
    for (int gI = 0; gI < SG; ++gI) {
      const float2 v = part[gI * DC + t];
      sx += v.x;
      sy += v.y;
      sd += dpart[gI * DC];  // every thread of a run holds the same den
    }
    if (sk != kNegInfM) sd += exp2f((sk - M) * kLog2e);
    const bool empty = M == kNegInfM || !(sd > 0.0f);
    const float inv = empty ? 0.0f : 1.0f / sd;
    put2<OT>(out + orow * D + 2 * t, sx * inv, sy * inv);
    if (out_lse != nullptr && t == 0) out_lse[orow] = empty ? kNegInfM : M + logf(sd);
  }
}

// Few parts (S < 16, e.g. a key-split prefill): one wave per (token, head),
// four rows per work group; lane l owns column pairs l, l + 64, ... and walks
// the S parts in ascending order.  One read of every record byte, no LDS, no
// barrier: a prefill with many rows and two to four parts is bound by HBM
// instead of by work-group launches.
template <typename OT>
__global__ __launch_bounds__(256) void merge_rows_kernel(const float* __restrict__ partials, int S, int D,
                                                         int64_t rows, OT* __restrict__ out,
                                                         float* __restrict__ out_lse,
                                                         const float* __restrict__ sinks, int H,
                                                         const int* __restrict__ tok_map) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int64_t orow = out_row(tok_map, row, H);
  if (orow < 0) return;
  const int R = D + 2;
  const float* rec = partials + row * (int64_t)S * R;
  float M = kNegInfM;
#pragma unroll 4
  for (int s = 0; s < S; ++s) M = fmaxf(M, rec[(int64_t)s * R + D]);
  const float sk = sinks ? sinks[row % H] : kNegInfM;  // one more logit with no value
  M = fmaxf(M, sk);
  const int DC = D >> 1;
  for (int dc = lane; dc < DC; dc += 64) {
    float ax = 0.0f, ay = 0.0f, den = 0.0f;
    if (M != kNegInfM) {
#pragma unroll 4
      for (int s = 0; s < S; ++s) {
        const float* r = rec + (int64_t)s * R;
        const float ls = r[D];
        const float2 v = *(const float2*)(r + 2 * dc);
        const bool live = ls != kNegInfM;
        const float ws = live ? exp2f((ls - M) * kLog2e) : 0.0f;
        ax = live ? fmaf(ws, v.x, ax) : ax;
        ay = live ? fmaf(ws, v.y, ay) : ay;
        den += ws;
      }
      if (sk != kNegInfM) den += exp2f((sk - M) * kLog2e);
    }
    const bool empty = M == kNegInfM || !(den > 0.0f);
    const float inv = empty ? 0.0f : 1.0f / den;
    put2<OT>(out + orow * D + 2 * dc, ax * inv, ay * inv);
    if (out_lse != nullptr && dc == 0) out_lse[orow] = empty ? kNegInfM : M + logf(den);
  }
}

template <typename OT>
static hipError_t launch_m(const float* partials, int S, int ntok, int H, int D, void* out, float* out_lse,
                           bool strided, const float* sinks, const int* tok_map, hipStream_t stream) {
  const int64_t rows = (int64_t)ntok * H;
  if (rows == 0) return hipSuccess;
  if (strided)
    hipLaunchKernelGGL((merge_kernel<OT, 1024, true>), dim3((unsigned)rows), dim3(1024), 0, stream, partials, S, D,
                       (OT*)out, out_lse, sinks, H, tok_map);
  else if (S >= 16)
    hipLaunchKernelGGL((merge_kernel<OT, 1024, false>), dim3((unsigned)rows), dim3(1024), 0, stream, partials, S, D,
                       (OT*)out, out_lse, sinks, H, tok_map);
  else
    hipLaunchKernelGGL((merge_rows_kernel<OT>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream, partials, S,
                       D, rows, (OT*)out, out_lse, sinks, H, tok_map);
  return hipGetLastError();
}

hipError_t launch_merge(const float* partials, int S, int ntok, int H, int D, void* out, int out_kind,
                        float* out_lse, bool strided, const float* sinks, const int* tok_map, hipStream_t stream) {
  switch (out_kind) {
    case KV_F32: return launch_m<float>(partials, S, ntok, H, D, out, out_lse, strided, sinks, tok_map, stream);
    case KV_F16: return launch_m<_Float16>(partials, S, ntok, H, D, out, out_lse, strided, sinks, tok_map, stream);
    case KV_BF16: return launch_m<__bf16>(partials, S, ntok, H, D, out, out_lse, strided, sinks, tok_map, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
