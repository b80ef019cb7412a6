// Paged attention pass 1 on the vector ALU, in fp32 with exact IEEE products.
//
// The FP32 path of the varlen paged prefill (InferMatrixLab/vllm-rlt PR #128,
// "Purpose", Prefill: exact IEEE products for FP32 inputs) and of pass 1 of
// the split-KV decode.  Every product is an fp32 fused multiply-add, no
// operand is rounded to a narrower type.  It accepts any KV storage type
// (converted to fp32 in LDS) but is dispatched for fp32 only.
//
// One work group = 16 GQA-packed query rows (4 per wave) of one sequence and
// one kv head over one part of the key range; 32-key tiles are gathered through
// the block table into LDS as fp32.  Per row and tile: lane (key k, half h)
// forms half of the dot product q.K_k, the partner lane the other half; the
// wave reduces the max and the sum over the 32 keys; each lane then updates
// DPAD/64 output columns from the tile's probabilities.

#include "pa_common.h"

namespace pa {

namespace {

constexpr int kRowsV = 16;
constexpr int kKTV = 32;
constexpr int kThreadsV = 256;
constexpr float kNegInfV = -__builtin_huge_valf();

template <int KVK> struct KvLoad;
template <> struct KvLoad<KV_F32> {
  static constexpr int esz = 4;
  static __device__ __forceinline__ float4 load4(const char* p) { return *(const float4*)p; }
};
template <> struct KvLoad<KV_F16> {
  static constexpr int esz = 2;
  static __device__ __forceinline__ float4 load4(const char* p) {
    typedef _Float16 h4 __attribute__((ext_vector_type(4)));
    h4 v = *(const h4*)p;
    return make_float4((float)v[0], (float)v[1], (float)v[2], (float)v[3]);
  }
};
template <> struct KvLoad<KV_BF16> {
  static constexpr int esz = 2;
  static __device__ __forceinline__ float4 load4(const char* p) {
    uint2 v = *(const uint2*)p;
    return make_float4(__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xFFFF0000u),
                       __uint_as_float(v.y << 16), __uint_as_float(v.y & 0xFFFF0000u));
  }
};
template <> struct KvLoad<KV_E5M2> {
  static constexpr int esz = 1;
  static __device__ __forceinline__ float4 load4(const char* p) {
    uint32_t x = *(const uint32_t*)p, lo, hi;
    e5m2x4_to_f16x4(x, lo, hi);
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    h2 a = __builtin_bit_cast(h2, lo), b = __builtin_bit_cast(h2, hi);
    return make_float4((float)a[0], (float)a[1], (float)b[0], (float)b[1]);
  }
};

template <typename QT> __device__ __forceinline__ float q_at(const QT* p) { return (float)*p; }
template <> __device__ __forceinline__ float q_at<__bf16>(const __bf16* p) {
  return __uint_as_float(((uint32_t)*(const uint16_t*)p) << 16);
}

template <typename QT> __device__ __forceinline__ void out_store(QT* p, float v) { *p = (QT)v; }

__device__ __forceinline__ float wave_max32(float v) {
#pragma unroll
  for (int o = 16; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum32(float v) {
#pragma unroll
  for (int o = 16; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

}  // namespace

// MOD: softcap / ALiBi score modifiers (mod_score) on every visible score.
template <typename QT, int KVK, int DPAD, bool MOD>
__global__ __launch_bounds__(kThreadsV) void attn_valu_kernel(const AttnParams p) {
  constexpr int KF = DPAD + 1;         // fp32 K row stride in LDS
  constexpr int NC = DPAD / 64;        // output columns per lane
  constexpr int HALF = DPAD / 2;
  constexpr int ESZ = KvLoad<KVK>::esz;
  __shared__ float kf[kKTV * KF];
  __shared__ float vf[kKTV * DPAD];
  __shared__ float qs[kRowsV * DPAD];
  __shared__ float ps[4][4][kKTV];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  WorkItem wi;
  if (!work_of_block(p, blockIdx.x, true, wi)) return;
  // a sequence's last query tiles see the most keys: they are handed out first
  const int qtile = wi.qtile, split = wi.split, kvh = wi.kvh;
  const float score_scale = head_score_scale(p, kvh), out_scale = head_v_scale(p, kvh);
  const int seq = wi.seqpos;

  const int q0 = p.cu_seqlens_q[seq];
  const int qlen = q_end_of(p, seq) - q0;
  const int g = p.group;
  const int nrows = qlen * g;
  const int row0 = qtile * kRowsV;
  if (row0 >= nrows) return;
  const int L = p.seq_lens[seq];
  int klo, khi;
  split_range(p, L, qlen, split, klo, khi);
  klo = window_klo(p, klo, khi, L - qlen + row0 / g);  // first tile: the earliest window start
  const int last_tok = (min(row0 + kRowsV, nrows) - 1) / g;
  const int kend = min(khi, L - qlen + last_tok + 1);

  // queries of the work group -> LDS (fp32)
  for (int e = tid; e < kRowsV * DPAD; e += kThreadsV) {
    const int r = e / DPAD, d = e % DPAD, prow = row0 + r;
    float v = 0.0f;
    if (prow < nrows && d < p.head_dim) {
      const int tok = prow / g, hq = kvh * g + prow % g;
      v = q_at<QT>((const QT*)p.q + ((int64_t)(q0 + tok) * p.num_q_heads + hq) * p.head_dim + d);
    }
    qs[e] = v;
  }

  // this wave's 4 rows
  int lim[4], lo[4], rowtok[4], rowhq[4];
  float slope[4];
  bool rvalid[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int prow = row0 + wave * 4 + i;
    rvalid[i] = prow < nrows;
    rowtok[i] = rvalid[i] ? prow / g : 0;
    rowhq[i] = kvh * g + (rvalid[i] ? prow % g : 0);
    lim[i] = rvalid[i] ? min(L - qlen + rowtok[i] + 1, khi) : 0;
    lo[i] = window_lo(p, L - qlen + rowtok[i]);
    slope[i] = MOD ? alibi_slope_l2(p, rowhq[i]) : 0.0f;
  }
  float m[4], l[4], o[4][NC];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    m[i] = kNegInfV;
    l[i] = 0.0f;
#pragma unroll
    for (int c = 0; c < NC; ++c) o[i][c] = 0.0f;
  }

  const int P = p.page_size;
  const int* bt = p.block_tables + (int64_t)seq * p.max_pages;
  const char* kbase = (const char*)p.k_pages + (int64_t)kvh * p.stride_head * ESZ;
  const char* vbase = (const char*)p.v_pages + (int64_t)kvh * p.stride_head * ESZ;
  const int key = lane & 31, half = lane >> 5;

  for (int j0 = klo; j0 < kend; j0 += kKTV) {
    __syncthreads();  // previous tile fully consumed (and qs written)
    for (int e = tid; e < kKTV * (DPAD / 4); e += kThreadsV) {
      const int kr = e / (DPAD / 4), d = (e % (DPAD / 4)) * 4;
      const int j = j0 + kr;
      float4 kv = make_float4(0, 0, 0, 0), vv = make_float4(0, 0, 0, 0);
      if (j < kend && d < p.head_dim) {
        const int64_t off = (int64_t)bt[j / P] * p.stride_page + (int64_t)(j % P) * p.stride_token + d;
        kv = KvLoad<KVK>::load4(kbase + off * ESZ);
        vv = KvLoad<KVK>::load4(vbase + off * ESZ);
      }
      float* kd = &kf[kr * KF + d];
      kd[0] = kv.x; kd[1] = kv.y; kd[2] = kv.z; kd[3] = kv.w;
      *(float4*)&vf[kr * DPAD + d] = vv;
    }
    __syncthreads();

#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float* qr = &qs[(wave * 4 + i) * DPAD + half * HALF];
      const float* kr = &kf[key * KF + half * HALF];
      float dot = 0.0f;
#pragma unroll 8
      for (int d = 0; d < HALF; ++d) dot = fmaf(qr[d], kr[d], dot);
      dot += __shfl_xor(dot, 32);
      float s = (j0 + key < lim[i] && j0 + key >= lo[i]) ? dot * score_scale : kNegInfV;
      if constexpr (MOD)
        if (s != kNegInfV) s = mod_score(p, s, slope[i], L - qlen + rowtok[i] - (j0 + key));
      const float tmax = wave_max32(s);
      const float mnew = fmaxf(m[i], tmax);
      const float alpha = mnew == kNegInfV ? 1.0f : exp2f(m[i] - mnew);
      const float pr = mnew == kNegInfV ? 0.0f : exp2f(s - mnew);
      l[i] = l[i] * alpha + wave_sum32(pr);
      m[i] = mnew;
      if (half == 0) ps[wave][i][key] = pr;
      __builtin_amdgcn_s_waitcnt(0xc07f);  // LDS writes of this wave visible to its own reads
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int d = lane + 64 * c;
        float acc = o[i][c] * alpha;
#pragma unroll 8
        for (int k = 0; k < kKTV; ++k) acc = fmaf(ps[wave][i][k], vf[k * DPAD + d], acc);
        o[i][c] = acc;
      }
      __builtin_amdgcn_wave_barrier();
    }
  }

  // epilogue
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (!rvalid[i]) continue;
    float inv, lse_nat;
    final_row(p.write_partial ? nullptr : p.sinks, rowhq[i], m[i], l[i], out_scale, inv, lse_nat);
    const int64_t rowidx = (int64_t)(q0 + rowtok[i]) * p.num_q_heads + rowhq[i];
    if (p.write_partial) {
      float* rec = p.partial + (rowidx * p.num_splits + split) * (int64_t)(p.head_dim + 2);
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int d = lane + 64 * c;
        if (d < p.head_dim) rec[d] = o[i][c] * inv;
      }
      if (lane == 0) {
        rec[p.head_dim] = lse_nat;
        rec[p.head_dim + 1] = 0.0f;
      }
    } else {
      QT* orow = (QT*)p.out + rowidx * p.head_dim;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int d = lane + 64 * c;
        if (d < p.head_dim) out_store<QT>(orow + d, o[i][c] * inv);
      }
      if (p.lse != nullptr && lane == 0) p.lse[rowidx] = lse_nat;
    }
  }
}

template <typename QT, int KVK, int DPAD>
static hipError_t launch_v(const AttnParams& p, int nblocks, hipStream_t stream) {
  if (has_score_mods(p))
    hipLaunchKernelGGL((attn_valu_kernel<QT, KVK, DPAD, true>), dim3(nblocks), dim3(kThreadsV), 0, stream, p);
  else
    hipLaunchKernelGGL((attn_valu_kernel<QT, KVK, DPAD, false>), dim3(nblocks), dim3(kThreadsV), 0, stream, p);
  return hipGetLastError();
}

// fp32 q with fp32 KV (the exact-product path).
hipError_t launch_attn_valu(const AttnParams& p, int q_kind, int kv_kind, int dpad, int nblocks,
                            hipStream_t stream) {
  if (q_kind != KV_F32 || kv_kind != KV_F32) return hipErrorInvalidValue;
  switch (dpad) {
    case 64: return launch_v<float, KV_F32, 64>(p, nblocks, stream);
    case 128: return launch_v<float, KV_F32, 128>(p, nblocks, stream);
    case 256: return launch_v<float, KV_F32, 256>(p, nblocks, stream);
    default: return hipErrorInvalidValue;
  }
}

int valu_rows_per_group() { return kRowsV; }

}  // namespace pa
