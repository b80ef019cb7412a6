// Paged attention pass 1 on MFMA (fp16 / bf16 queries; fp16, bf16 or fp8 E5M2 / E4M3 KV).
//
// One work group = 128 GQA-packed query rows (packed row r of a sequence is
// query token r / g, query head kv_head * g + r % g) of one sequence and one
// kv head, over one part of the key range.  It is the same kernel for the
// varlen prefill (InferMatrixLab/vllm-rlt PR #128, "Purpose", Prefill) and for
// pass 1 of the split-KV decode (same section, Decode): a decode row is a
// sequence with q <= 16 tokens whose keys are cut into parts.
//
// Per 32-key tile:
//   * K and V of the tile are gathered through the block table (key j is slot
//     j % P of page block_tables[b][j / P]) into LDS, double buffered: the
//     next tile's global loads are in flight in registers while the current
//     tile computes (the register-staged prefetch of 1CatAI/1Cat-vLLM PR #1279,
//     commit 1).  V is written transposed so that it can feed the MFMA.
//   * S^T = K Q^T with v_mfma_f32_32x32x16 (each lane then owns one query row
//     and 16 of the 32 keys), scale, bottom-right causal mask by select;
//   * online softmax: row max = 16 local values + the partner lane (lane^32);
//     the running max is only moved when a tile's max exceeds it by more than
//     2^8 (exponentials stay <= 256), so the O rescale is rare;
//   * O^T += V^T P^T with the same MFMA; P is rounded to the q dtype.
// Epilogue: O / l -> out (q dtype) and lse, or an FP32 partial record
// (o normalised, lse, pad) per (token, q head, part).

#include "pa_common.h"

namespace pa {

namespace {

constexpr int kRows = 128;     // packed query rows per work group
constexpr int kKT = 32;        // keys per tile
constexpr int kThreads = 256;  // 4 waves of 64
constexpr float kTau = 8.0f;   // lazy-rescale threshold (log2 units)
constexpr float kNegInf = -__builtin_huge_valf();

template <typename QT> struct Mfma;
template <> struct Mfma<_Float16> {
  static __device__ __forceinline__ f32x16_t run(uint4 a, uint4 b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8_t, a),
                                                  __builtin_bit_cast(half8_t, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack2(float a, float b) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    h2 v = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, v);
  }
  static __device__ __forceinline__ void store4(void* dst, float a, float b, float c, float d) {
    uint2 v = {pack2(a, b), pack2(c, d)};
    *(uint2*)dst = v;
  }
};
template <> struct Mfma<__bf16> {
  static __device__ __forceinline__ f32x16_t run(uint4 a, uint4 b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack2(float a, float b) {
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    b2 v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
  }
  static __device__ __forceinline__ void store4(void* dst, float a, float b, float c, float d) {
    uint2 v = {pack2(a, b), pack2(c, d)};
    *(uint2*)dst = v;
  }
};

// Raw 8-element chunk of the KV storage type.
template <int KVK> struct Chunk { typedef uint4 raw; };
template <> struct Chunk<KV_E5M2> { typedef uint2 raw; };
template <> struct Chunk<KV_E4M3> { typedef uint2 raw; };

// Eight KV elements -> eight values of the compute type QT (exact for fp8).
template <typename QT, int KVK>
__device__ __forceinline__ uint4 to_compute(typename Chunk<KVK>::raw x) {
  if constexpr ((KVK == KV_E5M2 || KVK == KV_E4M3) && __is_same(QT, __bf16)) {
    return make_uint4(fp8x2_to_bf16x2<KVK, false>(x.x), fp8x2_to_bf16x2<KVK, true>(x.x),
                      fp8x2_to_bf16x2<KVK, false>(x.y), fp8x2_to_bf16x2<KVK, true>(x.y));
  } else if constexpr (KVK == KV_E5M2) {
    uint4 r;
    e5m2x4_to_f16x4(x.x, r.x, r.y);
    e5m2x4_to_f16x4(x.y, r.z, r.w);
    return r;
  } else if constexpr (KVK == KV_E4M3) {
    return make_uint4(e4m3x2_to_f16x2<false>(x.x), e4m3x2_to_f16x2<true>(x.x), e4m3x2_to_f16x2<false>(x.y),
                      e4m3x2_to_f16x2<true>(x.y));
  } else {
    return x;
  }
}

// Position of key quad q (keys 4q..4q+3 of a tile) inside a transposed V row:
// the order in which the P^T operand of the PV product holds the keys.
__device__ __forceinline__ int vt_pos(int quad) {
  return 16 * (quad >> 2) + 8 * (quad & 1) + 4 * ((quad >> 1) & 1);
}

}  // namespace

// MOD: softcap / ALiBi score modifiers (mod_score) on every visible score.
template <typename QT, int KVK, int DPAD, bool MOD = false>
__global__ __launch_bounds__(kThreads) void attn_mfma_kernel(const AttnParams p) {
  constexpr int KS = DPAD + 8;     // K row stride in LDS (16-bit elements)
  constexpr int VS = kKT + 8;      // transposed V row stride
  constexpr int NKK = DPAD / 16;   // k-steps of S^T = K Q^T
  constexpr int NDB = DPAD / 32;   // 32-wide d blocks of O^T
  constexpr int CPK = DPAD / 8;    // 8-element chunks per key row
  constexpr int KPASS = CPK / 8;   // K chunks each thread loads per tile
  constexpr int KKEYS = kThreads / CPK;  // keys per K pass
  constexpr int ESZ = (KVK == KV_E5M2 || KVK == KV_E4M3) ? 1 : 2;
  typedef typename Chunk<KVK>::raw Raw;

  __shared__ __attribute__((aligned(16))) uint16_t k_lds[2][kKT * KS];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[2][DPAD * VS];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int hi = lane >> 5, r32 = lane & 31;

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
  const int row0 = qtile * kRows;
  if (row0 >= nrows) return;
  const int L = p.seq_lens[seq];
  int klo, khi;
  split_range(p, L, qlen, split, klo, khi);
  klo = window_klo(p, klo, khi, L - qlen + row0 / g);  // first tile: the earliest window start

  const int prow = row0 + wave * 32 + r32;
  const bool valid = prow < nrows;
  const int tok = valid ? prow / g : 0;
  const int hq = kvh * g + (valid ? prow - (prow / g) * g : 0);
  const int lim = valid ? min(L - qlen + tok + 1, khi) : 0;
  const int lo = window_lo(p, L - qlen + tok);
  const float slope = MOD ? alibi_slope_l2(p, hq) : 0.0f;
  const int last_tok = (min(row0 + kRows, nrows) - 1) / g;
  const int kend = min(khi, L - qlen + last_tok + 1);
  const int wrow_first = row0 + wave * 32;
  const bool wave_active = wrow_first < nrows;
  const int wave_kend =
      wave_active ? min(khi, L - qlen + (min(wrow_first + 32, nrows) - 1) / g + 1) : 0;

  // ---- Q^T fragments (B operand): lane holds row r32, d = 16 kk + 8 hi .. +7
  uint4 qf[NKK];
  {
    const QT* qrow = (const QT*)p.q + ((int64_t)(q0 + tok) * p.num_q_heads + hq) * p.head_dim;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const int d = kk * 16 + hi * 8;
      qf[kk] = (valid && d < p.head_dim) ? *(const uint4*)(qrow + d) : make_uint4(0, 0, 0, 0);
    }
  }

  f32x16_t oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = (f32x16_t)(0.0f);
  float m = kNegInf, lsum = 0.0f;

  const int ntiles = kend > klo ? (kend - klo + kKT - 1) / kKT : 0;
  const int P = p.page_size;
  const int* bt = p.block_tables + (int64_t)seq * p.max_pages;
  const char* kbase = (const char*)p.k_pages + (int64_t)kvh * p.stride_head * ESZ;
  const char* vbase = (const char*)p.v_pages + (int64_t)kvh * p.stride_head * ESZ;

  // per-thread load roles
  const int kc = tid % CPK, kkey0 = tid / CPK;            // K: chunk, first key
  const int vquad = tid & 7, vc = tid >> 3;               // V: key quad, chunk
  const bool v_loader = vc < CPK;

  Raw kst[KPASS], vst[4];

  auto load_tile = [&](int it) {
    const int j0 = klo + it * kKT;
    const int pg = j0 / P, off = j0 - pg * P;
    const int first_n = P - off;  // keys of this tile on the first page (multiple of 16)
    const int page_a = bt[pg];
    const int page_b = (first_n < kKT && (pg + 1) * P < kend) ? bt[pg + 1] : page_a;
    auto key_off = [&](int kr) -> int64_t {
      const int page = kr < first_n ? page_a : page_b;
      const int slot = kr < first_n ? off + kr : kr - first_n;
      return (int64_t)page * p.stride_page + (int64_t)slot * p.stride_token;
    };
#pragma unroll
    for (int ps = 0; ps < KPASS; ++ps) {
      const int kr = kkey0 + ps * KKEYS;
      const int d = kc * 8;
      Raw x = {};
      if (j0 + kr < kend && d < p.head_dim) x = *(const Raw*)(kbase + (key_off(kr) + d) * ESZ);
      kst[ps] = x;
    }
    if (v_loader) {
      const int d = vc * 8;
      const int64_t o0 = key_off(vquad * 4);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        Raw x = {};
        if (j0 + vquad * 4 + c < kend && d < p.head_dim)
          x = *(const Raw*)(vbase + (o0 + (int64_t)c * p.stride_token + d) * ESZ);
        vst[c] = x;
      }
    }
  };

  auto store_tile = [&](int buf) {
#pragma unroll
    for (int ps = 0; ps < KPASS; ++ps) {
      const int kr = kkey0 + ps * KKEYS;
      *(uint4*)&k_lds[buf][kr * KS + kc * 8] = to_compute<QT, KVK>(kst[ps]);
    }
    if (v_loader) {
      uint4 x0 = to_compute<QT, KVK>(vst[0]), x1 = to_compute<QT, KVK>(vst[1]);
      uint4 x2 = to_compute<QT, KVK>(vst[2]), x3 = to_compute<QT, KVK>(vst[3]);
      const uint32_t a0[4] = {x0.x, x0.y, x0.z, x0.w}, a1[4] = {x1.x, x1.y, x1.z, x1.w};
      const uint32_t a2[4] = {x2.x, x2.y, x2.z, x2.w}, a3[4] = {x3.x, x3.y, x3.z, x3.w};
      uint16_t* dst = &v_lds[buf][(vc * 8) * VS + vt_pos(vquad)];
#pragma unroll
      for (int dd = 0; dd < 8; ++dd) {
        const int wi = dd >> 1, sh = (dd & 1) * 16;
        uint2 v;
        v.x = ((a0[wi] >> sh) & 0xFFFFu) | (((a1[wi] >> sh) & 0xFFFFu) << 16);
        v.y = ((a2[wi] >> sh) & 0xFFFFu) | (((a3[wi] >> sh) & 0xFFFFu) << 16);
        *(uint2*)(dst + dd * VS) = v;
      }
    }
  };

  auto compute = [&](int buf, int j0) {
    if (!wave_active || j0 >= wave_kend) return;
    f32x16_t s = (f32x16_t)(0.0f);
    const uint16_t* kl = &k_lds[buf][r32 * KS + hi * 8];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) s = Mfma<QT>::run(*(const uint4*)(kl + kk * 16), qf[kk], s);

    float tmax = kNegInf;
    if constexpr (MOD) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] *= score_scale;
      mod_scores16(p, s, slope, L - qlen + tok - j0 - 4 * hi);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = j0 + 8 * (r >> 2) + 4 * hi + (r & 3);
      const float v = (key < lim && key >= lo) ? (MOD ? s[r] : s[r] * score_scale) : kNegInf;
      s[r] = v;
      tmax = fmaxf(tmax, v);
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    // per-row update of the running max (rows that do not need it are
    // multiplied by exactly 1), so a row's bits do not depend on its neighbours
    const bool upd = tmax > m + kTau;
    if (__any(upd)) {
      const float mnew = upd ? fmaxf(m, tmax) : m;
      const float alpha = (!upd || mnew == kNegInf) ? 1.0f : fast_exp2(m - mnew);
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
      m = mnew;
    }
    const float mref = m == kNegInf ? 0.0f : m;
    uint4 pf[2];
    uint32_t* pw = (uint32_t*)pf;
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const float e0 = fast_exp2(s[r] - mref), e1 = fast_exp2(s[r + 1] - mref);
      lsum += e0 + e1;
      pw[r >> 1] = Mfma<QT>::pack2(e0, e1);
    }
    const uint16_t* vl = &v_lds[buf][r32 * VS + hi * 8];
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      oacc[db] = Mfma<QT>::run(*(const uint4*)(vl + db * 32 * VS), pf[0], oacc[db]);
      oacc[db] = Mfma<QT>::run(*(const uint4*)(vl + db * 32 * VS + 16), pf[1], oacc[db]);
    }
  };

  if (ntiles > 0) {
    load_tile(0);
    store_tile(0);
    __syncthreads();
    for (int it = 0; it < ntiles; ++it) {
      const int buf = it & 1;
      const bool more = it + 1 < ntiles;
      if (more) load_tile(it + 1);
      compute(buf, klo + it * kKT);
      if (more) store_tile(buf ^ 1);
      __syncthreads();
    }
  }

  // ---- epilogue
  const float ltot = lsum + __shfl_xor(lsum, 32);
  if (!valid) return;
  float inv, lse_nat;
  final_row(p.write_partial ? nullptr : p.sinks, hq, m, ltot, out_scale, inv, lse_nat);
  const int64_t rowidx = (int64_t)(q0 + tok) * p.num_q_heads + hq;
  if (p.write_partial) {
    float* rec = p.partial + (rowidx * p.num_splits + split) * (int64_t)(p.head_dim + 2);
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int d = db * 32 + 8 * rr + 4 * hi;
        if (d < p.head_dim) {
          float2 a = {oacc[db][4 * rr + 0] * inv, oacc[db][4 * rr + 1] * inv};
          float2 b = {oacc[db][4 * rr + 2] * inv, oacc[db][4 * rr + 3] * inv};
          *(float2*)(rec + d) = a;
          *(float2*)(rec + d + 2) = b;
        }
      }
    }
    if (hi == 0) {
      float2 t = {lse_nat, 0.0f};
      *(float2*)(rec + p.head_dim) = t;
    }
  } else {
    QT* orow = (QT*)p.out + rowidx * p.head_dim;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int d = db * 32 + 8 * rr + 4 * hi;
        if (d < p.head_dim)
          Mfma<QT>::store4(orow + d, oacc[db][4 * rr + 0] * inv, oacc[db][4 * rr + 1] * inv,
                           oacc[db][4 * rr + 2] * inv, oacc[db][4 * rr + 3] * inv);
      }
    }
    if (p.lse != nullptr && hi == 0) p.lse[rowidx] = lse_nat;
  }
}

// ---- host side -------------------------------------------------------------

template <typename QT, int KVK, int DPAD>
static hipError_t launch_t(const AttnParams& p, int nblocks, hipStream_t stream) {
  // the calls routed here: fp8 KV at head dims up to 128
  constexpr bool kModVariant = (KVK == KV_E5M2 || KVK == KV_E4M3) && DPAD <= 128;
  if (has_score_mods(p)) {
    if constexpr (!kModVariant) return hipErrorInvalidValue;
    else hipLaunchKernelGGL((attn_mfma_kernel<QT, KVK, DPAD, true>), dim3(nblocks), dim3(kThreads), 0, stream, p);
  } else {
    hipLaunchKernelGGL((attn_mfma_kernel<QT, KVK, DPAD, false>), dim3(nblocks), dim3(kThreads), 0, stream, p);
  }
  return hipGetLastError();
}

template <typename QT, int KVK>
static hipError_t launch_d(const AttnParams& p, int dpad, int nblocks, hipStream_t stream) {
  switch (dpad) {
    case 64: return launch_t<QT, KVK, 64>(p, nblocks, stream);
    case 128: return launch_t<QT, KVK, 128>(p, nblocks, stream);
    case 256: return launch_t<QT, KVK, 256>(p, nblocks, stream);
    default: return hipErrorInvalidValue;
  }
}

// q_kind: KV_F16 or KV_BF16; kv_kind: same as q_kind, or KV_E5M2 / KV_E4M3.
hipError_t launch_attn_mfma(const AttnParams& p, int q_kind, int kv_kind, int dpad, int nblocks,
                            hipStream_t stream) {
  if (q_kind == KV_F16 && kv_kind == KV_F16) return launch_d<_Float16, KV_F16>(p, dpad, nblocks, stream);
  if (q_kind == KV_BF16 && kv_kind == KV_BF16) return launch_d<__bf16, KV_BF16>(p, dpad, nblocks, stream);
  if (q_kind == KV_F16 && kv_kind == KV_E5M2) return launch_d<_Float16, KV_E5M2>(p, dpad, nblocks, stream);
  if (q_kind == KV_F16 && kv_kind == KV_E4M3) return launch_d<_Float16, KV_E4M3>(p, dpad, nblocks, stream);
  if (q_kind == KV_BF16 && kv_kind == KV_E5M2) return launch_d<__bf16, KV_E5M2>(p, dpad, nblocks, stream);
  if (q_kind == KV_BF16 && kv_kind == KV_E4M3) return launch_d<__bf16, KV_E4M3>(p, dpad, nblocks, stream);
  return hipErrorInvalidValue;
}

int mfma_rows_per_group() { return kRows; }

}  // namespace pa

namespace pa {

template <typename QT, int KVK, int DPAD>
static hipError_t occ_t(int* n) {
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(n, attn_mfma_kernel<QT, KVK, DPAD>, kThreads, 0);
}

template <typename QT, int KVK>
static hipError_t occ_d(int dpad, int* n) {
  switch (dpad) {
    case 64: return occ_t<QT, KVK, 64>(n);
    case 128: return occ_t<QT, KVK, 128>(n);
    case 256: return occ_t<QT, KVK, 256>(n);
    default: return hipErrorInvalidValue;
  }
}

// Work groups of the MFMA kernel that fit on one compute unit.
hipError_t mfma_occupancy(int q_kind, int kv_kind, int dpad, int* blocks_per_cu) {
  if (q_kind == KV_F16 && kv_kind == KV_F16) return occ_d<_Float16, KV_F16>(dpad, blocks_per_cu);
  if (q_kind == KV_BF16 && kv_kind == KV_BF16) return occ_d<__bf16, KV_BF16>(dpad, blocks_per_cu);
  if (q_kind == KV_F16 && kv_kind == KV_E5M2) return occ_d<_Float16, KV_E5M2>(dpad, blocks_per_cu);
  if (q_kind == KV_F16 && kv_kind == KV_E4M3) return occ_d<_Float16, KV_E4M3>(dpad, blocks_per_cu);
  if (q_kind == KV_BF16 && kv_kind == KV_E5M2) return occ_d<__bf16, KV_E5M2>(dpad, blocks_per_cu);
  if (q_kind == KV_BF16 && kv_kind == KV_E4M3) return occ_d<__bf16, KV_E4M3>(dpad, blocks_per_cu);
  return hipErrorInvalidValue;
}

}  // namespace pa
