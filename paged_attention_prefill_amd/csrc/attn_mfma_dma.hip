// Paged attention pass 1 on MFMA with a multi-stage LDS pipeline (fp16 / bf16).
//
// Same computation and work decomposition as the register-staged kernel (one
// work group = 32 * WAVES GQA-packed query rows of one sequence and one kv
// head over one part of the key range, 32-key tiles, S^T = K Q^T and
// O^T += V^T P^T on v_mfma_f32_32x32x16, lazy online softmax), but the K/V
// gathers go straight from HBM into LDS:
//
//   * every 32-key tile is fetched with global_load_lds_dwordx4 (16 bytes per
//     lane, no staging registers); each lane computes its own page address
//     from the block table, so a tile may straddle two pages of any size
//     that is a multiple of 16 (1CatAI/1Cat-vLLM PR #616, the any-page gate);
//   * NST stages are in flight: while tile i is computed, tiles i+1 .. i+NST-1
//     are loading (the loads-overlap-math requirement of 1CatAI/1Cat-vLLM
//     PR #1279, commit 1, pushed to a deeper pipeline for HBM3E latency);
//   * K and V stay row-major in LDS with an XOR swizzle of the 16-byte chunks;
//     V^T reaches the MFMA through ds_read_b64_tr_b16 (transpose read), so no
//     transposing store is needed.
//
// The loads are issued from inline assembly so that the compiler does not
// insert a wait for all of them before every LDS read; completion is tracked
// by hand with s_waitcnt vmcnt(N) plus a work-group barrier.

#include "pa_common.h"

#include <cstdlib>

#pragma clang diagnostic ignored "-Winline-asm"

namespace pa {

namespace {

constexpr int kKT = 32;
constexpr float kTau = 8.0f;
constexpr float kNegInf = -__builtin_huge_valf();

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16_t;

__device__ __forceinline__ void dma16(const char* g, uint32_t lds_byte) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g),
               "s"(__builtin_amdgcn_readfirstlane(lds_byte))
               : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// XOR swizzles of the 16-byte chunks of a key row (chunk c of key `key` lives
// in slot swz(key, c)); chosen so that the MFMA operand reads are free of LDS
// bank conflicts.  Both are involutions.
template <int DPAD>
__device__ __forceinline__ int swz_k(int key, int c) {
  if constexpr (DPAD >= 128) return c ^ (key & 15);
  else return c ^ ((key >> 1) & 7);
}
template <int DPAD>
__device__ __forceinline__ int swz_v(int key, int c) {
  if constexpr (DPAD >= 128) return c ^ ((key & 3) << 2);
  else return c ^ (((key >> 1) & 1) << 2);
}

template <typename QT> struct Mf;
template <> struct Mf<_Float16> {
  static __device__ __forceinline__ f32x16_t run(uint4 a, uint4 b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8_t, a), __builtin_bit_cast(half8_t, b), c,
                                                  0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack2(float a, float b) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    h2 v = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, v);
  }
};
template <> struct Mf<__bf16> {
  static __device__ __forceinline__ f32x16_t run(uint4 a, uint4 b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                   c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack2(float a, float b) {
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    b2 v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
  }
};

}  // namespace

template <typename QT, int DPAD, int WAVES, int NST>
__global__ __launch_bounds__(64 * WAVES, (DPAD <= 128 ? 2 : 1)) void attn_mfma_dma_kernel(const AttnParams p) {
  constexpr int ROWS = 32 * WAVES;
  constexpr int CPK = DPAD / 8;                 // 16-byte chunks per key row
  constexpr int ROWB = CPK * 16;                // bytes per key row in LDS
  constexpr int TILE_BYTES = kKT * ROWB;        // one K (or V) tile
  constexpr int STAGE_BYTES = 2 * TILE_BYTES;
  constexpr int INSTR = STAGE_BYTES / 1024;     // 1 KB DMA instructions per stage
  static_assert(INSTR % WAVES == 0, "DMA instructions must split evenly over the waves");
  constexpr int LPW = INSTR / WAVES;            // DMA instructions per wave per tile
  constexpr int HALF = INSTR / 2;               // instructions per region (K or V)
  constexpr int NKK = DPAD / 16;
  constexpr int NDB = DPAD / 32;
  static_assert((NST - 2) * LPW <= 63, "vmcnt range");

  __shared__ __attribute__((aligned(1024))) char smem[NST * STAGE_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hi = lane >> 5, r32 = lane & 31;

  int w = xcd_remap(blockIdx.x);
  if (w >= p.num_work) return;
  const int qtile = w % p.qtiles;
  w /= p.qtiles;
  const int split = w % p.num_splits;
  w /= p.num_splits;
  const int kvh = w % p.num_kv_heads;
  const int seq = w / p.num_kv_heads;

  const int q0 = p.cu_seqlens_q[seq];
  const int qlen = p.cu_seqlens_q[seq + 1] - q0;
  const int g = p.group;
  const int nrows = qlen * g;
  const int row0 = qtile * ROWS;
  if (row0 >= nrows) return;
  const int L = p.seq_lens[seq];
  int klo, khi;
  split_range(L, p.num_splits, split, klo, khi);

  const int prow = row0 + wave * 32 + r32;
  const bool valid = prow < nrows;
  const int tok = valid ? prow / g : 0;
  const int hq = kvh * g + (valid ? prow - (prow / g) * g : 0);
  const int lim = valid ? min(L - qlen + tok + 1, khi) : 0;
  const int last_tok = (min(row0 + ROWS, nrows) - 1) / g;
  const int kend = min(khi, L - qlen + last_tok + 1);
  const int wrow_first = row0 + wave * 32;
  const bool wave_active = wrow_first < nrows;
  const int wave_kend = wave_active ? min(khi, L - qlen + (min(wrow_first + 32, nrows) - 1) / g + 1) : 0;

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
  const int64_t sp_b = p.stride_page * 2, st_b = p.stride_token * 2;
  const char* kbase = (const char*)p.k_pages + (int64_t)kvh * p.stride_head * 2;
  const char* vbase = (const char*)p.v_pages + (int64_t)kvh * p.stride_head * 2;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(&smem[0]);
  const int dchunks = p.head_dim >> 3;

  // ---- per-lane DMA roles (loop invariant): key, chunk offset, LDS slot
  int dkey[LPW];
  int doff[LPW];  // bytes; 32 keys * stride_token fits in 32 bits (checked on the host)
  const char* dbase[LPW];
  uint32_t dlds[LPW];
#pragma unroll
  for (int n = 0; n < LPW; ++n) {
    const int inst = wave * LPW + n;
    const int region = inst / HALF;  // 0: K, 1: V (wave-uniform)
    const int ri = inst - region * HALF;
    const int slot = ri * 64 + lane;
    const int key = slot / CPK, pos = slot % CPK;
    int c = region == 0 ? swz_k<DPAD>(key, pos) : swz_v<DPAD>(key, pos);
    c = c < dchunks ? c : dchunks - 1;  // head_dim < DPAD: any finite data (multiplied by 0 / discarded)
    dkey[n] = key;
    doff[n] = key * (int)st_b + c * 16;
    dbase[n] = region == 0 ? kbase : vbase;
    dlds[n] = lds0 + region * TILE_BYTES + ri * 1024;
  }

  // running page position of the next tile to issue
  int nx_pg = klo / P, nx_off = klo - (klo / P) * P;
  auto issue = [&](int it, int stage) {
    const int j0 = klo + it * kKT;
    const int pg = nx_pg, off = nx_off;
    nx_off += kKT;
    while (nx_off >= P) nx_off -= P, ++nx_pg;
    const int first_n = P - off;
    const int page_a = bt[pg];
    const int page_b = (first_n < kKT && (pg + 1) * P < kend) ? bt[pg + 1] : page_a;
    const int64_t A = (int64_t)page_a * sp_b + (int64_t)off * st_b;
    const int64_t B = (int64_t)page_b * sp_b - (int64_t)first_n * st_b;
    const int lastkey = kend - 1 - j0;
    const uint32_t sbase = stage * STAGE_BYTES;
#pragma unroll
    for (int n = 0; n < LPW; ++n) {
      int key = dkey[n];
      int o = doff[n];
      if (key > lastkey) {  // past the work group's last key: reload a valid key (finite data, masked)
        o += (lastkey - key) * (int)st_b;
        key = lastkey;
      }
      dma16(dbase[n] + (key < first_n ? A : B) + o, dlds[n] + sbase);
    }
  };

  // ---- per-lane LDS read offsets (loop invariant)
  const int sk = DPAD >= 128 ? (r32 & 15) : ((r32 >> 1) & 7);
  const int krow = r32 * ROWB;
  const int tg = lane >> 4, tk = lane & 15;
  const int vkey = 4 * hi + (tk >> 2);
  const int sv = DPAD >= 128 ? ((vkey & 3) << 2) : (((vkey >> 1) & 1) << 2);
  const int vcl = 2 * (tg & 1) + ((tk & 3) >> 1);
  const int vrow = vkey * ROWB + 8 * (tk & 1);

  auto compute = [&](int stage, int j0) {
    if (!wave_active || j0 >= wave_kend) return;
    const char* kt = smem + stage * STAGE_BYTES;
    const char* vt = kt + TILE_BYTES;
    f32x16_t s = (f32x16_t)(0.0f);
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const uint4 a = *(const uint4*)(kt + krow + (((2 * kk + hi) ^ sk) << 4));
      s = Mf<QT>::run(a, qf[kk], s);
    }
    float tmax = kNegInf;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = j0 + 8 * (r >> 2) + 4 * hi + (r & 3);
      const float v = key < lim ? s[r] * p.scale_log2 : kNegInf;
      s[r] = v;
      tmax = fmaxf(tmax, v);
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    if (__any(tmax > m + kTau)) {
      const float mnew = fmaxf(m, tmax);
      const float alpha = mnew == kNegInf ? 1.0f : fast_exp2(m - mnew);
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
      pw[r >> 1] = Mf<QT>::pack2(e0, e1);
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int coff = ((((4 * db) ^ sv) + vcl) << 4);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const char* a0 = vt + vrow + ks * 16 * ROWB + coff;
        const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)a0);
        const v4i16 hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(a0 + 8 * ROWB));
        uint4 a;
        a.x = __builtin_bit_cast(uint2, lo).x;
        a.y = __builtin_bit_cast(uint2, lo).y;
        a.z = __builtin_bit_cast(uint2, hi4).x;
        a.w = __builtin_bit_cast(uint2, hi4).y;
        oacc[db] = Mf<QT>::run(a, pf[ks], oacc[db]);
      }
    }
  };

  int issued = 0;
#pragma unroll
  for (int i = 0; i < NST - 1; ++i)
    if (issued < ntiles) issue(issued, issued), ++issued;

  for (int it = 0; it < ntiles; ++it) {
    const int ahead = issued - it - 1;  // tiles issued after this one
    if constexpr (NST >= 4) {
      if (ahead >= 2) wait_vmcnt<2 * LPW>();
      else if (ahead == 1) wait_vmcnt<LPW>();
      else wait_vmcnt<0>();
    } else {
      if (ahead >= 1) wait_vmcnt<LPW>();
      else wait_vmcnt<0>();
    }
    __syncthreads();
    if (issued < ntiles) issue(issued, issued % NST), ++issued;
    compute(it % NST, klo + it * kKT);
  }

  // ---- epilogue
  const float ltot = lsum + __shfl_xor(lsum, 32);
  if (!valid) return;
  const bool empty = (m == kNegInf) || !(ltot > 0.0f);
  const float inv = empty ? 0.0f : p.v_scale / ltot;
  const float lse_nat = empty ? kNegInf : (m + __log2f(ltot)) * 0.69314718055994530942f;
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
        if (d < p.head_dim) {
          uint2 v = {Mf<QT>::pack2(oacc[db][4 * rr + 0] * inv, oacc[db][4 * rr + 1] * inv),
                     Mf<QT>::pack2(oacc[db][4 * rr + 2] * inv, oacc[db][4 * rr + 3] * inv)};
          *(uint2*)(orow + d) = v;
        }
      }
    }
    if (p.lse != nullptr && hi == 0) p.lse[rowidx] = lse_nat;
  }
}

// ---- host side -------------------------------------------------------------

namespace {
struct DmaCfg {
  int waves, nst;
};
// Work-group shape per head-dim bucket (tuning knob while measuring).
int d256_waves() {
  static int w = [] {
    const char* e = getenv("PA_TUNE_D256_WAVES");
    return (e && atoi(e) == 4) ? 4 : 8;
  }();
  return w;
}
DmaCfg dma_cfg(int dpad) {
  switch (dpad) {
    case 64: return {4, 4};
    case 128: return {4, 4};
    default: return {d256_waves(), 4};
  }
}

template <typename QT, int DPAD, int WAVES, int NST>
hipError_t launch_cfg(const AttnParams& p, int nblocks, hipStream_t stream) {
  hipLaunchKernelGGL((attn_mfma_dma_kernel<QT, DPAD, WAVES, NST>), dim3(nblocks), dim3(64 * WAVES), 0, stream, p);
  return hipGetLastError();
}

template <typename QT, int DPAD, int WAVES, int NST>
hipError_t occ_cfg(int* n) {
  return hipOccupancyMaxActiveBlocksPerMultiprocessor(n, attn_mfma_dma_kernel<QT, DPAD, WAVES, NST>, 64 * WAVES, 0);
}

template <typename QT>
hipError_t launch_q(const AttnParams& p, int dpad, int nblocks, hipStream_t stream) {
  switch (dpad) {
    case 64: return launch_cfg<QT, 64, 4, 4>(p, nblocks, stream);
    case 128: return launch_cfg<QT, 128, 4, 4>(p, nblocks, stream);
    case 256:
      return d256_waves() == 4 ? launch_cfg<QT, 256, 4, 4>(p, nblocks, stream)
                               : launch_cfg<QT, 256, 8, 4>(p, nblocks, stream);
    default: return hipErrorInvalidValue;
  }
}

template <typename QT>
hipError_t occ_q(int dpad, int* n) {
  switch (dpad) {
    case 64: return occ_cfg<QT, 64, 4, 4>(n);
    case 128: return occ_cfg<QT, 128, 4, 4>(n);
    case 256: return d256_waves() == 4 ? occ_cfg<QT, 256, 4, 4>(n) : occ_cfg<QT, 256, 8, 4>(n);
    default: return hipErrorInvalidValue;
  }
}
}  // namespace

// fp16 or bf16 q with KV of the same dtype.
hipError_t launch_attn_mfma_dma(const AttnParams& p, int q_kind, int dpad, int nblocks, hipStream_t stream) {
  if (q_kind == KV_F16) return launch_q<_Float16>(p, dpad, nblocks, stream);
  if (q_kind == KV_BF16) return launch_q<__bf16>(p, dpad, nblocks, stream);
  return hipErrorInvalidValue;
}

hipError_t mfma_dma_occupancy(int q_kind, int dpad, int* blocks_per_cu) {
  if (q_kind == KV_F16) return occ_q<_Float16>(dpad, blocks_per_cu);
  if (q_kind == KV_BF16) return occ_q<__bf16>(dpad, blocks_per_cu);
  return hipErrorInvalidValue;
}

int mfma_dma_rows(int dpad) { return 32 * dma_cfg(dpad).waves; }

}  // namespace pa
