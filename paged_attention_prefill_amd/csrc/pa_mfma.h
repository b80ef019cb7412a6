// Device helpers shared by the MFMA attention kernels (gfx950): MFMA wrappers,
// the LDS DMA tile loader for paged K/V, LDS swizzles and barriers.
#pragma once

#include "pa_common.h"

#pragma clang diagnostic ignored "-Winline-asm"

namespace pa {
namespace mf {

constexpr int kKT = 32;       // keys per tile
constexpr float kTau = 8.0f;  // lazy-rescale threshold (log2 units)
constexpr float kNegInf = -__builtin_huge_valf();

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16_t;

// 16 bytes per lane from global memory straight into LDS at lds_byte + 16 * lane.
// Issued from inline assembly so that the compiler does not make every later LDS
// read wait for all of these loads; completion is tracked with wait_vmcnt.
__device__ __forceinline__ void dma16(const char* g, uint32_t lds_byte) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g),
               "s"(__builtin_amdgcn_readfirstlane(lds_byte))
               : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Wait until at most `ahead` tiles of LPW loads each are still in flight.
template <int LPW, int MAXA>
__device__ __forceinline__ void wait_tiles(int ahead) {
  static_assert(MAXA <= 3 && MAXA * LPW <= 63, "vmcnt range");
  if constexpr (MAXA >= 3) {
    if (ahead >= 3) return wait_vmcnt<3 * LPW>();
  }
  if constexpr (MAXA >= 2) {
    if (ahead >= 2) return wait_vmcnt<2 * LPW>();
  }
  if constexpr (MAXA >= 1) {
    if (ahead >= 1) return wait_vmcnt<LPW>();
  }
  wait_vmcnt<0>();
}

// Work-group barrier for the LDS ring.  __syncthreads() also waits for every
// outstanding vector-memory load (vmcnt(0)), which would drain the tile loads
// still in flight; here each wave has already waited for its own loads of the
// tile about to be read, so only LDS traffic has to settle before s_barrier.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Completes every load the compiler can see.  Placed before a tile pipeline
// starts so that the compiler puts no vmcnt wait inside the loop (such a wait
// would also drain the tile loads, which it does not track).
__device__ __forceinline__ void drain_visible_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// LDS layouts of a tile (32 keys, DPAD elements per key, 16-byte chunks):
//  * K is chunk-major: chunk c of key k at byte (c * 32 + k) * 16.  The S^T
//    operand read of lane (key k, half h) at k-step kk is chunk 2 kk + h, so
//    the 16 lanes of one LDS cycle read 16 consecutive 16-byte slots (no bank
//    conflict) and successive k-steps are immediate offsets of one address.
//  * V is row-major with an XOR swizzle of the chunks (chunk c of key k lives
//    in slot swz_v(k, c)), chosen so that the transpose reads of the PV
//    operand are free of bank conflicts.  The swizzle is an involution.
__device__ __forceinline__ int k_slot(int key, int c) { return c * kKT + key; }
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

// Byte offset of lane (key r32, half hi)'s S^T operand at k-step 0 inside a K
// tile; k-step kk adds kk * 2 * kKT * 16 bytes.
__device__ __forceinline__ uint32_t k_frag_lane(int r32, int hi) { return (uint32_t)k_slot(r32, hi) * 16; }
constexpr int kKStep = 2 * kKT * 16;

// V^T fragment of the PV product (A operand of 32x32x16): two transpose reads
// of four keys each, d = 32 db + lane % 32.
__device__ __forceinline__ uint4 read_vt(const char* a0, int eight_rows) {
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)a0);
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(a0 + eight_rows));
  uint4 a;
  a.x = __builtin_bit_cast(uint2, lo).x;
  a.y = __builtin_bit_cast(uint2, lo).y;
  a.z = __builtin_bit_cast(uint2, hi).x;
  a.w = __builtin_bit_cast(uint2, hi).y;
  return a;
}

// Gathers 32-key K and V tiles of one kv head through the block table into an
// LDS ring (16-bit KV).  Stage layout: K tile (chunk-major) then V tile
// (row-major, swizzled chunks), see above.  Every lane owns LPW 1 KB DMA
// instructions per tile; a tile may straddle two pages of any size that is a
// multiple of 16.  Keys at or past `kend` reload the last valid key (finite
// data that the softmax masks), so nothing past the sequence is ever read.
template <int DPAD, int WAVES>
struct TileLoader {
  static constexpr int CPK = DPAD / 8;
  static constexpr int ROWB = CPK * 16;
  static constexpr int TILE_BYTES = kKT * ROWB;
  static constexpr int STAGE_BYTES = 2 * TILE_BYTES;
  static constexpr int INSTR = STAGE_BYTES / 1024;
  static_assert(INSTR % WAVES == 0, "DMA instructions must split evenly over the waves");
  static constexpr int LPW = INSTR / WAVES;
  static constexpr int HALF = INSTR / 2;
  static constexpr int KPI = 64 / CPK;

  int doff[LPW];
  int dkey[LPW];
  int wave, lkey, klo, kend, P, st_b, nx_pg, nx_off;
  int64_t sp_b;
  const char* kbase;
  const char* vbase;
  const __attribute__((address_space(4))) int* btc;
  uint32_t lds0;

  __device__ __forceinline__ void init(const AttnParams& p, int seq, int kvh, int wave_, int lane, int klo_,
                                       int kend_, uint32_t lds0_) {
    wave = wave_;
    klo = klo_;
    kend = kend_;
    P = p.page_size;
    sp_b = p.stride_page * 2;
    st_b = (int)(p.stride_token * 2);  // 32 keys * stride fits in 32 bits (checked on the host)
    kbase = (const char*)p.k_pages + (int64_t)kvh * p.stride_head * 2;
    vbase = (const char*)p.v_pages + (int64_t)kvh * p.stride_head * 2;
    // page ids are read through the constant address space at a uniform index:
    // scalar loads, tracked by lgkmcnt, so they never drain the tile loads
    btc = (const __attribute__((address_space(4))) int*)(p.block_tables + (int64_t)seq * p.max_pages);
    lds0 = lds0_;
    nx_pg = klo / P;
    nx_off = klo - nx_pg * P;
    lkey = lane / CPK;
    const int lpos = lane % CPK, dchunks = p.head_dim >> 3;
#pragma unroll
    for (int n = 0; n < LPW; ++n) {
      const int inst = wave * LPW + n;
      const int region = inst / HALF;  // 0: K, 1: V (wave-uniform)
      const int ri = inst - region * HALF;
      int key, c;
      if (region == 0) {  // K: the instruction's 64 slots are chunks 2 ri, 2 ri + 1 of keys 0..31
        key = lane & (kKT - 1);
        c = 2 * ri + (lane >> 5);
      } else {
        key = ri * KPI + lkey;
        c = swz_v<DPAD>(key, lpos);
      }
      c = c < dchunks ? c : dchunks - 1;  // head_dim < DPAD: any finite data (multiplied by 0 / discarded)
      dkey[n] = key;
      doff[n] = key * st_b + c * 16;
    }
  }

  // Issues tile `it` (keys klo + 32 it ...) into `stage`; calls must come in order.
  __device__ __forceinline__ void issue(int it, int stage) {
    const int j0 = klo + it * kKT;
    const int pg = nx_pg, off = nx_off;
    nx_off += kKT;
    while (nx_off >= P) nx_off -= P, ++nx_pg;
    const int first_n = P - off;  // keys of the tile on the first page (a multiple of 16)
    const int page_a = btc[__builtin_amdgcn_readfirstlane(pg)];
    const int page_b =
        (first_n < kKT && (pg + 1) * P < kend) ? btc[__builtin_amdgcn_readfirstlane(pg + 1)] : page_a;
    const int64_t A = (int64_t)page_a * sp_b + (int64_t)off * st_b;
    const int64_t B = (int64_t)page_b * sp_b - (int64_t)first_n * st_b;
    const int lastkey = kend - 1 - j0;
    const uint32_t sbase = lds0 + stage * STAGE_BYTES;
#pragma unroll
    for (int n = 0; n < LPW; ++n) {
      const int inst = wave * LPW + n;
      const int region = inst / HALF;
      const int ri = inst - region * HALF;
      int key = dkey[n];
      int o = doff[n];
      if (key > lastkey) {  // past the work group's last key: reload a valid key (finite data, masked)
        o += (lastkey - key) * st_b;
        key = lastkey;
      }
      dma16((region == 0 ? kbase : vbase) + (key < first_n ? A : B) + o, sbase + region * TILE_BYTES + ri * 1024);
    }
  }
};

}  // namespace mf
}  // namespace pa
