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
// NT sets the non-temporal cache policy: data read once (a decode part's keys)
// streams past the caches instead of displacing lines, which measures about
// 10% faster for a plain streaming read on this chip.
template <bool NT = false>
__device__ __forceinline__ void dma16(const char* g, uint32_t lds_byte) {
  if constexpr (NT)
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off nt" ::"v"(g),
                 "s"(__builtin_amdgcn_readfirstlane(lds_byte))
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g),
                 "s"(__builtin_amdgcn_readfirstlane(lds_byte))
                 : "memory", "m0");
}

// Same with a wave-uniform 64-bit base in SGPRs and a 32-bit per-lane offset
// (the saddr form: no 64-bit address arithmetic per lane).
template <bool NT = false>
__device__ __forceinline__ void dma16_sb(const char* base, uint32_t voff, uint32_t lds_byte) {
  // readfirstlane works on (signed) int: widen through uint32_t so that the
  // low half is zero-extended, not sign-extended into the high half
  const uint64_t b = (uint64_t)(uintptr_t)base;
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
  const char* sbase = (const char*)(uintptr_t)((hi << 32) | lo);
  if constexpr (NT)
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(sbase),
                 "s"(__builtin_amdgcn_readfirstlane(lds_byte))
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase),
                 "s"(__builtin_amdgcn_readfirstlane(lds_byte))
                 : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Wait until at most `ahead` (<= MAXA) tiles of LPW loads each are still in flight.
template <int LPW, int MAXA>
__device__ __forceinline__ void wait_tiles(int ahead) {
  static_assert(MAXA * LPW <= 63, "vmcnt range");
  if constexpr (MAXA >= 1) {
    if (ahead >= MAXA) return wait_vmcnt<MAXA * LPW>();
    return wait_tiles<LPW, MAXA - 1>(ahead);
  } else {
    wait_vmcnt<0>();
  }
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
//  * K is stored in 1 KB blocks of 8 keys x 8 chunks (one 128-byte line of
//    each key): block (c / 8) * 4 + k / 8, row k % 8 of the block holding the
//    key's 8 chunks, chunk c at position (c % 8) ^ ((k / 2) % 8).  One DMA
//    instruction fills one block, eight consecutive lanes per key, so every
//    instruction reads whole 128-byte lines (a layout that takes 32 bytes of
//    32 keys per instruction streams about 20% slower).  The S^T operand read
//    of lane (key k, half h) at k-step kk is chunk 2 kk + h; the XOR spreads
//    the 16 keys of one LDS cycle over all 16 slots of a bank row.
//  * V is row-major with an XOR swizzle of the chunks (chunk c of key k lives
//    in slot swz_v(k, c)), chosen so that the transpose reads of the PV
//    operand are free of bank conflicts.  The swizzle is an involution.
__device__ __forceinline__ int k_swz(int key) { return (key >> 1) & 7; }
__device__ __forceinline__ int k_slot(int key, int c) { return (c >> 3) * (8 * kKT) + key * 8 + ((c & 7) ^ k_swz(key)); }
template <int DPAD, int ES = 2>
__device__ __forceinline__ int swz_v(int key, int c) {
  if constexpr (ES == 1) return c ^ (((key & 3) | ((key >> 1) & 4)) << 1);  // fp8, 16-chunk rows: see read_vt8
  else if constexpr (DPAD >= 128) return c ^ ((key & 3) << 2);
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
  // acc + both halves of a packed pair, products and sum in fp32 (one v_dot2)
  static __device__ __forceinline__ float sum2(uint32_t p, float acc) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, p), (h2){(_Float16)1.0f, (_Float16)1.0f}, acc, false);
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
  static __device__ __forceinline__ float sum2(uint32_t p, float acc) {
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2, p), (b2){(__bf16)1.0f, (__bf16)1.0f}, acc, false);
  }
};

// max(x[lane], x[lane ^ 32]) in every lane, through v_permlane32_swap (lanes
// 32..63 of the first operand trade places with lanes 0..31 of the second).
__device__ __forceinline__ float max_halves(float x) {
  float t;
  asm volatile(
      "v_mov_b32 %1, %0\n\ts_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1\n\tv_max_f32 %0, %0, %1"
      : "+v"(x), "=&v"(t));
  return x;
}

// The same with the minimum.
__device__ __forceinline__ float min_halves(float x) {
  float t;
  asm volatile(
      "v_mov_b32 %1, %0\n\ts_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1\n\tv_min_f32 %0, %0, %1"
      : "+v"(x), "=&v"(t));
  return x;
}

// max(a, b, c) without the canonicalizing moves the compiler adds around
// fmaxf of MFMA results (the scores are never signalling NaNs).
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float min3f(float a, float b, float c) {
  float r;
  asm("v_min3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
__device__ __forceinline__ float max2f(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// Byte offset of lane (key r32, half hi)'s S^T operand at k-step 0 inside a K
// tile, and at k-step kk (chunk 2 kk + hi): chunks 2 kk + hi of one 8-chunk
// line differ from chunk hi in bits 1..2 only, an XOR of the slot.
__device__ __forceinline__ uint32_t k_frag_lane(int r32, int hi) { return (uint32_t)k_slot(r32, hi) * 16; }
__device__ __forceinline__ uint32_t k_frag(uint32_t klane, int kk) {
  return (uint32_t)((kk >> 2) * (8 * kKT * 16)) + (klane ^ (uint32_t)((kk & 3) << 5));
}

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

// ---- fp8 (E5M2) KV operands.  An E5M2 byte is the high byte of the fp16 of
// the same value, so widening is a byte permute (exact).
__device__ __forceinline__ uint32_t e5m2_lo2(uint32_t x) { return __builtin_amdgcn_perm(0u, x, 0x010C000Cu); }
__device__ __forceinline__ uint32_t e5m2_hi2(uint32_t x) { return __builtin_amdgcn_perm(0u, x, 0x030C020Cu); }
__device__ __forceinline__ uint4 e5m2x8_to_f16(uint32_t a, uint32_t b) {
  return make_uint4(e5m2_lo2(a), e5m2_hi2(a), e5m2_lo2(b), e5m2_hi2(b));
}

// Eight fp8 bytes (a: elements 0..3, b: 4..7) -> eight values of the 16-bit
// compute type QT (fp16 or bf16, the query's type), F8 = KV_E5M2 or KV_E4M3.
// Exact: every fp8 value of both formats is representable in fp16 and in bf16.
template <typename QT, int F8>
__device__ __forceinline__ uint4 fp8x8_to(uint32_t a, uint32_t b) {
  if constexpr (__is_same(QT, __bf16))
    return make_uint4(fp8x2_to_bf16x2<F8, false>(a), fp8x2_to_bf16x2<F8, true>(a), fp8x2_to_bf16x2<F8, false>(b),
                      fp8x2_to_bf16x2<F8, true>(b));
  else if constexpr (F8 == KV_E4M3)
    return make_uint4(e4m3x2_to_f16x2<false>(a), e4m3x2_to_f16x2<true>(a), e4m3x2_to_f16x2<false>(b),
                      e4m3x2_to_f16x2<true>(b));
  else
    return e5m2x8_to_f16(a, b);
}

typedef int v2i32 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) v2i32 lds_v2i32_t;

// V^T fragment of the PV product from an fp8 V tile: one transpose read of
// 8-bit elements.  Within each 16-lane group, input lane k supplies 8 bytes
// (half k % 2 of a 16-byte chunk of row k / 2 of an 8-row block) and output
// lane j receives byte j of each of the 8 rows, in row order: 8 keys of one d,
// the A operand of a 32x32x16 MFMA after widening.  The rows a group
// addresses are the 8 keys that the P^T operand pairs with this lane's
// k-indices (16 ks + 8 (i / 4) + 4 (lane / 32) + i % 4, i = 0..7); the V chunk
// swizzle c ^ 2 f(key), f(key) = (key & 3) | (bit 3 of key) << 2, puts those 8
// rows' chunks in 8 different slots, so the reads are free of bank conflicts.
template <typename QT, int F8>
__device__ __forceinline__ uint4 read_vt8(const char* a) {
  const v2i32 r = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_v2i32_t*)a);
  return fp8x8_to<QT, F8>((uint32_t)r.x, (uint32_t)r.y);
}

// Gathers 32-key K and V tiles of one kv head through the block table into an
// LDS ring (ES = 2: 16-bit KV; ES = 1: fp8 KV, bytes copied as they are).
// Stage layout: K tile (8-key x 8-chunk blocks) then V tile
// (row-major, swizzled chunks), see above.  Every lane owns LPW 1 KB DMA
// instructions per tile; a tile may straddle two pages of any size that is a
// multiple of 16.  Keys at or past `kend` reload the last valid key (finite
// data that the softmax masks), so nothing past the sequence is ever read.
//
// A tile is loaded in three steps so that callers can spread the work:
// fetch(it) reads the tile's page ids (scalar loads), begin(stage) forms its
// page bases, part<FAST>(n) issues DMA instruction n of this wave.  FAST may
// be used when fast() holds (one page, every key inside the range).
// DESC: tiles are fetched in descending key order (a negative stride).
// PIDL: the page ids may come from a table in LDS (set_pid_table) instead of
// scalar loads of the block table.  A scalar load still in flight makes every
// later wait for an LDS read a wait for everything (scalar loads return out of
// order), so a loop that reads page ids from the block table while LDS reads
// are outstanding pays the scalar load's latency; from LDS it does not.
// Without a table, a fetch then waits for its own scalar loads.
template <int DPAD, int WAVES, int ES = 2, bool NT = false, bool DESC = false, bool PIDL = false>
struct TileLoader {
  static_assert(ES == 2 || (ES == 1 && DPAD == 256), "8-bit KV tiles are laid out for D 256");
  static constexpr int CPK = DPAD * ES / 16;
  static constexpr int ROWB = CPK * 16;
  static constexpr int TILE_BYTES = kKT * ROWB;
  static constexpr int STAGE_BYTES = 2 * TILE_BYTES;
  static constexpr int INSTR = STAGE_BYTES / 1024;
  static_assert(INSTR % WAVES == 0, "DMA instructions must split evenly over the waves");
  static constexpr int LPW = INSTR / WAVES;
  static constexpr int HALF = INSTR / 2;
  static constexpr int KPI = 64 / CPK;

  int doff[LPW];  // per lane: byte offset of its 16 bytes for instruction n, relative to the key-0 base
  int wave, lane, lkey, klo, kend, P, st_b;
  int nx_pg, nx_off, nx_key, kstep;   // page cursor and first key of the next tile to fetch
  int f_j0, f_off, f_first, f_pa, f_pb;  // the fetched tile
  int64_t sp_b;
  int64_t tA, tB;                     // byte offsets of key 0 on the first / second page
  int tfirst, tlast;
  uint32_t tsb;
  const char* kbase;
  const char* vbase;
  const __attribute__((address_space(4))) int* btc;
  uint32_t lds0;
  // PIDL: page ids pid_base .. of the group's keys in LDS (when pid_on)
  const __attribute__((address_space(3))) int* pid_tab;
  int pid_base;
  bool pid_on;

  __device__ __forceinline__ void init(const AttnParams& p, int seq, int kvh, int wave_, int lane_, int klo_,
                                       int kend_, uint32_t lds0_) {
    wave = wave_;
    lane = lane_;
    klo = __builtin_amdgcn_readfirstlane(klo_);
    kend = __builtin_amdgcn_readfirstlane(kend_);
    P = p.page_size;
    sp_b = p.stride_page * ES;
    st_b = (int)(p.stride_token * ES);  // 32 keys * stride fits in 32 bits (checked on the host)
    kbase = (const char*)p.k_pages + (int64_t)kvh * p.stride_head * ES;
    vbase = (const char*)p.v_pages + (int64_t)kvh * p.stride_head * ES;
    // page ids are read through the constant address space at a uniform index:
    // scalar loads, tracked by lgkmcnt, so they never drain the tile loads
    btc = (const __attribute__((address_space(4))) int*)(p.block_tables + (int64_t)seq * p.max_pages);
    lds0 = lds0_;
    nx_pg = __builtin_amdgcn_readfirstlane(klo / P);
    nx_off = __builtin_amdgcn_readfirstlane(klo - nx_pg * P);
    nx_key = klo;
    kstep = DESC ? -kKT : kKT;
    lkey = lane_ / CPK;
    const int lpos = lane_ % CPK, dchunks = (p.head_dim * ES) >> 4;
#pragma unroll
    for (int n = 0; n < LPW; ++n) {
      const int inst = wave * LPW + n;
      const int region = inst / HALF;  // 0: K, 1: V (wave-uniform)
      const int ri = inst - region * HALF;
      int key, c;
      key = inst_key(region, ri);
      if (region == 0) c = 8 * (ri >> 2) + ((lane_ & 7) ^ k_swz(key));  // K: block ri of 8 keys x 8 chunks
      else c = swz_v<DPAD, ES>(key, lpos);
      c = c < dchunks ? c : dchunks - 1;  // head_dim < DPAD: any finite data (multiplied by 0 / discarded)
      doff[n] = key * st_b + c * 16;
    }
  }

  // Tiles are fetched every `step` keys from klo (a multiple of 32, negative
  // with DESC; kKT unless set, -kKT with DESC).
  __device__ __forceinline__ void set_stride(int step) { kstep = step; }

  // PIDL: page ids from the table at LDS byte `tab_byte` (entry i = block-table
  // entry base + i, covering every page a fetch reads) when `on`, else from
  // the block table.
  __device__ __forceinline__ void set_pid_table(bool on, uint32_t tab_byte, int base) {
    pid_on = on;
    pid_tab = (const __attribute__((address_space(3))) int*)(uintptr_t)tab_byte;
    pid_base = base;
  }

  // Reads the page ids of the next tile (keys klo + step * it ...); calls come in tile order.
  __device__ __forceinline__ void fetch(int it) {
    (void)it;
    f_j0 = nx_key;
    nx_key += kstep;
    const int pg = nx_pg;
    f_off = nx_off;
    nx_off += kstep;
    if constexpr (DESC) {
      while (nx_off < 0) nx_off += P, --nx_pg;
    } else {
      while (nx_off >= P) nx_off -= P, ++nx_pg;
    }
    f_first = P - f_off;  // keys of the tile on the first page (a multiple of 16)
    // both ids are loaded without a branch on the first (the second page's id
    // is only used when the tile reaches it; otherwise the first is re-read),
    // so nothing waits for these loads before the tile's refill begins
    const int pg2 = (f_first < kKT && (pg + 1) * P < kend) ? pg + 1 : pg;
    if constexpr (PIDL) {
      if (pid_on) {
        // LDS reads into vector registers; begin() moves them to scalars
        f_pa = pid_tab[pg - pid_base];
        f_pb = pid_tab[pg2 - pid_base];
      } else {
        f_pa = btc[pg];
        f_pb = btc[pg2];
        asm volatile("" : "+s"(f_pa), "+s"(f_pb));  // the scalar loads complete here
      }
    } else {
      f_pa = btc[pg];
      f_pb = btc[pg2];
    }
  }

  // Page bases of the fetched tile, to be loaded into `stage`.
  __device__ __forceinline__ void begin(int stage) {
    if constexpr (PIDL) {
      f_pa = __builtin_amdgcn_readfirstlane(f_pa);
      f_pb = __builtin_amdgcn_readfirstlane(f_pb);
    }
    tA = (int64_t)f_pa * sp_b + (int64_t)f_off * st_b;
    tB = (int64_t)f_pb * sp_b - (int64_t)f_first * st_b;
    tfirst = f_first;
    tlast = kend - 1 - f_j0;
    tsb = lds0 + stage * STAGE_BYTES;
  }

  __device__ __forceinline__ bool fast() const { return tfirst >= kKT && tlast >= kKT - 1; }

  template <bool FAST>
  __device__ __forceinline__ void part(int n) {
    const int inst = wave * LPW + n;
    const int region = inst / HALF;
    const int ri = inst - region * HALF;
    const char* base = region == 0 ? kbase : vbase;
    const uint32_t dst = tsb + region * TILE_BYTES + ri * 1024;
    if constexpr (FAST) {
      dma16_sb<NT>(base + tA, (uint32_t)doff[n], dst);
    } else {
      int key = inst_key(region, ri);
      int o = doff[n];
      asm volatile("" : "+v"(o));  // keeps the per-lane 64-bit address out of loop-invariant code motion
      if (key > tlast) {  // past the work group's last key: reload a valid key (finite data, masked)
        o += (tlast - key) * st_b;
        key = tlast;
      }
      dma16<NT>(base + (key < tfirst ? tA : tB) + o, dst);
    }
  }

  // Issues tile `it` into `stage` in one go.
  __device__ __forceinline__ void issue(int it, int stage) {
    fetch(it);
    begin(stage);
    if (fast()) {
#pragma unroll
      for (int n = 0; n < LPW; ++n) part<true>(n);
    } else {
#pragma unroll
      for (int n = 0; n < LPW; ++n) part<false>(n);
    }
  }

  // Key (0..31 within the tile) that this lane loads in instruction `ri` of `region`.
  __device__ __forceinline__ int inst_key(int region, int ri) const {
    return region == 0 ? 8 * (ri & 3) + (lane >> 3) : ri * KPI + lkey;
  }
};

}  // namespace mf
}  // namespace pa
