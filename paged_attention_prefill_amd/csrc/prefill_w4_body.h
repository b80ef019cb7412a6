// Paged attention pass 1, one wave per SIMD, 64 query rows per wave (fp16 / bf16).
//
// Same computation and work decomposition as attn_mfma_dma.hip (GQA-packed
// query rows of one sequence and kv head over one key part, 32-key tiles from
// the LDS DMA ring, S^T = K Q^T and O^T += V^T P^T on v_mfma_f32_32x32x16, lazy
// online softmax), arranged for a higher MFMA share of the SIMD:
//
//   * every wave holds two blocks of 32 rows, so each K or V^T fragment read
//     from LDS feeds two MFMAs; LDS read traffic per flop is half that of a
//     32-row wave, which matters because at 32 rows per wave the LDS is nearly
//     as busy as the matrix cores;
//   * the 64 x DPAD output accumulators (256 registers at D = 256) live in the
//     AGPR file, the scores S^T in VGPRs (their MFMAs are issued from inline
//     assembly, so that the compiler does not place them in AGPRs too);
//   * the PV product of tile i - 1 is issued in the same basic block as the
//     softmax of tile i and the two are interleaved instruction by instruction
//     (a few VALU instructions run in the shadow of every MFMA), so the softmax
//     costs little beyond the MFMA time; the QK product of tile i runs alone;
//   * the row max is exchanged between the two lane halves with
//     v_permlane32_swap (one VALU instruction instead of an LDS permute), the
//     softmax scale is folded into the exponent's FMA, and the causal mask is
//     only applied on tiles that reach a row's last key.
//
// Inline-assembly MFMAs are not covered by the compiler's hazard recognizer,
// so the required wait states are written out where their results are read.

#ifndef PA_PREFILL_W4_BODY_H
#define PA_PREFILL_W4_BODY_H

#include <type_traits>

#include "pa_mfma.h"

namespace pa {

using namespace mf;

// Entries of a work group's page-id table in LDS (32 KB).
constexpr int kPidMax = 8192;

namespace {

// c = a * b (+ c unless `first`), accumulator in VGPRs.  VALU_A: `a` was just
// written by VALU instructions (the widened fp8 K operand), which an MFMA may
// read only after 2 wait states; the s_nop supplies 3.
template <typename QT, bool VALU_A = false>
__device__ __forceinline__ void mfma_s(f32x16_t& c, uint4 a, uint4 b, bool first) {
  typedef int i32x4 __attribute__((ext_vector_type(4)));
  const i32x4 av = __builtin_bit_cast(i32x4, a), bv = __builtin_bit_cast(i32x4, b);
#define PA_MFMA_S(OP)                                                                             \
  if (first) asm volatile(OP " %0, %1, %2, 0" : "=&v"(c) : "v"(av), "v"(bv));                     \
  else asm volatile(OP " %0, %1, %2, %0" : "+v"(c) : "v"(av), "v"(bv));
  if constexpr (__is_same(QT, _Float16)) {
    if constexpr (VALU_A) {
      PA_MFMA_S("s_nop 2\n\tv_mfma_f32_32x32x16_f16")
    } else {
      PA_MFMA_S("v_mfma_f32_32x32x16_f16")
    }
  } else {
    if constexpr (VALU_A) {
      PA_MFMA_S("s_nop 2\n\tv_mfma_f32_32x32x16_bf16")
    } else {
      PA_MFMA_S("v_mfma_f32_32x32x16_bf16")
    }
  }
#undef PA_MFMA_S
}

// Wait states between the last score MFMA and the first VALU read of its
// result (20 >= the 12 that an 8-pass XDL op needs); tying the scores to the
// statement keeps every read after it.
__device__ __forceinline__ void scores_ready(f32x16_t& s0, f32x16_t& s1) {
  asm volatile("s_nop 15\n\ts_nop 3" : "+v"(s0), "+v"(s1));
}

// In-place scale of an accumulator held in AGPRs (read, multiply, write back
// into the same register), so that the conditional rescale does not make the
// compiler keep a second copy of the accumulators.
__device__ __forceinline__ void scale_acc_agpr(f32x16_t& x, float s) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float e = x[i], t;
    asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %2, %1\n\tv_accvgpr_write_b32 %0, %1"
                 : "+a"(e), "=&v"(t)
                 : "v"(s));
    x[i] = e;
  }
}

// Pins the accumulators to the AGPR file and orders everything that defines
// them before everything that reads them next, with `N` + 1 wait states.
template <int NDB>
__device__ __forceinline__ void acc_fence(f32x16_t (&o)[NDB]) {
#pragma unroll
  for (int db = 0; db < NDB; ++db) asm volatile("s_nop 7" : "+a"(o[db]));
}

}  // namespace

// F8 = KV_E5M2 or KV_E4M3: K and V are fp8 (q fp16 or bf16); the tiles stay
// 8-bit in LDS and are widened to the query's type as their MFMA operands are read.  F8 = 0: KV of
// the q dtype.
// VAR 0: no options that touch the scores; 1: a left sliding window; 2: a
// logit softcap; 3: ALiBi; 4: both (2 to 4 with or without a window).  Each is its own instantiation, so that the
// default one keeps no per-row state in this tightly scheduled loop.
template <typename QT, int F8, int DPAD, int NST, int VAR>
__device__ __forceinline__ void prefill_w4_body(const AttnParams& p, int bid, char* smem) {
  constexpr bool KV8 = F8 != 0;
  constexpr bool WIN = VAR >= 1, MOD = VAR >= 2, CAP = VAR == 2;
  constexpr int WAVES = 4, RB = 2, WROWS = 64, ROWS = WAVES * WROWS;
  typedef TileLoader<DPAD, WAVES, KV8 ? 1 : 2, false, MOD, true> TL;
  constexpr int ROWB = TL::ROWB;
  constexpr int TILE_BYTES = TL::TILE_BYTES;
  constexpr int STAGE_BYTES = TL::STAGE_BYTES;
  constexpr int LPW = TL::LPW;
  constexpr int NKK = DPAD / 16, NDB = DPAD / 32, NST2 = 2 * NDB;
  constexpr int DIST = NST - 2;  // tile i - 1 is still read in iteration i
  constexpr int KPF = KV8 ? 2 : 3, VPF = 3;  // LDS operand reads issued ahead of their MFMA
  static_assert(NST * STAGE_BYTES <= 160 * 1024, "LDS");
  static_assert(DIST >= 1, "ring depth");


  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hi = lane >> 5, r32 = lane & 31;

  WorkItem wi;
  if (!work_of_block(p, bid, true, wi)) return;
  // a sequence's last query tiles see the most keys: they are handed out first
  // Uniform, and held in scalar registers (OPQ) so that nothing derived from
  // them takes a vector register across the tile loop.  Register allocation
  // is tight in every instantiation: this keeps the 16-bit default and window
  // ones free of scratch; the modifier and fp8 ones are free of it without
  // (and the fp8 ones ran 3 % slower with it).
  constexpr bool OPQ = !MOD && !KV8;
  const int qtile = OPQ ? __builtin_amdgcn_readfirstlane(wi.qtile) : wi.qtile;
  const int split = OPQ ? __builtin_amdgcn_readfirstlane(wi.split) : wi.split;
  const int kvh = OPQ ? __builtin_amdgcn_readfirstlane(wi.kvh) : wi.kvh;
  const float score_scale = head_score_scale(p, kvh), out_scale = head_v_scale(p, kvh);
  const int seq = seq_by_rank(p, wi.seqpos, (int*)smem, tid, 256);

  const int q0 = p.cu_seqlens_q[seq];
  const int qlen = q_end_of(p, seq) - q0;
  const int g = p.group;
  const int nrows = qlen * g;
  const int row0 = qtile * ROWS;
  if (row0 >= nrows) return;
  const int L = p.seq_lens[seq];
  int klo, khi;
  split_range(p, L, qlen, split, klo, khi);
  const int last_tok = (min(row0 + ROWS, nrows) - 1) / g;
  const int kend = min(khi, L - qlen + last_tok + 1);
  const int wrow0 = row0 + wave * WROWS;
  // first tile: the part's start, or the tile of the earliest window start
  const int kfirst = WIN ? window_klo(p, klo, khi, L - qlen + row0 / g) : klo;
  // mask bounds of this wave's rows (monotone in the row): tiles that end
  // past wlim or (window) start before wlo need the per-element mask
  const int wlim = wrow0 + WROWS > nrows ? 0 : min(L - qlen + wrow0 / g + 1, khi);
  const int wlo = (!WIN || wrow0 >= nrows) ? 0 : window_lo(p, L - qlen + (min(wrow0 + WROWS, nrows) - 1) / g);

  // this lane's rows (one per block) and their Q^T fragments (B operand).
  // lim: one past the row's last visible key (the part's end and the window
  // start are applied in the rare masked tiles: one register per row block).
  int lim[RB];
  uint4 qf[RB][NKK];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int prow = wrow0 + rb * 32 + r32;
    const bool valid = prow < nrows;
    const int tok = valid ? prow / g : 0;
    const int hq = kvh * g + (valid ? prow - tok * g : 0);
    lim[rb] = valid ? L - qlen + tok + 1 : 0;
    const QT* qrow = (const QT*)p.q + ((int64_t)(q0 + tok) * p.num_q_heads + hq) * p.head_dim;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      // 16-bit K: k-step kk covers d 16 kk + 8 hi ..; fp8 K: the pair of
      // k-steps 2j, 2j+1 covers the 16-byte chunk 2j + hi, low then high half
      const int d = KV8 ? 32 * (kk >> 1) + 16 * hi + 8 * (kk & 1) : kk * 16 + hi * 8;
      qf[rb][kk] = (valid && d < p.head_dim) ? *(const uint4*)(qrow + d) : make_uint4(0, 0, 0, 0);
    }
  }

  const int ntiles = kend > kfirst ? (kend - kfirst + kKT - 1) / kKT : 0;
  f32x16_t oacc[RB][NDB];
  float m[RB], lsum[RB];

  // ---- epilogue: o = O / l into out (+ lse), or the part's FP32 record.
  // ZERO: the group sees no key of its part, so every row gets o = 0 and lse
  // -inf (or its sink) without reading the accumulators.
  auto epilogue = [&](auto zero_tag) {
    constexpr bool ZERO = decltype(zero_tag)::value;
    // the lane index, the row offsets and the output factor formed again here
    // (mbcnt, a scalar load), so that nothing of the epilogue is kept alive
    // (in scratch memory) across the tile loop
    int lane_e = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    asm volatile("" : "+v"(lane_e));
    // (OPQ: the same for the scalars the row arithmetic starts from, opaque
    // copies, so that the division by g and the row offsets are not shared
    // with, and kept alive from, the same arithmetic before the loop)
    int g_e = g, kvh_e = kvh, q0_e = q0, wrow0_e = wrow0, nrows_e = nrows, split_e = split;
    if constexpr (OPQ) {
      g_e = __builtin_amdgcn_readfirstlane(g_e), q0_e = __builtin_amdgcn_readfirstlane(q0_e);
      wrow0_e = __builtin_amdgcn_readfirstlane(wrow0_e), nrows_e = __builtin_amdgcn_readfirstlane(nrows_e);
      asm volatile("" : "+s"(g_e), "+s"(kvh_e), "+s"(q0_e), "+s"(wrow0_e), "+s"(nrows_e), "+s"(split_e));
    }
    const int hi = lane_e >> 5, r32 = lane_e & 31;
    const float out_scale = head_v_scale(p, kvh_e);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float ltot = 0.0f, mrow = kNegInf;
      if constexpr (!ZERO) ltot = lsum[rb] + __shfl_xor(lsum[rb], 32), mrow = m[rb];
      const int prow = wrow0_e + rb * 32 + r32;
      if (prow >= nrows_e) continue;
      const int tok = prow / g_e;
      const int hq = kvh_e * g_e + (prow - tok * g_e);
      float inv, lse_nat;
      final_row(p.write_partial ? nullptr : p.sinks, hq, mrow, ltot, out_scale, inv, lse_nat);
      const int64_t rowidx = (int64_t)(q0_e + tok) * p.num_q_heads + hq;
      // element i of accumulator block db, normalised
      auto o = [&](int db, int i) {
        if constexpr (ZERO) return 0.0f;
        else return oacc[rb][db][i] * inv;
      };
      if (p.write_partial) {
        float* rec = p.partial + (rowidx * p.num_splits + split_e) * (int64_t)(p.head_dim + 2);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const int d = db * 32 + 8 * rr + 4 * hi;
            if (d < p.head_dim) {
              float2 a = {o(db, 4 * rr + 0), o(db, 4 * rr + 1)};
              float2 b = {o(db, 4 * rr + 2), o(db, 4 * rr + 3)};
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
              uint2 v = {Mf<QT>::pack2(o(db, 4 * rr + 0), o(db, 4 * rr + 1)),
                         Mf<QT>::pack2(o(db, 4 * rr + 2), o(db, 4 * rr + 3))};
              *(uint2*)(orow + d) = v;
            }
          }
        }
        if (p.lse != nullptr && hi == 0) p.lse[rowidx] = lse_nat;
      }
    }
  };
  // Written apart so that the accumulators' zero start values are not kept
  // alive across the tile loop for this path (the register allocator parked
  // all 256 of them in scratch memory to have them here).
  if (ntiles == 0) {
    epilogue(std::true_type());
    return;
  }

#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m[rb] = kNegInf;
    lsum[rb] = 0.0f;
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[rb][db] = (f32x16_t)(0.0f);
    acc_fence<NDB>(oacc[rb]);
  }

  // The modifier instantiation runs the tiles from the last one down: under
  // ALiBi a row's biased scores grow with the key, so in ascending order its
  // running max would rise by up to slope * 32 every tile and rescale the
  // accumulators each time; from the nearest keys down the max is set by the
  // first tile.
  const int kstart = MOD && ntiles > 0 ? kfirst + (ntiles - 1) * kKT : kfirst;
  const int kstep = MOD ? -kKT : kKT;
  TL tl;
  tl.init(p, seq, kvh, wave, lane, kstart, kend, (uint32_t)(uintptr_t)(&smem[0]));
  // The group's page ids (pages kfirst / P .. (kend - 1) / P) are copied to
  // the table after the ring, so that the tile loop reads them from LDS
  // instead of the block table; a group with more than kPidMax pages reads
  // the block table (and waits for it) at every tile.
  {
    const int pid_first = kfirst / p.page_size;
    const int pid_n = (kend - 1) / p.page_size - pid_first + 1;
    const bool pid_on = pid_n <= kPidMax;
    if (pid_on) {
      const int* bt = p.block_tables + (int64_t)seq * p.max_pages + pid_first;
      int* tab = (int*)(smem + NST * STAGE_BYTES);
      for (int i = tid; i < pid_n; i += ROWS) tab[i] = bt[i];
    }
    tl.set_pid_table(pid_on, (uint32_t)(uintptr_t)(&smem[0]) + NST * STAGE_BYTES, pid_first);
    __syncthreads();  // the table is complete before any wave fetches
  }

  const uint32_t klane = k_frag_lane(r32, hi);
  const int tg = lane >> 4, tk = lane & 15;
  const int vkey = 4 * hi + (tk >> 2);
  const int sv = DPAD >= 128 ? ((vkey & 3) << 2) : (((vkey >> 1) & 1) << 2);
  const int vcl = 2 * (tg & 1) + ((tk & 3) >> 1);
  // fp8 V^T (read_vt8): input lane tk of group tg addresses row kr = tk / 2 of
  // its 8-key block, key 8 (kr / 4) + 4 (tg / 2) + kr % 4, chunk 2 db + tg % 2
  // in slot (chunk) ^ 2 kr; the d block enters by an XOR of 32 db per fragment
  const int kr = tk >> 1;
  const uint32_t vlane = KV8 ? TILE_BYTES + (8 * (kr >> 2) + 4 * (tg >> 1) + (kr & 3)) * ROWB + 16 * (tg & 1) +
                                   8 * (tk & 1) + 32 * kr
                              : TILE_BYTES + vkey * ROWB + 16 * vcl + 8 * (tk & 1) + 16 * sv;
  // the modifier pass leaves the scores in log2 units
  const float c = MOD ? 1.0f : score_scale;
  // window of the per-element mask (the modifier instantiation also runs without one)
  const int wleft = (MOD && p.window_left < 0) ? (1 << 30) : p.window_left;
  float slope[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int prow = wrow0 + rb * 32 + r32;
    slope[rb] = MOD ? alibi_slope_l2(p, kvh * g + (prow < nrows ? prow % g : 0)) : 0.0f;
  }

  f32x16_t s[RB];
  uint4 pcur[RB][2], pnew[RB][2];
  bool need[RB];
  float alpha[RB];

  // S^T = K Q^T for both row blocks; each K fragment feeds two MFMAs.  The
  // DMA instructions of the tile being refilled are spread over the k-steps
  // (MODE 1: fast tile, 2: general tile, 0: nothing to load), so that the
  // vector memory unit takes them while the matrix cores are busy.
  auto qk = [&](int stage, auto mode_tag) {
    constexpr int MODE = decltype(mode_tag)::value;
    const uint32_t kls = stage * STAGE_BYTES;
    // 16-bit K: one read per k-step; fp8 K: one 16-byte read per pair of k-steps
    constexpr int NRD = KV8 ? NKK / 2 : NKK;
    uint4 kf[KPF];
#pragma unroll
    for (int i = 0; i < KPF; ++i) kf[i] = *(const uint4*)(smem + kls + k_frag(klane, i));
    uint4 kw = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const int rd = KV8 ? kk >> 1 : kk;
      uint4 a;
      if (!KV8 || (kk & 1) == 0) {
        kw = kf[rd % KPF];
        if (rd + KPF < NRD) kf[rd % KPF] = *(const uint4*)(smem + kls + k_frag(klane, rd + KPF));
      }
      if constexpr (KV8) a = (kk & 1) ? fp8x8_to<QT, F8>(kw.z, kw.w) : fp8x8_to<QT, F8>(kw.x, kw.y);
      else a = kw;
      mfma_s<QT, KV8>(s[0], a, qf[0][kk], kk == 0);
      mfma_s<QT>(s[1], a, qf[1][kk], kk == 0);
      if constexpr (MODE != 0) {
        constexpr int EVERY = NKK / LPW;
        static_assert(NKK % LPW == 0, "DMA spread");
        if (kk % EVERY == EVERY - 1) tl.template part<MODE == 1>(kk / EVERY);
      }
    }
    scores_ready(s[0], s[1]);
  };

  // Causal / key-range / window mask on the scores of the tile starting at
  // key j0; only tiles that reach some row's last key or start before some
  // row's window need it.
  // wave-uniform test: the tile ends past the wave's first row's limit (or
  // the wave has rows past the end), or (window) starts before the window
  // start of its last row
  auto tile_masked = [&](int j0) { return j0 + kKT > wlim || (WIN && j0 < wlo); };
  // value of a masked element: the scaled score -inf, or (CAP, below) the
  // reciprocal +inf that stands for it
  constexpr float kMasked = CAP ? __builtin_huge_valf() : kNegInf;
  auto mask_on = [&](f32x16_t(&sv)[RB], int j0) {
    if constexpr (WIN) {
      if (tile_masked(j0)) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          // key of element r: j0 + 8 (r / 4) + 4 hi + r % 4
          const int t = min(lim[rb], khi) - j0 - 4 * hi, u = lim[rb] - 1 - wleft - j0 - 4 * hi;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int c = 8 * (r >> 2) + (r & 3);
            sv[rb][r] = (c < t && c >= u) ? sv[rb][r] : kMasked;
          }
        }
      }
    } else {
      if (tile_masked(j0)) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const int t = min(lim[rb], khi) - j0 - 4 * hi;
#pragma unroll
          for (int r = 0; r < 16; ++r) sv[rb][r] = (8 * (r >> 2) + (r & 3)) < t ? sv[rb][r] : kMasked;
        }
      }
    }
  };

  auto mask_scores = [&](int j0) { mask_on(s, j0); };

  // Score modifiers of the tile starting at key j0, before its mask: raw score
  // s -> scaled score t = score_scale s -> modified score, in log2 units.
  // The softcap's c' tanh(t / c') (c' the cap in log2 units) is
  // c' - 2 c' / (1 + e^(2 t / c')) with e^(2 t / c') = 2^(ks s): one exp2 and
  // one reciprocal, the limits exact (2^x overflowing to inf gives c',
  // underflowing to 0 gives -c').  The ALiBi bias of element r is -slope dist,
  // dist = (lim - 1) - key, the distance from the row's own key position
  // (rows past the end are masked afterwards).
  // Without ALiBi (CAP) the softcap runs in steps of two scores (cap_step)
  // that the PV product of the previous tile places among its MFMAs, and it
  // stops at the reciprocal r = 1 / (1 + 2^(ks s)): the modified score
  // t = c' - 2 c' r is decreasing in r, so the softmax takes the row minimum
  // of r for its maximum and folds t into its exponent's FMA
  // (2^(t - m) = 2^(-2 c' r + (c' - m))); a masked element is r = +inf.
  constexpr int kCapSteps = CAP ? 16 : 0;
  auto cap_step = [&](int j) {
    const int rb = j & 1, q = j >> 1;
    const float ks = score_scale * p.softcap_k2;
#pragma unroll
    for (int r = 2 * q; r < 2 * q + 2; ++r) s[rb][r] = __builtin_amdgcn_rcpf(1.0f + fast_exp2(s[rb][r] * ks));
  };
  auto mod_mask = [&](int j0) {
    if constexpr (CAP) {
#pragma unroll
      for (int j = 0; j < kCapSteps; ++j) cap_step(j);
    } else if constexpr (VAR == 3) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const float b0 = -slope[rb] * (float)(lim[rb] - 1 - j0 - 4 * hi);
#pragma unroll
        for (int r = 0; r < 16; ++r)
          s[rb][r] = __builtin_fmaf(s[rb][r], score_scale, __builtin_fmaf(slope[rb], (float)(8 * (r >> 2) + (r & 3)), b0));
      }
    } else if constexpr (MOD) {
      // both: the scaled scores through mod_score, one modifier at a time
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[rb][r] *= score_scale;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) mod_scores16(p, s[rb], slope[rb], lim[rb] - 1 - j0 - 4 * hi);
    }
    mask_scores(j0);
  };

  // Online softmax of the (masked) scores in `s` -> pnew, cut into kSmSteps
  // small steps (15 per row block, the two blocks alternating) so that they
  // can be placed between MFMAs: per block, 4 steps of row max, the exchange
  // between lane halves and the rescale decision, the new reference max, 8
  // steps of two exponentials each, and the row-sum update.
  constexpr int kSmSteps = 30;
  float tmax[RB], nref[RB], ls[RB];
  // (CAP: the same steps on r, with minima for maxima)
  auto red3 = [&](float a, float b, float d) { return CAP ? min3f(a, b, d) : max3f(a, b, d); };
  auto sm_on = [&](f32x16_t& sv, int rb, int k) {
    if (k == 0) {  // elements 0..4
      tmax[rb] = red3(red3(sv[0], sv[1], sv[2]), sv[3], sv[4]);
    } else if (k < 3) {  // elements 4k + 1 .. 4k + 4
      tmax[rb] = red3(red3(tmax[rb], sv[4 * k + 1], sv[4 * k + 2]), sv[4 * k + 3], sv[4 * k + 4]);
    } else if (k == 3) {  // elements 13..15
      tmax[rb] = red3(red3(tmax[rb], sv[13], sv[14]), sv[15], sv[15]);
    } else if (k == 4) {
      if constexpr (CAP) tmax[rb] = __builtin_fmaf(min_halves(tmax[rb]), -2.0f * p.softcap_l2, p.softcap_l2);
      else tmax[rb] = max_halves(tmax[rb]) * c;
      need[rb] = __any(tmax[rb] > m[rb] + kTau);
    } else if (k == 5) {
      const float mnew = need[rb] ? max2f(m[rb], tmax[rb]) : m[rb];
      alpha[rb] = (need[rb] && mnew != kNegInf) ? fast_exp2(m[rb] - mnew) : 1.0f;
      m[rb] = mnew;
      nref[rb] = mnew == kNegInf ? 0.0f : -mnew;
      if constexpr (CAP) nref[rb] += p.softcap_l2;
    } else if (k < 14) {
      const int q = k - 6;  // elements 2q, 2q + 1 -> packed word q
      const float ce = CAP ? -2.0f * p.softcap_l2 : c;
      const float e0 = fast_exp2(__builtin_fmaf(sv[2 * q], ce, nref[rb]));
      const float e1 = fast_exp2(__builtin_fmaf(sv[2 * q + 1], ce, nref[rb]));
      const uint32_t pk = Mf<QT>::pack2(e0, e1);
      ((uint32_t*)pnew[rb])[q] = pk;
      // the row sum adds the rounded P that the PV product uses
      ls[rb] = Mf<QT>::sum2(pk, q == 0 ? 0.0f : ls[rb]);
    } else {
      lsum[rb] = __builtin_fmaf(lsum[rb], alpha[rb], ls[rb]);
    }
  };
  auto sm_step = [&](int j) { sm_on(s[j & 1], j & 1, j >> 1); };
  // Keeps the softmax results in the block that computed them (otherwise the
  // compiler sinks the exponentials below the rescale branch).
  auto pin_rb = [&](int rb) {
    typedef int i32x4 __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      i32x4 t = __builtin_bit_cast(i32x4, pnew[rb][ks]);
      asm volatile("" : "+v"(t));
      pnew[rb][ks] = __builtin_bit_cast(uint4, t);
    }
    asm volatile("" : "+v"(lsum[rb]));
  };
  auto pin_softmax = [&]() {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) pin_rb(rb);
  };
  auto softmax = [&]() {
#pragma unroll
    for (int j = 0; j < kSmSteps; ++j) sm_step(j);
    pin_softmax();
  };

  // V^T fragment n = (d block n / 2, key half n % 2)
  auto vt_read = [&](uint32_t vls, int n) {
    if constexpr (KV8) return read_vt8<QT, F8>(smem + ((vls + (n & 1) * 16 * ROWB) ^ ((n >> 1) << 5)));
    else return read_vt(smem + (vls ^ ((n >> 1) << 6)) + (n & 1) * 16 * ROWB, 8 * ROWB);
  };

  // O^T += V^T P^T for the tile in `stage` with the P in pcur.
  auto pv = [&](int stage) {
    const uint32_t vls = stage * STAGE_BYTES + vlane;
    uint4 vf[VPF];
#pragma unroll
    for (int i = 0; i < VPF; ++i) vf[i] = vt_read(vls, i);
#pragma unroll
    for (int st = 0; st < NST2; ++st) {
      const int db = st >> 1, ks = st & 1;
      const uint4 a = vf[st % VPF];
      if (st + VPF < NST2) vf[st % VPF] = vt_read(vls, st + VPF);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) oacc[rb][db] = Mf<QT>::run(a, pcur[rb][ks], oacc[rb][db]);
    }
  };

  // PV of the previous tile with the softmax of the current one placed between
  // its MFMAs by hand (scheduling barriers keep every group where it is).
  // CAP: the softcap steps of the current tile (key j0) come first, then its
  // mask (a wave-uniform branch, taken on the few tiles that need it).
  auto pv_softmax = [&](int pstage, int j0) {
    constexpr int NMF = RB * NST2, NSTEP = kCapSteps + kSmSteps;
    auto step = [&](int j) {
      if (j < kCapSteps) {
        cap_step(j);
        if (j == kCapSteps - 1) mask_scores(j0);
      } else {
        sm_step(j - kCapSteps);
      }
    };
    const uint32_t vls = pstage * STAGE_BYTES + vlane;
    uint4 vf[VPF];
#pragma unroll
    for (int i = 0; i < VPF; ++i) vf[i] = vt_read(vls, i);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int st = 0; st < NST2; ++st) {
      const int db = st >> 1, ks = st & 1;
      const uint4 a = vf[st % VPF];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        oacc[rb][db] = Mf<QT>::run(a, pcur[rb][ks], oacc[rb][db]);
        const int i = st * RB + rb;
#pragma unroll
        for (int j = i * NSTEP / NMF; j < (i + 1) * NSTEP / NMF; ++j) step(j);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (st + VPF < NST2) vf[st % VPF] = vt_read(vls, st + VPF);
      __builtin_amdgcn_sched_barrier(0);
    }
    pin_softmax();
  };

  auto rescale = [&]() {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      if (need[rb]) {
        // the accumulators were last written by MFMAs: wait states before the reads
        asm volatile("s_nop 15\n\ts_nop 7" ::: "memory");
#pragma unroll
        for (int db = 0; db < NDB; ++db) scale_acc_agpr(oacc[rb][db], alpha[rb]);
        acc_fence<NDB>(oacc[rb]);
      }
    }
  };

  drain_visible_loads();

  int issued = 0;
#pragma unroll
  for (int i = 0; i < DIST; ++i)
    if (issued < ntiles) tl.issue(issued, issued), ++issued;
  if (issued < ntiles) tl.fetch(issued);

  // QK of the tile in `stage`, issuing the next tile's loads on the way.
  auto qk_issue = [&](int stage) {
    if (issued < ntiles) {
      tl.begin(issued % NST);
      if (tl.fast()) qk(stage, std::integral_constant<int, 1>());
      else qk(stage, std::integral_constant<int, 2>());
      ++issued;
    } else {
      qk(stage, std::integral_constant<int, 0>());
    }
  };

  if (ntiles > 0) {
    // tile 0: QK and softmax only (no earlier PV to overlap with)
    wait_tiles<LPW, DIST - 1>(issued - 1);
    lds_barrier();
    qk_issue(0);
    mod_mask(kstart);
    softmax();
    if (issued < ntiles) tl.fetch(issued);
    // alpha of the first tile multiplies zero accumulators: nothing to rescale
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      pcur[rb][0] = pnew[rb][0];
      pcur[rb][1] = pnew[rb][1];
    }

    for (int it = 1; it < ntiles; ++it) {
      wait_tiles<LPW, DIST - 1>(issued - it - 1);
      lds_barrier();
      const int j0 = kstart + it * kstep;
      qk_issue(it % NST);
      if constexpr (!CAP) mod_mask(j0);
      pv_softmax((it - 1) % NST, j0);
      rescale();
      if (issued < ntiles) tl.fetch(issued);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        pcur[rb][0] = pnew[rb][0];
        pcur[rb][1] = pnew[rb][1];
      }
    }
    pv((ntiles - 1) % NST);
  }

  epilogue(std::false_type());
}

// LDS of the body: NST stages of one K and one V tile, then the page-id table.
template <int F8, int DPAD, int NST>
constexpr int prefill_w4_lds_bytes() {
  return NST * TileLoader<DPAD, 4, F8 != 0 ? 1 : 2>::STAGE_BYTES + kPidMax * 4;
}

}  // namespace pa

#endif  // PA_PREFILL_W4_BODY_H
