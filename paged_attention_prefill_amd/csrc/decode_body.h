// Split-KV decode pass 1 on MFMA (fp16 / bf16 q; KV of the same dtype, or
// fp8 E5M2 / E4M3 KV for head dims padded to 256).
//
// A decode row has q <= 16 tokens (InferMatrixLab/vllm-rlt PR #128, "Purpose",
// Decode; MTP verify rows q = K+1, 1CatAI/1Cat-vLLM PR #616, "Purpose"), so a
// work group holds one block of 32 GQA-packed query rows of one row and kv head
// over one part of its keys, and the pass is bound by HBM.  What limits it is
// how many bytes each CU keeps in flight and how little the waves wait on one
// another: each wave of the group walks its own 32-key tiles (every fourth
// one) with the whole head dimension, through an LDS ring of its own, and
// keeps its own online-softmax state; nothing in the tile loop waits for
// another wave.  The four states are combined in LDS at the end, in a fixed
// order, into one FP32 partial record per (token, q head, part) that the merge
// pass combines.
#ifndef PA_DECODE_BODY_H
#define PA_DECODE_BODY_H

#include "pa_mfma.h"

namespace pa {

using namespace mf;

// Wave w of the group owns tiles w, w + 4, w + 8, ... of the group's key range,
// NSW stages of (K, V) tiles in its own part of LDS.  The K half of a stage is
// refilled as soon as the wave's S^T = K Q^T has read it and the V half after
// O^T += V^T P^T, so that between one and 2 NSW half-tiles per wave are always
// in flight.  F8 = KV_E5M2 or KV_E4M3: K and V are fp8 (q fp16 or bf16), 8-bit
// tiles in LDS widened to the query's type as the MFMA operands are read.  The
// combined result depends only on the row's own length and the part count.
// Head dims up to 128 are held to 256 registers so that two groups share a CU
// (with one ring stage per wave at D 128: 64 KB of LDS per group): a decode
// batch has many short parts, and a second resident group hides each part's
// first-tile latency.  fp8 KV at D 256 (QLDS) does the same with one stage per
// wave: its query fragments stay in LDS (16 KB after the ring, written once by
// wave 0, read at every k-step) instead of 64 registers per lane, which brings
// a wave to 256 registers and a group to 80 KB of LDS.
// MOD: softcap / ALiBi score modifiers (mod_score) on every visible score.
template <typename QT, int F8, int DPAD, int NSW, bool MOD>
__device__ __forceinline__ void decode_body(const AttnParams& p, int bid, char* smem) {
  constexpr bool KV8 = F8 != 0;
  constexpr int WAVES = 4;
  typedef TileLoader<DPAD, 1, KV8 ? 1 : 2> TL;
  constexpr int ROWB = TL::ROWB;
  constexpr int TILE_BYTES = TL::TILE_BYTES;
  constexpr int STAGE_BYTES = TL::STAGE_BYTES;
  constexpr int HALF = TL::HALF;  // DMA instructions of one K (or V) tile
  constexpr int NKK = DPAD / 16, NDB = DPAD / 32;
  constexpr int RING = WAVES * NSW * STAGE_BYTES;
  constexpr bool QLDS = KV8 && DPAD == 256;
  constexpr int QOFF = RING;  // query fragments (QLDS): k-step kk at QOFF + 1 KB kk, 16 bytes per lane
  static_assert(NSW == 1 || NSW == 2, "ring depth");

  float2 (*mlx)[32] = (float2 (*)[32])(smem + RING);  // per wave and row: (m, l)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hi = lane >> 5, r32 = lane & 31;

  WorkItem wi;
  if (!work_of_block(p, bid, false, wi)) return;
  // (QLDS: held in scalar registers, so that none takes a vector register
  // across the tile loop; the others are free of scratch without that)
  const int qtile = QLDS ? __builtin_amdgcn_readfirstlane(wi.qtile) : wi.qtile;
  const int split = QLDS ? __builtin_amdgcn_readfirstlane(wi.split) : wi.split;
  const int kvh = QLDS ? __builtin_amdgcn_readfirstlane(wi.kvh) : wi.kvh;
  const float score_scale = head_score_scale(p, kvh), out_scale = head_v_scale(p, kvh);
  const int seq = wi.seqpos;

  const int q0 = p.cu_seqlens_q[seq];
  const int qlen = q_end_of(p, seq) - q0;
  const int g = p.group;
  const int nrows = qlen * g;
  const int row0 = qtile * 32;
  if (row0 >= nrows) return;
  const int L = p.seq_lens[seq];
  int klo, khi;
  split_range(p, L, qlen, split, klo, khi);
  const int last_tok = (min(row0 + 32, nrows) - 1) / g;
  const int kend = min(khi, L - qlen + last_tok + 1);

  const int prow = row0 + r32;
  const bool valid = prow < nrows;
  const int tok = valid ? prow / g : 0;
  const int hq = kvh * g + (valid ? prow - (prow / g) * g : 0);
  const int lim = valid ? min(L - qlen + tok + 1, khi) : 0;
  const int lo = window_lo(p, L - qlen + tok);
  const float slope = MOD ? alibi_slope_l2(p, hq) : 0.0f;

  // Q^T (B operand) over the whole head dimension: k-step kk holds d = 16 kk + 8 hi .. +7
  // (fp8 K: the pair of k-steps 2j, 2j+1 covers chunk 2j + hi, low then high half).
  // QLDS: the four waves hold the same rows, so wave 0 alone loads them and
  // stores them to LDS; the barrier before the tile loop publishes them.
  uint4 qf[QLDS ? 1 : NKK];
  if (!QLDS || wave == 0) {
    uint4 qv[NKK];
    const QT* qrow = (const QT*)p.q + ((int64_t)(q0 + tok) * p.num_q_heads + hq) * p.head_dim;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const int d = KV8 ? 32 * (kk >> 1) + 16 * hi + 8 * (kk & 1) : kk * 16 + hi * 8;
      qv[kk] = (valid && d < p.head_dim) ? *(const uint4*)(qrow + d) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      if constexpr (QLDS) *(uint4*)(smem + QOFF + kk * 1024 + lane * 16) = qv[kk];
      else qf[kk] = qv[kk];
    }
  }
  // B operand of k-step kk
  auto qfrag = [&](int kk) {
    if constexpr (QLDS) return *(const uint4*)(smem + QOFF + kk * 1024 + lane * 16);
    else return qf[kk];
  };

  f32x16_t oacc[NDB];
#pragma unroll
  for (int j = 0; j < NDB; ++j) oacc[j] = (f32x16_t)(0.0f);
  float m = kNegInf, lsum = 0.0f;

  const int ntiles = kend > klo ? (kend - klo + kKT - 1) / kKT : 0;
  // Tile t of the part (keys klo + 32 t ..) belongs to wave t % 4 whatever the
  // window: tiles before the earliest window start of the group's rows are
  // skipped, so each wave starts at its first tile at or after t0.  Anchoring
  // the assignment at the part's start keeps a row's bits independent of the
  // rows packed with it (the extra tiles of a verify row are masked no-ops).
  const int t0 = (window_klo(p, klo, khi, L - qlen + row0 / g) - klo) / kKT;
  const int tw = wave + WAVES * ((max(t0 - wave, 0) + WAVES - 1) / WAVES);
  const int nt_w = ntiles > tw ? (ntiles - tw + WAVES - 1) / WAVES : 0;
  const uint32_t wbase = wave * NSW * STAGE_BYTES;
  TL tl;
  tl.init(p, seq, kvh, 0, lane, klo + tw * kKT, kend, (uint32_t)(uintptr_t)(&smem[0]) + wbase);
  tl.set_stride(WAVES * kKT);

  const uint32_t klane = k_frag_lane(r32, hi);
  const int tg = lane >> 4, tk = lane & 15;
  const int vkey = 4 * hi + (tk >> 2);
  const int sv = DPAD >= 128 ? ((vkey & 3) << 2) : (((vkey >> 1) & 1) << 2);
  const int vcl = 2 * (tg & 1) + ((tk & 3) >> 1);
  const int kr = tk >> 1;  // fp8 V^T: see read_vt8
  const uint32_t vlane = KV8 ? TILE_BYTES + (8 * (kr >> 2) + 4 * (tg >> 1) + (kr & 3)) * ROWB + 16 * (tg & 1) +
                                   8 * (tk & 1) + 32 * kr
                              : TILE_BYTES + vkey * ROWB + 16 * vcl + 8 * (tk & 1) + 16 * sv;

  // DMA of the K or V half of the tile begun last (one wave issues all of a
  // tile's instructions), with the non-temporal cache policy: a part's keys
  // are read once, and streaming them past the caches instead of allocating
  // lines for them moves the q=1 row over a 152K-token cache 14 % faster.  K instruction ri fills block ri (keys 8 (ri % 4) ..,
  // chunks 8 (ri / 4) ..), V instruction ri keys KPI ri ..; the per-lane part
  // of the source offset repeats every 2 (K) or 4 (V) instructions and the rest
  // is uniform, so a whole-tile, whole-row load keeps 6 per-lane offsets
  // instead of one per instruction.
  constexpr int CPK = TL::CPK, KPI = TL::KPI, ES = KV8 ? 1 : 2;
  const int st_b = tl.st_b;
  const int dchunks = (p.head_dim * ES) >> 4;
  const bool full_d = dchunks == CPK;
  const int lkey = lane / CPK, lpos = lane % CPK;
  uint32_t klb[2], vlb[4];
#pragma unroll
  for (int r = 0; r < 2; ++r)
    klb[r] = (uint32_t)((lane >> 3) * st_b + 16 * ((lane & 7) ^ (4 * r + (lane >> 4))));
#pragma unroll
  for (int r = 0; r < 4; ++r) vlb[r] = (uint32_t)(lkey * st_b + 16 * swz_v<DPAD, ES>(r * KPI + lkey, lpos));

  auto issue_k = [&]() {
    const uint32_t dst0 = tl.tsb;
    if (full_d && tl.fast()) {
      const char* b = tl.kbase + tl.tA;
#pragma unroll
      for (int ri = 0; ri < HALF; ++ri)
        dma16_sb<true>(b + ((int64_t)(8 * (ri & 3)) * st_b + 128 * (ri >> 2)), klb[ri & 1], dst0 + ri * 1024);
    } else {
#pragma unroll
      for (int ri = 0; ri < HALF; ++ri) {
        int key = 8 * (ri & 3) + (lane >> 3);
        int c = 8 * (ri >> 2) + ((lane & 7) ^ k_swz(key));
        asm volatile("" : "+v"(key), "+v"(c));  // per tile, not hoisted into one register per instruction
        c = min(c, dchunks - 1);
        key = min(key, tl.tlast);  // past the group's last key: reload a valid key (finite data, masked)
        dma16<true>(tl.kbase + (key < tl.tfirst ? tl.tA : tl.tB) + (key * st_b + c * 16), dst0 + ri * 1024);
      }
    }
  };
  auto issue_v = [&]() {
    const uint32_t dst0 = tl.tsb + TILE_BYTES;
    if (full_d && tl.fast()) {
      const char* b = tl.vbase + tl.tA;
#pragma unroll
      for (int ri = 0; ri < HALF; ++ri) dma16_sb<true>(b + (int64_t)(ri * KPI) * st_b, vlb[ri & 3], dst0 + ri * 1024);
    } else {
#pragma unroll
      for (int ri = 0; ri < HALF; ++ri) {
        int key = ri * KPI + lkey;
        int c = swz_v<DPAD, ES>(key, lpos);
        asm volatile("" : "+v"(key), "+v"(c));
        c = min(c, dchunks - 1);
        key = min(key, tl.tlast);
        dma16<true>(tl.vbase + (key < tl.tfirst ? tl.tA : tl.tB) + (key * st_b + c * 16), dst0 + ri * 1024);
      }
    }
  };

  drain_visible_loads();
  int nh = 0;  // half-tiles issued, in the order K(0) V(0) K(1) V(1) ...
#pragma unroll
  for (int i = 0; i < NSW; ++i)
    if (i < nt_w) {
      tl.fetch(i);
      tl.begin(i);
      issue_k();
      issue_v();
      nh += 2;
    }
  // page ids are read one tile ahead of their use, so that the scalar loads
  // are never waited for on the way to a refill
  if (NSW < nt_w) tl.fetch(NSW);
  if constexpr (QLDS) lds_barrier();  // wave 0's query fragments are in LDS

  for (int i = 0; i < nt_w; ++i) {
    const int st = NSW == 1 ? 0 : (i & 1);
    const int j0 = klo + (tw + WAVES * i) * kKT;
    const uint32_t sb = wbase + st * STAGE_BYTES;
    const bool more = i + NSW < nt_w;

    wait_tiles<HALF, 2 * NSW - 1>(nh - 2 * i - 1);  // K(i) landed
    f32x16_t s0 = (f32x16_t)(0.0f), s1 = (f32x16_t)(0.0f);
    if constexpr (KV8) {
#pragma unroll
      for (int kp = 0; kp < NKK / 2; ++kp) {
        const uint4 kw = *(const uint4*)(smem + sb + k_frag(klane, kp));
        s0 = Mf<QT>::run(fp8x8_to<QT, F8>(kw.x, kw.y), qfrag(2 * kp), s0);
        s1 = Mf<QT>::run(fp8x8_to<QT, F8>(kw.z, kw.w), qfrag(2 * kp + 1), s1);
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < NKK; kk += 2) {
        s0 = Mf<QT>::run(*(const uint4*)(smem + sb + k_frag(klane, kk)), qfrag(kk), s0);
        s1 = Mf<QT>::run(*(const uint4*)(smem + sb + k_frag(klane, kk + 1)), qfrag(kk + 1), s1);
      }
    }
    f32x16_t s = s0 + s1;
    if (more) {  // refill the K half of this stage with tile i + NSW (page ids fetched before)
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      tl.begin(st);
      issue_k();
      ++nh;
    }

    // c: the factor from the scores in `s` to log2 units (the modifier pass
    // scales them itself; otherwise the softmax scale enters the row max once
    // and each exponent's FMA)
    const float c = MOD ? 1.0f : score_scale;
    if constexpr (MOD) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] *= score_scale;
      mod_scores16(p, s, slope, L - qlen + tok - j0 - 4 * hi);
    }
    // Only tiles that reach a valid row's last key (or the part's end) or start
    // before its window need the mask: on the others it is the identity for
    // every valid row.  Rows past the group's end (lim 0) have zero queries,
    // so their unmasked scores are finite, and their outputs are never written.
    if (MOD || __any(valid && (j0 + kKT > lim || j0 < lo))) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = j0 + 8 * (r >> 2) + 4 * hi + (r & 3);
        s[r] = (key < lim && key >= lo) ? s[r] : kNegInf;
      }
    }
    // row max in two chains of v_max3, then the other lane half of the row by
    // v_permlane32_swap (no LDS round trip)
    const float ma = max3f(max3f(max3f(s[0], s[1], s[2]), s[3], s[4]), s[5], s[6]);
    const float mb = max3f(max3f(max3f(s[7], s[8], s[9]), s[10], s[11]), s[12], s[13]);
    const float tmax = max_halves(max3f(ma, mb, max2f(s[14], s[15]))) * c;
    // the running max of a row moves on that row's own scores only (a row
    // that does not need it is multiplied by exactly 1), so a row's bits do
    // not depend on the other rows packed with it: a verify row's token
    // equals the q = 1 row of the same length
    const bool upd = tmax > m + kTau;
    if (__any(upd)) {
      const float mnew = upd ? fmaxf(m, tmax) : m;
      const float alpha = (!upd || mnew == kNegInf) ? 1.0f : fast_exp2(m - mnew);
      lsum *= alpha;
#pragma unroll
      for (int j = 0; j < NDB; ++j) oacc[j] *= alpha;
      m = mnew;
    }
    const float nref = m == kNegInf ? 0.0f : -m;
    uint4 pf[2];
    uint32_t* pw = (uint32_t*)pf;
    float ls = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const float e0 = fast_exp2(__builtin_fmaf(s[r], c, nref));
      const float e1 = fast_exp2(__builtin_fmaf(s[r + 1], c, nref));
      const uint32_t pk = Mf<QT>::pack2(e0, e1);
      pw[r >> 1] = pk;
      // the row sum adds the rounded P that the PV product uses
      ls = Mf<QT>::sum2(pk, ls);
    }
    lsum += ls;

    wait_tiles<HALF, 2 * NSW - 1>(nh - 2 * i - 2);  // V(i) landed
    const uint32_t vls = sb + vlane;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        uint4 a;
        if constexpr (KV8) a = read_vt8<QT, F8>(smem + ((vls + ks * 16 * ROWB) ^ (db << 5)));
        else a = read_vt(smem + (vls ^ (db << 6)) + ks * 16 * ROWB, 8 * ROWB);
        oacc[db] = Mf<QT>::run(a, pf[ks], oacc[db]);
      }
    }
    if (more) {  // and its V half
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      issue_v();
      ++nh;
      if (i + NSW + 1 < nt_w) tl.fetch(i + NSW + 1);
    }
  }

  // ---- combine the four waves' states, then the FP32 record of this part.
  // The waves' O go through the ring's LDS, in one round when the ring holds
  // all of them, else in ROUNDS rounds of DBR d blocks (wave w combining d
  // blocks w, w + 4, ... of a round, in the order of the waves either way).
  constexpr int ROUNDS = (WAVES * NDB * 4 * 1024 + RING - 1) / RING;
  constexpr int DBR = NDB / ROUNDS;
  static_assert(NDB % ROUNDS == 0 && WAVES * DBR * 4 * 1024 <= RING, "the O exchange reuses the ring");
  const float ltot = lsum + __shfl_xor(lsum, 32);
  lds_barrier();  // every wave is done with its ring (all of its loads were waited for) and the query fragments
  f32x4_t* ox = (f32x4_t*)smem;
  if constexpr (ROUNDS == 1) {
    if (hi == 0) mlx[wave][r32] = make_float2(m, ltot);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
        ox[((wave * NDB + db) * 4 + rr) * 64 + lane] =
            (f32x4_t){oacc[db][4 * rr], oacc[db][4 * rr + 1], oacc[db][4 * rr + 2], oacc[db][4 * rr + 3]};
    lds_barrier();
    float mv[WAVES], lv[WAVES];
#pragma unroll
    for (int v = 0; v < WAVES; ++v) {
      const float2 t = mlx[v][r32];
      mv[v] = t.x;
      lv[v] = t.y;
    }
    float mall = mv[0];
#pragma unroll
    for (int v = 1; v < WAVES; ++v) mall = fmaxf(mall, mv[v]);
    float av[WAVES];
    float lall = 0.0f;
#pragma unroll
    for (int v = 0; v < WAVES; ++v) {
      av[v] = (mv[v] == kNegInf) ? 0.0f : fast_exp2(mv[v] - mall);
      lall += av[v] * lv[v];
    }
    if (!valid) return;
    const bool empty = (mall == kNegInf) || !(lall > 0.0f);
    const float inv = empty ? 0.0f : out_scale / lall;
    const float lse_nat = empty ? kNegInf : (mall + __log2f(lall)) * 0.69314718055994530942f;
    const int64_t rowidx = (int64_t)(q0 + tok) * p.num_q_heads + hq;
    float* rec = p.partial + (rowidx * p.num_splits + split) * (int64_t)(p.head_dim + 2);
#pragma unroll
    for (int j = 0; j < (NDB + WAVES - 1) / WAVES; ++j) {
      const int db = wave + WAVES * j;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int d = db * 32 + 8 * rr + 4 * hi;
        if (db < NDB && d < p.head_dim) {
          f32x4_t o = (f32x4_t)(0.0f);
#pragma unroll
          for (int v = 0; v < WAVES; ++v) o += av[v] * ox[((v * NDB + db) * 4 + rr) * 64 + lane];
          *(float2*)(rec + d) = make_float2(o[0] * inv, o[1] * inv);
          *(float2*)(rec + d + 2) = make_float2(o[2] * inv, o[3] * inv);
        }
      }
    }
    if (wave == 0 && hi == 0) *(float2*)(rec + p.head_dim) = make_float2(lse_nat, 0.0f);
  } else {
    // every wave reaches every barrier of the rounds: the rows past the
    // group's last one skip only their stores.  The row's indices are formed
    // again here from the lane index and opaque copies of the group's scalars,
    // so that none of them is kept alive across the tile loop.
    int lane_e = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    asm volatile("" : "+v"(lane_e));
    int g_e = __builtin_amdgcn_readfirstlane(g), kvh_e = kvh, q0_e = __builtin_amdgcn_readfirstlane(q0),
        row0_e = __builtin_amdgcn_readfirstlane(row0), nrows_e = __builtin_amdgcn_readfirstlane(nrows),
        split_e = split;
    asm volatile("" : "+s"(g_e), "+s"(kvh_e), "+s"(q0_e), "+s"(row0_e), "+s"(nrows_e), "+s"(split_e));
    const int prow_e = row0_e + (lane_e & 31);
    const int hi_e = lane_e >> 5, r32_e = lane_e & 31;
    if (hi_e == 0) mlx[wave][r32_e] = make_float2(m, ltot);
    const bool valid_e = prow_e < nrows_e;
    const int tok_e = valid_e ? prow_e / g_e : 0;
    const int hq_e = kvh_e * g_e + (valid_e ? prow_e - tok_e * g_e : 0);
    float av[WAVES], inv = 0.0f, lse_nat = kNegInf;
    const int64_t rowidx = (int64_t)(q0_e + tok_e) * p.num_q_heads + hq_e;
    float* rec = p.partial + (rowidx * p.num_splits + split_e) * (int64_t)(p.head_dim + 2);
#pragma unroll
    for (int r = 0; r < ROUNDS; ++r) {
      if (r > 0) lds_barrier();  // the previous round's reads are done
#pragma unroll
      for (int b = 0; b < DBR; ++b)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int db = r * DBR + b;
          ox[((wave * DBR + b) * 4 + rr) * 64 + lane_e] =
              (f32x4_t){oacc[db][4 * rr], oacc[db][4 * rr + 1], oacc[db][4 * rr + 2], oacc[db][4 * rr + 3]};
        }
      lds_barrier();
      if (r == 0) {
        float mv[WAVES], lv[WAVES];
#pragma unroll
        for (int v = 0; v < WAVES; ++v) {
          const float2 t = mlx[v][r32_e];
          mv[v] = t.x;
          lv[v] = t.y;
        }
        float mall = mv[0];
#pragma unroll
        for (int v = 1; v < WAVES; ++v) mall = fmaxf(mall, mv[v]);
        float lall = 0.0f;
#pragma unroll
        for (int v = 0; v < WAVES; ++v) {
          av[v] = (mv[v] == kNegInf) ? 0.0f : fast_exp2(mv[v] - mall);
          lall += av[v] * lv[v];
        }
        const bool empty = (mall == kNegInf) || !(lall > 0.0f);
        inv = empty ? 0.0f : out_scale / lall;
        lse_nat = empty ? kNegInf : (mall + __log2f(lall)) * 0.69314718055994530942f;
      }
#pragma unroll
      for (int j = 0; j < (DBR + WAVES - 1) / WAVES; ++j) {
        const int b = wave + WAVES * j, db = r * DBR + b;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int d = db * 32 + 8 * rr + 4 * hi_e;
          if (valid_e && b < DBR && d < p.head_dim) {
            f32x4_t o = (f32x4_t)(0.0f);
#pragma unroll
            for (int v = 0; v < WAVES; ++v) o += av[v] * ox[((v * DBR + b) * 4 + rr) * 64 + lane_e];
            *(float2*)(rec + d) = make_float2(o[0] * inv, o[1] * inv);
            *(float2*)(rec + d + 2) = make_float2(o[2] * inv, o[3] * inv);
          }
        }
      }
    }
    if (valid_e && wave == 0 && hi_e == 0) *(float2*)(rec + p.head_dim) = make_float2(lse_nat, 0.0f);
  }
}

// LDS of the body: the ring of NSW stages per wave, then the (m, l) exchange,
// which QLDS places over the query fragments (free once the tile loop is done).
template <int F8, int DPAD, int NSW>
constexpr int decode_lds_bytes() {
  constexpr int qbytes = (F8 != 0 && DPAD == 256) ? (DPAD / 16) * 1024 : 0;
  constexpr int mlx = 4 * 32 * (int)sizeof(float2);
  return 4 * NSW * TileLoader<DPAD, 1, F8 != 0 ? 1 : 2>::STAGE_BYTES + (qbytes > mlx ? qbytes : mlx);
}

}  // namespace pa

#endif  // PA_DECODE_BODY_H
