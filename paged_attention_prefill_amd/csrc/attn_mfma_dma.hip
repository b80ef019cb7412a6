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

#include "pa_mfma.h"

namespace pa {

using namespace mf;

// MOD: softcap / ALiBi score modifiers (mod_score) on every visible score.
template <typename QT, int DPAD, int WAVES, int RB, int NST, bool MOD = false>
__global__ __launch_bounds__(64 * WAVES, 1) void attn_mfma_dma_kernel(
    const AttnParams p) {
  constexpr int WROWS = 32 * RB;                // query rows per wave (RB blocks of 32)
  constexpr int ROWS = WROWS * WAVES;
  typedef TileLoader<DPAD, WAVES> TL;
  constexpr int ROWB = TL::ROWB;                // bytes per key row in LDS
  constexpr int TILE_BYTES = TL::TILE_BYTES;    // one K (or V) tile
  constexpr int STAGE_BYTES = TL::STAGE_BYTES;
  constexpr int NKK = DPAD / 16;
  constexpr int NDB = DPAD / 32;
  static_assert(NST * STAGE_BYTES <= 160 * 1024, "LDS");

  __shared__ __attribute__((aligned(1024))) char smem[NST * STAGE_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hi = lane >> 5, r32 = lane & 31;

  WorkItem wi;
  if (!work_of_block(p, blockIdx.x, true, wi)) return;
  // a sequence's last query tiles see the most keys: they are handed out first
  const int qtile = wi.qtile, split = wi.split, kvh = wi.kvh;
  const float score_scale = head_score_scale(p, kvh), out_scale = head_v_scale(p, kvh);
  const int seq = seq_by_rank(p, wi.seqpos, (int*)smem, tid, 64 * WAVES);

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
  const bool wave_active = wrow0 < nrows;
  const int wave_kend = wave_active ? min(khi, L - qlen + (min(wrow0 + WROWS, nrows) - 1) / g + 1) : 0;
  // first tile: the part's start, or the tile of the earliest window start
  const int kfirst = window_klo(p, klo, khi, L - qlen + row0 / g);

  // ---- this lane's rows (one per block) and their Q^T fragments (B operand):
  // lane holds row r32 of each block, d = 16 kk + 8 hi .. +7
  bool valid[RB], rb_on[RB];
  int tok[RB], hq[RB], lim[RB], lo[RB];
  float slope[RB];
  uint4 qf[RB][NKK];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int prow = wrow0 + rb * 32 + r32;
    valid[rb] = prow < nrows;
    rb_on[rb] = wrow0 + rb * 32 < nrows;
    tok[rb] = valid[rb] ? prow / g : 0;
    hq[rb] = kvh * g + (valid[rb] ? prow - (prow / g) * g : 0);
    lim[rb] = valid[rb] ? min(L - qlen + tok[rb] + 1, khi) : 0;
    lo[rb] = window_lo(p, L - qlen + tok[rb]);
    if constexpr (MOD) slope[rb] = alibi_slope_l2(p, hq[rb]);
    const QT* qrow = (const QT*)p.q + ((int64_t)(q0 + tok[rb]) * p.num_q_heads + hq[rb]) * p.head_dim;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const int d = kk * 16 + hi * 8;
      qf[rb][kk] = (valid[rb] && d < p.head_dim) ? *(const uint4*)(qrow + d) : make_uint4(0, 0, 0, 0);
    }
  }

  f32x16_t oacc[RB][NDB];
  float m[RB], lsum[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m[rb] = kNegInf;
    lsum[rb] = 0.0f;
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[rb][db] = (f32x16_t)(0.0f);
  }

  const int ntiles = kend > kfirst ? (kend - kfirst + kKT - 1) / kKT : 0;
  // With score modifiers the tiles run from the highest key down: ALiBi
  // raises a row's biased maximum with every key, so in ascending order the
  // running max would grow and the accumulators be rescaled tile after tile.
  const int kstep = MOD ? -kKT : kKT;
  const int kstart = MOD && ntiles > 0 ? kfirst + (ntiles - 1) * kKT : kfirst;

  // Ping-pong (two waves per SIMD): the late wave group runs each tile's PV
  // one iteration after its softmax, so one group's softmax overlaps the
  // other group's MFMAs.  The late group carries that PV between the barrier
  // and its softmax, the early group its own PV after its softmax and then
  // waits at the next barrier, so the early group alone loads the tiles
  // (all of a tile's DMA instructions, the page ids of the next tile read
  // one tile ahead): the load issue and its scalar-load latency leave the
  // late group's path.
  constexpr bool PP = (WAVES == 8);
  constexpr int IW = PP ? WAVES / 2 : WAVES;  // waves that load the tiles
  const bool late = PP && wave >= WAVES / 2;
  typedef TileLoader<DPAD, IW, 2, false, MOD> TLI;
  constexpr int ILPW = TLI::LPW;  // DMA instructions per loading wave per tile
  TLI tl;
  // (initialised in every wave, so that it stays in registers; the late
  // waves never use it)
  tl.init(p, seq, kvh, late ? wave - IW : wave, lane, kstart, kend, (uint32_t)(uintptr_t)(&smem[0]));

  // ---- per-lane LDS read offsets (loop invariant).  The swizzled chunk index
  // is an XOR of a lane constant with the loop index on bits that do not
  // overlap the row and stage parts of the address, so each read costs one XOR.
  const uint32_t klane = k_frag_lane(r32, hi);
  const int tg = lane >> 4, tk = lane & 15;
  const int vkey = 4 * hi + (tk >> 2);
  const int sv = DPAD >= 128 ? ((vkey & 3) << 2) : (((vkey >> 1) & 1) << 2);
  const int vcl = 2 * (tg & 1) + ((tk & 3) >> 1);
  const uint32_t vlane = TILE_BYTES + vkey * ROWB + 16 * vcl + 8 * (tk & 1) + 16 * sv;

  uint4 pf[RB][2];  // P of the last tile whose softmax ran (kept across iterations by the late group)

  // S^T = K Q^T for this wave's rows, scale + mask, online softmax -> pf
  auto qk_softmax = [&](int stage, int j0) {
    const uint32_t kls = stage * STAGE_BYTES;
    f32x16_t s[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) s[rb] = (f32x16_t)(0.0f);
    // each K fragment read is issued one k-step ahead of the MFMA that uses it
    uint4 a = *(const uint4*)(smem + kls + k_frag(klane, 0));
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      uint4 an;
      if (kk + 1 < NKK) an = *(const uint4*)(smem + kls + k_frag(klane, kk + 1));
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        if (rb_on[rb]) s[rb] = Mf<QT>::run(a, qf[rb][kk], s[rb]);
      a = an;
    }
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float tmax;
      // c: the factor from the scores in `s` to log2 units (the modifier
      // pass scales them itself; otherwise the softmax scale enters the row
      // max once and each exponent's FMA)
      const float c = MOD ? 1.0f : score_scale;
      if constexpr (MOD) {
        if (p.softcap_k2 == 0.0f) {
          // ALiBi alone: the scaled score and its bias -slope (lim - 1 - key)
          // in two FMAs
          const float b0 = -slope[rb] * (float)(L - qlen + tok[rb] - j0 - 4 * hi);
#pragma unroll
          for (int r = 0; r < 16; ++r)
            s[rb][r] = __builtin_fmaf(s[rb][r], score_scale,
                                      __builtin_fmaf(slope[rb], (float)(8 * (r >> 2) + (r & 3)), b0));
        } else {
#pragma unroll
          for (int r = 0; r < 16; ++r) s[rb][r] *= score_scale;
          mod_scores16(p, s[rb], slope[rb], L - qlen + tok[rb] - j0 - 4 * hi);
        }
      }
      // the modified scores are finite, so the mask stays an identity on the
      // tiles that no row's bounds cut
      if (__any(j0 + kKT > lim[rb] || j0 < lo[rb])) {  // causal diagonal / key-range end / window start
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = j0 + 8 * (r >> 2) + 4 * hi + (r & 3);
          s[rb][r] = (key < lim[rb] && key >= lo[rb]) ? s[rb][r] : kNegInf;
        }
      }
      // row max of the 16 scores in two chains of v_max3, then the other lane
      // half of the row by v_permlane32_swap (no LDS round trip)
      const float ma = max3f(max3f(max3f(s[rb][0], s[rb][1], s[rb][2]), s[rb][3], s[rb][4]), s[rb][5], s[rb][6]);
      const float mb = max3f(max3f(max3f(s[rb][7], s[rb][8], s[rb][9]), s[rb][10], s[rb][11]), s[rb][12], s[rb][13]);
      tmax = max_halves(max3f(ma, mb, max2f(s[rb][14], s[rb][15]))) * c;
      if (__any(tmax > m[rb] + kTau)) {
        const float mnew = fmaxf(m[rb], tmax);
        const float alpha = mnew == kNegInf ? 1.0f : fast_exp2(m[rb] - mnew);
        lsum[rb] *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db) oacc[rb][db] *= alpha;
        m[rb] = mnew;
      }
      const float nref = m[rb] == kNegInf ? 0.0f : -m[rb];
      uint32_t* pw = (uint32_t*)pf[rb];
      float ls = 0.0f;
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float e0 = fast_exp2(__builtin_fmaf(s[rb][r], c, nref));
        const float e1 = fast_exp2(__builtin_fmaf(s[rb][r + 1], c, nref));
        const uint32_t pk = Mf<QT>::pack2(e0, e1);
        pw[r >> 1] = pk;
        // the row sum adds the rounded P that the PV product uses
        ls = Mf<QT>::sum2(pk, ls);
      }
      lsum[rb] += ls;
    }
  };

  // O^T += V^T P^T with the P of the tile in `stage`
  auto pv = [&](int stage) {
    const uint32_t vls = stage * STAGE_BYTES + vlane;
    // each V^T fragment (two transpose reads) is issued one step ahead of its MFMA
    uint4 a = read_vt(smem + vls, 8 * ROWB);
#pragma unroll
    for (int st = 0; st < 2 * NDB; ++st) {
      const int db = st >> 1, ks = st & 1;
      uint4 an;
      if (st + 1 < 2 * NDB) {
        const int db1 = (st + 1) >> 1, ks1 = (st + 1) & 1;
        an = read_vt(smem + (vls ^ (db1 << 6)) + ks1 * 16 * ROWB, 8 * ROWB);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        if (rb_on[rb]) oacc[rb][db] = Mf<QT>::run(a, pf[rb][ks], oacc[rb][db]);
      a = an;
    }
  };

  // With ping-pong, tiles are read up to one iteration after their barrier,
  // so the loads run DIST = NST - 2 tiles ahead instead of NST - 1.
  constexpr int DIST = PP ? NST - 2 : NST - 1;

  drain_visible_loads();

  // `issued` advances in every wave (the ring's bookkeeping), the loads
  // only in the loading waves
  int issued = 0;
#pragma unroll
  for (int i = 0; i < DIST; ++i)
    if (issued < ntiles) {
      if (!late) tl.issue(issued, issued);
      ++issued;
    }
  if (!late && issued < ntiles) tl.fetch(issued);

  for (int it = 0; it < ntiles; ++it) {
    // a loading wave waits for its own loads of this tile; the barrier then
    // covers every wave
    if (!late) wait_tiles<ILPW, DIST - 1>(issued - it - 1);
    lds_barrier();
    if (issued < ntiles) {
      if (!late) {
        tl.begin(issued % NST);
        if (tl.fast()) {
#pragma unroll
          for (int n = 0; n < ILPW; ++n) tl.template part<true>(n);
        } else {
#pragma unroll
          for (int n = 0; n < ILPW; ++n) tl.template part<false>(n);
        }
      }
      ++issued;
    }
    const int j0 = kstart + it * kstep;
    const bool live = wave_active && j0 < wave_kend;
    if (late && it > 0 && wave_active && j0 - kstep < wave_kend) pv((it - 1) % NST);
    if (live) qk_softmax(it % NST, j0);
    if (!late && live) pv(it % NST);
    // page ids of the next tile to load, read during the next barrier's wait
    if (!late && issued < ntiles) tl.fetch(issued);
  }
  if (late && ntiles > 0 && wave_active && kstart + (ntiles - 1) * kstep < wave_kend) pv((ntiles - 1) % NST);

  // ---- epilogue
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const float ltot = lsum[rb] + __shfl_xor(lsum[rb], 32);
    if (!valid[rb]) continue;
    float inv, lse_nat;
    final_row(p.write_partial ? nullptr : p.sinks, hq[rb], m[rb], ltot, out_scale, inv, lse_nat);
    const int64_t rowidx = (int64_t)(q0 + tok[rb]) * p.num_q_heads + hq[rb];
    if (p.write_partial) {
      float* rec = p.partial + (rowidx * p.num_splits + split) * (int64_t)(p.head_dim + 2);
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int d = db * 32 + 8 * rr + 4 * hi;
          if (d < p.head_dim) {
            float2 a = {oacc[rb][db][4 * rr + 0] * inv, oacc[rb][db][4 * rr + 1] * inv};
            float2 b = {oacc[rb][db][4 * rr + 2] * inv, oacc[rb][db][4 * rr + 3] * inv};
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
            uint2 v = {Mf<QT>::pack2(oacc[rb][db][4 * rr + 0] * inv, oacc[rb][db][4 * rr + 1] * inv),
                       Mf<QT>::pack2(oacc[rb][db][4 * rr + 2] * inv, oacc[rb][db][4 * rr + 3] * inv)};
            *(uint2*)(orow + d) = v;
          }
        }
      }
      if (p.lse != nullptr && hi == 0) p.lse[rowidx] = lse_nat;
    }
  }
}

// ---- host side -------------------------------------------------------------

namespace {
template <typename QT, int DPAD, int WAVES, int RB, int NST>
struct Cfg {
  static hipError_t launch(const AttnParams& p, int nblocks, hipStream_t stream) {
    if (has_score_mods(p))
      hipLaunchKernelGGL((attn_mfma_dma_kernel<QT, DPAD, WAVES, RB, NST, true>), dim3(nblocks), dim3(64 * WAVES), 0,
                         stream, p);
    else
      hipLaunchKernelGGL((attn_mfma_dma_kernel<QT, DPAD, WAVES, RB, NST, false>), dim3(nblocks), dim3(64 * WAVES), 0,
                         stream, p);
    return hipGetLastError();
  }
  static hipError_t occ(int* n) {
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(n, attn_mfma_dma_kernel<QT, DPAD, WAVES, RB, NST>,
                                                        64 * WAVES, 0);
  }
};

// Head dims padded to 64 or 128: 8 waves x 32 rows, two waves per SIMD in
// ping-pong.  (Padded to 256: the one-wave-per-SIMD kernel of
// attn_prefill_w4.hip, 4 waves x 64 rows.)  Both take 256 rows per group.
template <typename QT, typename F>
hipError_t with_cfg(int dpad, F&& f) {
  switch (dpad) {
    case 64: return f(Cfg<QT, 64, 8, 1, 4>());
    case 128: return f(Cfg<QT, 128, 8, 1, 4>());
    default: return hipErrorInvalidValue;
  }
}
}  // namespace

hipError_t launch_attn_prefill_w4(const AttnParams& p, int q_kind, int kv_kind, int dpad, int nblocks,
                                  hipStream_t stream);
hipError_t prefill_w4_occupancy(int q_kind, int dpad, int* blocks_per_cu);

// Prefill pass 1 for fp16 or bf16 q with KV of the same dtype.
hipError_t launch_attn_mfma_dma(const AttnParams& p, int q_kind, int dpad, int nblocks, hipStream_t stream) {
  if (dpad == 256) return launch_attn_prefill_w4(p, q_kind, q_kind, dpad, nblocks, stream);
  auto go = [&](auto cfg) { return decltype(cfg)::launch(p, nblocks, stream); };
  if (q_kind == KV_F16) return with_cfg<_Float16>(dpad, go);
  if (q_kind == KV_BF16) return with_cfg<__bf16>(dpad, go);
  return hipErrorInvalidValue;
}

hipError_t mfma_dma_occupancy(int q_kind, int dpad, int* blocks_per_cu) {
  if (dpad == 256) return prefill_w4_occupancy(q_kind, dpad, blocks_per_cu);
  auto go = [&](auto cfg) { return decltype(cfg)::occ(blocks_per_cu); };
  if (q_kind == KV_F16) return with_cfg<_Float16>(dpad, go);
  if (q_kind == KV_BF16) return with_cfg<__bf16>(dpad, go);
  return hipErrorInvalidValue;
}

int mfma_dma_rows(int dpad) { return dpad == 64 || dpad == 128 || dpad == 256 ? 256 : 0; }

}  // namespace pa
