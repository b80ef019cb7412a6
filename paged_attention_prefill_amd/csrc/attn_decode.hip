// Split-KV decode pass 1 on MFMA (fp16 / bf16): the head dimension of every
// tile is split over the four waves of a work group.
//
// A decode row has q <= 16 tokens (InferMatrixLab/vllm-rlt PR #128, "Purpose",
// Decode; MTP verify rows q = K+1, 1CatAI/1Cat-vLLM PR #616, "Purpose"), so a
// work group holds one block of 32 GQA-packed query rows of one row and kv head
// over one part of its keys.  With so few rows the attention is bound by HBM,
// and a single wave doing the whole tile's math would stall on its own LDS
// operand reads; instead all four waves work on every 32-key tile:
//   * wave w forms the partial S^T = K Q^T over its quarter of the head
//     dimension and leaves it in LDS;
//   * after a barrier every wave adds the four partials in the same order (so
//     all waves hold bit-identical scores), runs the same online softmax, and
//     accumulates O^T += V^T P^T for its own quarter of the output columns.
// The K/V tiles come through the same LDS DMA ring as the prefill kernel.  The
// ring is kept shallow (one or two tiles in flight) so that two to four groups
// share a CU: a group's own chain of LDS reads, MFMAs and softmax sets its
// rate, and more resident groups hide it better than a deeper ring does.  The
// output is an FP32 partial record per (token, q head, part) that the merge
// pass combines.

#include "pa_mfma.h"

namespace pa {

using namespace mf;

// KV8: K and V are fp8 E5M2 (q fp16): 8-bit tiles in LDS, widened to fp16 as
// the MFMA operands are read (same layouts as the prefill kernel's fp8 path).
template <typename QT, bool KV8, int DPAD, int NST>
__global__ __launch_bounds__(256) void attn_decode_kernel(const AttnParams p) {
  constexpr int WAVES = 4;
  typedef TileLoader<DPAD, WAVES, KV8 ? 1 : 2> TL;
  constexpr int ROWB = TL::ROWB;
  constexpr int TILE_BYTES = TL::TILE_BYTES;
  constexpr int STAGE_BYTES = TL::STAGE_BYTES;
  constexpr int LPW = TL::LPW;
  constexpr int NKK = DPAD / 16, NDB = DPAD / 32;
  constexpr int KKW = NKK / WAVES;            // k-steps of S^T per wave
  constexpr int NDBW = (NDB + WAVES - 1) / WAVES;  // output d blocks per wave
  constexpr int DIST = NST - 1;

  __shared__ __attribute__((aligned(1024))) char smem[NST * STAGE_BYTES];
  __shared__ f32x4_t sx[WAVES][4][64];  // partial scores: [wave][quarter][lane]

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
  const int row0 = qtile * 32;
  if (row0 >= nrows) return;
  const int L = p.seq_lens[seq];
  int klo, khi;
  split_range(L, p.num_splits, split, klo, khi);
  const int last_tok = (min(row0 + 32, nrows) - 1) / g;
  const int kend = min(khi, L - qlen + last_tok + 1);

  const int prow = row0 + r32;
  const bool valid = prow < nrows;
  const int tok = valid ? prow / g : 0;
  const int hq = kvh * g + (valid ? prow - (prow / g) * g : 0);
  const int lim = valid ? min(L - qlen + tok + 1, khi) : 0;

  // this wave's quarter of Q^T (B operand), kk in [wave*KKW, +KKW): d = 16 kk + 8 hi .. +7
  // (fp8 K: the pair of k-steps 2j, 2j+1 covers chunk 2j + hi, low then high half)
  static_assert(!KV8 || KKW % 2 == 0, "fp8 K is read in pairs of k-steps");
  uint4 qf[KKW];
  {
    const QT* qrow = (const QT*)p.q + ((int64_t)(q0 + tok) * p.num_q_heads + hq) * p.head_dim;
#pragma unroll
    for (int i = 0; i < KKW; ++i) {
      const int kk = wave * KKW + i;
      const int d = KV8 ? 32 * (kk >> 1) + 16 * hi + 8 * (kk & 1) : kk * 16 + hi * 8;
      qf[i] = (valid && d < p.head_dim) ? *(const uint4*)(qrow + d) : make_uint4(0, 0, 0, 0);
    }
  }

  f32x16_t oacc[NDBW];
#pragma unroll
  for (int j = 0; j < NDBW; ++j) oacc[j] = (f32x16_t)(0.0f);
  float m = kNegInf, lsum = 0.0f;

  const int ntiles = kend > klo ? (kend - klo + kKT - 1) / kKT : 0;
  TL tl;
  tl.init(p, seq, kvh, wave, lane, klo, kend, (uint32_t)(uintptr_t)(&smem[0]));

  const uint32_t klane = k_frag_lane(r32, hi);
  const int tg = lane >> 4, tk = lane & 15;
  const int vkey = 4 * hi + (tk >> 2);
  const int sv = DPAD >= 128 ? ((vkey & 3) << 2) : (((vkey >> 1) & 1) << 2);
  const int vcl = 2 * (tg & 1) + ((tk & 3) >> 1);
  const int kr = tk >> 1;  // fp8 V^T: see read_vt8
  const uint32_t vlane = KV8 ? TILE_BYTES + (8 * (kr >> 2) + 4 * (tg >> 1) + (kr & 3)) * ROWB + 16 * (tg & 1) +
                                   8 * (tk & 1) + 32 * kr
                              : TILE_BYTES + vkey * ROWB + 16 * vcl + 8 * (tk & 1) + 16 * sv;

  drain_visible_loads();
  int issued = 0;
#pragma unroll
  for (int i = 0; i < DIST; ++i)
    if (issued < ntiles) tl.issue(issued, issued), ++issued;

  for (int it = 0; it < ntiles; ++it) {
    wait_tiles<LPW, DIST - 1>(issued - it - 1);
    lds_barrier();  // tile landed for all waves; previous partial scores consumed
    if (issued < ntiles) tl.issue(issued, issued % NST), ++issued;
    const int stage = it % NST;
    const int j0 = klo + it * kKT;
    const uint32_t sb = stage * STAGE_BYTES;

    // partial S^T over this wave's quarter of the head dimension
    f32x16_t s = (f32x16_t)(0.0f);
    uint4 kw = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < KKW; ++i) {
      const int kk = wave * KKW + i;
      uint4 a;
      if constexpr (KV8) {
        if ((i & 1) == 0) kw = *(const uint4*)(smem + sb + klane + (kk >> 1) * kKStep);
        a = (i & 1) ? e5m2x8_to_f16(kw.z, kw.w) : e5m2x8_to_f16(kw.x, kw.y);
      } else {
        a = *(const uint4*)(smem + sb + klane + kk * kKStep);
      }
      s = Mf<QT>::run(a, qf[i], s);
    }
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) sx[wave][q4][lane] = (f32x4_t){s[4 * q4], s[4 * q4 + 1], s[4 * q4 + 2], s[4 * q4 + 3]};
    lds_barrier();
    // full scores, summed in the same order by every wave
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      f32x4_t t = sx[0][q4][lane];
#pragma unroll
      for (int v = 1; v < WAVES; ++v) t += sx[v][q4][lane];
      s[4 * q4] = t[0];
      s[4 * q4 + 1] = t[1];
      s[4 * q4 + 2] = t[2];
      s[4 * q4 + 3] = t[3];
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
      for (int j = 0; j < NDBW; ++j) oacc[j] *= alpha;
      m = mnew;
    }
    const float mref = m == kNegInf ? 0.0f : m;
    uint4 pf[2];
    uint32_t* pw = (uint32_t*)pf;
    float ls = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const float e0 = fast_exp2(s[r] - mref), e1 = fast_exp2(s[r + 1] - mref);
      ls += e0 + e1;
      pw[r >> 1] = Mf<QT>::pack2(e0, e1);
    }
    lsum += ls;

    // O^T += V^T P^T for this wave's output columns
    const uint32_t vls = sb + vlane;
#pragma unroll
    for (int j = 0; j < NDBW; ++j) {
      const int db = wave * NDBW + j;
      if (db < NDB) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          uint4 a;
          if constexpr (KV8) a = read_vt8(smem + ((vls + ks * 16 * ROWB) ^ (db << 5)));
          else a = read_vt(smem + (vls ^ (db << 6)) + ks * 16 * ROWB, 8 * ROWB);
          oacc[j] = Mf<QT>::run(a, pf[ks], oacc[j]);
        }
      }
    }
  }

  // ---- epilogue: FP32 record (o normalised, lse, pad); this wave's columns
  const float ltot = lsum + __shfl_xor(lsum, 32);
  if (!valid) return;
  const bool empty = (m == kNegInf) || !(ltot > 0.0f);
  const float inv = empty ? 0.0f : p.v_scale / ltot;
  const float lse_nat = empty ? kNegInf : (m + __log2f(ltot)) * 0.69314718055994530942f;
  const int64_t rowidx = (int64_t)(q0 + tok) * p.num_q_heads + hq;
  float* rec = p.partial + (rowidx * p.num_splits + split) * (int64_t)(p.head_dim + 2);
#pragma unroll
  for (int j = 0; j < NDBW; ++j) {
    const int db = wave * NDBW + j;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int d = db * 32 + 8 * rr + 4 * hi;
      if (db < NDB && d < p.head_dim) {
        float2 a = {oacc[j][4 * rr + 0] * inv, oacc[j][4 * rr + 1] * inv};
        float2 b = {oacc[j][4 * rr + 2] * inv, oacc[j][4 * rr + 3] * inv};
        *(float2*)(rec + d) = a;
        *(float2*)(rec + d + 2) = b;
      }
    }
  }
  if (wave == 0 && hi == 0) {
    float2 t = {lse_nat, 0.0f};
    *(float2*)(rec + p.head_dim) = t;
  }
}

// ---- host side -------------------------------------------------------------

namespace {
template <typename QT, bool KV8, int DPAD, int NST>
hipError_t launch_dec(const AttnParams& p, int nblocks, hipStream_t stream) {
  hipLaunchKernelGGL((attn_decode_kernel<QT, KV8, DPAD, NST>), dim3(nblocks), dim3(256), 0, stream, p);
  return hipGetLastError();
}
template <typename QT>
hipError_t launch_dec_d(const AttnParams& p, int dpad, int nblocks, hipStream_t stream) {
  switch (dpad) {
    case 64: return launch_dec<QT, false, 64, 3>(p, nblocks, stream);
    case 128: return launch_dec<QT, false, 128, 2>(p, nblocks, stream);
    case 256: return launch_dec<QT, false, 256, 2>(p, nblocks, stream);
    default: return hipErrorInvalidValue;
  }
}
}  // namespace

// Decode pass 1, 32 rows per group: fp16 / bf16 q with KV of the same dtype
// (kv_kind = q_kind), or fp16 q with fp8 E5M2 KV for head dims padded to 256.
hipError_t launch_attn_decode(const AttnParams& p, int q_kind, int kv_kind, int dpad, int nblocks,
                              hipStream_t stream) {
  if (kv_kind == KV_E5M2) {
    if (q_kind == KV_F16 && dpad == 256) return launch_dec<_Float16, true, 256, 3>(p, nblocks, stream);
    return hipErrorInvalidValue;
  }
  if (q_kind != kv_kind) return hipErrorInvalidValue;
  if (q_kind == KV_F16) return launch_dec_d<_Float16>(p, dpad, nblocks, stream);
  if (q_kind == KV_BF16) return launch_dec_d<__bf16>(p, dpad, nblocks, stream);
  return hipErrorInvalidValue;
}

int decode_rows_per_group() { return 32; }

}  // namespace pa
