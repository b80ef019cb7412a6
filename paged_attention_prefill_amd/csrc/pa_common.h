// Shared device-side definitions of the paged-attention kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

enum KvKind : int { KV_F32 = 0, KV_F16 = 1, KV_BF16 = 2, KV_E5M2 = 3, KV_E4M3 = 4 };

// Keys per tile of the split partition (the decode parts and the prefill parts
// are both cut on this grid).
constexpr int kSplitTile = 32;

// Everything a pass-1 kernel needs; passed by value.
struct AttnParams {
  const void* q;           // [total_q, Hq, D]
  void* out;               // [total_q, Hq, D] (written when num_splits == 1 and !force_partial)
  float* lse;              // [total_q, Hq] nullable
  float* partial;          // [total_q, Hq, S, D + 2] when writing partial records
  const int* cu_seqlens_q; // [B + 1]: sequence b's tokens are [cu[b], cu[b + 1]) ...
  const int* q_end;        // ... or, when set, [cu[b], q_end[b]) (sequences addressed in place)
  const int* seq_lens;     // [B]
  const int* block_tables; // [B, max_pages]
  const void* k_pages;
  const void* v_pages;
  int64_t stride_page, stride_token, stride_head;  // elements
  int num_seqs, max_pages, num_q_heads, num_kv_heads, group, head_dim, page_size;
  int num_splits;
  int part_keys;           // 0: parts cut from each row's own length; > 0: absolute parts of this many keys
  int write_partial;       // 1: records to `partial`; 0: final out/lse
  int qtiles;              // q tiles per (sequence, kv head, key part) in the grid
  int chunks;              // runs per group of q tiles (see work_of_block)
  int run_len;             // q tiles per run
  int num_runs;            // groups * chunks
  float scale_log2;        // scale * k_scale * log2(e)
  float v_scale;
  const float* k_head_scale;  // [Hkv] or null: fp8 K of head h is decode(byte) * k_scale * k_head_scale[h]
  const float* v_head_scale;  // [Hkv] or null
  const float* sinks;         // [Hq] or null: one more logit per q head in the softmax denominator
  int window_left;            // < 0: none; the token at key p sees keys >= p - window_left
  float softcap_k2;           // 2 / softcap (0: no softcap)
  float softcap_l2;           // softcap * log2(e)
  const float* alibi_slopes;  // [Hq] or null (natural units per key of distance)
};

// One past the last query token of sequence `seq` (see AttnParams::q_end).
__device__ __forceinline__ int q_end_of(const AttnParams& p, int seq) {
  return p.q_end != nullptr ? p.q_end[seq] : p.cu_seqlens_q[seq + 1];
}

// First key visible to the token at key position `pos` under the left window.
__device__ __forceinline__ int window_lo(const AttnParams& p, int pos) {
  return p.window_left < 0 ? 0 : max(0, pos - p.window_left);
}

// Start of a work group's tiles: klo moved up to the tile that holds the
// earliest window start of its rows (first_pos = key position of its first
// token), staying on the klo + 32 t grid.
__device__ __forceinline__ int window_klo(const AttnParams& p, int klo, int khi, int first_pos) {
  const int lo = window_lo(p, first_pos);
  if (lo <= klo) return klo;
  const int t = min(lo, khi) - klo;
  return klo + (t / 32) * 32;
}

// Epilogue of an unsplit row: output factor and natural-log lse from the row
// state (m: running max in log2 units of the scaled scores, l: the sum of
// exp2(s - m)), with the head's sink taken into the denominator.
// `sinks` is p.sinks for a final output and null for a partial record.
__device__ __forceinline__ void final_row(const float* sinks, int hq, float m, float l, float out_scale,
                                          float& inv, float& lse_nat) {
  const float kNegInfF = -__builtin_huge_valf();
  if (sinks == nullptr) {
    const bool empty = (m == kNegInfF) || !(l > 0.0f);
    inv = empty ? 0.0f : out_scale / l;
    lse_nat = empty ? kNegInfF : (m + __log2f(l)) * 0.69314718055994530942f;
    return;
  }
  const float sk = sinks[hq] * 1.4426950408889634f;
  const float M = fmaxf(m, sk);
  if (M == kNegInfF) {  // no visible key and a sink of -inf
    inv = 0.0f;
    lse_nat = kNegInfF;
    return;
  }
  const float a = m == kNegInfF ? 0.0f : exp2f(m - M);
  const float l2 = l * a + exp2f(sk - M);
  inv = out_scale * a / l2;
  lse_nat = (M + __log2f(l2)) * 0.69314718055994530942f;
}

// The score factor (scale * k_scale * log2 e, times the head's K scale) and the
// output factor (v_scale times the head's V scale) of kv head h.
__device__ __forceinline__ float head_score_scale(const AttnParams& p, int h) {
  return p.k_head_scale ? p.scale_log2 * p.k_head_scale[h] : p.scale_log2;
}
__device__ __forceinline__ float head_v_scale(const AttnParams& p, int h) {
  return p.v_head_scale ? p.v_scale * p.v_head_scale[h] : p.v_scale;
}

// Arguments of the KV write (new tokens' K and V into their cache pages).
struct KvWriteParams {
  const void* k_new;       // [total_q, Hkv, D], source dtype
  const void* v_new;
  const int* cu_seqlens_q; // [B + 1]: the new tokens of each sequence
  const int* seq_lens;     // [B]: lengths after the write
  const int* block_tables; // [B, max_pages]
  void* k_pages;           // cache pages (cache dtype)
  void* v_pages;
  int64_t stride_page, stride_token, stride_head;  // elements of the cache dtype
  int num_seqs, max_pages, max_q, num_kv_heads, head_dim, page_size;
  float k_scale, v_scale;  // fp8 cache: byte = fp8(x / scale), scale = k_scale * k_head_scale[h]
  const float* k_head_scale;  // [Hkv] or null
  const float* v_head_scale;
};

// Routing of a mixed step (mixed_route.hip): what the route kernels read and
// write, all of the written arrays inside the call's workspace.
struct RouteParams {
  const int* cu;        // [B + 1]
  const int* seq_lens;  // [B]
  const int* bt;        // [B, max_pages]
  const char* q;        // [total_q, row_bytes]
  int B, max_pages, decode_max_q;
  int n_dec, n_pre, nt_cap;  // rows of each class and small-q tokens (the host's count; every write is bounded by them)
  int64_t row_bytes;    // one token's q (or out) row, a multiple of 16
  // small-q rows, compact
  int* dec_cu;          // [n_dec + 1]
  int* dec_seq_lens;    // [n_dec]
  int* dec_src;         // [n_dec]: batch index of compact row i (-1: none)
  int* dec_tok;         // [nt_cap]: batch token of compact token k (-1: none)
  int* dec_bt;          // [n_dec, max_pages]
  char* dec_q;          // [nt_cap, row_bytes]
  // chunks, in place
  int* pre_qs;          // [n_pre] first token
  int* pre_qe;          // [n_pre] one past the last token
  int* pre_seq_lens;    // [n_pre]
  int* pre_src;         // [n_pre]
  int* pre_bt;          // [n_pre, max_pages]
};

// Block index -> work item.  A group is the query tiles of one (sequence
// position, kv head, key part): they all read the same K/V.  Its qtiles tiles
// are cut into `chunks` runs of run_len consecutive tiles, and every run stays
// on one XCD, so each XCD's L2 fetches a group's K/V once per run it holds
// (the host makes whole groups one run where that keeps the 8 XCDs evenly
// loaded).  Work groups go to the 8 XCDs round robin (block b to XCD b % 8);
// row r of 8 runs is dealt to the XCDs rotated by r, so a pattern of busy and
// empty runs that repeats every 2, 4 or 8 runs (a static grid sized for the
// longest sequence leaves such holes behind the shorter ones) is spread over
// all XCDs.  Within a run the tiles come in order; `reverse` hands out a
// group's last tiles (the ones that see the most keys) first.  Returns false
// for a padding block.  The mapping is a bijection on the padded grid, so it
// only affects locality and balance.
struct WorkItem {
  int qtile, split, kvh, seqpos;  // seqpos: position in the grid's sequence order
};
__device__ __forceinline__ bool work_of_block(const AttnParams& p, int bid, bool reverse, WorkItem& wi) {
  const int R = p.run_len;
  const int xcd = bid & 7, k = bid >> 3;
  const int row = k / R, pos = k - row * R;
  const int run = row * 8 + ((xcd - row) & 7);
  if (run >= p.num_runs) return false;
  int grp = run / p.chunks;
  const int qi = (run - grp * p.chunks) * R + pos;
  if (qi >= p.qtiles) return false;
  wi.qtile = reverse ? p.qtiles - 1 - qi : qi;
  wi.split = grp % p.num_splits;
  grp /= p.num_splits;
  wi.kvh = grp % p.num_kv_heads;
  wi.seqpos = grp / p.num_kv_heads;
  return true;
}

// Sequence taken at position r of the grid's sequence order: longest first
// (seq_lens descending, ties by index), so that the work groups of the longest
// sequences, which set the end of a varlen call, are handed out before the
// short ones.  Every thread of the group calls it (it holds two barriers);
// `lds` is at least kRankMaxSeqs + 1 ints of LDS that the group does not
// otherwise use yet.  Beyond kRankMaxSeqs sequences the order is the given one.
constexpr int kRankMaxSeqs = 256;
__device__ __forceinline__ int seq_by_rank(const AttnParams& p, int r, int* lds, int tid, int nthreads) {
  const int B = p.num_seqs;
  if (B <= 1 || B > kRankMaxSeqs) return r;
  for (int b = tid; b < B; b += nthreads) lds[b] = p.seq_lens[b];
  __syncthreads();
  if (tid < B) {
    const int L = lds[tid];
    int rank = 0;
    for (int j = 0; j < B; ++j) {
      const int Lj = lds[j];
      rank += (Lj > L) || (Lj == L && j < tid);
    }
    if (rank == r) lds[kRankMaxSeqs] = tid;
  }
  __syncthreads();
  // the same word in every lane: kept in a scalar register, so that what is
  // derived from it (the sequence's offsets and lengths) is scalar too
  const int seq = __builtin_amdgcn_readfirstlane(lds[kRankMaxSeqs]);
  __syncthreads();  // the scratch is free again
  return seq;
}

// Key range [lo, hi) of part `s` of a sequence with L keys and qlen query
// tokens.  part_keys == 0: S parts of whole kSplitTile-key tiles cut from the
// keys the sequence can see, [base, L) with base the tile that holds its first
// token's window start (0 without a window): per = ceil(ceil((L - base) / T) /
// S) tiles each, a function of the sequence's own length (and window).
// part_keys > 0 (a multiple of T): absolute parts [s * part_keys,
// (s + 1) * part_keys), the last part (s = S - 1) running on to L, so that the
// boundaries do not depend on L at all.
__device__ __forceinline__ void split_range(const AttnParams& p, int L, int qlen, int s, int& lo, int& hi) {
  const int S = p.num_splits;
  long long a, b;
  if (p.part_keys > 0) {
    a = (long long)s * p.part_keys;
    b = s == S - 1 ? (long long)L : a + p.part_keys;
  } else {
    const int base = p.window_left < 0 ? 0 : (max(0, L - qlen - p.window_left) / kSplitTile) * kSplitTile;
    const int tiles = (L - base + kSplitTile - 1) / kSplitTile;
    const int per = (tiles + S - 1) / S;
    a = base + (long long)s * per * kSplitTile;
    b = a + (long long)per * kSplitTile;
  }
  lo = (int)(a < L ? a : L);
  hi = (int)(b < L ? b : L);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ALiBi slope of q head hq in the kernels' log2 units (0 without ALiBi).
__device__ __forceinline__ float alibi_slope_l2(const AttnParams& p, int hq) {
  return p.alibi_slopes == nullptr ? 0.0f : p.alibi_slopes[hq] * 1.4426950408889634f;
}

// Score modifiers on a scaled score t = log2(e) * z of a visible key (z = the
// natural-unit logit).  Softcap z -> c tanh(z / c) is t -> c' tanh(t / c')
// with c' = c log2(e), and tanh(y) = 1 - 2 / (1 + e^(2y)), where e^(2 t / c') =
// 2^(2 t / c): one exp2 and one reciprocal (the limits come out exact: 2^x
// overflowing to inf gives 1, underflowing to 0 gives -1).  Then ALiBi: t
// loses slope_l2 * dist, dist = p - j for the token at key position p.
__device__ __forceinline__ float mod_score(const AttnParams& p, float t, float slope_l2, int dist) {
  if (p.softcap_k2 != 0.0f) {
    const float e = fast_exp2(t * p.softcap_k2);
    t = p.softcap_l2 * __builtin_fmaf(-2.0f, __builtin_amdgcn_rcpf(1.0f + e), 1.0f);
  }
  return __builtin_fmaf(-slope_l2, (float)dist, t);
}

// The two modifiers one at a time, for loops that test each flag once per tile.
__device__ __forceinline__ float softcap_score(const AttnParams& p, float t) {
  const float e = fast_exp2(t * p.softcap_k2);
  return p.softcap_l2 * __builtin_fmaf(-2.0f, __builtin_amdgcn_rcpf(1.0f + e), 1.0f);
}

// Softcap then ALiBi on the 16 scaled scores of one lane of a 32x32 MFMA
// score tile (element r: key 8 (r / 4) + r % 4 after the lane's first key,
// whose distance from the row's key position is d0).  Each modifier is tested
// once per fragment; masked elements are selected away afterwards.
template <typename V16>
__device__ __forceinline__ void mod_scores16(const AttnParams& p, V16& s, float slope_l2, int d0) {
  if (p.softcap_k2 != 0.0f) {
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = softcap_score(p, s[r]);
  }
  if (p.alibi_slopes != nullptr) {
    const float a = -slope_l2 * (float)d0;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] += __builtin_fmaf(slope_l2, (float)(8 * (r >> 2) + (r & 3)), a);
  }
}

// Whether a call carries score modifiers (they select the kernels' MOD instantiations).
inline bool has_score_mods(const AttnParams& p) { return p.softcap_k2 != 0.0f || p.alibi_slopes != nullptr; }

// Two fp8 E4M3 bytes (byte 2 w and 2 w + 1 of x) -> two fp16 in one 32-bit
// word, lower byte in the lower half: the gfx950 conversion with a scale of 1
// (every E4M3 value is exact in fp16).
template <bool HI>
__device__ __forceinline__ uint32_t e4m3x2_to_f16x2(uint32_t x) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x, 1.0f, HI));
}

// Two fp8 bytes (byte 2 w and 2 w + 1 of x) -> two bf16 in one 32-bit word,
// lower byte in the lower half: the gfx950 conversions with a scale of 1
// (every E5M2 and every E4M3 value is exact in bf16).
template <int F8, bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t x) {
  if constexpr (F8 == KV_E4M3)
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, HI));
  else
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(x, 1.0f, HI));
}

// fp8 E5M2 byte -> fp16 bits: E5M2 is the high byte of an fp16 with the same
// sign/exponent/mantissa layout, so the conversion is exact.
__device__ __forceinline__ void e5m2x4_to_f16x4(uint32_t x, uint32_t& lo, uint32_t& hi) {
  lo = ((x & 0x000000FFu) << 8) | ((x & 0x0000FF00u) << 16);
  hi = ((x & 0x00FF0000u) >> 8) | (x & 0xFF000000u);
}

}  // namespace pa
