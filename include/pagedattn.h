/*
 * pagedattn.h -- C ABI of libpagedattn.so: paged softmax attention over a
 * block-table KV cache, hand-written HIP kernels for AMD gfx950 (MI355X).
 *
 * What the calls compute (the pages this library follows):
 *  - pa_paged_prefill: the varlen paged prefill of InferMatrixLab/vllm-rlt
 *    PR #128 ("Purpose", Prefill): packed queries addressed by cu_seqlens_q,
 *    one block table per sequence, causal mask aligned bottom-right (query
 *    token i of a sequence with Q query tokens and L keys sees keys
 *    j < L - Q + i + 1), GQA, exact products for FP32 inputs; optionally the
 *    key range of every query tile is split in whole tiles and merged by
 *    log-sum-exp (1CatAI/1Cat-vLLM PR #1279, commit 5, split-KV by waves).
 *  - pa_split_kv_decode: the split-KV decode of PR #128 ("Purpose", Decode)
 *    for small-q rows (q = 1, or an MTP verify row q = K+1 as in
 *    1CatAI/1Cat-vLLM PR #616, "Purpose"): each row's keys are cut into
 *    num_splits equal parts of whole 32-key tiles, a function of the row's own
 *    length only, each part writes an FP32 partial softmax state, and a second
 *    launch merges them.  A row's output is bitwise independent of the other
 *    rows in the call for fixed (num_splits, max_q_per_row, dtypes, head_dim).
 *  - pa_merge_states: that second pass on its own (also used by prefill
 *    splits).
 *  - fp8 KV (1CatAI/1Cat-vLLM PR #616, fp8_e5m2 paragraph of "Test Result";
 *    the same page's "Test Plan" names an e4m3 path too): E5M2 or E4M3 bytes
 *    are dequantized inside the kernels, value = decode(byte) * k_scale (or
 *    v_scale); q and out stay fp16 or bf16 (every fp8 value widens exactly
 *    to either).
 *  - pa_split_kv_decode_fixed: decode with absolute part boundaries, so that
 *    a verify row equals serial decoding bit for bit.
 *  - pa_write_kv: the new tokens' K/V into their pages (fp8: quantised).
 *
 * Conventions shared by all calls
 *  - Every data pointer is DEVICE memory owned by the caller; the library
 *    allocates nothing, keeps no state besides a per-device cache of the
 *    compute-unit count, and is safe to call from several threads.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = default
 *    stream).  The launch grid depends only on the host scalars, so the calls
 *    can be captured in a HIP graph.
 *  - Device-side metadata (cu_seqlens_q, seq_lens, block_tables) is trusted:
 *    checking it would need a device-to-host copy.  pa_validate_metadata
 *    checks host copies of it.
 *  - Layouts: q and out are [total_q, num_q_heads, head_dim], contiguous.
 *    lse is [total_q, num_q_heads] float32, natural log, -inf for a row that
 *    sees no key (its output is 0).  cu_seqlens_q is int32 [num_seqs + 1]
 *    with cu_seqlens_q[0] = 0 and cu_seqlens_q[num_seqs] = total_q;
 *    seq_lens is int32 [num_seqs] (keys of the sequence, the chunk's own keys
 *    included: the caller writes the chunk's K/V into the pages first);
 *    block_tables is int32 [num_seqs, max_pages_per_seq], row-major.
 *  - KV pages: element (page p, slot s, kv head h, dim d) of K is at
 *    k_pages + p*stride_page + s*stride_token + h*stride_head + d (in
 *    elements of the KV dtype); V uses the same geometry.  The layouts
 *    [pages, page_size, Hkv, D] and [pages, Hkv, page_size, D] are both
 *    expressible.  page_size is any multiple of 16 (1CatAI/1Cat-vLLM PR #616,
 *    the any-page gate).  Strides and base pointers must be 16-byte aligned.
 *  - Query head hq reads kv head hq / (num_q_heads / num_kv_heads).
 *  - Supported dtypes: (q, KV) = (F32, F32), (F16, F16), (BF16, BF16),
 *    (F16 or BF16, FP8_E5M2), (F16 or BF16, FP8_E4M3); out has q's dtype.
 *    head_dim is a multiple of 16 in [16, 256].
 *
 * Errors: every call returns PA_OK (0) or a negative pa_status; nothing is
 * launched when an argument is rejected.  pa_last_error() gives a message
 * for the last failure on the calling thread.
 */
#ifndef PAGEDATTN_H
#define PAGEDATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_VERSION 3
#define PA_DECODE_MAX_Q 16       /* largest q of a decode / verify row */
#define PA_DECODE_SPLIT_TILE 32  /* keys per tile of the split partition */
#define PA_PREFILL_MAX_AUTO_SPLITS 16

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_INVALID_ARGUMENT = -1, /* null pointer, negative size, bad stride */
  PA_ERR_UNSUPPORTED = -2,      /* dtype pair, head_dim, page_size, GQA ratio, q > 16 */
  PA_ERR_WORKSPACE = -3,        /* workspace missing or too small */
  PA_ERR_HIP = -4,              /* HIP runtime / launch failure */
  PA_ERR_METADATA = -5          /* pa_validate_metadata found an inconsistency */
} pa_status;

typedef enum pa_dtype {
  PA_F32 = 0,
  PA_F16 = 1,
  PA_BF16 = 2,
  PA_FP8_E5M2 = 3,  /* OCP E5M2 bytes: bias 15, infinities and NaNs */
  PA_FP8_E4M3 = 4   /* OCP E4M3 ("fn") bytes: bias 7, no infinities, 0x7F / 0xFF NaN, max 448 */
} pa_dtype;

/* One paged KV cache (K and V share the geometry). Host struct, device pointers. */
typedef struct pa_kv_cache {
  const void *k_pages;   /* device, caller-owned */
  const void *v_pages;   /* device, caller-owned */
  int64_t stride_page;   /* elements between pages */
  int64_t stride_token;  /* elements between slots of a page */
  int64_t stride_head;   /* elements between kv heads */
  int32_t num_pages;
  int32_t page_size;     /* multiple of 16 */
  int32_t num_kv_heads;
  int32_t head_dim;      /* multiple of 16 in [16, 256]; contiguous */
  int32_t dtype;         /* pa_dtype */
  float k_scale;         /* fp8 KV only (must be 1 otherwise): value = decode(byte) * scale */
  float v_scale;
  /* fp8 KV only, nullable: device float[num_kv_heads] per-head factors, value =
   * decode(byte) * k_scale * k_head_scales[h] (V likewise).  Trusted like the
   * other device data: positive and finite. */
  const float *k_head_scales;
  const float *v_head_scales;
} pa_kv_cache;

/*
 * Optional variants of the attention calls (the *_ex entry points).  The
 * pages' Turing prefill gate lists sinks and sliding windows among what it
 * does not take (1CatAI/1Cat-vLLM PR #1279, commit 1, the selection rule);
 * here they are options of every kernel.
 *   sinks: device float[num_q_heads] or NULL.  Head h's softmax gets one more
 *     logit sinks[h] (natural units, compared with scale * q.k) that carries
 *     no value: o = sum_j e^{s_j} v_j / (sum_j e^{s_j} + e^{sinks[h]}), lse =
 *     log(sum_j e^{s_j} + e^{sinks[h]}); a row with no visible key gets o = 0,
 *     lse = sinks[h].  Applied once per row, in the unsplit epilogue or in the
 *     merge; the FP32 records of pass 1 (out = NULL) stay sink-free.
 *   window_left: < 0 for none; otherwise the token at key position p (p =
 *     seq_len - q_len + i) sees keys p - window_left .. p only.
 * The same gate lists logit softcapping and ALiBi; the pages define neither,
 * and these are FlashAttention's conventions, applied to the natural-unit
 * logit z = scale * q.k of every visible key before the softmax:
 *   softcap: > 0 (finite): z -> softcap * tanh(z / softcap); 0: none.
 *   alibi_slopes: device float[num_q_heads] or NULL; for head h, the token
 *     at key position p and key j <= p: z -> z - alibi_slopes[h] * (p - j)
 *     (after the softcap).
 * The score modifiers run in a separate instantiation of each kernel (the
 * default one is unchanged); tanh is evaluated as 1 - 2 / (1 + e^(2x)) with
 * the hardware exp2 and reciprocal, so the softcapped logits carry an
 * absolute error of a few fp32 ulps of softcap.
 */
typedef struct pa_attn_options {
  const float *sinks;
  int32_t window_left;
  float softcap;
  const float *alibi_slopes;
} pa_attn_options;

/*
 * Varlen paged prefill (InferMatrixLab/vllm-rlt PR #128, "Purpose", Prefill).
 *   q [total_q, num_q_heads, head_dim] (q_dtype); out same shape and dtype;
 *   lse nullable; scale (positive, finite) multiplies q.k (k_scale, also
 *   positive, folded in for fp8): the kernels take row maxima of the unscaled
 *   scores, which commutes with a positive scale only.
 *   max_seqlen_q bounds every cu_seqlens_q[b+1] - cu_seqlens_q[b] (it sizes the
 *   static grid).  num_kv_splits: 1 = no key split; 2..64 = split every query
 *   tile's keys into that many whole-tile parts and merge; 0 = choose by how
 *   many full waves of work groups fill the device (1CatAI/1Cat-vLLM PR #1279,
 *   commit 5): up to 4 parts when the query tiles alone cover the device, up
 *   to PA_PREFILL_MAX_AUTO_SPLITS when they do not, and never more than the
 *   workspace holds (no workspace: 1).  The choice depends on the shape of the
 *   call and the device, so num_kv_splits = 0 is not batch-invariant; any
 *   fixed count is.  With num_kv_splits >= 2 the workspace must hold
 *   pa_prefill_workspace_bytes(total_q, num_q_heads, head_dim, num_kv_splits)
 *   bytes of device memory (8-byte aligned); pa_prefill_workspace_bytes(...,
 *   0) is the size that lets the automatic choice use every option.
 *   out (with lse) may be NULL when num_kv_splits >= 2: then only the first
 *   pass runs and the workspace holds the FP32 records [total_q, num_q_heads,
 *   num_kv_splits, head_dim + 2] for pa_merge_states (a caller that merges
 *   these states with others, or times the passes apart).
 */
int pa_paged_prefill(const void *q, int32_t q_dtype, void *out, float *lse,
                     const int32_t *cu_seqlens_q, const int32_t *seq_lens,
                     const int32_t *block_tables, int32_t num_seqs, int32_t max_pages_per_seq,
                     int32_t total_q, int32_t max_seqlen_q, int32_t num_q_heads,
                     const pa_kv_cache *kv, float scale, int32_t num_kv_splits,
                     void *workspace, size_t workspace_bytes, void *stream);

/* pa_paged_prefill with options (opts may be NULL: none). */
int pa_paged_prefill_ex(const void *q, int32_t q_dtype, void *out, float *lse,
                        const int32_t *cu_seqlens_q, const int32_t *seq_lens,
                        const int32_t *block_tables, int32_t num_seqs, int32_t max_pages_per_seq,
                        int32_t total_q, int32_t max_seqlen_q, int32_t num_q_heads,
                        const pa_kv_cache *kv, float scale, int32_t num_kv_splits,
                        const pa_attn_options *opts, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Split-KV decode / verify (InferMatrixLab/vllm-rlt PR #128, "Purpose", Decode).
 *   Rows are the sequences of the call; row b has q_len = cu_seqlens_q[b+1] -
 *   cu_seqlens_q[b] <= max_q_per_row <= PA_DECODE_MAX_Q query tokens (q_len 0
 *   is allowed).  Row b's keys [0, L) are cut with T = PA_DECODE_SPLIT_TILE and
 *   per = ceil(ceil(L / T) / num_splits) tiles per part; part s covers
 *   [s*per*T, min((s+1)*per*T, L)).  Pass 1 writes, for every (token, q head,
 *   part), an FP32 record of head_dim + 2 floats -- the part's normalised
 *   output, its lse, one pad -- into the workspace laid out
 *   [total_q, num_q_heads, num_splits, head_dim + 2]; pass 2 (the merge)
 *   writes out and lse.  workspace_bytes >= pa_decode_workspace_bytes(...).
 *   out (with lse) may be NULL: then only pass 1 runs and the records are left
 *   in the workspace for pa_merge_states.
 */
int pa_split_kv_decode(const void *q, int32_t q_dtype, void *out, float *lse,
                       const int32_t *cu_seqlens_q, const int32_t *seq_lens,
                       const int32_t *block_tables, int32_t num_rows, int32_t max_pages_per_seq,
                       int32_t total_q, int32_t max_q_per_row, int32_t num_q_heads,
                       const pa_kv_cache *kv, float scale, int32_t num_splits,
                       void *workspace, size_t workspace_bytes, void *stream);

/*
 * Split-KV decode / verify with absolute part boundaries.  Speculative
 * verification checks a verify row against serial decoding token by token, so
 * it needs the packed row to match the decode bit for bit (InferMatrixLab/
 * vllm-rlt PR #128, "Purpose", Prefill, the paragraph after the change list);
 * a verify row of K+1 tokens stands for K+1 decode steps (1CatAI/1Cat-vLLM
 * PR #616 original, "Purpose", the token-wise expansion of small-q rows).  Same arguments, layouts and ownership as pa_split_kv_decode,
 * except the partition: part s of every row covers keys
 * [s*part_keys, (s+1)*part_keys) intersected with [0, L), and the last part
 * (s = num_parts - 1) runs on to L, so rows longer than num_parts*part_keys
 * are still exact (their last part is just longer).  part_keys is a positive
 * multiple of PA_DECODE_SPLIT_TILE.  Because the boundaries do not depend on
 * the row's length, the running max of every query row moves on that row's
 * own scores only, and the merge associates its sums by part index alone
 * (empty trailing parts add exact zeros), token i of a verify row of q
 * tokens at length L gives the same bits as a q = 1 row at length L - q + 1 + i,
 * in any batch and with any num_parts that covers it.  With out = NULL only
 * pass 1 runs, as for pa_split_kv_decode; pa_merge_states then combines the
 * records in its own order (equal within rounding, not bit for bit, to this
 * call's merge, which groups parts by index modulo a count fixed by head_dim).
 * workspace_bytes >=
 * pa_decode_workspace_bytes(total_q, num_q_heads, head_dim, num_parts).
 * Returns PA_ERR_INVALID_ARGUMENT for a bad part_keys, otherwise as
 * pa_split_kv_decode.
 */
int pa_split_kv_decode_fixed(const void *q, int32_t q_dtype, void *out, float *lse,
                             const int32_t *cu_seqlens_q, const int32_t *seq_lens,
                             const int32_t *block_tables, int32_t num_rows, int32_t max_pages_per_seq,
                             int32_t total_q, int32_t max_q_per_row, int32_t num_q_heads,
                             const pa_kv_cache *kv, float scale, int32_t part_keys, int32_t num_parts,
                             void *workspace, size_t workspace_bytes, void *stream);

/*
 * Split-KV decode with options: part_keys = 0 is pa_split_kv_decode (parts cut
 * from each row's own length, num_splits of them), part_keys > 0 is
 * pa_split_kv_decode_fixed (num_splits absolute parts of part_keys keys);
 * opts may be NULL.
 */
int pa_split_kv_decode_ex(const void *q, int32_t q_dtype, void *out, float *lse,
                          const int32_t *cu_seqlens_q, const int32_t *seq_lens,
                          const int32_t *block_tables, int32_t num_rows, int32_t max_pages_per_seq,
                          int32_t total_q, int32_t max_q_per_row, int32_t num_q_heads,
                          const pa_kv_cache *kv, float scale, int32_t num_splits, int32_t part_keys,
                          const pa_attn_options *opts, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Split-KV decode that allocates nothing and takes no workspace: for callers
 * that cannot allocate device memory (code under HIP graph capture, serving
 * loops and harnesses that forbid allocation).  Computes exactly what
 * pa_split_kv_decode_ex computes with the same arguments (the same kernels and
 * partition, so the same bits), but the FP32 records live in a buffer the
 * library itself holds on each GPU: PA_NOALLOC_SCRATCH_BYTES of device memory
 * per GPU, reserved when the library's code is loaded on that GPU and kept
 * until the process ends.  The records of a call need
 * pa_decode_workspace_bytes(total_q, num_q_heads, head_dim, num_splits) bytes;
 * a call that needs more returns PA_ERR_WORKSPACE without launching.  out must
 * not be NULL (the records cannot be handed out); lse nullable.  Nothing in the
 * buffer has to start at zero (every record the merge reads is written by the
 * same call's first pass).  The buffer is shared by every call on one GPU:
 * calls that overlap on one GPU (on different streams, or from several
 * threads) race on it and must be ordered by the caller.  The first call on a
 * device looks the buffer's address up (hipGetSymbolAddress, no allocation
 * and no stream work).  Other arguments and errors as pa_split_kv_decode_ex.
 */
#define PA_NOALLOC_SCRATCH_BYTES (64 * 1024 * 1024)
int pa_split_kv_decode_noalloc(const void *q, int32_t q_dtype, void *out, float *lse,
                               const int32_t *cu_seqlens_q, const int32_t *seq_lens,
                               const int32_t *block_tables, int32_t num_rows, int32_t max_pages_per_seq,
                               int32_t total_q, int32_t max_q_per_row, int32_t num_q_heads,
                               const pa_kv_cache *kv, float scale, int32_t num_splits, int32_t part_keys,
                               const pa_attn_options *opts, void *stream);

/*
 * One mixed step: small-q rows (decode / MTP verify) and prefill chunks over
 * one KV cache, routed by their query length in one call (1CatAI/1Cat-vLLM
 * PR #1279: a step carries chunks next to decode and verify rows; rows of a
 * few tokens are expanded token-wise into decode rows, 1CatAI/1Cat-vLLM PR #616
 * original, "Purpose"; the Turing prefill route starts at a minimum query
 * length, PR #1279 commit 1).
 *   The batch is in any order and is described as for pa_paged_prefill_ex,
 *   plus host_q_lens: a HOST copy of the rows' query lengths (host_q_lens[b]
 *   = cu_seqlens_q[b+1] - cu_seqlens_q[b], summing to total_q; read during the
 *   call only).  Every row with 1 <= q <= decode_max_q (0:
 *   PA_MIXED_DECODE_MAX_Q; at most PA_DECODE_MAX_Q, the decode kernels' limit)
 *   is computed exactly as by pa_split_kv_decode_ex(decode_splits,
 *   decode_part_keys) on the small-q rows, the other rows as by
 *   pa_paged_prefill_ex(prefill_splits; 0 = the automatic count of that call
 *   on the chunks alone, capped by the workspace) on the chunks: the same
 *   work items and kernel code, so the same bits.  The default threshold is
 *   the measured crossover on MI355X: for every q up to 16 (D 256 GQA 6 and
 *   D 128 GQA 4, 2K to 128K keys) one row takes less time through the decode
 *   than through the prefill.
 *   The host counts each class from host_q_lens, which sizes the grids and
 *   the workspace exactly; on the device a small kernel classifies the rows
 *   from cu_seqlens_q, gathers the small-q rows' queries and metadata into the
 *   workspace, the attention runs (head dims padded to 256 with fp16 / bf16 /
 *   fp8 KV and no window or score modifier: one grid, chunk groups first, the
 *   decode groups filling the compute units the chunks' last wave leaves
 *   idle; otherwise the two pass-1 kernels back to back), and the merges
 *   follow, the small-q rows' merge writing each row to its batch tokens.  out
 *   must not be NULL; lse nullable; opts as for the _ex calls (both classes).
 *   Workspace: pa_mixed_workspace_bytes(host_q_lens, ...) bytes, 256-byte
 *   aligned (prefill_splits 0 sizes it for every automatic count).
 *   Device metadata is trusted as for the other calls, and must agree with
 *   host_q_lens (if they disagree, rows are missed, but nothing is written
 *   outside the workspace and out).
 */
#define PA_MIXED_DECODE_MAX_Q 16
size_t pa_mixed_workspace_bytes(const int32_t *host_q_lens, int32_t num_seqs, int32_t max_pages_per_seq,
                                int32_t num_q_heads, int32_t head_dim, int32_t q_dtype, int32_t decode_max_q,
                                int32_t decode_splits, int32_t prefill_splits);
int pa_mixed_step(const void *q, int32_t q_dtype, void *out, float *lse, const int32_t *cu_seqlens_q,
                  const int32_t *host_q_lens, const int32_t *seq_lens, const int32_t *block_tables, int32_t num_seqs,
                  int32_t max_pages_per_seq, int32_t total_q, int32_t num_q_heads, const pa_kv_cache *kv, float scale,
                  int32_t decode_max_q, int32_t decode_splits, int32_t decode_part_keys, int32_t prefill_splits,
                  const pa_attn_options *opts, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Merge of FP32 partial softmax states (InferMatrixLab/vllm-rlt PR #128,
 * "Purpose", Decode: the second kernel).
 *   partials [num_tokens, num_heads, num_splits, head_dim + 2] float32, record =
 *   (o_s normalised, lse_s, pad).  For every (token, head): M = max_s lse_s,
 *   w_s = exp(lse_s - M), o = sum_s w_s o_s / sum_s w_s, lse = M + log(sum_s
 *   w_s), summed in a fixed order that depends only on num_splits and
 *   head_dim; all parts empty (lse = -inf) gives o = 0, lse = -inf.
 *   out [num_tokens, num_heads, head_dim] in out_dtype (F32, F16, BF16);
 *   out_lse nullable.  o_s of an empty part is ignored.  head_dim must be
 *   even and <= 256; partials 8-byte aligned.
 */
int pa_merge_states(const float *partials, int32_t num_splits, int32_t num_tokens,
                    int32_t num_heads, int32_t head_dim, void *out, int32_t out_dtype,
                    float *out_lse, void *stream);

/*
 * KV write: the new tokens' K and V into their cache pages, before the
 * attention that reads them (a chunk's keys are in the cache when its prefill
 * runs: 1CatAI/1Cat-vLLM PR #1279, commit 3, the second half reading the first
 * half's KV writes; fp8_e5m2 cache with a per-tensor scale: 1CatAI/1Cat-vLLM
 * PR #616 original, "Test Result", fp8_e5m2 KV paragraph).
 *   k_new, v_new [total_q, kv->num_kv_heads, kv->head_dim] in src_dtype,
 *   contiguous, 16-byte aligned (device, caller-owned, read only).  Sequence b's
 *   new tokens are rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 (q_len of them,
 *   q_len <= max_q); token t goes to position seq_lens[b] - q_len + t (its last
 *   q_len slots, seq_lens counting the new tokens), i.e. page
 *   block_tables[b][pos / page_size], slot pos % page_size.  Tokens with a
 *   negative position (q_len > seq_len) are not written.
 *   The cache (kv->k_pages, kv->v_pages: written through, despite the const of
 *   the descriptor) has src_dtype, which is copied exactly, or FP8_E5M2 (with
 *   F16 or BF16 src) or FP8_E4M3 (with F16 or BF16 src), byte = the fp8 code of (x / scale)
 *   computed in fp32, scale = k_scale (v_scale for V, both positive) times the
 *   head's k_head_scales[h] when given (the product rounded to fp32), rounded to
 *   nearest with ties to even and saturated to the largest finite magnitude
 *   (57344 for E5M2, 448 for E4M3); NaN stays NaN (0x7F with its sign).  Nothing else in
 *   the cache is touched.  Device metadata is trusted (pa_validate_metadata
 *   checks host copies); two new tokens must not map to the same slot.
 *   Asynchronous on `stream`; returns the argument / support statuses of
 *   pa_paged_prefill.
 */
int pa_write_kv(const void *k_new, const void *v_new, int32_t src_dtype, const int32_t *cu_seqlens_q,
                const int32_t *seq_lens, const int32_t *block_tables, int32_t num_seqs,
                int32_t max_pages_per_seq, int32_t total_q, int32_t max_q, const pa_kv_cache *kv,
                void *stream);

/* Workspace sizes in bytes (host-only, no HIP call). */
size_t pa_prefill_workspace_bytes(int32_t total_q, int32_t num_q_heads, int32_t head_dim,
                                  int32_t num_kv_splits);
size_t pa_decode_workspace_bytes(int32_t total_q, int32_t num_q_heads, int32_t head_dim,
                                 int32_t num_splits);

/*
 * Capability check without launching (host-only): returns PA_OK or the status
 * a call with these scalars would return, and a static rejection reason.
 */
int pa_check_supported(int32_t q_dtype, int32_t kv_dtype, int32_t head_dim, int32_t page_size,
                       int32_t num_q_heads, int32_t num_kv_heads, const char **reason);

/*
 * Host-side metadata check (debugging and tests; host pointers).  Checks that
 * cu_seqlens_q starts at 0, is non-decreasing and ends at total_q; that every
 * q length is <= max_q (when max_q > 0) and every seq_len is >= 0 and fits
 * max_pages_per_seq pages; and that every block-table entry a sequence reads
 * lies in [0, num_pages).  Returns PA_OK or PA_ERR_METADATA.
 */
int pa_validate_metadata(const int32_t *cu_seqlens_q, const int32_t *seq_lens,
                         const int32_t *block_tables, int32_t num_seqs,
                         int32_t max_pages_per_seq, int32_t total_q, int32_t max_q,
                         int32_t page_size, int32_t num_pages);

/* Number of key splits pa_paged_prefill picks for num_kv_splits = 0 (uses the
 * current device's compute-unit count); negative pa_status on failure. */
int pa_prefill_auto_splits(int32_t total_q, int32_t num_seqs, int32_t max_seqlen_q,
                           int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                           int32_t q_dtype, int32_t kv_dtype);

const char *pa_status_string(int status);
const char *pa_last_error(void);
int pa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_H */
