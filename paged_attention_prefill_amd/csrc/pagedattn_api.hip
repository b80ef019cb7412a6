// C ABI of libpagedattn.so: argument checks, launch plans and dispatch.
// The operations are described in include/pagedattn.h.  Every check here runs
// on host scalars before any HIP call, so a rejected call launches nothing.

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "pa_common.h"
#include "../../include/pagedattn.h"

namespace pa {
hipError_t launch_attn_mfma(const AttnParams& p, int q_kind, int kv_kind, int dpad, int nblocks,
                            hipStream_t stream);
hipError_t launch_attn_valu(const AttnParams& p, int q_kind, int kv_kind, int dpad, int nblocks,
                            hipStream_t stream);
// tok_map (nullable): record token t's output goes to token tok_map[t] (none if negative)
hipError_t launch_merge(const float* partials, int S, int ntok, int H, int D, void* out, int out_kind,
                        float* out_lse, bool strided, const float* sinks, const int* tok_map, hipStream_t stream);
hipError_t mfma_occupancy(int q_kind, int kv_kind, int dpad, int* blocks_per_cu);
hipError_t launch_attn_mfma_dma(const AttnParams& p, int q_kind, int dpad, int nblocks,
                                hipStream_t stream);
hipError_t launch_attn_prefill_w4(const AttnParams& p, int q_kind, int kv_kind, int dpad, int nblocks,
                                  hipStream_t stream);
hipError_t mfma_dma_occupancy(int q_kind, int dpad, int* blocks_per_cu);
int mfma_dma_rows(int dpad);
hipError_t launch_attn_mixed(const AttnParams& pp, const AttnParams& pd, int q_kind, int kv_kind, int dpad,
                             int prefill_blocks, int decode_blocks, hipStream_t stream);
hipError_t launch_attn_decode(const AttnParams& p, int q_kind, int kv_kind, int dpad, int nblocks,
                              hipStream_t stream);
int decode_rows_per_group();
hipError_t launch_kv_write(const KvWriteParams& w, int src_kind, int cache_kind, hipStream_t stream);
int mfma_rows_per_group();
int valu_rows_per_group();
}  // namespace pa

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_err[0] = 0;
  return PA_OK;
}

size_t dtype_size(int dt) {
  switch (dt) {
    case PA_F32: return 4;
    case PA_F16: return 2;
    case PA_BF16: return 2;
    case PA_FP8_E5M2: return 1;
    case PA_FP8_E4M3: return 1;
    default: return 0;
  }
}

bool is_fp8(int dt) { return dt == PA_FP8_E5M2 || dt == PA_FP8_E4M3; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Supported (q, kv) pairs, head dims and page sizes; returns status + reason.
int check_supported(int q_dtype, int kv_dtype, int head_dim, int page_size, int hq, int hkv,
                    const char** reason) {
  const char* r = nullptr;
  int st = PA_OK;
  if (dtype_size(q_dtype) == 0 || is_fp8(q_dtype)) {
    st = PA_ERR_UNSUPPORTED, r = "q dtype must be F32, F16 or BF16";
  } else if (dtype_size(kv_dtype) == 0) {
    st = PA_ERR_UNSUPPORTED, r = "unknown KV dtype";
  } else if (!(kv_dtype == q_dtype || (is_fp8(kv_dtype) && (q_dtype == PA_F16 || q_dtype == PA_BF16)))) {
    st = PA_ERR_UNSUPPORTED, r = "KV dtype must equal q dtype, or be FP8_E5M2 / FP8_E4M3 with F16 or BF16 q";
  } else if (head_dim < 16 || head_dim > 256 || head_dim % 16 != 0) {
    st = PA_ERR_UNSUPPORTED, r = "head_dim must be a multiple of 16 in [16, 256]";
  } else if (page_size < 16 || page_size % 16 != 0) {
    st = PA_ERR_UNSUPPORTED, r = "page_size must be a positive multiple of 16";
  } else if (hq < 1 || hkv < 1) {
    st = PA_ERR_INVALID_ARGUMENT, r = "head counts must be positive";
  } else if (hq % hkv != 0) {
    st = PA_ERR_UNSUPPORTED, r = "num_q_heads must be a multiple of num_kv_heads";
  }
  if (reason) *reason = r ? r : "supported";
  return st;
}

int dpad_of(int head_dim) { return head_dim <= 64 ? 64 : head_dim <= 128 ? 128 : 256; }

int kind_of(int dt) {
  switch (dt) {
    case PA_F32: return pa::KV_F32;
    case PA_F16: return pa::KV_F16;
    case PA_BF16: return pa::KV_BF16;
    case PA_FP8_E4M3: return pa::KV_E4M3;
    default: return pa::KV_E5M2;
  }
}

int check_kv(const pa_kv_cache* kv, int q_dtype, int hq) {
  if (kv == nullptr) return fail(PA_ERR_INVALID_ARGUMENT, "kv is NULL");
  const char* reason = nullptr;
  int st = check_supported(q_dtype, kv->dtype, kv->head_dim, kv->page_size, hq, kv->num_kv_heads, &reason);
  if (st != PA_OK) return fail(st, "%s", reason);
  if (kv->num_pages < 1) return fail(PA_ERR_INVALID_ARGUMENT, "num_pages must be >= 1");
  if (kv->k_pages == nullptr || kv->v_pages == nullptr)
    return fail(PA_ERR_INVALID_ARGUMENT, "k_pages / v_pages is NULL");
  if (!aligned16(kv->k_pages) || !aligned16(kv->v_pages))
    return fail(PA_ERR_INVALID_ARGUMENT, "k_pages / v_pages must be 16-byte aligned");
  const int64_t es = (int64_t)dtype_size(kv->dtype);
  const int64_t st3[3] = {kv->stride_page, kv->stride_token, kv->stride_head};
  for (int i = 0; i < 3; ++i)
    if (st3[i] <= 0 || (st3[i] * es) % 16 != 0)
      return fail(PA_ERR_INVALID_ARGUMENT, "KV strides must be positive and 16-byte multiples");
  if (kv->stride_token * es * 32 >= ((int64_t)1 << 31))
    return fail(PA_ERR_UNSUPPORTED, "stride_token too large (32 slots must span < 2 GiB)");
  if (!std::isfinite(kv->k_scale) || !std::isfinite(kv->v_scale))
    return fail(PA_ERR_INVALID_ARGUMENT, "k_scale / v_scale must be finite");
  if (!(kv->k_scale > 0.0f)) return fail(PA_ERR_INVALID_ARGUMENT, "k_scale must be positive");
  if (!is_fp8(kv->dtype) && (kv->k_scale != 1.0f || kv->v_scale != 1.0f))
    return fail(PA_ERR_UNSUPPORTED, "k_scale / v_scale apply to fp8 KV only (must be 1)");
  if (!is_fp8(kv->dtype) && (kv->k_head_scales != nullptr || kv->v_head_scales != nullptr))
    return fail(PA_ERR_UNSUPPORTED, "per-head scales apply to fp8 KV only");
  if (((uintptr_t)kv->k_head_scales & 3u) || ((uintptr_t)kv->v_head_scales & 3u))
    return fail(PA_ERR_INVALID_ARGUMENT, "per-head scales must be 4-byte aligned");
  return PA_OK;
}

std::atomic<int> g_cu_count[64];

int device_cus(int* cus) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(PA_ERR_HIP, "hipGetDevice failed");
  if (dev >= 0 && dev < 64) {
    int c = g_cu_count[dev].load(std::memory_order_relaxed);
    if (c > 0) {
      *cus = c;
      return PA_OK;
    }
  }
  int c = 0;
  if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0)
    return fail(PA_ERR_HIP, "hipDeviceGetAttribute(MultiprocessorCount) failed");
  if (dev >= 0 && dev < 64) g_cu_count[dev].store(c, std::memory_order_relaxed);
  *cus = c;
  return PA_OK;
}

// Split count for num_kv_splits = 0, by full waves of work groups on this
// device (1CatAI/1Cat-vLLM PR #1279, commit 5, which picks <= 4 on Turing):
// cost(S) = ceil(A S / slots) / S, the makespan in units of one unsplit group,
// plus 0.2 % per extra part for the merge and the per-group start-up.  When
// the A active groups already cover the slots, parts only trade granularity
// and S stays <= 4; when they do not (a long chunk of few query tiles), up to
// max_s parts fill the device (a 784-token chunk after 104K keys: 76 groups,
// 10 parts run 8 % faster than 3).  Ties go to fewer parts.
int auto_splits(int64_t active_groups, int slots, int max_s) {
  const int cap = active_groups >= slots ? (max_s < 4 ? max_s : 4) : max_s;
  int best = 1;
  double best_cost = 1e300;
  for (int s = 1; s <= cap; ++s) {
    const int64_t waves = (active_groups * s + slots - 1) / slots;
    const double cost = (double)waves / s + 0.002 * (s - 1);
    if (cost < best_cost - 1e-9) best_cost = cost, best = s;
  }
  return best;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// gcd(n, 8) for n >= 1
int64_t gcd8(int64_t n) { return (n & 7) == 0 ? 8 : (n & 3) == 0 ? 4 : (n & 1) == 0 ? 2 : 1; }

// Which pass-1 kernel serves a call: fp32 -> exact-product VALU kernel;
// fp16/bf16 with same-dtype KV -> MFMA kernels with the LDS DMA pipeline;
// fp16 / bf16 q with fp8 KV -> the DMA kernels (8-bit tiles widened to the
// query's type at the operand reads) for head dims padded to 256, otherwise
// the MFMA kernel with register-staged dequant.
enum KernelKind { K_VALU, K_DMA, K_REGSTAGE };
// Bytes of one q / out element.
size_t elem_size(int dtype) { return dtype == PA_F32 ? 4 : 2; }

KernelKind kernel_for(int q_dtype, int kv_dtype, int dpad, bool decode) {
  if (q_dtype == PA_F32) return K_VALU;
  if (is_fp8(kv_dtype)) return dpad == 256 ? K_DMA : K_REGSTAGE;
  (void)decode;
  return K_DMA;
}
int rows_for(KernelKind k, int dpad, bool decode) {
  if (k == K_VALU) return pa::valu_rows_per_group();
  if (k == K_DMA) return decode ? pa::decode_rows_per_group() : pa::mfma_dma_rows(dpad);
  return pa::mfma_rows_per_group();
}

}  // namespace

extern "C" {

int pa_version(void) { return PA_VERSION; }

const char* pa_last_error(void) { return g_err; }

const char* pa_status_string(int status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_INVALID_ARGUMENT: return "invalid argument";
    case PA_ERR_UNSUPPORTED: return "unsupported configuration";
    case PA_ERR_WORKSPACE: return "workspace missing or too small";
    case PA_ERR_HIP: return "HIP runtime error";
    case PA_ERR_METADATA: return "inconsistent metadata";
    default: return "unknown status";
  }
}

int pa_check_supported(int32_t q_dtype, int32_t kv_dtype, int32_t head_dim, int32_t page_size,
                       int32_t num_q_heads, int32_t num_kv_heads, const char** reason) {
  return check_supported(q_dtype, kv_dtype, head_dim, page_size, num_q_heads, num_kv_heads, reason);
}

size_t pa_prefill_workspace_bytes(int32_t total_q, int32_t num_q_heads, int32_t head_dim,
                                  int32_t num_kv_splits) {
  if (total_q <= 0 || num_q_heads <= 0 || head_dim <= 0) return 0;
  const int s = num_kv_splits == 0 ? PA_PREFILL_MAX_AUTO_SPLITS : num_kv_splits;
  if (s <= 1) return 0;
  return (size_t)total_q * num_q_heads * s * (size_t)(head_dim + 2) * sizeof(float);
}

size_t pa_decode_workspace_bytes(int32_t total_q, int32_t num_q_heads, int32_t head_dim,
                                 int32_t num_splits) {
  if (total_q <= 0 || num_q_heads <= 0 || head_dim <= 0 || num_splits <= 0) return 0;
  return (size_t)total_q * num_q_heads * num_splits * (size_t)(head_dim + 2) * sizeof(float);
}

int pa_validate_metadata(const int32_t* cu, const int32_t* seq_lens, const int32_t* bt,
                         int32_t num_seqs, int32_t max_pages, int32_t total_q, int32_t max_q,
                         int32_t page_size, int32_t num_pages) {
  if (num_seqs < 0 || max_pages < 1 || page_size < 1 || num_pages < 1)
    return fail(PA_ERR_INVALID_ARGUMENT, "bad scalar");
  if (num_seqs == 0) return ok();
  if (!cu || !seq_lens || !bt) return fail(PA_ERR_INVALID_ARGUMENT, "NULL metadata pointer");
  if (cu[0] != 0) return fail(PA_ERR_METADATA, "cu_seqlens_q[0] = %d, expected 0", cu[0]);
  for (int b = 0; b < num_seqs; ++b) {
    const int ql = cu[b + 1] - cu[b];
    if (ql < 0) return fail(PA_ERR_METADATA, "cu_seqlens_q decreases at %d", b);
    if (max_q > 0 && ql > max_q) return fail(PA_ERR_METADATA, "sequence %d has q_len %d > %d", b, ql, max_q);
    const int L = seq_lens[b];
    if (L < 0) return fail(PA_ERR_METADATA, "seq_lens[%d] = %d < 0", b, L);
    const int64_t need = ((int64_t)L + page_size - 1) / page_size;
    if (need > max_pages)
      return fail(PA_ERR_METADATA, "sequence %d needs %lld pages > max_pages_per_seq %d", b,
                  (long long)need, max_pages);
    for (int64_t i = 0; i < need; ++i) {
      const int pg = bt[(int64_t)b * max_pages + i];
      if (pg < 0 || pg >= num_pages)
        return fail(PA_ERR_METADATA, "block_tables[%d][%lld] = %d out of [0, %d)", b, (long long)i, pg,
                    num_pages);
    }
  }
  if (cu[num_seqs] != total_q)
    return fail(PA_ERR_METADATA, "cu_seqlens_q[%d] = %d != total_q %d", num_seqs, cu[num_seqs], total_q);
  return ok();
}

int pa_prefill_auto_splits(int32_t total_q, int32_t num_seqs, int32_t max_seqlen_q,
                           int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                           int32_t q_dtype, int32_t kv_dtype) {
  const char* reason;
  int st = check_supported(q_dtype, kv_dtype, head_dim, 16, num_q_heads, num_kv_heads, &reason);
  if (st != PA_OK) return fail(st, "%s", reason);
  if (total_q <= 0 || num_seqs <= 0) return 1;
  const int g = num_q_heads / num_kv_heads;
  const KernelKind kk = kernel_for(q_dtype, kv_dtype, dpad_of(head_dim), false);
  const int rows = rows_for(kk, dpad_of(head_dim), false);
  int cus = 0;
  st = device_cus(&cus);
  if (st != PA_OK) return st;
  int occ = 1;
  hipError_t oe = hipSuccess;
  if (kk == K_DMA) oe = pa::mfma_dma_occupancy(kind_of(q_dtype), dpad_of(head_dim), &occ);
  else if (kk == K_REGSTAGE) oe = pa::mfma_occupancy(kind_of(q_dtype), kind_of(kv_dtype), dpad_of(head_dim), &occ);
  if (oe != hipSuccess || occ < 1) occ = 1;
  const int64_t tiles_grid = ceil_div((int64_t)max_seqlen_q * g, rows) * num_seqs;
  const int64_t tiles_est = ceil_div((int64_t)total_q * g, rows) + num_seqs - 1;
  const int64_t active = (tiles_grid < tiles_est ? tiles_grid : tiles_est) * num_kv_heads;
  return auto_splits(active, cus * occ, PA_PREFILL_MAX_AUTO_SPLITS);
}

// Plan of one pass-1 launch: the work decomposition (groups of query tiles
// cut into XCD runs) and the kernel parameters.  nblocks = 0: nothing to run.
static int plan_attention(pa::AttnParams& p, int64_t& nblocks, const void* q, int q_dtype, void* out, float* lse,
                          const int32_t* cu, const int32_t* seq_lens, const int32_t* bt, int num_seqs,
                          int max_pages, int total_q, int max_q, int hq, const pa_kv_cache* kv, float scale,
                          int splits, int part_keys, bool is_decode, const pa_attn_options* opts, void* workspace) {
  const int g = hq / kv->num_kv_heads;
  const KernelKind kind = kernel_for(q_dtype, kv->dtype, dpad_of(kv->head_dim), is_decode);
  const int rows = rows_for(kind, dpad_of(kv->head_dim), is_decode);
  const int qtiles = (int)ceil_div((int64_t)max_q * g, rows);
  // Groups (sequence, kv head, part) of qtiles query tiles each, cut into runs
  // that stay on one XCD: whole groups when the group count spreads evenly over
  // the 8 XCDs, otherwise the fewest cuts that make the run count a multiple of
  // 8, and runs of at most 64 tiles (two waves of one XCD's compute units).
  const int64_t groups = (int64_t)num_seqs * kv->num_kv_heads * splits;
  int64_t chunks = 8 / gcd8(groups);
  if (chunks > qtiles) chunks = qtiles;
  while (ceil_div(qtiles, chunks) > 64) chunks *= 2;
  const int64_t run_len = ceil_div(qtiles, chunks);
  const int64_t runs = groups * chunks;
  nblocks = ceil_div(runs, 8) * 8 * run_len;
  if (nblocks >= (int64_t)1 << 31) return fail(PA_ERR_UNSUPPORTED, "grid too large (%lld groups)", (long long)nblocks);
  if (groups == 0 || total_q == 0) nblocks = 0;
  const bool partial = is_decode || splits > 1;

  p.q = q;
  p.out = out;
  p.lse = lse;
  p.partial = (float*)workspace;
  p.cu_seqlens_q = cu;
  p.q_end = nullptr;
  p.seq_lens = seq_lens;
  p.block_tables = bt;
  p.k_pages = kv->k_pages;
  p.v_pages = kv->v_pages;
  p.stride_page = kv->stride_page;
  p.stride_token = kv->stride_token;
  p.stride_head = kv->stride_head;
  p.num_seqs = num_seqs;
  p.max_pages = max_pages;
  p.num_q_heads = hq;
  p.num_kv_heads = kv->num_kv_heads;
  p.group = g;
  p.head_dim = kv->head_dim;
  p.page_size = kv->page_size;
  p.num_splits = splits;
  p.part_keys = part_keys;
  p.write_partial = partial ? 1 : 0;
  p.qtiles = qtiles;
  p.chunks = (int)chunks;
  p.run_len = (int)run_len;
  p.num_runs = (int)runs;
  p.scale_log2 = scale * (is_fp8(kv->dtype) ? kv->k_scale : 1.0f) * 1.4426950408889634f;
  p.v_scale = is_fp8(kv->dtype) ? kv->v_scale : 1.0f;
  p.k_head_scale = kv->k_head_scales;
  p.v_head_scale = kv->v_head_scales;
  p.sinks = opts ? opts->sinks : nullptr;
  p.window_left = opts ? opts->window_left : -1;
  const float cap = opts ? opts->softcap : 0.0f;
  p.softcap_k2 = cap > 0.0f ? 2.0f / cap : 0.0f;
  p.softcap_l2 = cap * 1.4426950408889634f;
  p.alibi_slopes = opts ? opts->alibi_slopes : nullptr;

  return PA_OK;
}

// Pass 1 of one planned call on its own kernel.
static hipError_t launch_pass1(const pa::AttnParams& p, int q_dtype, const pa_kv_cache* kv, bool is_decode,
                               int64_t nblocks, hipStream_t stream) {
  const KernelKind kind = kernel_for(q_dtype, kv->dtype, dpad_of(kv->head_dim), is_decode);
  const int qk = kind_of(q_dtype), kk = kind_of(kv->dtype), dp = dpad_of(kv->head_dim);
  return kind == K_VALU ? pa::launch_attn_valu(p, qk, kk, dp, (int)nblocks, stream)
         : kind == K_DMA ? (is_decode ? pa::launch_attn_decode(p, qk, kk, dp, (int)nblocks, stream)
                            : (kk == pa::KV_E5M2 || kk == pa::KV_E4M3)
                                ? pa::launch_attn_prefill_w4(p, qk, kk, dp, (int)nblocks, stream)
                                : pa::launch_attn_mfma_dma(p, qk, dp, (int)nblocks, stream))
                         : pa::launch_attn_mfma(p, qk, kk, dp, (int)nblocks, stream);
}

static int run_attention(const void* q, int q_dtype, void* out, float* lse, const int32_t* cu,
                         const int32_t* seq_lens, const int32_t* bt, int num_seqs, int max_pages,
                         int total_q, int max_q, int hq, const pa_kv_cache* kv, float scale,
                         int splits, int part_keys, bool is_decode, const pa_attn_options* opts,
                         void* workspace, size_t ws_bytes, hipStream_t stream) {
  pa::AttnParams p;
  int64_t nblocks = 0;
  int st = plan_attention(p, nblocks, q, q_dtype, out, lse, cu, seq_lens, bt, num_seqs, max_pages, total_q, max_q,
                          hq, kv, scale, splits, part_keys, is_decode, opts, workspace);
  if (st != PA_OK) return st;
  if (nblocks == 0) return ok();
  hipError_t e = launch_pass1(p, q_dtype, kv, is_decode, nblocks, stream);
  if (e != hipSuccess) return fail(PA_ERR_HIP, "attention launch failed: %s", hipGetErrorString(e));
  if (p.write_partial && out != nullptr) {  // out NULL: pass 1 only, the records stay in the workspace
    e = pa::launch_merge((const float*)workspace, splits, total_q, hq, kv->head_dim, out, kind_of(q_dtype), lse,
                         part_keys > 0, p.sinks, nullptr, stream);
    if (e != hipSuccess) return fail(PA_ERR_HIP, "merge launch failed: %s", hipGetErrorString(e));
  }
  (void)ws_bytes;
  return ok();
}

static int check_options(const pa_attn_options* opts) {
  if (opts == nullptr) return PA_OK;
  if ((uintptr_t)opts->sinks & 3u) return fail(PA_ERR_INVALID_ARGUMENT, "sinks must be 4-byte aligned");
  if (!std::isfinite(opts->softcap) || opts->softcap < 0.0f)
    return fail(PA_ERR_INVALID_ARGUMENT, "softcap must be 0 (none) or positive and finite");
  if ((uintptr_t)opts->alibi_slopes & 3u) return fail(PA_ERR_INVALID_ARGUMENT, "alibi_slopes must be 4-byte aligned");
  return PA_OK;
}

static int check_common(const void* q, int q_dtype, void* out, const int32_t* cu, const int32_t* seq_lens,
                        const int32_t* bt, int num_seqs, int max_pages, int total_q, int max_q, int hq,
                        const pa_kv_cache* kv) {
  if (num_seqs < 0 || total_q < 0 || max_q < 0 || max_pages < 1 || hq < 1)
    return fail(PA_ERR_INVALID_ARGUMENT, "negative size or max_pages_per_seq < 1 or num_q_heads < 1");
  int st = check_kv(kv, q_dtype, hq);
  if (st != PA_OK) return st;
  if (num_seqs == 0 || total_q == 0) return PA_OK;
  if (!q || !cu || !seq_lens || !bt) return fail(PA_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  if (!aligned16(q) || (out && !aligned16(out))) return fail(PA_ERR_INVALID_ARGUMENT, "q / out must be 16-byte aligned");
  if (max_q < 1) return fail(PA_ERR_INVALID_ARGUMENT, "max q length must be >= 1 when total_q > 0");
  return PA_OK;
}

int pa_paged_prefill_ex(const void* q, int32_t q_dtype, void* out, float* lse, const int32_t* cu_seqlens_q,
                        const int32_t* seq_lens, const int32_t* block_tables, int32_t num_seqs,
                        int32_t max_pages_per_seq, int32_t total_q, int32_t max_seqlen_q,
                        int32_t num_q_heads, const pa_kv_cache* kv, float scale, int32_t num_kv_splits,
                        const pa_attn_options* opts, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_common(q, q_dtype, out, cu_seqlens_q, seq_lens, block_tables, num_seqs, max_pages_per_seq,
                        total_q, max_seqlen_q, num_q_heads, kv);
  if (st != PA_OK) return st;
  st = check_options(opts);
  if (st != PA_OK) return st;
  if (!std::isfinite(scale) || !(scale > 0.0f))
    return fail(PA_ERR_INVALID_ARGUMENT, "scale must be positive and finite");
  if (num_kv_splits < 0 || num_kv_splits > 64) return fail(PA_ERR_INVALID_ARGUMENT, "num_kv_splits must be in [0, 64]");
  if (out == nullptr && (num_kv_splits < 2 || lse != nullptr))
    return fail(PA_ERR_INVALID_ARGUMENT, "out may be NULL only with num_kv_splits >= 2 and lse NULL");
  if (num_seqs == 0 || total_q == 0) return ok();
  int splits = num_kv_splits;
  if (splits == 0) {
    splits = pa_prefill_auto_splits(total_q, num_seqs, max_seqlen_q, num_q_heads, kv->num_kv_heads,
                                    kv->head_dim, q_dtype, kv->dtype);
    if (splits < 0) return splits;
    // at most the parts the workspace holds (records of one part: total_q * Hq * (D + 2) floats)
    const size_t per = pa_prefill_workspace_bytes(total_q, num_q_heads, kv->head_dim, 2) / 2;
    const size_t fit = (workspace == nullptr || ((uintptr_t)workspace & 7u)) ? 0 : workspace_bytes / per;
    if ((size_t)splits > fit) splits = fit >= 2 ? (int)fit : 1;
  }
  if (splits != 1) {
    const size_t need = pa_prefill_workspace_bytes(total_q, num_q_heads, kv->head_dim, splits);
    if (workspace == nullptr || workspace_bytes < need || ((uintptr_t)workspace & 7u))
      return fail(PA_ERR_WORKSPACE, "prefill with %d splits needs %zu bytes of 8-byte aligned workspace (got %zu)",
                  splits, need, workspace == nullptr ? (size_t)0 : workspace_bytes);
  }
  return run_attention(q, q_dtype, out, lse, cu_seqlens_q, seq_lens, block_tables, num_seqs,
                       max_pages_per_seq, total_q, max_seqlen_q, num_q_heads, kv, scale, splits, 0, false, opts,
                       workspace, workspace_bytes, (hipStream_t)stream);
}

int pa_paged_prefill(const void* q, int32_t q_dtype, void* out, float* lse, const int32_t* cu_seqlens_q,
                     const int32_t* seq_lens, const int32_t* block_tables, int32_t num_seqs,
                     int32_t max_pages_per_seq, int32_t total_q, int32_t max_seqlen_q,
                     int32_t num_q_heads, const pa_kv_cache* kv, float scale, int32_t num_kv_splits,
                     void* workspace, size_t workspace_bytes, void* stream) {
  return pa_paged_prefill_ex(q, q_dtype, out, lse, cu_seqlens_q, seq_lens, block_tables, num_seqs,
                             max_pages_per_seq, total_q, max_seqlen_q, num_q_heads, kv, scale, num_kv_splits,
                             nullptr, workspace, workspace_bytes, stream);
}

static int decode_call(const void* q, int32_t q_dtype, void* out, float* lse, const int32_t* cu_seqlens_q,
                       const int32_t* seq_lens, const int32_t* block_tables, int32_t num_rows,
                       int32_t max_pages_per_seq, int32_t total_q, int32_t max_q_per_row,
                       int32_t num_q_heads, const pa_kv_cache* kv, float scale, int32_t num_splits,
                       int32_t part_keys, const pa_attn_options* opts, void* workspace, size_t workspace_bytes,
                       void* stream) {
  int st = check_common(q, q_dtype, out, cu_seqlens_q, seq_lens, block_tables, num_rows, max_pages_per_seq,
                        total_q, max_q_per_row, num_q_heads, kv);
  if (st != PA_OK) return st;
  if (!std::isfinite(scale) || !(scale > 0.0f))
    return fail(PA_ERR_INVALID_ARGUMENT, "scale must be positive and finite");
  if (max_q_per_row > PA_DECODE_MAX_Q)
    return fail(PA_ERR_UNSUPPORTED, "max_q_per_row %d > %d (longer rows go to pa_paged_prefill)", max_q_per_row,
                PA_DECODE_MAX_Q);
  if (num_splits < 1 || num_splits > 4096) return fail(PA_ERR_INVALID_ARGUMENT, "num_splits must be in [1, 4096]");
  if (part_keys < 0 || part_keys % PA_DECODE_SPLIT_TILE != 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "part_keys must be 0 or a positive multiple of %d", PA_DECODE_SPLIT_TILE);
  st = check_options(opts);
  if (st != PA_OK) return st;
  if (out == nullptr && lse != nullptr) return fail(PA_ERR_INVALID_ARGUMENT, "lse must be NULL when out is NULL");
  if (num_rows == 0 || total_q == 0) return ok();
  const size_t need = pa_decode_workspace_bytes(total_q, num_q_heads, kv->head_dim, num_splits);
  if (workspace == nullptr || workspace_bytes < need || ((uintptr_t)workspace & 7u))
    return fail(PA_ERR_WORKSPACE, "decode needs %zu bytes of 8-byte aligned workspace (got %zu)", need,
                workspace == nullptr ? (size_t)0 : workspace_bytes);
  return run_attention(q, q_dtype, out, lse, cu_seqlens_q, seq_lens, block_tables, num_rows, max_pages_per_seq,
                       total_q, max_q_per_row, num_q_heads, kv, scale, num_splits, part_keys, true, opts, workspace,
                       workspace_bytes, (hipStream_t)stream);
}

int pa_split_kv_decode(const void* q, int32_t q_dtype, void* out, float* lse, const int32_t* cu_seqlens_q,
                       const int32_t* seq_lens, const int32_t* block_tables, int32_t num_rows,
                       int32_t max_pages_per_seq, int32_t total_q, int32_t max_q_per_row,
                       int32_t num_q_heads, const pa_kv_cache* kv, float scale, int32_t num_splits,
                       void* workspace, size_t workspace_bytes, void* stream) {
  return decode_call(q, q_dtype, out, lse, cu_seqlens_q, seq_lens, block_tables, num_rows, max_pages_per_seq,
                     total_q, max_q_per_row, num_q_heads, kv, scale, num_splits, 0, nullptr, workspace,
                     workspace_bytes, stream);
}

int pa_split_kv_decode_fixed(const void* q, int32_t q_dtype, void* out, float* lse, const int32_t* cu_seqlens_q,
                             const int32_t* seq_lens, const int32_t* block_tables, int32_t num_rows,
                             int32_t max_pages_per_seq, int32_t total_q, int32_t max_q_per_row,
                             int32_t num_q_heads, const pa_kv_cache* kv, float scale, int32_t part_keys,
                             int32_t num_parts, void* workspace, size_t workspace_bytes, void* stream) {
  if (part_keys < PA_DECODE_SPLIT_TILE || part_keys % PA_DECODE_SPLIT_TILE != 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "part_keys must be a positive multiple of %d", PA_DECODE_SPLIT_TILE);
  return decode_call(q, q_dtype, out, lse, cu_seqlens_q, seq_lens, block_tables, num_rows, max_pages_per_seq,
                     total_q, max_q_per_row, num_q_heads, kv, scale, num_parts, part_keys, nullptr, workspace,
                     workspace_bytes, stream);
}

}  // extern "C"

// Workspace of pa_mixed_step, every region 256-byte aligned: the route's int32
// metadata, the small-q rows' block-table rows and the chunks', the small-q
// rows' gathered q, their compact out and lse, their FP32 records, then the
// chunks' records (indexed by batch token, when the chunks are split).
namespace {
// The two classes of a batch, counted from the host copy of its query lengths.
struct MixedSplit {
  int n_dec = 0, n_pre = 0, max_dec_q = 0, max_pre_q = 0;
  int64_t dec_tokens = 0, pre_tokens = 0;
};

struct MixedLayout {
  size_t meta, dec_bt, pre_bt, dec_q, dec_rec, pre_rec, total;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int mixed_decode_max_q(int32_t decode_max_q) { return decode_max_q == 0 ? PA_MIXED_DECODE_MAX_Q : decode_max_q; }

// Rows with 1 <= q <= dmq are small-q rows, rows with q > dmq chunks, q = 0 neither.
int mixed_split(const int32_t* host_q_lens, int B, int dmq, MixedSplit& s) {
  if (host_q_lens == nullptr) return fail(PA_ERR_INVALID_ARGUMENT, "host_q_lens is NULL");
  for (int b = 0; b < B; ++b) {
    const int q = host_q_lens[b];
    if (q < 0) return fail(PA_ERR_INVALID_ARGUMENT, "host_q_lens[%d] = %d < 0", b, q);
    if (q == 0) continue;
    if (q <= dmq) {
      ++s.n_dec;
      s.dec_tokens += q;
      if (q > s.max_dec_q) s.max_dec_q = q;
    } else {
      ++s.n_pre;
      s.pre_tokens += q;
      if (q > s.max_pre_q) s.max_pre_q = q;
    }
  }
  return PA_OK;
}

MixedLayout mixed_layout(int64_t total_q, const MixedSplit& s, int64_t max_pages, int64_t hq, int64_t d, int64_t es,
                         int64_t dsplits, int64_t psplits) {
  const int64_t nt = s.dec_tokens, nd = s.n_dec, np = s.n_pre;
  MixedLayout m;
  size_t o = 0;
  m.meta = o;
  o += align256(sizeof(int) * (size_t)(3 * nd + 1 + 4 * np + nt));
  m.dec_bt = o;
  o += align256(sizeof(int) * (size_t)(nd * max_pages));
  m.pre_bt = o;
  o += align256(sizeof(int) * (size_t)(np * max_pages));
  m.dec_q = o;
  o += align256((size_t)(nt * hq * d * es));
  m.dec_rec = o;
  o += align256(sizeof(float) * (size_t)(nt * hq * dsplits * (d + 2)));
  m.pre_rec = o;
  if (np > 0 && psplits > 1) o += align256(sizeof(float) * (size_t)(total_q * hq * psplits * (d + 2)));
  m.total = o;
  return m;
}
}  // namespace

namespace pa {
hipError_t launch_route(const RouteParams& r, hipStream_t stream);
}  // namespace pa

extern "C" {

size_t pa_mixed_workspace_bytes(const int32_t* host_q_lens, int32_t num_seqs, int32_t max_pages_per_seq,
                                int32_t num_q_heads, int32_t head_dim, int32_t q_dtype, int32_t decode_max_q,
                                int32_t decode_splits, int32_t prefill_splits) {
  if (num_seqs <= 0 || max_pages_per_seq <= 0 || num_q_heads <= 0 || head_dim <= 0 || decode_splits <= 0 ||
      decode_max_q < 0 || decode_max_q > PA_DECODE_MAX_Q || prefill_splits < 0 || elem_size(q_dtype) == 0)
    return 0;
  MixedSplit s;
  if (mixed_split(host_q_lens, num_seqs, mixed_decode_max_q(decode_max_q), s) != PA_OK) return 0;
  const int sp = prefill_splits == 0 ? PA_PREFILL_MAX_AUTO_SPLITS : prefill_splits;
  return mixed_layout(s.dec_tokens + s.pre_tokens, s, max_pages_per_seq, num_q_heads, head_dim,
                      (int64_t)elem_size(q_dtype), decode_splits, sp)
      .total;
}

int pa_mixed_step(const void* q, int32_t q_dtype, void* out, float* lse, const int32_t* cu_seqlens_q,
                  const int32_t* host_q_lens, const int32_t* seq_lens, const int32_t* block_tables, int32_t num_seqs,
                  int32_t max_pages_per_seq, int32_t total_q, int32_t num_q_heads, const pa_kv_cache* kv, float scale,
                  int32_t decode_max_q, int32_t decode_splits, int32_t decode_part_keys, int32_t prefill_splits,
                  const pa_attn_options* opts, void* workspace, size_t workspace_bytes, void* stream) {
  if (decode_max_q < 0 || decode_max_q > PA_DECODE_MAX_Q)
    return fail(PA_ERR_UNSUPPORTED, "decode_max_q must be 0 (the default, %d) or in [1, %d]", PA_MIXED_DECODE_MAX_Q,
                PA_DECODE_MAX_Q);
  if (num_seqs < 0 || total_q < 0) return fail(PA_ERR_INVALID_ARGUMENT, "negative size");
  const int dmq = mixed_decode_max_q(decode_max_q);
  MixedSplit ms;
  int st = num_seqs > 0 ? mixed_split(host_q_lens, num_seqs, dmq, ms) : PA_OK;
  if (st != PA_OK) return st;
  if (ms.dec_tokens + ms.pre_tokens != total_q)
    return fail(PA_ERR_INVALID_ARGUMENT, "host_q_lens sum to %lld, total_q is %d",
                (long long)(ms.dec_tokens + ms.pre_tokens), total_q);
  const int max_q = ms.max_pre_q > ms.max_dec_q ? ms.max_pre_q : ms.max_dec_q;
  st = check_common(q, q_dtype, out, cu_seqlens_q, seq_lens, block_tables, num_seqs, max_pages_per_seq, total_q,
                    max_q, num_q_heads, kv);
  if (st != PA_OK) return st;
  st = check_options(opts);
  if (st != PA_OK) return st;
  if (!std::isfinite(scale) || !(scale > 0.0f))
    return fail(PA_ERR_INVALID_ARGUMENT, "scale must be positive and finite");
  if (out == nullptr) return fail(PA_ERR_INVALID_ARGUMENT, "out is NULL");
  if (decode_splits < 1 || decode_splits > 4096)
    return fail(PA_ERR_INVALID_ARGUMENT, "decode_splits must be in [1, 4096]");
  if (decode_part_keys < 0 || decode_part_keys % PA_DECODE_SPLIT_TILE != 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "decode_part_keys must be 0 or a positive multiple of %d",
                PA_DECODE_SPLIT_TILE);
  if (prefill_splits < 0 || prefill_splits > 64)
    return fail(PA_ERR_INVALID_ARGUMENT, "prefill_splits must be in [0, 64]");
  if (total_q == 0 || num_seqs == 0) return ok();
  const int D = kv->head_dim;
  const int64_t es = (int64_t)elem_size(q_dtype);
  // the chunks' part count: as a prefill call on the chunks alone would pick
  // it, capped by the workspace
  int sp = prefill_splits;
  if (sp == 0 && ms.n_pre > 0) {
    sp = pa_prefill_auto_splits((int32_t)ms.pre_tokens, ms.n_pre, ms.max_pre_q, num_q_heads, kv->num_kv_heads, D,
                                q_dtype, kv->dtype);
    if (sp < 0) return sp;
    while (sp > 1 && (workspace == nullptr ||
                      mixed_layout(total_q, ms, max_pages_per_seq, num_q_heads, D, es, decode_splits, sp).total >
                          workspace_bytes))
      --sp;
  }
  if (sp == 0) sp = 1;
  const MixedLayout ml = mixed_layout(total_q, ms, max_pages_per_seq, num_q_heads, D, es, decode_splits, sp);
  if (workspace == nullptr || workspace_bytes < ml.total || ((uintptr_t)workspace & 255u))
    return fail(PA_ERR_WORKSPACE, "mixed step needs %zu bytes of 256-byte aligned workspace (got %zu)", ml.total,
                workspace == nullptr ? (size_t)0 : workspace_bytes);
  const int nd = ms.n_dec, np = ms.n_pre, nt = (int)ms.dec_tokens;
  char* ws = (char*)workspace;
  int* meta = (int*)(ws + ml.meta);
  pa::RouteParams r;
  r.cu = cu_seqlens_q;
  r.seq_lens = seq_lens;
  r.bt = block_tables;
  r.q = (const char*)q;
  r.B = num_seqs;
  r.max_pages = max_pages_per_seq;
  r.decode_max_q = dmq;
  r.n_dec = nd;
  r.n_pre = np;
  r.nt_cap = nt;
  r.row_bytes = (int64_t)num_q_heads * D * es;
  r.dec_cu = meta;
  r.dec_seq_lens = r.dec_cu + (nd + 1);
  r.dec_src = r.dec_seq_lens + nd;
  r.pre_qs = r.dec_src + nd;
  r.pre_qe = r.pre_qs + np;
  r.pre_seq_lens = r.pre_qe + np;
  r.pre_src = r.pre_seq_lens + np;
  r.dec_tok = r.pre_src + np;
  r.dec_bt = (int*)(ws + ml.dec_bt);
  r.pre_bt = (int*)(ws + ml.pre_bt);
  r.dec_q = ws + ml.dec_q;
  hipStream_t strm = (hipStream_t)stream;

  // each class planned exactly as its own call on its sub-batch would be
  pa::AttnParams pd, pp;
  int64_t nb_d = 0, nb_p = 0;
  if (nd > 0) {
    // (decode pass 1 writes records only; the merge puts the rows into out)
    st = plan_attention(pd, nb_d, r.dec_q, q_dtype, out, lse, r.dec_cu,
                        r.dec_seq_lens, r.dec_bt, nd, max_pages_per_seq, nt, ms.max_dec_q, num_q_heads, kv, scale,
                        decode_splits, decode_part_keys, true, opts, ws + ml.dec_rec);
    if (st != PA_OK) return st;
  }
  if (np > 0) {
    st = plan_attention(pp, nb_p, q, q_dtype, out, lse, r.pre_qs, r.pre_seq_lens, r.pre_bt, np, max_pages_per_seq,
                        total_q, ms.max_pre_q, num_q_heads, kv, scale, sp, 0, false, opts, ws + ml.pre_rec);
    if (st != PA_OK) return st;
    pp.q_end = r.pre_qe;
  }
  if (nb_d + nb_p >= (int64_t)1 << 31) return fail(PA_ERR_UNSUPPORTED, "grid too large");

  hipError_t e = pa::launch_route(r, strm);
  if (e != hipSuccess) return fail(PA_ERR_HIP, "route launch failed: %s", hipGetErrorString(e));
  // one grid for the default instantiations at D padded to 256 (with a window
  // or score modifiers the fused kernel spills: the two kernels run instead)
  const bool fused = nb_d > 0 && nb_p > 0 && dpad_of(D) == 256 &&
                     kernel_for(q_dtype, kv->dtype, 256, false) == K_DMA && pp.window_left < 0 &&
                     !pa::has_score_mods(pp);
  if (fused) {
    e = pa::launch_attn_mixed(pp, pd, kind_of(q_dtype), kind_of(kv->dtype), 256, (int)nb_p, (int)nb_d, strm);
  } else {  // other shapes: the two pass-1 kernels back to back
    if (nb_p > 0) e = launch_pass1(pp, q_dtype, kv, false, nb_p, strm);
    if (e == hipSuccess && nb_d > 0) e = launch_pass1(pd, q_dtype, kv, true, nb_d, strm);
  }
  if (e != hipSuccess) return fail(PA_ERR_HIP, "mixed-step attention launch failed: %s", hipGetErrorString(e));
  // the chunks' merge runs over every token of the batch (records indexed by
  // batch token); the small-q rows' tokens get values from records no chunk
  // wrote and are overwritten by the decode merge that follows, which writes
  // each compact token's rows to its batch token (dec_tok)
  if (nb_p > 0 && sp > 1) {
    e = pa::launch_merge((const float*)(ws + ml.pre_rec), sp, total_q, num_q_heads, D, out, kind_of(q_dtype), lse,
                         false, pp.sinks, nullptr, strm);
    if (e != hipSuccess) return fail(PA_ERR_HIP, "merge launch failed: %s", hipGetErrorString(e));
  }
  if (nb_d > 0) {
    e = pa::launch_merge((const float*)(ws + ml.dec_rec), decode_splits, nt, num_q_heads, D, out, kind_of(q_dtype),
                         lse, decode_part_keys > 0, pd.sinks, r.dec_tok, strm);
    if (e != hipSuccess) return fail(PA_ERR_HIP, "merge launch failed: %s", hipGetErrorString(e));
  }
  return ok();
}

int pa_write_kv(const void* k_new, const void* v_new, int32_t src_dtype, const int32_t* cu_seqlens_q,
                const int32_t* seq_lens, const int32_t* block_tables, int32_t num_seqs, int32_t max_pages_per_seq,
                int32_t total_q, int32_t max_q, const pa_kv_cache* kv, void* stream) {
  if (num_seqs < 0 || total_q < 0 || max_q < 0 || max_pages_per_seq < 1)
    return fail(PA_ERR_INVALID_ARGUMENT, "negative size or max_pages_per_seq < 1");
  if (kv == nullptr) return fail(PA_ERR_INVALID_ARGUMENT, "kv is NULL");
  int st = check_kv(kv, src_dtype, kv->num_kv_heads);
  if (st != PA_OK) return st;
  if (is_fp8(kv->dtype) && !(kv->v_scale > 0.0f))
    return fail(PA_ERR_INVALID_ARGUMENT, "v_scale must be positive for an fp8 cache");
  if (num_seqs == 0 || total_q == 0) return ok();
  if (!k_new || !v_new || !cu_seqlens_q || !seq_lens || !block_tables)
    return fail(PA_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  if (!aligned16(k_new) || !aligned16(v_new)) return fail(PA_ERR_INVALID_ARGUMENT, "k_new / v_new must be 16-byte aligned");
  if (max_q < 1) return fail(PA_ERR_INVALID_ARGUMENT, "max_q must be >= 1 when total_q > 0");
  const int64_t bps = ((int64_t)max_q * kv->num_kv_heads * (kv->head_dim / 8) + 255) / 256;
  if (bps * num_seqs >= ((int64_t)1 << 31)) return fail(PA_ERR_UNSUPPORTED, "grid too large");
  pa::KvWriteParams w;
  w.k_new = k_new;
  w.v_new = v_new;
  w.cu_seqlens_q = cu_seqlens_q;
  w.seq_lens = seq_lens;
  w.block_tables = block_tables;
  w.k_pages = const_cast<void*>(kv->k_pages);
  w.v_pages = const_cast<void*>(kv->v_pages);
  w.stride_page = kv->stride_page;
  w.stride_token = kv->stride_token;
  w.stride_head = kv->stride_head;
  w.num_seqs = num_seqs;
  w.max_pages = max_pages_per_seq;
  w.max_q = max_q;
  w.num_kv_heads = kv->num_kv_heads;
  w.head_dim = kv->head_dim;
  w.page_size = kv->page_size;
  w.k_scale = kv->k_scale;
  w.v_scale = kv->v_scale;
  w.k_head_scale = kv->k_head_scales;
  w.v_head_scale = kv->v_head_scales;
  hipError_t e = pa::launch_kv_write(w, kind_of(src_dtype), is_fp8(kv->dtype) ? kind_of(kv->dtype) : 0,
                                     (hipStream_t)stream);
  if (e != hipSuccess) return fail(PA_ERR_HIP, "KV write launch failed: %s", hipGetErrorString(e));
  return ok();
}

int pa_split_kv_decode_ex(const void* q, int32_t q_dtype, void* out, float* lse, const int32_t* cu_seqlens_q,
                          const int32_t* seq_lens, const int32_t* block_tables, int32_t num_rows,
                          int32_t max_pages_per_seq, int32_t total_q, int32_t max_q_per_row,
                          int32_t num_q_heads, const pa_kv_cache* kv, float scale, int32_t num_splits,
                          int32_t part_keys, const pa_attn_options* opts, void* workspace, size_t workspace_bytes,
                          void* stream) {
  return decode_call(q, q_dtype, out, lse, cu_seqlens_q, seq_lens, block_tables, num_rows, max_pages_per_seq,
                     total_q, max_q_per_row, num_q_heads, kv, scale, num_splits, part_keys, opts, workspace,
                     workspace_bytes, stream);
}

}  // extern "C"

// The FP32 records of pa_split_kv_decode_noalloc: a buffer the library owns
// on every GPU it runs on (a device-code variable, loaded with the library's
// code object and held until the process ends), so that the call allocates
// nothing.  Host code never uses the name itself (on the host it stands for
// a host-side handle): its device address, looked up once per device with
// that device current, is what the kernels get.
static __device__ __align__(256) char scratch[PA_NOALLOC_SCRATCH_BYTES];

namespace {
std::atomic<void*> g_scratch_ptr[64];

// Device address of `scratch` on the current device (looked up on the first
// call on that device; no allocation, no stream work).
int scratch_address(void** ptr) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(PA_ERR_HIP, "hipGetDevice failed");
  if (dev < 0 || dev >= 64) return fail(PA_ERR_UNSUPPORTED, "device index %d out of range", dev);
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(PA_ERR_HIP, "hipGetSymbolAddress(scratch) failed: %s", hipGetErrorString(e));
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *ptr = p;
  return PA_OK;
}
}  // namespace

extern "C" {

int pa_split_kv_decode_noalloc(const void* q, int32_t q_dtype, void* out, float* lse, const int32_t* cu_seqlens_q,
                               const int32_t* seq_lens, const int32_t* block_tables, int32_t num_rows,
                               int32_t max_pages_per_seq, int32_t total_q, int32_t max_q_per_row,
                               int32_t num_q_heads, const pa_kv_cache* kv, float scale, int32_t num_splits,
                               int32_t part_keys, const pa_attn_options* opts, void* stream) {
  if (out == nullptr) return fail(PA_ERR_INVALID_ARGUMENT, "out is NULL (the records stay in the library's buffer)");
  if (kv == nullptr) return fail(PA_ERR_INVALID_ARGUMENT, "kv is NULL");
  if (total_q < 0 || num_q_heads < 1 || num_splits < 1)
    return fail(PA_ERR_INVALID_ARGUMENT, "negative total_q, or num_q_heads / num_splits < 1");
  const size_t need = pa_decode_workspace_bytes(total_q, num_q_heads, kv->head_dim, num_splits);
  if (need > (size_t)PA_NOALLOC_SCRATCH_BYTES)
    return fail(PA_ERR_WORKSPACE, "the records need %zu bytes, more than the %zu of the library's buffer", need,
                (size_t)PA_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if (num_rows > 0 && total_q > 0) {
    const int st = scratch_address(&ws);
    if (st != PA_OK) return st;
  }
  return decode_call(q, q_dtype, out, lse, cu_seqlens_q, seq_lens, block_tables, num_rows, max_pages_per_seq,
                     total_q, max_q_per_row, num_q_heads, kv, scale, num_splits, part_keys, opts, ws,
                     (size_t)PA_NOALLOC_SCRATCH_BYTES, stream);
}

int pa_merge_states(const float* partials, int32_t num_splits, int32_t num_tokens, int32_t num_heads,
                    int32_t head_dim, void* out, int32_t out_dtype, float* out_lse, void* stream) {
  if (num_splits < 1 || num_tokens < 0 || num_heads < 1 || head_dim < 2 || head_dim > 256 || head_dim % 2)
    return fail(PA_ERR_INVALID_ARGUMENT, "bad merge sizes (head_dim must be even, <= 256)");
  if (out_dtype != PA_F32 && out_dtype != PA_F16 && out_dtype != PA_BF16)
    return fail(PA_ERR_UNSUPPORTED, "merge output dtype must be F32, F16 or BF16");
  if (num_tokens == 0) return ok();
  if (!partials || !out) return fail(PA_ERR_INVALID_ARGUMENT, "NULL pointer argument");
  if (((uintptr_t)partials & 7u) || ((uintptr_t)out & 3u))
    return fail(PA_ERR_INVALID_ARGUMENT, "partials must be 8-byte and out 4-byte aligned");
  if ((int64_t)num_tokens * num_heads >= ((int64_t)1 << 31))
    return fail(PA_ERR_UNSUPPORTED, "too many rows");
  hipError_t e = pa::launch_merge(partials, num_splits, num_tokens, num_heads, head_dim, out, kind_of(out_dtype),
                                  out_lse, false, nullptr, nullptr, (hipStream_t)stream);
  if (e != hipSuccess) return fail(PA_ERR_HIP, "merge launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"
