// Routing of a mixed step's rows by their query length, on the device.
//
// A serving step carries prefill chunks next to decode and MTP verify rows
// (1CatAI/1Cat-vLLM PR #1279); rows of a few query tokens are expanded
// token-wise into decode rows (1CatAI/1Cat-vLLM PR #616 original, "Purpose"),
// the others take the prefill kernel, which on the pages' Turing route only
// starts from a minimum query length (PR #1279, commit 1).  pa_mixed_step takes
// the batch in any order.  The host counts each class from its copy of the
// query lengths (the grids and the workspace are sized exactly from them);
// these kernels read cu_seqlens_q on the device, split the rows into the two
// classes in batch order, and lay out what each class's kernels read:
//
//   * small-q rows (1 <= q <= decode_max_q): compact metadata (cu_seqlens_q
//     from 0, seq_lens, block-table rows) and their query rows gathered into a
//     compact q, so that their FP32 records are indexed by a compact token
//     number; the decode merge writes each compact token's rows to its batch
//     token;
//   * chunks (q > decode_max_q): addressed in place ([start, end) token
//     ranges, AttnParams::q_end), with their seq_lens and block-table rows.
//
// Every write is bounded by the host's counts; entries the device does not
// fill (were the two copies of the lengths to disagree) are empty rows.

#include "pa_common.h"

namespace pa {

namespace {

constexpr int kPlanThreads = 1024;

// Inclusive scans over the work group of three values per thread (a scan
// within each wave by lane shuffles, then one over the 16 wave totals):
// returns the inclusive prefixes and leaves the group's totals in tot.
__device__ __forceinline__ int3 block_scan3(int3 x, int3* lds, int3* tot) {
  constexpr int NW = kPlanThreads / 64;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int a = __shfl_up(x.x, off), b = __shfl_up(x.y, off), c = __shfl_up(x.z, off);
    if (lane >= off) x.x += a, x.y += b, x.z += c;
  }
  if (lane == 63) lds[w] = x;
  __syncthreads();
  if (t == 0) {
    for (int i = 1; i < NW; ++i) lds[i] = make_int3(lds[i].x + lds[i - 1].x, lds[i].y + lds[i - 1].y,
                                                     lds[i].z + lds[i - 1].z);
  }
  __syncthreads();
  if (w > 0) x = make_int3(x.x + lds[w - 1].x, x.y + lds[w - 1].y, x.z + lds[w - 1].z);
  *tot = lds[NW - 1];
  __syncthreads();  // lds is free for the next call
  return x;
}

// One work group: classifies the rows in batch order and writes both classes'
// metadata (everything except the block-table rows and the gathered q).
__global__ __launch_bounds__(kPlanThreads) void route_plan_kernel(RouteParams r) {
  __shared__ int3 lds[kPlanThreads / 64];
  int n_dec = 0, n_pre = 0, n_tok = 0;  // running totals (uniform)
  for (int c0 = 0; c0 < r.B; c0 += kPlanThreads) {
    const int b = c0 + (int)threadIdx.x;
    int q = 0, L = 0, start = 0;
    if (b < r.B) {
      start = r.cu[b];
      q = r.cu[b + 1] - start;
      L = r.seq_lens[b];
    }
    const bool is_dec = b < r.B && q >= 1 && q <= r.decode_max_q;
    const bool is_pre = b < r.B && q > r.decode_max_q;
    const int3 mine = make_int3(is_dec ? 1 : 0, is_pre ? 1 : 0, is_dec ? q : 0);
    int3 tot;
    const int3 incl = block_scan3(mine, lds, &tot);
    const int id = incl.x - mine.x, ip = incl.y - mine.y, it = incl.z - mine.z;
    const int td = tot.x, tp = tot.y, tt = tot.z;
    const int i = n_dec + id, j = n_pre + ip, k0 = n_tok + it;
    if (is_dec && i < r.n_dec) {
      r.dec_src[i] = b;
      r.dec_seq_lens[i] = L;
      r.dec_cu[i] = min(k0, r.nt_cap);
      for (int t = 0; t < q && k0 + t < r.nt_cap; ++t) r.dec_tok[k0 + t] = start + t;
    }
    if (is_pre && j < r.n_pre) {
      r.pre_src[j] = b;
      r.pre_qs[j] = start;
      r.pre_qe[j] = start + q;
      r.pre_seq_lens[j] = L;
    }
    n_dec += td;
    n_pre += tp;
    n_tok += tt;
  }
  // every entry up to the host's counts is written: rows the device did not
  // find (host and device lengths disagree) are empty
  for (int i = n_dec + (int)threadIdx.x; i <= r.n_dec; i += kPlanThreads) {
    r.dec_cu[i] = min(n_tok, r.nt_cap);
    if (i < r.n_dec) {
      r.dec_seq_lens[i] = 0;
      r.dec_src[i] = -1;
    }
  }
  if (threadIdx.x == 0 && n_dec > r.n_dec) r.dec_cu[r.n_dec] = r.nt_cap;
  for (int k = n_tok + (int)threadIdx.x; k < r.nt_cap; k += kPlanThreads) r.dec_tok[k] = -1;
  for (int j = n_pre + (int)threadIdx.x; j < r.n_pre; j += kPlanThreads) {
    r.pre_qs[j] = 0;
    r.pre_qe[j] = 0;
    r.pre_seq_lens[j] = 0;
    r.pre_src[j] = -1;
  }
}

// Block-table rows of both classes (work groups [0, n_dec + n_pre)) and the
// small-q rows' query tokens (the nt_cap work groups after them), 16 bytes
// per thread.
__global__ __launch_bounds__(256) void route_copy_kernel(RouteParams r) {
  const int blk = (int)blockIdx.x;
  if (blk < r.n_dec + r.n_pre) {
    const bool dec = blk < r.n_dec;
    const int i = dec ? blk : blk - r.n_dec;
    const int src = dec ? r.dec_src[i] : r.pre_src[i];
    int* dst = (dec ? r.dec_bt : r.pre_bt) + (int64_t)i * r.max_pages;
    for (int c = (int)threadIdx.x; c < r.max_pages; c += 256)
      dst[c] = src >= 0 ? r.bt[(int64_t)src * r.max_pages + c] : 0;
    return;
  }
  const int k = blk - r.n_dec - r.n_pre;
  const int g = r.dec_tok[k];
  if (g < 0) return;
  const uint4* s = (const uint4*)(r.q + (int64_t)g * r.row_bytes);
  uint4* d = (uint4*)(r.dec_q + (int64_t)k * r.row_bytes);
  for (int64_t c = threadIdx.x; c < r.row_bytes / 16; c += 256) d[c] = s[c];
}

}  // namespace

hipError_t launch_route(const RouteParams& r, hipStream_t stream) {
  hipLaunchKernelGGL(route_plan_kernel, dim3(1), dim3(kPlanThreads), 0, stream, r);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int blocks = r.n_dec + r.n_pre + r.nt_cap;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(route_copy_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, r);
  return hipGetLastError();
}

}  // namespace pa
