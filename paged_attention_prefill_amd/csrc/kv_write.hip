// KV write: the new tokens' K and V into their cache pages, the step before
// attention (the chunk's keys must be in the cache before the prefill reads
// them; 1CatAI/1Cat-vLLM PR #1279, commit 3, the second half reading the first
// half's KV writes).  Same dtype: an exact copy.  fp8 E5M2 cache (1CatAI/
// 1Cat-vLLM PR #616 original, "Test Result", fp8_e5m2 KV paragraph, per-tensor
// scale; the same page's "Test Plan" names an e4m3 path): byte = the fp8 code
// of (x / scale) computed in fp32, rounded to nearest with ties to even,
// saturated to the largest finite value (57344 for E5M2, 448 for E4M3), NaN
// kept NaN.
//
// One thread per 8 elements of one (token, kv head) row: a 16-byte load of
// fp16 / bf16 (32 of fp32) and a 16-byte store (8 for E5M2), coalesced along
// the head dimension.  Grid: blocks_per_seq groups (enough for the longest
// sequence's rows) per sequence, one-dimensional.
// HBM-bound: reads and writes every new element once.

#include "pa_common.h"

namespace pa {

namespace {

template <typename T> __device__ __forceinline__ float to_f32(T x) { return (float)x; }

// E5M2 byte of a float32: round to nearest even on the 21 dropped mantissa
// bits of a normal result, an exact scaling to units of 2^-16 for the
// subnormal range, saturation to 0x7B, NaN -> 0x7F (sign kept).
__device__ __forceinline__ uint32_t f32_to_e5m2_sat(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return sign | 0x7Fu;  // NaN
  uint32_t code;
  if (a >= 0x38800000u) {  // |x| >= 2^-14: normal in E5M2
    const uint32_t r = (a + 0x000FFFFFu + ((a >> 21) & 1u)) >> 21;
    code = r - (112u << 2);
    code = code > 0x7Bu ? 0x7Bu : code;  // past 57344 (and infinities): saturate
  } else {
    // |x| < 2^-14: multiples of 2^-16; the product is exact, rintf rounds to even
    code = (uint32_t)rintf(__uint_as_float(a) * 65536.0f);  // 0..4 (4 = 2^-14, the smallest normal)
  }
  return sign | code;
}

// E4M3 byte of a float32: nearest even on the 20 dropped mantissa bits of a
// normal result (|x| >= 2^-6), units of 2^-9 below, saturation to 0x7E (448;
// 0x7F is the format's NaN), NaN -> 0x7F (sign kept).
__device__ __forceinline__ uint32_t f32_to_e4m3_sat(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return sign | 0x7Fu;  // NaN
  uint32_t code;
  if (a >= 0x3C800000u) {
    const uint32_t r = (a + 0x0007FFFFu + ((a >> 20) & 1u)) >> 20;
    code = r - (120u << 3);
    code = code > 0x7Eu ? 0x7Eu : code;  // past 448 (and infinities): saturate
  } else {
    code = (uint32_t)rintf(__uint_as_float(a) * 512.0f);  // 0..8 (8 = 2^-6, the smallest normal)
  }
  return sign | code;
}

template <int F8>
__device__ __forceinline__ uint32_t f32_to_fp8_sat(float x) {
  if constexpr (F8 == KV_E4M3) return f32_to_e4m3_sat(x);
  else return f32_to_e5m2_sat(x);
}

// F8 = 0: copy; KV_E5M2 / KV_E4M3: quantise.
template <typename ST, int F8>
__global__ __launch_bounds__(256) void kv_write_kernel(const ST* __restrict__ k_new, const ST* __restrict__ v_new,
                                                       const int* __restrict__ cu_seqlens_q,
                                                       const int* __restrict__ seq_lens,
                                                       const int* __restrict__ block_tables, int max_pages,
                                                       char* __restrict__ k_pages, char* __restrict__ v_pages,
                                                       int64_t stride_page, int64_t stride_token,
                                                       int64_t stride_head, int page_size, int num_kv_heads,
                                                       int head_dim, int blocks_per_seq, float k_scale,
                                                       float v_scale, const float* __restrict__ k_head_scale,
                                                       const float* __restrict__ v_head_scale) {
  const int seq = blockIdx.x / blocks_per_seq;
  const int chunks = head_dim >> 3;  // 8 elements each
  const int64_t item = (int64_t)(blockIdx.x - seq * blocks_per_seq) * 256 + threadIdx.x;
  const int64_t row = item / chunks;  // (token of the sequence, kv head)
  const int c = (int)(item - row * chunks);
  const int q0 = cu_seqlens_q[seq];
  const int qlen = cu_seqlens_q[seq + 1] - q0;
  if (row >= (int64_t)qlen * num_kv_heads) return;
  const int tok = (int)(row / num_kv_heads), h = (int)(row - (int64_t)tok * num_kv_heads);
  const int pos = seq_lens[seq] - qlen + tok;  // the sequence's last qlen slots
  if (pos < 0) return;                         // no slot for this token (q_len > seq_len)
  const int page = block_tables[(int64_t)seq * max_pages + pos / page_size];
  const int64_t dst = (int64_t)page * stride_page + (int64_t)(pos % page_size) * stride_token +
                      (int64_t)h * stride_head + 8 * c;  // elements of the cache dtype
  const int64_t src = ((int64_t)(q0 + tok) * num_kv_heads + h) * head_dim + 8 * c;
#pragma unroll
  for (int kvi = 0; kvi < 2; ++kvi) {
    const ST* s = (kvi == 0 ? k_new : v_new) + src;
    char* base = kvi == 0 ? k_pages : v_pages;
    if constexpr (F8 != 0) {
      // the head's scale: the per-tensor factor times the per-head one (rounded to fp32)
      const float* hs = kvi == 0 ? k_head_scale : v_head_scale;
      const float sc = (kvi == 0 ? k_scale : v_scale) * (hs ? hs[h] : 1.0f);
      float x[8];
      if constexpr (sizeof(ST) == 4) {
        const float4 a = ((const float4*)s)[0], b = ((const float4*)s)[1];
        x[0] = a.x, x[1] = a.y, x[2] = a.z, x[3] = a.w, x[4] = b.x, x[5] = b.y, x[6] = b.z, x[7] = b.w;
      } else {
        const uint4 w = *(const uint4*)s;
        const ST* e = (const ST*)&w;
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = to_f32(e[i]);
      }
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        lo |= f32_to_fp8_sat<F8>(x[i] / sc) << (8 * i);
        hi |= f32_to_fp8_sat<F8>(x[i + 4] / sc) << (8 * i);
      }
      *(uint2*)(base + dst) = make_uint2(lo, hi);
    } else {
      ST* d = (ST*)base + dst;
      if constexpr (sizeof(ST) == 4) {
        ((float4*)d)[0] = ((const float4*)s)[0];
        ((float4*)d)[1] = ((const float4*)s)[1];
      } else {
        *(uint4*)d = *(const uint4*)s;
      }
    }
  }
}

template <typename ST, int F8>
hipError_t launch_kv_f(const KvWriteParams& w, hipStream_t stream) {
  const int64_t items = (int64_t)w.max_q * w.num_kv_heads * (w.head_dim >> 3);
  const int bps = (int)((items + 255) / 256);
  const dim3 grid((unsigned)((int64_t)bps * w.num_seqs));
  hipLaunchKernelGGL((kv_write_kernel<ST, F8>), grid, dim3(256), 0, stream, (const ST*)w.k_new, (const ST*)w.v_new,
                     w.cu_seqlens_q, w.seq_lens, w.block_tables, w.max_pages, (char*)w.k_pages, (char*)w.v_pages,
                     w.stride_page, w.stride_token, w.stride_head, w.page_size, w.num_kv_heads, w.head_dim, bps,
                     w.k_scale, w.v_scale, w.k_head_scale, w.v_head_scale);
  return hipGetLastError();
}

template <typename ST>
hipError_t launch_kv(const KvWriteParams& w, int cache_kind, hipStream_t stream) {
  if (cache_kind == KV_E5M2) return launch_kv_f<ST, KV_E5M2>(w, stream);
  if (cache_kind == KV_E4M3) return launch_kv_f<ST, KV_E4M3>(w, stream);
  return launch_kv_f<ST, 0>(w, stream);
}

}  // namespace

hipError_t launch_kv_write(const KvWriteParams& w, int src_kind, int cache_kind, hipStream_t stream) {
  switch (src_kind) {
    case KV_F32: return launch_kv<float>(w, cache_kind, stream);
    case KV_F16: return launch_kv<_Float16>(w, cache_kind, stream);
    case KV_BF16: return launch_kv<__bf16>(w, cache_kind, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
