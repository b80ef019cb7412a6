// Measured ceilings of the chip, reported beside the published peaks: a pure
// MFMA loop (v_mfma_f32_32x32x16_f16, four independent accumulators per wave,
// one wave per SIMD) on fixed operands, the same loop fed a fresh A fragment
// from LDS for every pair of MFMAs (the operand traffic of attention's S^T
// phase: new K data each k-step, two query blocks per fragment), the same
// loop with vector-ALU instructions after every MFMA (how much of a softmax
// one wave hides behind its MFMAs), and a streaming read.  Not part of the
// attention path.
//
// The MFMA loop also reads the shader clock (s_memtime) and the 100 MHz
// real-time counter (s_memrealtime) at its start and end, so the clock the
// chip actually ran at under that load can be stated.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_ceilings.h"

namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256, 1) void mfma_loop(const uint4* __restrict__ operands, float* __restrict__ sink,
                                                     int iters, unsigned long long* __restrict__ clocks) {
  const int lane = threadIdx.x & 63;
  const uint4 a = operands[lane], b = operands[64 + lane];
  const uint64_t t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  f32x16_t c0 = (f32x16_t)(0.0f), c1 = c0, c2 = c0, c3 = c0;
  const half8_t ah = __builtin_bit_cast(half8_t, a), bh = __builtin_bit_cast(half8_t, b);
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, bh, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, bh, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, bh, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_f16(ah, bh, c3, 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  sink[blockIdx.x * 256 + threadIdx.x] = s;
  const uint64_t t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0) {
    clocks[2 * blockIdx.x] = t1 - t0;
    clocks[2 * blockIdx.x + 1] = r1 - r0;
  }
}

// operands: 2048 16-byte fragments (32 KB, copied to LDS) then 4 x 64 B
// fragments kept in registers
__global__ __launch_bounds__(256, 1) void mfma_lds_loop(const uint4* __restrict__ operands,
                                                         float* __restrict__ sink, int iters,
                                                         unsigned long long* __restrict__ clocks) {
  __shared__ uint4 pool[2048];
  const int tid = threadIdx.x, lane = tid & 63;
  for (int i = tid; i < 2048; i += 256) pool[i] = operands[i];
  const half8_t b0 = __builtin_bit_cast(half8_t, operands[2048 + lane]);
  const half8_t b1 = __builtin_bit_cast(half8_t, operands[2048 + 64 + lane]);
  const half8_t b2 = __builtin_bit_cast(half8_t, operands[2048 + 128 + lane]);
  const half8_t b3 = __builtin_bit_cast(half8_t, operands[2048 + 192 + lane]);
  __syncthreads();
  const uint64_t t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  f32x16_t c0 = (f32x16_t)(0.0f), c1 = c0, c2 = c0, c3 = c0;
  // fragment f (of 32) is pool[64 f + lane]; iteration it uses fragments 2 it, 2 it + 1 (mod 32),
  // read one iteration ahead.  The reads are issued from inline assembly with the wait written
  // out (lgkmcnt(2): the pair read last may still be in flight), so the loop measures the
  // matrix cores and not the LDS latency.
  typedef int i32x4 __attribute__((ext_vector_type(4)));
  const uint32_t base = (uint32_t)(uintptr_t)&pool[lane];
  i32x4 a0, a1, n0, n1;
  uint32_t addr = base;
  asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %2 offset:1024" : "=v"(a0), "=v"(a1) : "v"(addr) : "memory");
  for (int it = 0; it + 1 < iters; it += 2) {
    const uint32_t af = base + (uint32_t)(((2 * it + 2) & 31) * 1024);
    const uint32_t ag = base + (uint32_t)(((2 * it + 4) & 31) * 1024);
    asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %2 offset:1024" : "=v"(n0), "=v"(n1) : "v"(af) : "memory");
    asm volatile("s_waitcnt lgkmcnt(2)" : "+v"(a0), "+v"(a1) :: "memory");
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8_t, a0), b0, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8_t, a0), b1, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8_t, a1), b2, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8_t, a1), b3, c3, 0, 0, 0);
    asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %2 offset:1024" : "=v"(a0), "=v"(a1) : "v"(ag) : "memory");
    asm volatile("s_waitcnt lgkmcnt(2)" : "+v"(n0), "+v"(n1) :: "memory");
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8_t, n0), b0, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8_t, n0), b1, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8_t, n1), b2, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(half8_t, n1), b3, c3, 0, 0, 0);
  }
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a0), "+v"(a1) :: "memory");
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  sink[blockIdx.x * 256 + threadIdx.x] = s;
  const uint64_t t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0) {
    clocks[2 * blockIdx.x] = t1 - t0;
    clocks[2 * blockIdx.x + 1] = r1 - r0;
  }
}

// How much vector-ALU work one wave can place in the shadow of its own MFMAs:
// the loop of mfma_loop with NV independent VALU instructions after every
// MFMA (KIND 0: v_fma_f32, 1: v_exp_f32), one wave per SIMD.  MFMAs and VALU
// instructions are written in inline assembly so that the compiler keeps
// their order; the VALU operands never touch the accumulators.
template <int NV, int KIND>
__global__ __launch_bounds__(256, 1) void mfma_valu_loop(const uint4* __restrict__ operands, float* __restrict__ sink,
                                                          int iters, unsigned long long* __restrict__ clocks) {
  typedef int i32x4 __attribute__((ext_vector_type(4)));
  const int lane = threadIdx.x & 63;
  const i32x4 a = __builtin_bit_cast(i32x4, operands[lane]), b = __builtin_bit_cast(i32x4, operands[64 + lane]);
  float v[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = -1e-3f * (float)(lane + i);
  const uint64_t t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  f32x16_t c0 = (f32x16_t)(0.0f), c1 = c0, c2 = c0, c3 = c0;
  for (int it = 0; it < iters; ++it) {
#define PA_CEIL_STEP(c)                                                                            \
  asm volatile("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));               \
  _Pragma("unroll") for (int j = 0; j < NV; ++j) {                                                  \
    if constexpr (KIND == 0) asm volatile("v_fma_f32 %0, %0, %0, %0" : "+v"(v[j & 7]));             \
    else asm volatile("v_exp_f32 %0, %0" : "+v"(v[j & 7]));                                         \
  }
    PA_CEIL_STEP(c0)
    PA_CEIL_STEP(c1)
    PA_CEIL_STEP(c2)
    PA_CEIL_STEP(c3)
#undef PA_CEIL_STEP
  }
  // wait states before the VALU reads the accumulators of the last MFMAs
  asm volatile("s_nop 15\n\ts_nop 15" : "+v"(c0), "+v"(c1), "+v"(c2), "+v"(c3));
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
#pragma unroll
  for (int i = 0; i < 8; ++i) s += v[i];
  sink[blockIdx.x * 256 + threadIdx.x] = s;
  const uint64_t t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  if (threadIdx.x == 0) {
    clocks[2 * blockIdx.x] = t1 - t0;
    clocks[2 * blockIdx.x + 1] = r1 - r0;
  }
}

template <int NV>
hipError_t launch_valu_loop(int kind, const uint4* operands, float* sink, int blocks, int iters,
                            unsigned long long* clocks, hipStream_t stream) {
  if (kind == 0)
    hipLaunchKernelGGL((mfma_valu_loop<NV, 0>), dim3(blocks), dim3(256), 0, stream, operands, sink, iters, clocks);
  else
    hipLaunchKernelGGL((mfma_valu_loop<NV, 1>), dim3(blocks), dim3(256), 0, stream, operands, sink, iters, clocks);
  return hipGetLastError();
}

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// Each block reads one contiguous range, eight 16-byte non-temporal loads per
// lane in flight; every loaded word feeds the result so none is dropped.
__global__ __launch_bounds__(256) void stream_read(const u32x4* __restrict__ src, long long n16,
                                                   float* __restrict__ sink) {
  const long long per = ((n16 + gridDim.x - 1) / gridDim.x + 2047) / 2048 * 2048;
  const long long lo = (long long)blockIdx.x * per;
  const long long hi = lo + per < n16 ? lo + per : n16;
  uint32_t acc = 0;
  long long i = lo + threadIdx.x;
  for (; i + 7 * 256 < hi; i += 8 * 256) {
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(src + i + u * 256);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < hi; i += 256) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  sink[blockIdx.x * blockDim.x + threadIdx.x] = (float)(acc & 1u);
}

}  // namespace

extern "C" {

int pa_ceiling_mfma(const void* operands, float* sink, int32_t blocks, int32_t iters,
                    unsigned long long* clocks, void* stream_) {
  const hipStream_t stream = (hipStream_t)stream_;
  if (!operands || !sink || !clocks || blocks <= 0 || iters <= 0) return -1;
  hipLaunchKernelGGL(mfma_loop, dim3(blocks), dim3(256), 0, stream, (const uint4*)operands, sink, iters, clocks);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int pa_ceiling_mfma_lds(const void* operands, float* sink, int32_t blocks, int32_t iters,
                        unsigned long long* clocks, void* stream_) {
  const hipStream_t stream = (hipStream_t)stream_;
  if (!operands || !sink || !clocks || blocks <= 0 || iters <= 0) return -1;
  hipLaunchKernelGGL(mfma_lds_loop, dim3(blocks), dim3(256), 0, stream, (const uint4*)operands, sink, iters,
                     clocks);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

int pa_ceiling_mfma_valu(const void* operands, float* sink, int32_t blocks, int32_t iters, int32_t nvalu,
                         int32_t kind, unsigned long long* clocks, void* stream_) {
  const hipStream_t stream = (hipStream_t)stream_;
  if (!operands || !sink || !clocks || blocks <= 0 || iters <= 0 || (kind != 0 && kind != 1)) return -1;
  const uint4* o = (const uint4*)operands;
  hipError_t e;
  switch (nvalu) {
    case 0: e = launch_valu_loop<0>(kind, o, sink, blocks, iters, clocks, stream); break;
    case 2: e = launch_valu_loop<2>(kind, o, sink, blocks, iters, clocks, stream); break;
    case 4: e = launch_valu_loop<4>(kind, o, sink, blocks, iters, clocks, stream); break;
    case 6: e = launch_valu_loop<6>(kind, o, sink, blocks, iters, clocks, stream); break;
    case 8: e = launch_valu_loop<8>(kind, o, sink, blocks, iters, clocks, stream); break;
    default: return -1;
  }
  return e == hipSuccess ? 0 : -4;
}

int pa_ceiling_stream_read(const void* src, int64_t bytes, float* sink, int32_t blocks, void* stream_) {
  const hipStream_t stream = (hipStream_t)stream_;
  if (!src || !sink || blocks <= 0 || bytes < 16 || bytes % 16 != 0 || ((uintptr_t)src & 15) != 0) return -1;
  hipLaunchKernelGGL(stream_read, dim3(blocks), dim3(256), 0, stream, (const u32x4*)src, (long long)(bytes / 16), sink);
  return hipGetLastError() == hipSuccess ? 0 : -4;
}

}  // extern "C"
