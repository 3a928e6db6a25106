// Measurement kernels for the achievable ceilings of gfx950 (the declarations and
// their contract are in include/dg_probe.h). Not part of the denoising step.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/dg_probe.h"

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

constexpr int kThreads = 256;
constexpr int kUnroll = 8;  // 16-byte loads in flight per thread

// Each work group takes runs of kUnroll * kThreads consecutive 16-byte words (grid
// stride between runs); a thread issues its kUnroll loads of a run, guarded by the end,
// before it uses any of them.
__global__ __launch_bounds__(kThreads) void probe_read(const uint4* __restrict__ src, int64_t n,
                                                       uint32_t* __restrict__ sink) {
  const int64_t step = (int64_t)gridDim.x * kThreads * kUnroll;
  uint32_t acc = 0;
  for (int64_t base = (int64_t)blockIdx.x * kThreads * kUnroll + threadIdx.x; base < n; base += step) {
    uint4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = base + u * kThreads;
      v[u] = i < n ? src[i] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  // one word per work group: XOR over the block through LDS
  __shared__ uint32_t red[kThreads / 64];
  for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

__global__ __launch_bounds__(kThreads) void probe_copy(uint4* __restrict__ dst, const uint4* __restrict__ src,
                                                       int64_t n) {
  const int64_t step = (int64_t)gridDim.x * kThreads * kUnroll;
  for (int64_t base = (int64_t)blockIdx.x * kThreads * kUnroll + threadIdx.x; base < n; base += step) {
    uint4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = base + u * kThreads;
      if (i < n) v[u] = src[i];
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = base + u * kThreads;
      if (i < n) dst[i] = v[u];
    }
  }
}

// 8 independent accumulation chains per wave, operands in registers. With `ops`, each
// lane takes 4 A and 4 B operand vectors from memory and every MFMA of an unrolled
// group of 4 iterations uses a different (A, B) pair, so the matrix inputs change from
// instruction to instruction as a GEMM's do; without it, one fixed pair.
__global__ __launch_bounds__(kThreads) void probe_mfma_bf16(const uint4* __restrict__ ops, float* __restrict__ sink,
                                                            int iters) {
  bf16x8 a[4], b[4];
  if (ops) {
    const uint4* o = ops + ((int64_t)blockIdx.x * kThreads + threadIdx.x) * 8;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      a[t] = __builtin_bit_cast(bf16x8, o[t]);
      b[t] = __builtin_bit_cast(bf16x8, o[4 + t]);
    }
  } else {
    const float x = (float)(threadIdx.x & 7) * 0.125f;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        a[t][e] = (__bf16)(x + 0.0078125f * e);
        b[t][e] = (__bf16)(0.5f - 0.0078125f * e);
      }
  }
  f32x16 acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[c][e] = 0.f;
  for (int it = 0; it < iters; it += 4) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int c = 0; c < 8; ++c)
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(c + u) & 3], b[(3 * c + u) & 3], acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[c][e];
  sink[(int64_t)blockIdx.x * kThreads + threadIdx.x] = s;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

extern "C" {

int dg_probe_read(const void* src, size_t bytes, uint32_t* sink, int blocks, void* stream) {
  if (!src || !sink || !aligned16(src) || bytes % 16 || blocks < 1 || blocks > 65536) return -1;
  hipLaunchKernelGGL(probe_read, dim3(blocks), dim3(kThreads), 0, reinterpret_cast<hipStream_t>(stream),
                     reinterpret_cast<const uint4*>(src), (int64_t)(bytes / 16), sink);
  return (int)hipGetLastError();
}

int dg_probe_copy(void* dst, const void* src, size_t bytes, int blocks, void* stream) {
  if (!src || !dst || !aligned16(src) || !aligned16(dst) || bytes % 16 || blocks < 1 || blocks > 65536) return -1;
  const char* s = reinterpret_cast<const char*>(src);
  const char* d = reinterpret_cast<const char*>(dst);
  if (s < d + bytes && d < s + bytes) return -1;
  hipLaunchKernelGGL(probe_copy, dim3(blocks), dim3(kThreads), 0, reinterpret_cast<hipStream_t>(stream),
                     reinterpret_cast<uint4*>(dst), reinterpret_cast<const uint4*>(src), (int64_t)(bytes / 16));
  return (int)hipGetLastError();
}

int dg_probe_mfma_bf16(const void* ops, float* sink, int blocks, int iters, void* stream) {
  if (!sink || blocks < 1 || blocks > 65536 || iters < 4 || iters > (1 << 24) || iters % 4) return -1;
  if (ops && !aligned16(ops)) return -1;
  hipLaunchKernelGGL(probe_mfma_bf16, dim3(blocks), dim3(kThreads), 0, reinterpret_cast<hipStream_t>(stream),
                     reinterpret_cast<const uint4*>(ops), sink, iters);
  return (int)hipGetLastError();
}

}  // extern "C"
