// Device helpers shared by the libdg kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace dg {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

// bf16 pair in a 32-bit word -> two floats (exact).
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two floats -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
// Two floats to bf16 (round to nearest even), lo in the low half: one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  typedef float f32x2_v __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
  const f32x2_v v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_v));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---- wave64 reductions (all lanes get the result) ------------------------------
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ int wave_min_int(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ int wave_max_int(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, 64));
  return v;
}
// Inclusive prefix sum over the lanes, in lane order.
__device__ __forceinline__ float wave_incl_scan(float x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  return x;
}
// The value of the previous lane (0 in lane 0): an exclusive scan from an inclusive one.
__device__ __forceinline__ float wave_shift_up(float x) {
  const float y = __shfl_up(x, 1, 64);
  return (threadIdx.x & 63) ? y : 0.f;
}

// ---- Philox4x64-10 (Salmon, Moraes, Dror, Shaw, SC'11) ---------------------------
// One round maps (x0,x1,x2,x3) under key (k0,k1) to
//   (hi(M1*x2)^x1^k0, lo(M1*x2), hi(M0*x0)^x3^k1, lo(M0*x0));
// the key advances by the Weyl constants between rounds. Only word 0 is used here.
__device__ __forceinline__ uint64_t philox_word0(uint64_t seed, uint64_t c0, uint64_t c1, uint64_t c2) {
  const uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
  const uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
  uint64_t x0 = c0, x1 = c1, x2 = c2, x3 = 0, k0 = seed, k1 = 0;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) { k0 += W0; k1 += W1; }
    const uint64_t lo0 = M0 * x0, hi0 = __umul64hi(M0, x0);
    const uint64_t lo1 = M1 * x2, hi1 = __umul64hi(M1, x2);
    const uint64_t n0 = hi1 ^ x1 ^ k0, n2 = hi0 ^ x3 ^ k1;
    x0 = n0; x1 = lo1; x2 = n2; x3 = lo0;
  }
  return x0;
}

// tanh-approximated GELU: x/2 * (1 + tanh(sqrt(2/pi) * (x + 0.044715 x^3)))
__device__ __forceinline__ float gelu_tanh(float x) {
  const float k = 0.7978845608028654f;  // sqrt(2 / pi)
  return 0.5f * x * (1.f + tanhf(k * fmaf(0.044715f * x, x * x, x)));
}

}  // namespace dg
