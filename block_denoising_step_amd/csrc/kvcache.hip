// Paged K/V writes on gfx950: new key rows (a prefill, a committed block or this
// step's canvas draft) are scattered into the K and V pools through each request's
// block table, the layout that dg_attn_mixed reads with block_size > 0.
//
// What is written follows [P1] ("DiffusionGemma: vLLM에서 네이티브로 처음 지원되는
// 첫 번째 Diffusion LLM") sections "샘플링 루프와 엔트로피 경계 디노이징" (a block is
// committed to the cache once it has converged) and "ModelState 인터페이스" (the
// canvas is redrafted at every step), on the paged cache that [P3] ("DiffusionGemma u
// vLLM: ...") section "Integracija u vLLM infrastrukturu" keeps from vLLM.
//
// A plain copy: HBM-bound, one 16-byte load and store per thread for K and for V,
// consecutive threads on consecutive bytes of a row (rows are Hkv x D contiguous in
// both the source and the pool).
//
// FP8 pools (the FP8 configuration the pages measure, [P1] section "성능 및 양자화"):
// each thread quantizes 8 consecutive values of a row to OCP E4M3 codes and stores
// them as 8 bytes; the rounding is done on the fp32 bits (round to nearest, ties to
// the even code), so it does not depend on a conversion instruction's modes.
#include "dg_common.cuh"
#include "dg_internal.h"

namespace dg {
namespace {

constexpr int kThreads = 256;

struct KvSeqTable {
  int32_t n;
  int32_t row_begin[DG_MAX_SEQS + 1];  // first written row of each request, over all requests
  int32_t src_start[DG_MAX_SEQS];
  int32_t table_start[DG_MAX_SEQS];
  int32_t pos[DG_MAX_SEQS];
};

__global__ __launch_bounds__(kThreads) void kv_write(KvSeqTable t, const int32_t* __restrict__ table,
                                                     int64_t pool_blocks, int shift, int vecs_per_row,
                                                     int64_t row_bytes, uint32_t total_vecs,
                                                     const char* __restrict__ k_new, const char* __restrict__ v_new,
                                                     char* __restrict__ k_pool, char* __restrict__ v_pool) {
  const uint32_t idx = blockIdx.x * kThreads + threadIdx.x;
  if (idx >= total_vecs) return;
  const int r = (int)(idx / (uint32_t)vecs_per_row);
  const int c = (int)(idx - (uint32_t)r * (uint32_t)vecs_per_row);
  int s = 0;
  for (int i = 1; i < t.n; ++i)
    if (r >= t.row_begin[i]) s = i;
  const int i = r - t.row_begin[s];
  const int p = t.pos[s] + i;  // key position within the request
  const int32_t e = table[t.table_start[s] + (p >> shift)];
  if (e < 0 || e >= pool_blocks) return;  // an entry outside the pool: nothing is written
  const int64_t dst_row = ((int64_t)e << shift) + (p & ((1 << shift) - 1));
  const int64_t src_off = (int64_t)(t.src_start[s] + i) * row_bytes + 16 * c;
  const int64_t dst_off = dst_row * row_bytes + 16 * c;
  const uint4 kx = *reinterpret_cast<const uint4*>(k_new + src_off);
  const uint4 vx = *reinterpret_cast<const uint4*>(v_new + src_off);
  *reinterpret_cast<uint4*>(k_pool + dst_off) = kx;
  *reinterpret_cast<uint4*>(v_pool + dst_off) = vx;
}

// One value as an E4M3 code: |y| clamped to 448 (NaN passes), then the nearest E4M3
// value, ties to the even code. Below 2^-6 the codes are the subnormal steps of
// 2^-9, so the code is |y| * 2^9 rounded to an integer (8 is 2^-6, the first normal
// code). Above, the code is the fp32 exponent (rebiased from 127 to 7) and the top 3
// mantissa bits, plus one when the remaining 20 bits are above half, or exactly half
// with the code odd; a carry steps into the exponent as the code increments.
__device__ __forceinline__ uint32_t e4m3_code(float y) {
  const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
  float a = fabsf(y);
  if (a != a) return sign | 0x7Fu;
  a = fminf(a, 448.f);
  if (a < 0.015625f) return sign | (uint32_t)__builtin_rintf(a * 512.f);
  const uint32_t b = __float_as_uint(a);
  uint32_t c = (((b >> 23) - 120u) << 3) | ((b >> 20) & 7u);
  const uint32_t rem = b & 0xFFFFFu;
  c += (rem > 0x80000u || (rem == 0x80000u && (c & 1u))) ? 1u : 0u;
  return sign | c;
}

// 8 consecutive values of a source row as fp32
template <bool kBf16>
__device__ __forceinline__ void load8(const char* src, int64_t elem, float (&x)[8]) {
  if constexpr (kBf16) {
    const uint4 v = *reinterpret_cast<const uint4*>(src + elem * 2);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[2 * k] = __uint_as_float(w[k] << 16);
      x[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
    }
  } else {
    const float4 a = *reinterpret_cast<const float4*>(src + elem * 4);
    const float4 b = *reinterpret_cast<const float4*>(src + elem * 4 + 16);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
}

__device__ __forceinline__ uint2 quantize8(const float (&x)[8], float inv) {
  uint32_t w[2] = {0u, 0u};
#pragma unroll
  for (int k = 0; k < 8; ++k) w[k >> 2] |= e4m3_code(x[k] * inv) << (8 * (k & 3));
  return make_uint2(w[0], w[1]);
}

// one thread per 8 values of a row: vecs_per_row = Hkv * D / 8
template <bool kBf16>
__global__ __launch_bounds__(kThreads) void kv_write_fp8(KvSeqTable t, const int32_t* __restrict__ table,
                                                         int64_t pool_blocks, int shift, int vecs_per_row,
                                                         uint32_t total_vecs, const char* __restrict__ k_new,
                                                         const char* __restrict__ v_new, char* __restrict__ k_pool,
                                                         char* __restrict__ v_pool, float k_inv, float v_inv) {
  const uint32_t idx = blockIdx.x * kThreads + threadIdx.x;
  if (idx >= total_vecs) return;
  const int r = (int)(idx / (uint32_t)vecs_per_row);
  const int c = (int)(idx - (uint32_t)r * (uint32_t)vecs_per_row);
  int s = 0;
  for (int i = 1; i < t.n; ++i)
    if (r >= t.row_begin[i]) s = i;
  const int i = r - t.row_begin[s];
  const int p = t.pos[s] + i;
  const int32_t e = table[t.table_start[s] + (p >> shift)];
  if (e < 0 || e >= pool_blocks) return;
  const int64_t row_elems = (int64_t)vecs_per_row * 8;
  const int64_t dst_row = ((int64_t)e << shift) + (p & ((1 << shift) - 1));
  const int64_t src = (int64_t)(t.src_start[s] + i) * row_elems + 8 * c;
  const int64_t dst = dst_row * row_elems + 8 * c;  // one byte per element
  float x[8];
  load8<kBf16>(k_new, src, x);
  *reinterpret_cast<uint2*>(k_pool + dst) = quantize8(x, k_inv);
  load8<kBf16>(v_new, src, x);
  *reinterpret_cast<uint2*>(v_pool + dst) = quantize8(x, v_inv);
}

}  // namespace

int launch_kv_write(const dg_kv_write_args* a, const KvWritePlan& plan, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  KvSeqTable t{};
  t.n = a->num_seqs;
  int32_t rows = 0;
  for (int i = 0; i < a->num_seqs; ++i) {
    t.row_begin[i] = rows;
    t.src_start[i] = a->seqs[i].src_start;
    t.table_start[i] = a->seqs[i].table_start;
    t.pos[i] = a->seqs[i].pos;
    rows += a->seqs[i].num;
  }
  t.row_begin[a->num_seqs] = rows;
  if (plan.pool_fp8) {
    const int vpr = a->num_kv_heads * a->head_dim / 8;
    const uint32_t total = (uint32_t)(plan.total_rows * vpr);
    const dim3 grid((total + kThreads - 1) / kThreads);
    if (a->dtype == DG_BF16)
      hipLaunchKernelGGL(kv_write_fp8<true>, grid, dim3(kThreads), 0, s, t, a->block_table,
                         a->pool_rows / a->block_size, plan.block_shift, vpr, total,
                         reinterpret_cast<const char*>(a->k_new), reinterpret_cast<const char*>(a->v_new),
                         reinterpret_cast<char*>(a->k_pool), reinterpret_cast<char*>(a->v_pool), plan.k_inv, plan.v_inv);
    else
      hipLaunchKernelGGL(kv_write_fp8<false>, grid, dim3(kThreads), 0, s, t, a->block_table,
                         a->pool_rows / a->block_size, plan.block_shift, vpr, total,
                         reinterpret_cast<const char*>(a->k_new), reinterpret_cast<const char*>(a->v_new),
                         reinterpret_cast<char*>(a->k_pool), reinterpret_cast<char*>(a->v_pool), plan.k_inv, plan.v_inv);
    return (int)hipGetLastError();
  }
  const int vecs_per_row = (int)(plan.row_bytes / 16);
  const uint32_t total = (uint32_t)(plan.total_rows * vecs_per_row);
  const dim3 grid((total + kThreads - 1) / kThreads);
  hipLaunchKernelGGL(kv_write, grid, dim3(kThreads), 0, s, t, a->block_table, a->pool_rows / a->block_size,
                     plan.block_shift, vecs_per_row, plan.row_bytes, total, reinterpret_cast<const char*>(a->k_new),
                     reinterpret_cast<const char*>(a->v_new), reinterpret_cast<char*>(a->k_pool),
                     reinterpret_cast<char*>(a->v_pool));
  return (int)hipGetLastError();
}

}  // namespace dg
