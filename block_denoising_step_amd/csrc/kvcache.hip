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
