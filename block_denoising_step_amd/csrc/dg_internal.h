// Internal interface between the host half of libdg (validation, planning,
// workspace layout) and the HIP launchers. No HIP types appear here, so the host
// half compiles and is testable without a GPU.
#pragma once

#include <cstddef>
#include <cstdint>

#include "../../include/dg.h"

namespace dg {

// ---- attention ---------------------------------------------------------------
//
// Work is laid out per request as [key chunk][kv head][q tile] in the bf16 head_dim-256
// kernels and [kv head][q tile][key chunk] in the general one. A q tile holds
// tile_rows query rows (tokens x grouped heads); a key chunk is a run of 64-key
// tiles. Every q tile of a request gets the same number of chunks (a chunk past a
// tile's keys is empty and exits at once). The kernel finds its (request, head,
// tile, chunk) from this table, so no work list has to be copied to the device.

constexpr int kAttnKeyTile = 64;
constexpr int kAttnTileRows = 128;      // q tile of the general kernel
constexpr int kAttnWideTileRows = 256;  // q tile of the bf16 head_dim-256 kernel (64 rows per wave)
// Rows of one merge work group (256 threads, one per 16 bytes of a partial row).
constexpr int attn_merge_rows_per_group(bool bf16, int head_dim) { return 256 / (head_dim / (bf16 ? 8 : 4)); }

struct AttnSeqPlan {
  int32_t q_start, num_q, kv_start, prefix_len, mode;
  int32_t tile_rows;        // query rows per q tile: kAttnWideTileRows or kAttnTileRows
  int32_t tokens_per_tile;  // tile_rows / G
  int32_t num_chunks;       // key chunks per q tile
  int32_t chunk_tiles;      // 64-key tiles per chunk (depends on this request only)
  int32_t work_begin;       // first work-group index of this request
  int32_t work_count;       // its work groups
  int32_t merge_begin;      // first merge work group (requests with num_chunks > 1)
  int32_t merge_count;      // its merge work groups
  int32_t part_begin;       // first partial row (requests with num_chunks > 1)
};

struct AttnPlan {
  int num_seqs;
  int group;            // G = Hq / Hkv
  int num_wide;         // work groups of the 64-rows-per-wave kernel: work [0, num_wide)
  int num_dma;          // end of the 128-row LDS-DMA kernel's work: [num_wide, num_dma)
  int num_work;         // all attention work groups; [num_dma, num_work) run the register-staged kernel
  int num_merge;        // work groups of the merge kernel
  int64_t part_rows;    // partial rows (each D wide)
  int block_shift;      // paged K/V: log2(block_size); -1 for the contiguous layout
  int kv_fp8;           // K/V hold E4M3 codes (bf16 queries, register-staged kernel)
  size_t part_o_offset;   // workspace: [part_rows][D] partial outputs, input dtype
  size_t part_ml_offset;  // workspace: [part_rows][2] fp32 (max, sum) in log2 units
  size_t bytes;
  AttnSeqPlan seqs[DG_MAX_SEQS];
};

// Validates args (everything but the workspace) and fills the plan.
dg_status attn_plan(const dg_attn_args* a, AttnPlan* plan, const char** msg);

// ---- sampler -----------------------------------------------------------------

struct SamplerPlan {
  int chunk;              // vocabulary entries per row-pass work group
  int num_chunks;         // chunks per row
  size_t sub_offset;      // workspace: sub-chunk masses [rows][chunks][32] fp32
  size_t bytes;           // workspace bytes (per-chunk statistics, sub-chunk masses)
};
dg_status sampler_plan(const dg_sampler_args* a, SamplerPlan* plan, const char** msg);

// ---- self-conditioning -------------------------------------------------------

struct SelfcondPlan {
  int dma;                     // 1: LDS-DMA kernel (bf16, V % 32 == 0); 0: register-staged kernel
  int tile_m, tile_n, tile_k;  // output tile per work group, K step
  int m_tiles, n_tiles;
  int splits;                  // split-K slices over V
  int k_per_split;             // vocabulary rows per slice (multiple of tile_k)
  size_t part_offset;          // workspace: partials per split and output tile (bf16 for bf16, else fp32; splits > 1)
  size_t p_offset;             // workspace: rebuilt bf16 probabilities [M][V] (logits mode, DMA kernel)
  size_t bytes;
};
dg_status selfcond_plan(const dg_selfcond_args* a, SelfcondPlan* plan, const char** msg);

// ---- paged K/V writes ----------------------------------------------------------

struct KvWritePlan {
  int64_t row_bytes;   // bytes of one source row (Hkv * D * element size of dtype)
  int64_t total_rows;  // rows written over all requests
  int block_shift;     // log2(block_size)
  int pool_fp8;        // pools hold E4M3 codes: values are quantized
  float k_inv, v_inv;  // pool_fp8: 1 / k_scale and 1 / v_scale, rounded to fp32
};
dg_status kv_write_plan(const dg_kv_write_args* a, KvWritePlan* plan, const char** msg);

// ---- self-conditioning injection ------------------------------------------------

struct InjectPlan {
  dg_selfcond_args gemm1;   // s . w_gate_up -> gu [M, 2 hidden] (workspace)
  dg_selfcond_args gemm2;   // h . w_down -> out
  SelfcondPlan plan1, plan2;
  size_t gu_offset, h_offset, gemm_ws_offset;  // workspace layout
  size_t bytes;
};
// Validates args (everything but the workspace) and fills the plan; the GEMM argument
// structs get their workspace pointers when the workspace is known (the call).
dg_status inject_plan(const dg_inject_args* a, InjectPlan* plan, const char** msg);

// Thread-local message for dg_last_error (the entry points in the .hip files use these).
dg_status record_error(dg_status s, const char* msg);
void clear_error();

// ---- launchers (HIP side); return 0 on success or a hipError_t value ---------

int launch_attn(const dg_attn_args* a, const AttnPlan& plan, void* stream);
int launch_sampler(const dg_sampler_args* a, const SamplerPlan& plan, void* stream);
// Epilogue of the split-K reduce, for the injection's two bf16 products (plain: the
// product itself).
enum { kReducePlain = 0, kReduceGeglu = 1, kReduceAddRows = 2 };
struct ReduceEpi {
  int mode;
  int half_tiles;          // geglu: column tiles of the gate half (hidden / tile_n); out is [M][hidden]
  const void* embed;       // add rows: [vocab][d] bf16
  const int32_t* tokens;   // add rows: [M], clamped to [0, vocab)
  int vocab;
};
int launch_selfcond(const dg_selfcond_args* a, const SelfcondPlan& plan, void* stream,
                    const ReduceEpi* epi = nullptr);
int launch_kv_write(const dg_kv_write_args* a, const KvWritePlan& plan, void* stream);
int launch_inject(const dg_inject_args* a, InjectPlan& plan, void* stream);
const char* hip_error_name(int err);

}  // namespace dg
