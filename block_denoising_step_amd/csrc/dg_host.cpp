// Host half of libdg: argument validation, work planning, workspace sizing and the
// extern "C" entry points declared in include/dg.h. Nothing here touches HIP: a
// call either fails validation here (nothing launched, nothing written) or is
// handed to the launchers in the .hip files.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <vector>

#include "dg_internal.h"

namespace dg {
namespace {

thread_local char g_last_error[512] = "";
// Test hook (dg_test_force_register_staged): plan every request on the register-staged
// attention kernel.
std::atomic<int> g_force_register_staged{0};
// Test hook (dg_test_wide_min_sub): the sub-tiles per work group from which a request runs
// on the 64-rows-per-wave attention kernel.
constexpr int kWideMinSubDefault = 64;
std::atomic<int> g_wide_min_sub{kWideMinSubDefault};

dg_status fail(dg_status s, const char* msg) {
  std::snprintf(g_last_error, sizeof(g_last_error), "%s", msg);
  return s;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Request-local key range [lo, hi] of new token i ([P1] section
// "대칭 슬라이딩 윈도우 어텐션": one-sided window for causal requests, symmetric for
// bidirectional ones; global layers use window < 0).
void key_range(int mode, int prefix, int num_q, int window, int i, int* lo, int* hi) {
  const int p = prefix + i;
  const int last = prefix + num_q - 1;
  *lo = window < 0 ? 0 : std::max(0, p - window);
  if (mode == DG_CAUSAL) *hi = p;
  else *hi = window < 0 ? last : std::min(last, p + window);
}

}  // namespace

dg_status record_error(dg_status s, const char* msg) { return fail(s, msg); }
void clear_error() { g_last_error[0] = 0; }

// ---- attention plan ----------------------------------------------------------
//
// A request with a single chunk per q tile writes its output directly; one with
// several writes partials (each chunk's output normalised by that chunk's sum, in the
// input dtype, plus its (max, sum) in fp32) that the merge kernel combines in chunk order.
// A request's chunk length gives it about kTargetGroups work groups (one per compute
// unit: a work group of the bf16 head_dim-256 kernels fills a CU), but never under
// kMinChunkTiles tiles, since every partial costs a [tile rows x D] write and read,
// unless the request is too small to reach kTargetGroups work groups at all.

static constexpr int kKeyTile = kAttnKeyTile;
static constexpr int kTargetGroups = 256;
static constexpr int kMinChunkTiles = 4;

dg_status attn_plan(const dg_attn_args* a, AttnPlan* plan, const char** msg) {
  auto bad = [&](dg_status s, const char* m) { *msg = m; return s; };
  if (!a) return bad(DG_ERR_INVALID_ARG, "args is NULL");
  if (a->num_seqs < 1 || a->num_seqs > DG_MAX_SEQS) return bad(DG_ERR_INVALID_ARG, "num_seqs must be in [1, DG_MAX_SEQS]");
  if (!a->seqs) return bad(DG_ERR_INVALID_ARG, "seqs is NULL");
  if (a->dtype != DG_F32 && a->dtype != DG_BF16) return bad(DG_ERR_INVALID_ARG, "dtype must be DG_F32 or DG_BF16");
  if (a->num_q_heads < 1 || a->num_kv_heads < 1) return bad(DG_ERR_INVALID_ARG, "head counts must be >= 1");
  if (a->num_q_heads % a->num_kv_heads) return bad(DG_ERR_INVALID_ARG, "num_q_heads must be a multiple of num_kv_heads");
  const int G = a->num_q_heads / a->num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16 && G != 32)
    return bad(DG_ERR_UNSUPPORTED, "num_q_heads / num_kv_heads must be a power of two <= 32");
  if (a->head_dim != 64 && a->head_dim != 128 && a->head_dim != 256)
    return bad(DG_ERR_UNSUPPORTED, "head_dim must be 64, 128 or 256");
  if (a->dtype == DG_F32 && a->head_dim > 128) return bad(DG_ERR_UNSUPPORTED, "fp32 attention supports head_dim 64 and 128");
  if (a->window < -1) return bad(DG_ERR_INVALID_ARG, "window must be -1 (global) or >= 0");
  if (!std::isfinite(a->scale) || a->scale < 0.f) return bad(DG_ERR_INVALID_ARG, "scale must be finite and >= 0");
  if (a->total_q < 0 || a->total_kv < 0) return bad(DG_ERR_INVALID_ARG, "total_q and total_kv must be >= 0");
  if (a->kv_chunk < 0 || a->kv_chunk % kKeyTile) return bad(DG_ERR_INVALID_ARG, "kv_chunk must be 0 or a positive multiple of 64");
  if (!a->q || !a->k || !a->v || !a->out) return bad(DG_ERR_INVALID_ARG, "q, k, v and out must be non-NULL");
  if (!aligned16(a->q) || !aligned16(a->k) || !aligned16(a->v) || !aligned16(a->out))
    return bad(DG_ERR_INVALID_ARG, "q, k, v and out must be 16-byte aligned");
  if (a->lse && !aligned4(a->lse)) return bad(DG_ERR_INVALID_ARG, "lse must be 4-byte aligned");
  // FP8 K/V: E4M3 codes with per-tensor scales, bf16 queries; the register-staged kernel
  if (a->kv_fp8 != 0 && a->kv_fp8 != 1) return bad(DG_ERR_INVALID_ARG, "kv_fp8 must be 0 or 1");
  plan->kv_fp8 = a->kv_fp8;
  if (a->kv_fp8) {
    if (a->dtype != DG_BF16) return bad(DG_ERR_UNSUPPORTED, "kv_fp8 needs dtype DG_BF16");
    if (!std::isfinite(a->k_scale) || !(a->k_scale > 0.f) || !std::isfinite(a->v_scale) || !(a->v_scale > 0.f))
      return bad(DG_ERR_INVALID_ARG, "k_scale and v_scale must be finite and > 0 with kv_fp8");
  }
  // paged K/V: pools of block_size-row blocks, a block table per request
  const bool paged = a->block_size != 0;
  plan->block_shift = -1;
  if (paged) {
    if (a->block_size < kKeyTile || (a->block_size & (a->block_size - 1)))
      return bad(DG_ERR_INVALID_ARG, "block_size must be 0 or a power of two >= 64");
    if (a->total_kv < a->block_size || a->total_kv % a->block_size)
      return bad(DG_ERR_INVALID_ARG, "total_kv must be a positive multiple of block_size in paged mode");
    if (!a->block_table || !aligned4(a->block_table)) return bad(DG_ERR_INVALID_ARG, "block_table must be non-NULL and 4-byte aligned");
    if (a->block_table_len < 1) return bad(DG_ERR_INVALID_ARG, "block_table_len must be >= 1 in paged mode");
    int sh = 0;
    while ((1 << sh) < a->block_size) ++sh;
    plan->block_shift = sh;
  }

  // request geometry
  std::vector<std::pair<int64_t, int64_t>> qranges;
  for (int s = 0; s < a->num_seqs; ++s) {
    const dg_seq& q = a->seqs[s];
    if (q.mode != DG_CAUSAL && q.mode != DG_BIDIR) return bad(DG_ERR_INVALID_ARG, "seq mode must be DG_CAUSAL or DG_BIDIR");
    if (q.q_start < 0 || q.num_q < 0 || q.kv_start < 0 || q.prefix_len < 0)
      return bad(DG_ERR_INVALID_ARG, "seq offsets and lengths must be >= 0");
    if ((int64_t)q.q_start + q.num_q > a->total_q) return bad(DG_ERR_INVALID_ARG, "seq query rows exceed total_q");
    if (!paged && (int64_t)q.kv_start + q.prefix_len + q.num_q > a->total_kv)
      return bad(DG_ERR_INVALID_ARG, "seq key rows exceed total_kv");
    if (paged && (int64_t)q.kv_start + ceil_div((int64_t)q.prefix_len + q.num_q, a->block_size) > a->block_table_len)
      return bad(DG_ERR_INVALID_ARG, "seq block table entries exceed block_table_len");
    if (paged && (int64_t)q.kv_start + ceil_div((int64_t)q.prefix_len + q.num_q, a->block_size) > INT32_MAX)
      return bad(DG_ERR_UNSUPPORTED, "seq block table entries past index 2^31 - 1");
    if ((int64_t)q.prefix_len + q.num_q > INT32_MAX - kKeyTile) return bad(DG_ERR_INVALID_ARG, "seq too long");
    if (q.num_q > 0) qranges.push_back({q.q_start, (int64_t)q.q_start + q.num_q});
  }
  std::sort(qranges.begin(), qranges.end());
  for (size_t i = 1; i < qranges.size(); ++i)
    if (qranges[i].first < qranges[i - 1].second) return bad(DG_ERR_INVALID_ARG, "seq query ranges overlap");

  // tiles and chunks; the split of a request, and the kernel that runs it, depend on
  // that request alone, so its result is the same whatever else is in the batch.
  // The LDS-DMA kernels (bf16 queries, head_dim 256; K/V in bf16 or, with kv_fp8, E4M3
  // codes) take 32-bit byte offsets within a request's K/V,
  // so a contiguous request whose K/V span passes 2^31 - 1 bytes runs on the
  // register-staged kernel; paged requests are addressed per sub-tile and have no limit.
  const bool dma_ok = a->dtype == DG_BF16 && a->head_dim == 256 &&
                      !g_force_register_staged.load(std::memory_order_relaxed);
  const int64_t kv_elem_bytes = a->kv_fp8 ? 1 : 2;
  bool dma[DG_MAX_SEQS];
  for (int s = 0; s < a->num_seqs; ++s) {
    const dg_seq& q = a->seqs[s];
    dma[s] = dma_ok && (paged || ((int64_t)q.prefix_len + q.num_q) * a->num_kv_heads * a->head_dim * kv_elem_bytes <=
                                     INT32_MAX);
  }
  // q tiles and key chunks of request q at a given tile height
  struct Split { int64_t ntiles_q, nch, chunk_tiles, sub_tiles; };
  auto split = [&](const dg_seq& q, int tile_rows) {
    const int tok = tile_rows / G;
    Split r{ceil_div(q.num_q, tok), 0, 0, 0};
    int64_t max_tiles = 0, units = 0;
    for (int t = 0; t < r.ntiles_q; ++t) {
      const int i0 = t * tok, i1 = std::min<int>(q.num_q, i0 + tok) - 1;
      int lo0, hi0, lo1, hi1;
      key_range(q.mode, q.prefix_len, q.num_q, a->window, i0, &lo0, &hi0);
      key_range(q.mode, q.prefix_len, q.num_q, a->window, i1, &lo1, &hi1);
      const int64_t nt = hi1 / kKeyTile - lo0 / kKeyTile + 1;
      max_tiles = std::max(max_tiles, nt);
      units += nt * a->num_kv_heads;
    }
    if (a->kv_chunk > 0) r.chunk_tiles = a->kv_chunk / kKeyTile;
    // a request too small to fill the GPU even at one tile per chunk takes one-tile chunks;
    // otherwise every q tile gets as many chunks as its longest key range needs, so the
    // chunk is sized from that range: about kTargetGroups work groups in all (a causal
    // request's shorter q tiles leave some of their chunks empty)
    else r.chunk_tiles = units < kTargetGroups
                             ? 1
                             : std::max<int64_t>(kMinChunkTiles,
                                                 ceil_div(max_tiles * r.ntiles_q * a->num_kv_heads, kTargetGroups));
    r.nch = max_tiles > 0 ? ceil_div(max_tiles, r.chunk_tiles) : 0;
    r.sub_tiles = units * (kKeyTile / 32);  // 32-key sub-tiles over all (q tile, kv head) units
    return r;
  };
  // The 64-rows-per-wave kernel reads each K/V byte into LDS for twice the rows, but has
  // the larger fixed cost (prologue, epilogue, twice the rows per work group) and, per
  // row, a loop no faster than the 128-row kernel's: it takes a request whose work
  // groups average at least kWideMinSubDefault sub-tiles (measured: a 16384-key denoise
  // request runs faster on the 128-row kernel, a 262144-key one on this one).
  const int64_t wide_min_sub = g_wide_min_sub.load(std::memory_order_relaxed);
  bool wide[DG_MAX_SEQS];
  Split sq[DG_MAX_SEQS];
  for (int s = 0; s < a->num_seqs; ++s) {
    const dg_seq& q = a->seqs[s];
    wide[s] = false;
    if (dma[s] && q.num_q > 0) {
      const Split w = split(q, kAttnWideTileRows);
      const int64_t groups = w.ntiles_q * w.nch * a->num_kv_heads;
      wide[s] = groups > 0 && w.sub_tiles >= wide_min_sub * groups;
      if (wide[s]) sq[s] = w;
    }
    if (!wide[s]) sq[s] = split(q, kAttnTileRows);
  }
  const int mrpg = attn_merge_rows_per_group(a->dtype == DG_BF16, a->head_dim);
  int64_t num_work = 0, num_merge = 0, part_rows = 0, num_wide = 0, num_dma = 0;
  plan->num_seqs = a->num_seqs;
  // Work list: the wide kernel's requests, then the 128-row LDS-DMA kernel's, then the
  // register-staged kernel's (one launch each); within each,
  // requests with the longest work groups first, so that the short ones fill the tail.
  // The order changes no result: every work group computes the same thing wherever it runs.
  int order[DG_MAX_SEQS];
  double per_group[DG_MAX_SEQS];
  for (int s = 0; s < a->num_seqs; ++s) {
    order[s] = s;
    const int64_t groups = a->num_kv_heads * sq[s].ntiles_q * sq[s].nch;
    per_group[s] = groups > 0 ? (double)sq[s].sub_tiles / (double)groups : 0.0;
  }
  std::stable_sort(order, order + a->num_seqs, [&](int x, int y) { return per_group[x] > per_group[y]; });
  for (int pass = 0; pass < 3; ++pass)
    for (int oi = 0; oi < a->num_seqs; ++oi) {
      const int s = order[oi];
      if ((wide[s] ? 0 : dma[s] ? 1 : 2) != pass) continue;
      const dg_seq& q = a->seqs[s];
      const Split& r = sq[s];
      const int tile_rows = wide[s] ? kAttnWideTileRows : kAttnTileRows;
      AttnSeqPlan& sp = plan->seqs[s];
      sp.q_start = q.q_start;
      sp.num_q = q.num_q;
      sp.kv_start = q.kv_start;
      sp.prefix_len = q.prefix_len;
      sp.mode = q.mode;
      sp.tile_rows = tile_rows;
      sp.tokens_per_tile = tile_rows / G;
      sp.num_chunks = (int32_t)r.nch;
      sp.chunk_tiles = (int32_t)std::min<int64_t>(r.chunk_tiles, INT32_MAX);
      const int64_t units = a->num_kv_heads * r.ntiles_q;
      sp.work_begin = (int32_t)num_work;
      sp.work_count = (int32_t)std::min<int64_t>(units * r.nch, INT32_MAX);
      sp.merge_begin = (int32_t)num_merge;
      sp.merge_count = 0;
      sp.part_begin = (int32_t)std::min<int64_t>(part_rows, INT32_MAX);
      num_work += units * r.nch;
      if (wide[s]) num_wide += units * r.nch;
      if (dma[s]) num_dma += units * r.nch;
      if (r.nch > 1) {
        sp.merge_count = (int32_t)std::min<int64_t>(units * (tile_rows / mrpg), INT32_MAX);
        num_merge += units * (tile_rows / mrpg);
        part_rows += units * r.nch * tile_rows;
      }
      if (num_work > INT32_MAX / 2 || num_merge > INT32_MAX / 2 || part_rows > INT32_MAX / 2)
        return bad(DG_ERR_UNSUPPORTED, "too much work for one call");
    }
  plan->group = G;
  plan->num_wide = (int)num_wide;
  plan->num_dma = (int)num_dma;
  plan->num_work = (int)num_work;
  plan->num_merge = (int)num_merge;
  plan->part_rows = part_rows;
  plan->part_o_offset = 0;
  const size_t o_bytes = (size_t)part_rows * a->head_dim * (a->dtype == DG_BF16 ? 2 : 4);
  plan->part_ml_offset = align_up(o_bytes, 256);
  const size_t ml_bytes = (size_t)part_rows * 2 * sizeof(float);
  plan->bytes = part_rows ? align_up(plan->part_ml_offset + ml_bytes, 256) : 0;
  return DG_OK;
}

// ---- sampler plan ------------------------------------------------------------

dg_status sampler_plan(const dg_sampler_args* a, SamplerPlan* plan, const char** msg) {
  auto bad = [&](dg_status s, const char* m) { *msg = m; return s; };
  if (!a) return bad(DG_ERR_INVALID_ARG, "args is NULL");
  if (a->num_reqs < 1 || a->num_reqs > DG_MAX_REQS) return bad(DG_ERR_INVALID_ARG, "num_reqs must be in [1, DG_MAX_REQS]");
  if (!a->reqs) return bad(DG_ERR_INVALID_ARG, "reqs is NULL");
  if (a->num_rows < 1) return bad(DG_ERR_INVALID_ARG, "num_rows must be >= 1");
  if (a->vocab < 1) return bad(DG_ERR_INVALID_ARG, "vocab must be >= 1");
  if (a->dtype != DG_F32 && a->dtype != DG_BF16) return bad(DG_ERR_INVALID_ARG, "dtype must be DG_F32 or DG_BF16");
  const bool reads_logits = !(a->flags & (DG_INIT_CANVAS | DG_SELECT_ONLY));
  if (reads_logits && (a->ld < a->vocab || a->ld % 8)) return bad(DG_ERR_INVALID_ARG, "ld must be >= vocab and a multiple of 8");
  if (!std::isfinite(a->budget) || a->budget < 0.f) return bad(DG_ERR_INVALID_ARG, "budget must be finite and >= 0");
  if (!std::isfinite(a->tau) || a->tau < 0.f) return bad(DG_ERR_INVALID_ARG, "tau must be finite and >= 0");
  if (a->min_accept < 0) return bad(DG_ERR_INVALID_ARG, "min_accept must be >= 0");
  if (a->conf_mode != DG_CONF_NEG_ENTROPY && a->conf_mode != DG_CONF_MAX_PROB) return bad(DG_ERR_INVALID_ARG, "bad conf_mode");
  if (a->combine != DG_CONV_AND && a->combine != DG_CONV_OR) return bad(DG_ERR_INVALID_ARG, "bad combine");
  if (a->renoise != 0 && a->renoise != 1) return bad(DG_ERR_INVALID_ARG, "renoise must be 0 or 1");
  if (a->stable_k < 1 || a->step_limit < 1) return bad(DG_ERR_INVALID_ARG, "stable_k and step_limit must be >= 1");
  if (a->flags & ~(DG_ENTROPY_IN | DG_INIT_CANVAS | DG_SKIP_SELECT | DG_SELECT_ONLY))
    return bad(DG_ERR_INVALID_ARG, "unknown flag bits");
  const bool init = a->flags & DG_INIT_CANVAS;
  const bool select_only = a->flags & DG_SELECT_ONLY;
  if ((a->flags & DG_SKIP_SELECT) && (select_only || init))
    return bad(DG_ERR_INVALID_ARG, "DG_SKIP_SELECT excludes DG_SELECT_ONLY and DG_INIT_CANVAS");
  if (select_only && init) return bad(DG_ERR_INVALID_ARG, "DG_SELECT_ONLY excludes DG_INIT_CANVAS");
  if (!init && !select_only && !a->logits) return bad(DG_ERR_INVALID_ARG, "logits is NULL");
  if (a->logits && !aligned16(a->logits)) return bad(DG_ERR_INVALID_ARG, "logits must be 16-byte aligned");
  const void* ptrs[] = {a->entropy, a->conf, a->row_max, a->row_sum, a->argmax, a->cand, a->canvas,
                        a->prev_argmax, a->stable_count, a->num_accepted, a->converged, a->mean_entropy};
  for (const void* p : ptrs)
    if (!p || !aligned4(p)) return bad(DG_ERR_INVALID_ARG, "every output/state pointer must be non-NULL and 4-byte aligned");
  if (!a->accept) return bad(DG_ERR_INVALID_ARG, "accept is NULL");
  if ((a->probs == nullptr) != (a->probs_scale == nullptr)) return bad(DG_ERR_INVALID_ARG, "set both probs and probs_scale, or neither");
  if (a->probs && (!aligned16(a->probs) || !aligned4(a->probs_scale))) return bad(DG_ERR_INVALID_ARG, "probs must be 16-byte aligned");
  if (a->step_counter && !aligned4(a->step_counter)) return bad(DG_ERR_INVALID_ARG, "step_counter must be 4-byte aligned");
  if (a->probs && (a->ldq < a->vocab || a->ldq % 8)) return bad(DG_ERR_INVALID_ARG, "ldq must be >= vocab and a multiple of 8");
  std::vector<std::pair<int64_t, int64_t>> r;
  for (int i = 0; i < a->num_reqs; ++i) {
    const dg_sreq& q = a->reqs[i];
    if (q.num_rows < 1 || q.num_rows > DG_MAX_CANVAS) return bad(DG_ERR_INVALID_ARG, "request num_rows must be in [1, DG_MAX_CANVAS]");
    if (q.row_start < 0 || (int64_t)q.row_start + q.num_rows > a->num_rows) return bad(DG_ERR_INVALID_ARG, "request rows exceed num_rows");
    if (q.step < 0) return bad(DG_ERR_INVALID_ARG, "request step must be >= 0");
    if (q.reserved != 0) return bad(DG_ERR_INVALID_ARG, "request reserved field must be 0");
    r.push_back({q.row_start, (int64_t)q.row_start + q.num_rows});
  }
  std::sort(r.begin(), r.end());
  for (size_t i = 1; i < r.size(); ++i)
    if (r[i].first < r[i - 1].second) return bad(DG_ERR_INVALID_ARG, "request row ranges overlap");
  plan->chunk = a->dtype == DG_BF16 ? 16384 : 8192;
  plan->num_chunks = (int)ceil_div(a->vocab, plan->chunk);
  if (plan->num_chunks > 1024) return bad(DG_ERR_UNSUPPORTED, "vocab too large (more than 1024 row-pass chunks)");
  plan->sub_offset = align_up((size_t)a->num_rows * plan->num_chunks * 16, 256);
  plan->bytes = init || select_only ? 0 : plan->sub_offset + align_up((size_t)a->num_rows * plan->num_chunks * 32 * sizeof(float), 256);
  return DG_OK;
}

// ---- self-conditioning plan --------------------------------------------------

dg_status selfcond_plan(const dg_selfcond_args* a, SelfcondPlan* plan, const char** msg) {
  auto bad = [&](dg_status s, const char* m) { *msg = m; return s; };
  if (!a) return bad(DG_ERR_INVALID_ARG, "args is NULL");
  if (a->M < 1 || a->V < 1 || a->d < 1) return bad(DG_ERR_INVALID_ARG, "M, V and d must be >= 1");
  if (a->dtype != DG_F32 && a->dtype != DG_BF16) return bad(DG_ERR_INVALID_ARG, "dtype must be DG_F32 or DG_BF16");
  if (a->d % 128) return bad(DG_ERR_UNSUPPORTED, "d must be a multiple of 128");
  if (a->ldp < a->V || a->ldp % 8) return bad(DG_ERR_INVALID_ARG, "ldp must be >= V and a multiple of 8");
  if (a->lde < a->d || a->lde % 8) return bad(DG_ERR_INVALID_ARG, "lde must be >= d and a multiple of 8");
  if (a->ldo < a->d || a->ldo % 8) return bad(DG_ERR_INVALID_ARG, "ldo must be >= d and a multiple of 8");
  if (!a->p || !a->embed || !a->out) return bad(DG_ERR_INVALID_ARG, "p, embed and out must be non-NULL");
  if (!aligned16(a->p) || !aligned16(a->embed) || !aligned16(a->out)) return bad(DG_ERR_INVALID_ARG, "p, embed and out must be 16-byte aligned");
  if ((a->row_max == nullptr) != (a->row_sum == nullptr)) return bad(DG_ERR_INVALID_ARG, "set both row_max and row_sum, or neither");
  if (a->p_scale && a->row_max) return bad(DG_ERR_INVALID_ARG, "p_scale and row_max/row_sum are exclusive");
  const bool scaled = a->p_scale != nullptr;
  const bool fused = a->row_max != nullptr;
  plan->dma = a->dtype == DG_BF16 && a->V % 32 == 0;
  // The DMA kernel's 128 x 512 tile spends less of its LDS ring on P (an L2-resident
  // operand shared by the tile's neighbours) and more on E, the stream from HBM.
  // A small unscaled product (a weight matrix, K <= 16384, at most 256 rows) takes a
  // 256 x 128 tile: every byte of E read by one work group, and twice the work groups of
  // a 64K-value tile, so that the few K steps of each still fill the GPU.
  const bool narrow = plan->dma && !scaled && a->M <= 256 && a->V <= 16384 && a->d % 128 == 0;
  const bool wide = plan->dma && !narrow && a->d % 512 == 0;
  // An fp32 product with fewer than 16 tiles of 256 x 256 takes 64 x 128 tiles: at one
  // K step per slice, 256 x 256 tiles would leave half the CUs idle (a slice must hold a
  // whole step) and write a 256 KB partial per step.
  const bool small_f32 = !plan->dma && a->dtype == DG_F32 && ceil_div(a->M, 256) * ceil_div(a->d, 256) < 16;
  plan->tile_m = wide ? 128 : small_f32 ? 64 : 256;
  plan->tile_n = wide ? 512 : narrow || small_f32 ? 128 : 256;
  plan->tile_k = plan->dma ? 32 : (a->dtype == DG_BF16 ? 64 : 32);
  plan->m_tiles = (int)ceil_div(a->M, plan->tile_m);
  plan->n_tiles = (int)ceil_div(a->d, plan->tile_n);
  // split-K: about one work group per CU, in slices of at least kMinSteps K steps (one
  // for fp32, whose MFMA rate makes a single 256 x 256 tile's slice compute-bound)
  constexpr int64_t kCUs = 256;
  const int64_t kMinSteps = a->dtype == DG_F32 ? 1 : 8;
  const int64_t base = (int64_t)plan->m_tiles * plan->n_tiles;
  const int64_t target = std::max<int64_t>(1, ceil_div(kCUs, base));
  int64_t k_per_split;
  if (scaled) {
    // every slice inside one scale block: a power-of-two fraction of DG_PROB_BLOCK
    k_per_split = DG_PROB_BLOCK;
    while (k_per_split > plan->tile_k * kMinSteps && ceil_div(a->V, k_per_split) < target) k_per_split /= 2;
  } else {
    const int64_t ksteps = ceil_div(a->V, plan->tile_k);
    const int64_t splits = std::max<int64_t>(1, std::min<int64_t>(target, ksteps / kMinSteps));
    k_per_split = ceil_div(ksteps, splits) * plan->tile_k;
  }
  plan->splits = (int)ceil_div(a->V, k_per_split);
  plan->k_per_split = (int)k_per_split;
  plan->part_offset = 0;
  // partials in whole tiles (MFMA register layout)
  // partials: bf16 for bf16 products, fp32 for fp32 ones
  size_t bytes = plan->splits > 1 ? align_up((size_t)plan->splits * plan->m_tiles * plan->n_tiles *
                                             plan->tile_m * plan->tile_n * (a->dtype == DG_BF16 ? 2 : 4), 256) : 0;
  plan->p_offset = bytes;
  if (plan->dma && fused) bytes += align_up((size_t)a->M * a->V * 2, 256);
  plan->bytes = bytes;
  return DG_OK;
}

// ---- paged K/V writes ----------------------------------------------------------

dg_status kv_write_plan(const dg_kv_write_args* a, KvWritePlan* plan, const char** msg) {
  auto bad = [&](dg_status s, const char* m) { *msg = m; return s; };
  if (!a) return bad(DG_ERR_INVALID_ARG, "args is NULL");
  if (a->num_seqs < 1 || a->num_seqs > DG_MAX_SEQS) return bad(DG_ERR_INVALID_ARG, "num_seqs must be in [1, DG_MAX_SEQS]");
  if (!a->seqs) return bad(DG_ERR_INVALID_ARG, "seqs is NULL");
  if (a->dtype != DG_F32 && a->dtype != DG_BF16) return bad(DG_ERR_INVALID_ARG, "dtype must be DG_F32 or DG_BF16");
  if (a->pool_fp8 != 0 && a->pool_fp8 != 1) return bad(DG_ERR_INVALID_ARG, "pool_fp8 must be 0 or 1");
  if (a->pool_fp8 && (!std::isfinite(a->k_scale) || !(a->k_scale > 0.f) || !std::isfinite(a->v_scale) ||
                      !(a->v_scale > 0.f)))
    return bad(DG_ERR_INVALID_ARG, "k_scale and v_scale must be finite and > 0 with pool_fp8");
  if (a->num_kv_heads < 1) return bad(DG_ERR_INVALID_ARG, "num_kv_heads must be >= 1");
  if (a->head_dim < 8 || a->head_dim % 8) return bad(DG_ERR_INVALID_ARG, "head_dim must be a positive multiple of 8");
  if (a->block_size < 1 || (a->block_size & (a->block_size - 1)))
    return bad(DG_ERR_INVALID_ARG, "block_size must be a power of two");
  if (a->pool_rows < a->block_size || a->pool_rows % a->block_size)
    return bad(DG_ERR_INVALID_ARG, "pool_rows must be a positive multiple of block_size");
  if (a->total_new < 0 || a->block_table_len < 1) return bad(DG_ERR_INVALID_ARG, "total_new must be >= 0 and block_table_len >= 1");
  if (!a->block_table || !aligned4(a->block_table)) return bad(DG_ERR_INVALID_ARG, "block_table must be non-NULL and 4-byte aligned");
  if (!a->k_new || !a->v_new || !a->k_pool || !a->v_pool) return bad(DG_ERR_INVALID_ARG, "k_new, v_new, k_pool and v_pool must be non-NULL");
  if (!aligned16(a->k_new) || !aligned16(a->v_new) || !aligned16(a->k_pool) || !aligned16(a->v_pool))
    return bad(DG_ERR_INVALID_ARG, "k_new, v_new, k_pool and v_pool must be 16-byte aligned");
  int64_t rows = 0;
  for (int s = 0; s < a->num_seqs; ++s) {
    const dg_kv_seq& q = a->seqs[s];
    if (q.src_start < 0 || q.num < 0 || q.table_start < 0 || q.pos < 0)
      return bad(DG_ERR_INVALID_ARG, "seq offsets and counts must be >= 0");
    if ((int64_t)q.src_start + q.num > a->total_new) return bad(DG_ERR_INVALID_ARG, "seq source rows exceed total_new");
    if ((int64_t)q.table_start + ceil_div((int64_t)q.pos + q.num, a->block_size) > a->block_table_len)
      return bad(DG_ERR_INVALID_ARG, "seq block table entries exceed block_table_len");
    if ((int64_t)q.table_start + ceil_div((int64_t)q.pos + q.num, a->block_size) > INT32_MAX ||
        (int64_t)q.pos + q.num > INT32_MAX)
      return bad(DG_ERR_UNSUPPORTED, "seq block table entries or positions past 2^31 - 1");
    rows += q.num;
  }
  plan->row_bytes = (int64_t)a->num_kv_heads * a->head_dim * (a->dtype == DG_BF16 ? 2 : 4);
  plan->pool_fp8 = a->pool_fp8;
  // the reciprocals of the scales, rounded to fp32 once, here
  plan->k_inv = a->pool_fp8 ? 1.0f / a->k_scale : 0.f;
  plan->v_inv = a->pool_fp8 ? 1.0f / a->v_scale : 0.f;
  plan->total_rows = rows;
  int sh = 0;
  while ((1 << sh) < a->block_size) ++sh;
  plan->block_shift = sh;
  // threads: one per 16 source bytes (a copy) or per 8 elements (quantized)
  const int64_t per_row = a->pool_fp8 ? (int64_t)a->num_kv_heads * a->head_dim / 8 : plan->row_bytes / 16;
  if (rows * per_row > INT32_MAX) return bad(DG_ERR_UNSUPPORTED, "too many rows for one call");
  return DG_OK;
}

// ---- self-conditioning injection ------------------------------------------------

dg_status inject_plan(const dg_inject_args* a, InjectPlan* plan, const char** msg) {
  auto bad = [&](dg_status s, const char* m) { *msg = m; return s; };
  if (!a) return bad(DG_ERR_INVALID_ARG, "args is NULL");
  if (a->M < 1 || a->vocab < 1) return bad(DG_ERR_INVALID_ARG, "M and vocab must be >= 1");
  if (a->d < 128 || a->d % 128 || a->hidden < 128 || a->hidden % 128)
    return bad(DG_ERR_UNSUPPORTED, "d and hidden must be positive multiples of 128");
  if (a->dtype != DG_F32 && a->dtype != DG_BF16) return bad(DG_ERR_INVALID_ARG, "dtype must be DG_F32 or DG_BF16");
  if (!a->tokens || !a->embed || !a->s || !a->w_gate_up || !a->w_down || !a->out)
    return bad(DG_ERR_INVALID_ARG, "tokens, embed, s, w_gate_up, w_down and out must be non-NULL");
  if (!aligned4(a->tokens) || !aligned16(a->embed) || !aligned16(a->s) || !aligned16(a->w_gate_up) ||
      !aligned16(a->w_down) || !aligned16(a->out))
    return bad(DG_ERR_INVALID_ARG, "tokens must be 4-byte and the other tensors 16-byte aligned");
  const size_t esz = a->dtype == DG_BF16 ? 2 : 4;
  void* const fake = reinterpret_cast<void*>(uintptr_t{256});  // a workspace address, set at launch
  dg_selfcond_args& g1 = plan->gemm1;
  g1 = dg_selfcond_args{};
  g1.M = a->M;
  g1.V = a->d;
  g1.d = 2 * a->hidden;
  g1.dtype = a->dtype;
  g1.p = a->s;
  g1.ldp = a->d;
  g1.embed = a->w_gate_up;
  g1.lde = 2 * a->hidden;
  g1.out = fake;
  g1.ldo = 2 * a->hidden;
  dg_selfcond_args& g2 = plan->gemm2;
  g2 = dg_selfcond_args{};
  g2.M = a->M;
  g2.V = a->hidden;
  g2.d = a->d;
  g2.dtype = a->dtype;
  g2.p = fake;
  g2.ldp = a->hidden;
  g2.embed = a->w_down;
  g2.lde = a->d;
  g2.out = a->out;
  g2.ldo = a->d;
  dg_status st = selfcond_plan(&g1, &plan->plan1, msg);
  if (st != DG_OK) return st;
  st = selfcond_plan(&g2, &plan->plan2, msg);
  if (st != DG_OK) return st;
  plan->gu_offset = 0;
  plan->h_offset = align_up((size_t)a->M * 2 * a->hidden * esz, 256);
  plan->gemm_ws_offset = plan->h_offset + align_up((size_t)a->M * a->hidden * esz, 256);
  plan->bytes = plan->gemm_ws_offset + std::max(plan->plan1.bytes, plan->plan2.bytes);
  return DG_OK;
}

}  // namespace dg

// ---- C ABI -------------------------------------------------------------------

using namespace dg;

extern "C" {

const char* dg_status_string(dg_status s) {
  switch (s) {
    case DG_OK: return "DG_OK";
    case DG_ERR_INVALID_ARG: return "DG_ERR_INVALID_ARG";
    case DG_ERR_UNSUPPORTED: return "DG_ERR_UNSUPPORTED";
    case DG_ERR_WORKSPACE: return "DG_ERR_WORKSPACE";
    case DG_ERR_HIP: return "DG_ERR_HIP";
  }
  return "unknown dg_status";
}

const char* dg_last_error(void) { return g_last_error; }
int dg_abi_version(void) { return DG_ABI_VERSION; }

int dg_test_force_register_staged(int on) { return g_force_register_staged.exchange(on != 0); }
int dg_test_wide_min_sub(int n) { return g_wide_min_sub.exchange(n >= 1 ? n : kWideMinSubDefault); }

size_t dg_attn_workspace_size(const dg_attn_args* a) {
  AttnPlan plan;
  const char* msg = "";
  if (attn_plan(a, &plan, &msg) != DG_OK) return (size_t)-1;
  return plan.bytes;
}

dg_status dg_attn_mixed(const dg_attn_args* a, void* stream) {
  AttnPlan plan;
  const char* msg = "";
  dg_status s = attn_plan(a, &plan, &msg);
  if (s != DG_OK) return fail(s, msg);
  if (plan.bytes && (!a->workspace || a->workspace_bytes < plan.bytes || !aligned16(a->workspace)))
    return fail(DG_ERR_WORKSPACE, "workspace missing, misaligned or smaller than dg_attn_workspace_size");
  if (plan.num_work == 0) { g_last_error[0] = 0; return DG_OK; }
  int e = launch_attn(a, plan, stream);
  if (e) return fail(DG_ERR_HIP, hip_error_name(e));
  g_last_error[0] = 0;
  return DG_OK;
}

size_t dg_sampler_workspace_size(const dg_sampler_args* a) {
  SamplerPlan plan;
  const char* msg = "";
  if (sampler_plan(a, &plan, &msg) != DG_OK) return (size_t)-1;
  return plan.bytes;
}

dg_status dg_sampler_step(const dg_sampler_args* a, void* stream) {
  SamplerPlan plan;
  const char* msg = "";
  dg_status s = sampler_plan(a, &plan, &msg);
  if (s != DG_OK) return fail(s, msg);
  if (plan.bytes && (!a->workspace || a->workspace_bytes < plan.bytes || !aligned16(a->workspace)))
    return fail(DG_ERR_WORKSPACE, "workspace missing, misaligned or smaller than dg_sampler_workspace_size");
  int e = launch_sampler(a, plan, stream);
  if (e) return fail(DG_ERR_HIP, hip_error_name(e));
  g_last_error[0] = 0;
  return DG_OK;
}

size_t dg_selfcond_workspace_size(const dg_selfcond_args* a) {
  SelfcondPlan plan;
  const char* msg = "";
  if (selfcond_plan(a, &plan, &msg) != DG_OK) return (size_t)-1;
  return plan.bytes;
}

dg_status dg_selfcond_embed(const dg_selfcond_args* a, void* stream) {
  SelfcondPlan plan;
  const char* msg = "";
  dg_status s = selfcond_plan(a, &plan, &msg);
  if (s != DG_OK) return fail(s, msg);
  if (plan.bytes && (!a->workspace || a->workspace_bytes < plan.bytes || !aligned16(a->workspace)))
    return fail(DG_ERR_WORKSPACE, "workspace missing, misaligned or smaller than dg_selfcond_workspace_size");
  int e = launch_selfcond(a, plan, stream);
  if (e) return fail(DG_ERR_HIP, hip_error_name(e));
  g_last_error[0] = 0;
  return DG_OK;
}

size_t dg_selfcond_inject_workspace_size(const dg_inject_args* a) {
  InjectPlan plan;
  const char* msg = "";
  if (inject_plan(a, &plan, &msg) != DG_OK) return (size_t)-1;
  return plan.bytes;
}

dg_status dg_selfcond_inject(const dg_inject_args* a, void* stream) {
  InjectPlan plan;
  const char* msg = "";
  dg_status s = inject_plan(a, &plan, &msg);
  if (s != DG_OK) return fail(s, msg);
  if (!a->workspace || a->workspace_bytes < plan.bytes || !aligned16(a->workspace))
    return fail(DG_ERR_WORKSPACE, "workspace missing, misaligned or smaller than dg_selfcond_inject_workspace_size");
  int e = launch_inject(a, plan, stream);
  if (e) return fail(DG_ERR_HIP, hip_error_name(e));
  g_last_error[0] = 0;
  return DG_OK;
}

dg_status dg_kv_write(const dg_kv_write_args* a, void* stream) {
  KvWritePlan plan;
  const char* msg = "";
  dg_status s = kv_write_plan(a, &plan, &msg);
  if (s != DG_OK) return fail(s, msg);
  if (plan.total_rows == 0) { g_last_error[0] = 0; return DG_OK; }
  int e = launch_kv_write(a, plan, stream);
  if (e) return fail(DG_ERR_HIP, hip_error_name(e));
  g_last_error[0] = 0;
  return DG_OK;
}

}  // extern "C"
