// DiffusionSampler denoise step on gfx950: three launches.
//
//   sampler_rowpass   one streaming, read-only pass over the logits. Each work group
//                     owns one 32 KB chunk of one row, holds it in registers, and
//                     writes the chunk's (max, sum of 2^y, sum of 2^y*y, argmax) with
//                     y = l*log2(e) - max*log2(e). 16-byte loads, all issued before
//                     the first use, give 32 KB in flight per work group.
//   sampler_finalize  one work group per row: merges the chunk statistics in chunk
//                     order, writes max, sum, entropy, confidence and argmax, then
//                     draws the candidate by inverse CDF - walk the chunk masses to
//                     the chunk holding u*Z, re-read that one chunk.
//   sampler_select    one work group per request: rank sort by confidence, exact
//                     integer prefix sum of entropies, budget cut, canvas update and
//                     convergence bookkeeping.
//
// What these compute is stated in [P1] ("DiffusionGemma: vLLM에서 네이티브로 처음
// 지원되는 첫 번째 Diffusion LLM") section "샘플링 루프와 엔트로피 경계 디노이징",
// [P3] ("DiffusionGemma u vLLM: ...") section "Mehanizam odlučivanja o gotovim
// tokenima", and, for re-noising, [P2] ("DiffusionGemma 개발자 가이드") sections
// "아키텍처 (The Architecture)" and "Diffusion에 스도쿠가 흥미로운 이유".
#include <climits>

#include "dg_common.cuh"
#include "dg_internal.h"

namespace dg {
namespace {

constexpr int kThreads = 256;
constexpr int kLoads = 8;  // 16-byte loads per thread per chunk
constexpr int kSelectThreads = DG_MAX_CANVAS;
constexpr int kFixedShift = 40;

struct ReqTable {
  int32_t n;
  int32_t row_start[DG_MAX_REQS];
  int32_t num_rows[DG_MAX_REQS];
  int32_t step[DG_MAX_REQS];
  uint64_t seed[DG_MAX_REQS];
};

// Elements of a 16-byte load.
template <bool kBf16> struct Vec;
template <> struct Vec<true> {
  static constexpr int n = 8;
  __device__ static float get(const uint4& v, int e) {
    const uint32_t w = (&v.x)[e >> 1];
    return (e & 1) ? bf16hi(w) : bf16lo(w);
  }
  __device__ static uint4 neg_inf() { return make_uint4(0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u); }
  __device__ static float scalar(const void* p, int64_t i) {
    return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(p)[i] << 16);
  }
};
template <> struct Vec<false> {
  static constexpr int n = 4;
  __device__ static float get(const uint4& v, int e) { return __uint_as_float((&v.x)[e]); }
  __device__ static uint4 neg_inf() { return make_uint4(0xFF800000u, 0xFF800000u, 0xFF800000u, 0xFF800000u); }
  __device__ static float scalar(const void* p, int64_t i) { return reinterpret_cast<const float*>(p)[i]; }
};

// Load 16 bytes of row elements [v0, v0 + n) with -inf past V.
template <bool kBf16>
__device__ __forceinline__ uint4 load_vec(const void* rowp, int v0, int V) {
  using VT = Vec<kBf16>;
  if (v0 + VT::n <= V) {
    const char* p = reinterpret_cast<const char*>(rowp) + (int64_t)v0 * (kBf16 ? 2 : 4);
    return *reinterpret_cast<const uint4*>(p);
  }
  uint4 r = VT::neg_inf();
  if (kBf16) {
    uint16_t* h = reinterpret_cast<uint16_t*>(&r);
    for (int e = 0; e < VT::n && v0 + e < V; ++e) h[e] = reinterpret_cast<const uint16_t*>(rowp)[v0 + e];
  } else {
    float* f = reinterpret_cast<float*>(&r);
    for (int e = 0; e < VT::n && v0 + e < V; ++e) f[e] = reinterpret_cast<const float*>(rowp)[v0 + e];
  }
  return r;
}

__device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int i = 1; i < kThreads / 64; ++i) r = fmaxf(r, red[i]);
  return r;
}
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int i = 1; i < kThreads / 64; ++i) r += red[i];
  return r;
}
__device__ __forceinline__ int block_min_int(int v, int* red) {
  v = wave_min_int(v);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  int r = red[0];
#pragma unroll
  for (int i = 1; i < kThreads / 64; ++i) r = min(r, red[i]);
  return r;
}

// ---- row pass ---------------------------------------------------------------------
template <bool kBf16>
__global__ __launch_bounds__(kThreads) void sampler_rowpass(const void* __restrict__ logits, int64_t ld, int V,
                                                            int chunk, int num_chunks, float4* __restrict__ stats) {
  using VT = Vec<kBf16>;
  __shared__ float redf[kThreads / 64];
  __shared__ int redi[kThreads / 64];
  const int c = blockIdx.x % num_chunks, row = blockIdx.x / num_chunks, tid = threadIdx.x;
  const char* rowp = reinterpret_cast<const char*>(logits) + (int64_t)row * ld * (kBf16 ? 2 : 4);
  const int c0 = c * chunk;
  uint4 buf[kLoads];
  if (c0 + chunk <= V) {
#pragma unroll
    for (int i = 0; i < kLoads; ++i)
      buf[i] = *reinterpret_cast<const uint4*>(rowp + ((int64_t)c0 + (i * kThreads + tid) * VT::n) * (kBf16 ? 2 : 4));
  } else {
#pragma unroll
    for (int i = 0; i < kLoads; ++i) buf[i] = load_vec<kBf16>(rowp, c0 + (i * kThreads + tid) * VT::n, V);
  }
  float mx = kNegInf;
#pragma unroll
  for (int i = 0; i < kLoads; ++i)
#pragma unroll
    for (int e = 0; e < VT::n; ++e) mx = fmaxf(mx, VT::get(buf[i], e));
  const float m = block_max(mx, redf);
  if (m == kNegInf) {  // chunk without a finite logit carries no mass
    if (tid == 0) stats[(int64_t)row * num_chunks + c] = make_float4(kNegInf, 0.f, 0.f, __int_as_float(INT_MAX));
    return;
  }
  const float nm2 = -m * kLog2e;
  float z = 0.f, t = 0.f;
  int first = INT_MAX;
#pragma unroll
  for (int i = kLoads - 1; i >= 0; --i) {
#pragma unroll
    for (int e = VT::n - 1; e >= 0; --e) {
      const float v = VT::get(buf[i], e);
      const float y = fmaxf(fmaf(v, kLog2e, nm2), -200.f);  // clamp keeps 0 * y finite for -inf logits
      const float w = fast_exp2(y);
      z += w;
      t = fmaf(w, y, t);
      if (v == m) first = c0 + (i * kThreads + tid) * VT::n + e;  // ends at the lowest index
    }
  }
  const float zs = block_sum(z, redf);
  const float ts = block_sum(t, redf);
  const int am = block_min_int(first, redi);
  if (tid == 0) stats[(int64_t)row * num_chunks + c] = make_float4(m, zs, ts, __int_as_float(am));
}

// ---- finalize: per-row statistics and candidate draw ---------------------------
template <bool kBf16>
__global__ __launch_bounds__(kThreads) void sampler_finalize(
    const void* __restrict__ logits, int64_t ld, int V, int chunk, int num_chunks, const float4* __restrict__ stats,
    ReqTable reqs, uint32_t flags, int conf_mode, float* __restrict__ entropy, float* __restrict__ conf,
    float* __restrict__ row_max, float* __restrict__ row_sum, int* __restrict__ argmax, int* __restrict__ cand) {
  using VT = Vec<kBf16>;
  __shared__ float redf[kThreads / 64];
  __shared__ int redi[kThreads / 64];
  __shared__ float mass[1024];
  __shared__ float seg[kThreads];
  __shared__ int pick_chunk, pick_seg, fallback;
  __shared__ float before, seg_before;
  const int row = blockIdx.x, tid = threadIdx.x;
  const float4* st = stats + (int64_t)row * num_chunks;

  float mx = kNegInf;
  for (int c = tid; c < num_chunks; c += kThreads) mx = fmaxf(mx, st[c].x);
  const float m = block_max(mx, redf);
  const float nm2 = -m * kLog2e;
  float z = 0.f, t = 0.f;
  int am = INT_MAX;
  for (int c = tid; c < num_chunks; c += kThreads) {
    const float4 s = st[c];
    float mc = 0.f;
    if (s.x != kNegInf) {
      const float delta = nm2 - (-s.x * kLog2e);  // <= 0: chunk's y offset relative to the row
      const float f = fast_exp2(delta);
      mc = s.y * f;
      z += mc;
      t += f * fmaf(delta, s.y, s.z);
      if (s.x == m) am = min(am, __float_as_int(s.w));
    }
    mass[c] = mc;
  }
  const float Z = block_sum(z, redf);
  const float T = block_sum(t, redf);
  const int amax = block_min_int(am, redi);

  if (tid == 0) {
    // entropy in nats: ln Z - (sum p*y) * ln 2, with y the log2-scaled logit offsets
    const double h = (double)kLn2 * (log2((double)Z) - (double)T / (double)Z);
    const float H = fmaxf(0.f, (float)h);
    // Z sums 2^y with y offset by the rounding of -m*log2e; fma recovers that offset
    // exactly, so the row sum is sum exp(l - m) (the entropy is offset-invariant).
    const float zsum = Z * fast_exp2(-fmaf(m, kLog2e, nm2));
    const bool ent_in = flags & DG_ENTROPY_IN;
    if (!ent_in) entropy[row] = H;
    if (conf_mode == DG_CONF_NEG_ENTROPY) conf[row] = -(ent_in ? entropy[row] : H);
    else if (!ent_in) conf[row] = 1.f / zsum;
    row_max[row] = m;
    row_sum[row] = zsum;
    argmax[row] = amax;
  }

  // which request (if any) owns this row
  int r = -1;
  for (int i = 0; i < reqs.n; ++i)
    if (row >= reqs.row_start[i] && row < reqs.row_start[i] + reqs.num_rows[i]) r = i;
  if (r < 0) {
    if (tid == 0) cand[row] = -1;
    return;
  }
  const int j = row - reqs.row_start[r];
  const uint64_t x0 = philox_word0(reqs.seed[r], (uint64_t)reqs.step[r], (uint64_t)j, 0);
  const float u = (float)(x0 >> 40) * 0x1p-24f;
  const float target = u * Z;
  __syncthreads();  // mass[] complete
  if (tid == 0) {
    float cum = 0.f;
    int pc = -1, last = 0;
    for (int c = 0; c < num_chunks; ++c) {
      if (mass[c] > 0.f) last = c;
      if (pc < 0 && cum + mass[c] > target) { pc = c; break; }
      cum += mass[c];
    }
    fallback = pc < 0;
    pick_chunk = pc < 0 ? last : pc;
    before = cum;
  }
  __syncthreads();
  // re-read the chosen chunk: thread tid owns a contiguous run of chunk/256 elements
  const int per = chunk / kThreads;
  const int e0 = pick_chunk * chunk + tid * per;
  const char* rowp = reinterpret_cast<const char*>(logits) + (int64_t)row * ld * (kBf16 ? 2 : 4);
  float w[64];
  float s = 0.f;
  int last_pos = -1;
#pragma unroll
  for (int i = 0; i < 64; ++i) {
    if (i < per) {
      const int v = e0 + i;
      const float l = v < V ? VT::scalar(rowp, v) : kNegInf;
      w[i] = fast_exp2(fmaf(l, kLog2e, nm2));
      s += w[i];
      if (w[i] > 0.f) last_pos = v;
    }
  }
  seg[tid] = s;
  __syncthreads();
  if (tid == 0) {
    const float rem = target - before;
    float pre = 0.f;
    int ps = -1;
    if (!fallback)
      for (int i = 0; i < kThreads; ++i) {
        if (pre + seg[i] > rem) { ps = i; break; }
        pre += seg[i];
      }
    pick_seg = ps;
    seg_before = pre;
  }
  __syncthreads();
  if (pick_seg < 0) {  // rounding left u*Z past the re-read mass: last token with mass
    const int lp = -block_min_int(-last_pos, redi);
    if (tid == 0) cand[row] = lp;
    return;
  }
  if (tid == pick_seg) {
    const float rem = target - before;
    float acc = 0.f;
    int got = last_pos;
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      if (i < per) {
        acc += w[i];
        if (seg_before + acc > rem) { got = e0 + i; break; }
      }
    }
    cand[row] = got;
  }
}

// ---- selection, canvas update, convergence -------------------------------------
__global__ __launch_bounds__(kSelectThreads) void sampler_select(
    ReqTable reqs, int vocab, float budget, int min_accept, int conf_mode, int renoise, int stable_k, float tau,
    int step_limit, int combine, uint32_t flags, const float* __restrict__ entropy, const float* __restrict__ conf,
    const int* __restrict__ argmax, const int* __restrict__ cand, uint8_t* __restrict__ accept,
    int* __restrict__ canvas, int* __restrict__ prev_argmax, int* __restrict__ stable_count,
    int* __restrict__ num_accepted, int* __restrict__ converged, float* __restrict__ mean_entropy) {
  __shared__ float key[kSelectThreads];
  __shared__ long long scan[2][kSelectThreads];
  __shared__ long long wsum[kSelectThreads / 64];
  __shared__ int conv_flag;
  const int r = blockIdx.x, j = threadIdx.x;
  const int n = reqs.num_rows[r], step = reqs.step[r];
  const uint64_t seed = reqs.seed[r];
  const bool active = j < n;
  const int row = reqs.row_start[r] + j;

  if (flags & DG_INIT_CANVAS) {
    if (active) {
      const uint64_t x = philox_word0(seed, (uint64_t)step, (uint64_t)j, 2);
      canvas[row] = (int)(((x >> 32) * (uint64_t)vocab) >> 32);
      prev_argmax[row] = -1;
      accept[row] = 0;
    }
    if (j == 0) {
      stable_count[r] = 0;
      converged[r] = 0;
      num_accepted[r] = 0;
      mean_entropy[r] = 0.f;
    }
    return;
  }

  const float h = active ? entropy[row] : 0.f;
  const float c = active ? (conf_mode == DG_CONF_NEG_ENTROPY ? -h : conf[row]) : kNegInf;
  key[j] = c;
  __syncthreads();
  int rank = 0;
  if (active)
    for (int i = 0; i < n; ++i) {
      const float ki = key[i];
      rank += (ki > c) || (ki == c && i < j);
    }
  // exact fixed point: floor(h * 2^40); h * 2^40 is exact in double
  const long long fx = active ? (long long)floor((double)h * 0x1p40) : 0;
  scan[0][j] = 0;
  __syncthreads();
  if (active) scan[0][rank] = fx;
  __syncthreads();
  int cur = 0;
  for (int off = 1; off < n; off <<= 1) {
    const long long v = scan[cur][j] + (j >= off ? scan[cur][j - off] : 0);
    scan[cur ^ 1][j] = v;
    cur ^= 1;
    __syncthreads();
  }
  const long long limit = (long long)floor((double)budget * 0x1p40);
  const bool acc = active && (scan[cur][rank] <= limit || rank < min_accept);
  const int count = __syncthreads_count(acc);
  const int same = __syncthreads_and(!active || argmax[row] == prev_argmax[row]);
  // exact total entropy of the request
  long long tot = fx;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) tot += __shfl_xor(tot, o, 64);
  if ((j & 63) == 0) wsum[j >> 6] = tot;
  __syncthreads();
  if (j == 0) {
    long long total = 0;
    for (int i = 0; i < kSelectThreads / 64; ++i) total += wsum[i];
    const int stable = (step > 0 && same) ? stable_count[r] + 1 : 0;
    const long long thr = (long long)ceil((double)tau * (double)n * 0x1p40);
    const bool low = total < thr;
    const bool done = step + 1 >= step_limit;
    const bool conv = combine == DG_CONV_AND ? ((stable >= stable_k && low) || done)
                                             : (stable >= stable_k || low || done);
    stable_count[r] = stable;
    converged[r] = conv;
    num_accepted[r] = count;
    mean_entropy[r] = (float)((double)total * 0x1p-40 / (double)n);
    conv_flag = conv;
  }
  __syncthreads();
  if (active) {
    const int am = argmax[row];
    int tok;
    if (acc) tok = cand[row];
    else if (conv_flag) tok = am;
    else if (renoise) {
      const uint64_t x = philox_word0(seed, (uint64_t)step, (uint64_t)j, 1);
      tok = (int)(((x >> 32) * (uint64_t)vocab) >> 32);
    } else tok = canvas[row];
    canvas[row] = tok;
    accept[row] = acc;
    prev_argmax[row] = am;
  }
}

}  // namespace

int launch_sampler(const dg_sampler_args* a, const SamplerPlan& plan, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  ReqTable t{};
  t.n = a->num_reqs;
  for (int i = 0; i < a->num_reqs; ++i) {
    t.row_start[i] = a->reqs[i].row_start;
    t.num_rows[i] = a->reqs[i].num_rows;
    t.step[i] = a->reqs[i].step;
    t.seed[i] = a->reqs[i].seed;
  }
  if (!(a->flags & DG_INIT_CANVAS)) {
    float4* stats = reinterpret_cast<float4*>(a->workspace);
    const dim3 grid(plan.num_chunks * a->num_rows);
    if (a->dtype == DG_BF16) {
      hipLaunchKernelGGL(sampler_rowpass<true>, grid, dim3(kThreads), 0, s, a->logits, a->ld, a->vocab, plan.chunk,
                         plan.num_chunks, stats);
      hipLaunchKernelGGL(sampler_finalize<true>, dim3(a->num_rows), dim3(kThreads), 0, s, a->logits, a->ld, a->vocab,
                         plan.chunk, plan.num_chunks, stats, t, a->flags, a->conf_mode, a->entropy, a->conf,
                         a->row_max, a->row_sum, a->argmax, a->cand);
    } else {
      hipLaunchKernelGGL(sampler_rowpass<false>, grid, dim3(kThreads), 0, s, a->logits, a->ld, a->vocab, plan.chunk,
                         plan.num_chunks, stats);
      hipLaunchKernelGGL(sampler_finalize<false>, dim3(a->num_rows), dim3(kThreads), 0, s, a->logits, a->ld, a->vocab,
                         plan.chunk, plan.num_chunks, stats, t, a->flags, a->conf_mode, a->entropy, a->conf,
                         a->row_max, a->row_sum, a->argmax, a->cand);
    }
  }
  hipLaunchKernelGGL(sampler_select, dim3(a->num_reqs), dim3(kSelectThreads), 0, s, t, a->vocab, a->budget,
                     a->min_accept, a->conf_mode, a->renoise, a->stable_k, a->tau, a->step_limit, a->combine, a->flags,
                     a->entropy, a->conf, a->argmax, a->cand, a->accept, a->canvas, a->prev_argmax, a->stable_count,
                     a->num_accepted, a->converged, a->mean_entropy);
  return (int)hipGetLastError();
}

const char* hip_error_name(int err) { return hipGetErrorString((hipError_t)err); }

}  // namespace dg
