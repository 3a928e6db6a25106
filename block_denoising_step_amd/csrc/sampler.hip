// DiffusionSampler denoise step on gfx950: three launches, none of which waits on
// another work group (no atomics, no device-scope fences: on a multi-XCD part a
// device-scope release writes back the L2, which costs more than a kernel boundary).
//
//   sampler_rowpass   one streaming, read-only pass over the logits. Each work group
//                     owns one 32 KB chunk of one row, holds it in registers, and
//                     writes the chunk's (max, sum of 2^y, sum of 2^y*y, argmax) with
//                     y = l*log2(e) - max*log2(e), plus 32 sub-chunk masses (one per
//                     wave and 16-byte load: 64 * 16 contiguous bytes each). 16-byte
//                     loads, all issued before the first use, give 32 KB in flight
//                     per work group. Optionally it writes w = 2^y (block-scaled
//                     probabilities for self-conditioning).
//   sampler_finalize  one wave per row: merges the chunk statistics in chunk order,
//                     writes max, sum, entropy, confidence and argmax, then draws the
//                     candidate by inverse CDF at u*Z - a wave prefix scan over the
//                     chunk masses, then over the chosen chunk's sub-chunk masses,
//                     then over one re-read 16-byte vector per lane.
//   sampler_select    one work group per request: rank sort by confidence, exact
//                     integer prefix sum of entropies, budget cut, canvas update and
//                     convergence bookkeeping.
//   sampler_init      start of a block: random canvas, state reset.
//
// What these compute is stated in [P1] ("DiffusionGemma: vLLM에서 네이티브로 처음
// 지원되는 첫 번째 Diffusion LLM") section "샘플링 루프와 엔트로피 경계 디노이징",
// [P3] ("DiffusionGemma u vLLM: ...") section "Mehanizam odlučivanja o gotovim
// tokenima", and, for re-noising, [P2] ("DiffusionGemma 개발자 가이드") sections
// "아키텍처 (The Architecture)" and "Diffusion에 스도쿠가 흥미로운 이유".
#include <climits>
#include <mutex>

#include "dg_common.cuh"
#include "dg_internal.h"

namespace dg {
namespace {

constexpr int kThreads = 256;
constexpr int kLoads = 8;  // 16-byte loads per thread per chunk
constexpr int kWaves = kThreads / 64;
constexpr int kSubs = kLoads * kWaves;  // sub-chunks per chunk: one per (load, wave)
constexpr int kPerThread = DG_MAX_CANVAS / kThreads;  // canvas positions per thread in the selection

struct ReqTable {
  int32_t n;
  int32_t row_start[DG_MAX_REQS];
  int32_t num_rows[DG_MAX_REQS];
  int32_t step[DG_MAX_REQS];
  uint64_t seed[DG_MAX_REQS];
  int32_t* step_dev;  // device step counters [n], or null: the steps above
};

// Request r's denoise step: the device counter when there is one (a recorded step
// replays with the step that the previous replay's selection stored), else the
// call's argument.
__device__ __forceinline__ int req_step(const ReqTable& t, int r) { return t.step_dev ? t.step_dev[r] : t.step[r]; }

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
__device__ __forceinline__ int block_max_int(int v, int* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, 64));
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  int r = red[0];
#pragma unroll
  for (int i = 1; i < kThreads / 64; ++i) r = max(r, red[i]);
  return r;
}
// Exclusive prefix sum over the block in thread order (fixed association).
__device__ __forceinline__ float block_exclusive_scan(float v, float* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  float x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  __syncthreads();
  if (lane == 63) red[w] = x;
  __syncthreads();
  float off = 0.f;
  for (int i = 0; i < w; ++i) off += red[i];
  return off + x - v;
}
__device__ __forceinline__ long long block_sum_ll(long long v, long long* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  long long r = 0;
#pragma unroll
  for (int i = 0; i < kThreads / 64; ++i) r += red[i];
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
// kTail: the launch covers only the last, partial chunk of every row (elements past V
// read as -inf); otherwise it covers the first `nfull` whole chunks of every row and
// needs no bounds checks, which keeps its register use low.
template <bool kBf16, bool kStore, bool kTail>
__global__ __launch_bounds__(kThreads) void sampler_rowpass(const void* __restrict__ logits, int64_t ld, int V,
                                                            int chunk, int num_chunks, int nfull,
                                                            float4* __restrict__ stats, float* __restrict__ sub,
                                                            void* __restrict__ probs, int64_t ldq) {
  using VT = Vec<kBf16>;
  __shared__ float redf[kThreads / 64];
  __shared__ int redi[kThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63;
  // sub-chunk (load i, wave w) holds elements c0 + (i * kThreads + 64 w) * n + [0, 64 n)
  float* subp = sub + (((int64_t)(kTail ? blockIdx.x : blockIdx.x / nfull) * num_chunks +
                        (kTail ? num_chunks - 1 : blockIdx.x % nfull)) * kWaves + (tid >> 6)) * kLoads;
  const int c = kTail ? num_chunks - 1 : blockIdx.x % nfull;
  const int row = kTail ? blockIdx.x : blockIdx.x / nfull;
  const char* rowp = reinterpret_cast<const char*>(logits) + (int64_t)row * ld * (kBf16 ? 2 : 4);
  const int c0 = c * chunk;
  uint4 buf[kLoads];
  if (!kTail) {
    // non-temporal loads: the logits are read once, and streamed this way they leave the
    // probabilities this pass writes (which self-conditioning reads next) in the caches
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const u32x4 x = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(rowp + ((int64_t)c0 + (i * kThreads + tid) * VT::n) * (kBf16 ? 2 : 4)));
      buf[i] = make_uint4(x.x, x.y, x.z, x.w);
    }
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
    subp[lane >> 3] = 0.f;
    if (kStore) {
      char* qrow = reinterpret_cast<char*>(probs) + (int64_t)row * ldq * (kBf16 ? 2 : 4);
      for (int i = 0; i < kLoads; ++i)
        for (int e = 0; e < VT::n; ++e) {
          const int v = c0 + (i * kThreads + tid) * VT::n + e;
          if (v < V) {
            if (kBf16) reinterpret_cast<uint16_t*>(qrow)[v] = 0;
            else reinterpret_cast<float*>(qrow)[v] = 0.f;
          }
        }
    }
    return;
  }
  const float nm2 = -m * kLog2e;
  float z = 0.f, t = 0.f;
  float zl[kLoads];  // this lane's mass in each load
  int first = INT_MAX;
  // With kStore the pass also writes w = 2^y of the chunk (block-scaled probabilities).
  char* qrow = kStore ? reinterpret_cast<char*>(probs) + (int64_t)row * ldq * (kBf16 ? 2 : 4) : nullptr;
#pragma unroll
  for (int i = kLoads - 1; i >= 0; --i) {
    float wl[VT::n];
    zl[i] = 0.f;
#pragma unroll
    for (int e = VT::n - 1; e >= 0; --e) {
      const float v = VT::get(buf[i], e);
      const float y = fmaxf(fmaf(v, kLog2e, nm2), -200.f);  // clamp keeps 0 * y finite for -inf logits
      const float w = fast_exp2(y);
      wl[e] = w;
      zl[i] += w;
      z += w;
      t = fmaf(w, y, t);
      if (v == m) first = c0 + (i * kThreads + tid) * VT::n + e;  // ends at the lowest index
    }
    if (kStore) {
      const int v0 = c0 + (i * kThreads + tid) * VT::n;
      if (!kTail) {
        const uint4 wv = kBf16 ? make_uint4(pack_bf16(wl[0], wl[1]), pack_bf16(wl[2], wl[3]),
                                            pack_bf16(wl[4], wl[5]), pack_bf16(wl[6], wl[7]))
                               : make_uint4(__float_as_uint(wl[0]), __float_as_uint(wl[1]), __float_as_uint(wl[2]),
                                            __float_as_uint(wl[3]));
        *reinterpret_cast<uint4*>(qrow + (int64_t)v0 * (kBf16 ? 2 : 4)) = wv;
      } else {
#pragma unroll
        for (int e = 0; e < VT::n; ++e)
          if (v0 + e < V) {
            if (kBf16) reinterpret_cast<__bf16*>(qrow)[v0 + e] = (__bf16)wl[e];
            else reinterpret_cast<float*>(qrow)[v0 + e] = wl[e];
          }
      }
      __builtin_amdgcn_sched_barrier(0);  // keep one 16-byte group's values live at a time
    }
  }
  // sub-chunk masses: sum each load's values over the wave by halving exchanges
  // (xor 32 keeps 4 of the 8 sums, xor 16 keeps 2, xor 8 keeps 1, then xor 4/2/1
  // finish), after which lane 8i holds the sum of load i
  {
    float k4[4], k2[2], k1;
    const bool b5 = lane & 32, b4 = lane & 16, b3 = lane & 8;
#pragma unroll
    for (int k = 0; k < 4; ++k) k4[k] = (b5 ? zl[k + 4] : zl[k]) + __shfl_xor(b5 ? zl[k] : zl[k + 4], 32, 64);
#pragma unroll
    for (int k = 0; k < 2; ++k) k2[k] = (b4 ? k4[k + 2] : k4[k]) + __shfl_xor(b4 ? k4[k] : k4[k + 2], 16, 64);
    k1 = (b3 ? k2[1] : k2[0]) + __shfl_xor(b3 ? k2[0] : k2[1], 8, 64);
    k1 += __shfl_xor(k1, 4, 64);
    k1 += __shfl_xor(k1, 2, 64);
    k1 += __shfl_xor(k1, 1, 64);
    subp[lane >> 3] = k1;  // the 8 lanes of a group hold the same sum (a branch here costs registers)
  }
  const float zs = block_sum(z, redf);
  const float ts = block_sum(t, redf);
  const int am = block_min_int(first, redi);
  if (tid == 0) stats[(int64_t)row * num_chunks + c] = make_float4(m, zs, ts, __int_as_float(am));
}

// ---- finalize: per-row statistics, candidate draw, and (last row of a request) the selection

struct SelectParams {
  int vocab, min_accept, conf_mode, renoise, stable_k, step_limit, combine;
  float budget, tau;
  uint32_t flags;
};

struct RowOut {
  float *entropy, *conf, *row_max, *row_sum;
  int *argmax, *cand;
  float* probs_scale;
  uint8_t* accept;
  int *canvas, *prev_argmax, *stable_count, *num_accepted, *converged;
  float* mean_entropy;
};

__device__ __forceinline__ int renoise_token(uint64_t seed, int step, int j, int stream, int vocab) {
  const uint64_t x = philox_word0(seed, (uint64_t)step, (uint64_t)j, (uint64_t)stream);
  return (int)(((x >> 32) * (uint64_t)vocab) >> 32);
}

// Exclusive prefix sum of int64 values over the block in thread order.
__device__ __forceinline__ long long block_exclusive_scan_ll(long long v, long long* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  long long x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const long long y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  __syncthreads();
  if (lane == 63) red[w] = x;
  __syncthreads();
  long long off = 0;
  for (int i = 0; i < w; ++i) off += red[i];
  return off + x - v;
}

// Selection for request r by one work group of kThreads: rank sort by (confidence
// desc, position asc), exact integer prefix sum of floor(H * 2^40), budget cut, canvas
// update and convergence bookkeeping. Every input is loaded up front.
// Sort key of position j with confidence c: c's bits made order-preserving as an
// unsigned integer (-0 folded into +0 first, so that equal confidences give equal
// keys) in the high word, ~j in the low word. key_i > key_j exactly when c_i > c_j,
// or c_i == c_j and i < j (confidences are finite).
__device__ __forceinline__ uint64_t rank_key(float c, int j) {
  const uint32_t u = __float_as_uint(c + 0.f);
  const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)ord << 32) | (uint32_t)~(uint32_t)j;
}

__device__ void select_request(int r, const ReqTable& reqs, const SelectParams& sp, const RowOut& o) {
  __shared__ __attribute__((aligned(16))) uint64_t key[DG_MAX_CANVAS + 16];
  __shared__ long long sorted[DG_MAX_CANVAS];
  __shared__ long long wred[kWaves];
  __shared__ int ired[kWaves];
  __shared__ int conv_flag;
  const int tid = threadIdx.x;
  const int n = reqs.num_rows[r], step = req_step(reqs, r), row0 = reqs.row_start[r];
  const uint64_t seed = reqs.seed[r];
  const int prev_stable = o.stable_count[r];  // loaded early: the bookkeeping at the end needs it
  float c[kPerThread];
  uint64_t kj[kPerThread];
  long long fx[kPerThread];
  int am[kPerThread], cand[kPerThread], old[kPerThread];
  long long sum = 0;
  int same = 1;
#pragma unroll
  for (int q = 0; q < kPerThread; ++q) {
    const int j = tid + kThreads * q;
    c[q] = kNegInf;
    kj[q] = 0;
    fx[q] = 0;
    am[q] = cand[q] = old[q] = 0;
    if (j < n) {
      const float h = o.entropy[row0 + j];
      c[q] = sp.conf_mode == DG_CONF_NEG_ENTROPY ? -h : o.conf[row0 + j];
      fx[q] = (long long)floor((double)h * 0x1p40);  // exact: h * 2^40 is exact in double
      am[q] = o.argmax[row0 + j];
      same &= am[q] == o.prev_argmax[row0 + j];
      cand[q] = o.cand[row0 + j];
      old[q] = o.canvas[row0 + j];
      sum += fx[q];
      kj[q] = rank_key(c[q], j);
      key[j] = kj[q];
    }
  }
  // pad to a multiple of 16 with 0, below every position's key
  if (tid < 16) key[n + tid] = 0;
  __syncthreads();
  int rank[kPerThread];
#pragma unroll
  for (int q = 0; q < kPerThread; ++q) rank[q] = 0;
  // rank_j = #{i : key_i > key_j} = #{i : c_i > c_j or (c_i == c_j and i < j)};
  // 16 keys per iteration, read 2 per 16-byte load so the loads pipeline
  for (int i0 = 0; i0 < n; i0 += 16) {
    ulonglong2 k2[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) k2[u] = *reinterpret_cast<const ulonglong2*>(&key[i0 + 2 * u]);
#pragma unroll
    for (int q = 0; q < kPerThread; ++q) {
      if (kThreads * q >= n) break;  // no thread has a position here (uniform)
#pragma unroll
      for (int u = 0; u < 8; ++u) rank[q] += (int)(k2[u].x > kj[q]) + (int)(k2[u].y > kj[q]);
    }
  }
#pragma unroll
  for (int q = 0; q < kPerThread; ++q) {
    const int j = tid + kThreads * q;
    if (j < n) sorted[rank[q]] = fx[q];
  }
  __syncthreads();
  // inclusive scan of sorted[0, n): each thread owns kPerThread consecutive ranks
  long long part[kPerThread];
  long long run = 0;
#pragma unroll
  for (int q = 0; q < kPerThread; ++q) {
    const int i = tid * kPerThread + q;
    run += i < n ? sorted[i] : 0;
    part[q] = run;
  }
  const long long off = block_exclusive_scan_ll(run, wred);
  __syncthreads();  // every thread has read sorted[] before it is overwritten
#pragma unroll
  for (int q = 0; q < kPerThread; ++q) {
    const int i = tid * kPerThread + q;
    if (i < n) sorted[i] = off + part[q];
  }
  __syncthreads();
  const long long limit = (long long)floor((double)sp.budget * 0x1p40);
  bool acc[kPerThread];
  int cnt = 0;
#pragma unroll
  for (int q = 0; q < kPerThread; ++q) {
    const int j = tid + kThreads * q;
    acc[q] = j < n && (sorted[rank[q]] <= limit || rank[q] < sp.min_accept);
    cnt += acc[q];
  }
  // one reduction for the entropy total, the accepted count and "argmax unchanged"
  long long tsum = sum;
  int tcnt = cnt, tsame = same;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    tsum += __shfl_xor(tsum, off, 64);
    tcnt += __shfl_xor(tcnt, off, 64);
    tsame &= __shfl_xor(tsame, off, 64);
  }
  if ((tid & 63) == 0) {
    wred[tid >> 6] = tsum;
    ired[tid >> 6] = tcnt | (tsame << 30);
  }
  __syncthreads();
  long long total = 0;
  int count = 0, all_same = 1;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    total += wred[w];
    count += ired[w] & ((1 << 30) - 1);
    all_same &= ired[w] >> 30;
  }
  if (tid == 0) {
    const int stable = (step > 0 && all_same) ? prev_stable + 1 : 0;
    const long long thr = (long long)ceil((double)sp.tau * (double)n * 0x1p40);
    const bool low = total < thr;
    const bool done = step + 1 >= sp.step_limit;
    const bool conv = sp.combine == DG_CONV_AND ? ((stable >= sp.stable_k && low) || done)
                                                : (stable >= sp.stable_k || low || done);
    o.stable_count[r] = stable;
    o.converged[r] = conv;
    o.num_accepted[r] = count;
    o.mean_entropy[r] = (float)((double)total * 0x1p-40 / (double)n);
    if (reqs.step_dev) reqs.step_dev[r] = step + 1;  // every read of it in this call is done
    conv_flag = conv;
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < kPerThread; ++q) {
    const int j = tid + kThreads * q;
    if (j >= n) continue;
    const int row = row0 + j;
    int tok;
    if (acc[q]) tok = cand[q];
    else if (conv_flag) tok = am[q];
    else if (sp.renoise) tok = renoise_token(seed, step, j, 1, sp.vocab);
    else tok = old[q];
    o.canvas[row] = tok;
    o.accept[row] = acc[q];
    o.prev_argmax[row] = am[q];
  }
}

// One wave per row (kWaves rows per work group, no barriers).
template <bool kBf16>
__global__ __launch_bounds__(kThreads) void sampler_finalize(const void* __restrict__ logits, int64_t ld, int V,
                                                             int chunk, int num_chunks, int num_rows,
                                                             const float4* __restrict__ stats,
                                                             const float* __restrict__ sub, ReqTable reqs,
                                                             SelectParams sp, RowOut o) {
  using VT = Vec<kBf16>;
  __shared__ float mass_s[kWaves][1024];
  // the wave index (so the row and its request) is uniform: scalar loads and branches
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int row = blockIdx.x * kWaves + wave;
  if (row >= num_rows) return;
  float* mass = mass_s[wave];
  const float4* st = stats + (int64_t)row * num_chunks;

  // this lane's first chunk statistics, loaded before the work below so that it waits
  // on them: which request (if any) owns this row, and its candidate's uniform u
  // (Philox counter (step, position, stream 0))
  const float4 s_first = lane < num_chunks ? st[lane] : make_float4(kNegInf, 0.f, 0.f, 0.f);
  int r = -1;
  for (int i = 0; i < reqs.n; ++i)
    if (row >= reqs.row_start[i] && row < reqs.row_start[i] + reqs.num_rows[i]) r = i;
  float u = 0.f;
  if (r >= 0) {
    const uint64_t x0 = philox_word0(reqs.seed[r], (uint64_t)req_step(reqs, r), (uint64_t)(row - reqs.row_start[r]), 0);
    u = (float)(x0 >> 40) * 0x1p-24f;
  }

  // merge the chunk statistics (lane c, c + 64, ... in order)
  float mx = s_first.x;
  for (int c = lane + 64; c < num_chunks; c += 64) mx = fmaxf(mx, st[c].x);
  const float m = wave_max(mx);
  const float nm2 = -m * kLog2e;
  float z = 0.f, t = 0.f;
  int am = INT_MAX;
  for (int c = lane; c < num_chunks; c += 64) {
    const float4 s = c == lane ? s_first : st[c];
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
  const float Z = wave_sum(z);
  const float T = wave_sum(t);
  const int amax = wave_min_int(am);
  if (o.probs_scale) {
    // p = w * 2^(chunk offset) / Z: one scale per DG_PROB_BLOCK entries (a chunk spans
    // chunk / DG_PROB_BLOCK blocks, all with the chunk's scale)
    const int per = chunk / DG_PROB_BLOCK;
    const int nblocks = (V + DG_PROB_BLOCK - 1) / DG_PROB_BLOCK;
    const float invz = 1.f / Z;
    for (int c = lane; c < num_chunks; c += 64) {
      const float sc = mass[c] > 0.f ? mass[c] / st[c].y * invz : 0.f;
      for (int b = c * per; b < min(nblocks, (c + 1) * per); ++b) o.probs_scale[(int64_t)row * nblocks + b] = sc;
    }
  }
  if (lane == 0) {
    // entropy in nats: ln Z - (sum p*y) * ln 2, with y the log2-scaled logit offsets
    const double h = (double)kLn2 * (log2((double)Z) - (double)T / (double)Z);
    const float H = fmaxf(0.f, (float)h);
    // Z sums 2^y with y offset by the rounding of -m*log2e; fma recovers that offset
    // exactly, so the row sum is sum exp(l - m) (the entropy is offset-invariant).
    const float zsum = Z * fast_exp2(-fmaf(m, kLog2e, nm2));
    const bool ent_in = sp.flags & DG_ENTROPY_IN;
    if (!ent_in) o.entropy[row] = H;
    if (sp.conf_mode == DG_CONF_NEG_ENTROPY) o.conf[row] = -(ent_in ? o.entropy[row] : H);
    else if (!ent_in) o.conf[row] = 1.f / zsum;
    o.row_max[row] = m;
    o.row_sum[row] = zsum;
    o.argmax[row] = amax;
  }

  if (r < 0) {
    if (lane == 0) o.cand[row] = -1;
    return;
  }
  // candidate: the first token whose cumulative mass exceeds u*Z. Rounding can leave
  // u*Z past the mass a level sums to; then the last token with mass is taken.
  const float target = u * Z;
  // level 1: chunks
  float carry = 0.f, rem = 0.f;
  int pc = -1, last = 0;
  for (int base = 0; base < num_chunks; base += 64) {
    const int c = base + lane;
    const float mc = c < num_chunks ? mass[c] : 0.f;
    const float incl = wave_incl_scan(mc);
    const uint64_t pos = __ballot(mc > 0.f);
    if (pos) last = base + 63 - __clzll(pos);
    const uint64_t hit = __ballot(carry + incl > target);
    if (hit) {
      const int k = __ffsll((long long)hit) - 1;
      pc = base + k;
      rem = target - (carry + __shfl(wave_shift_up(incl), k, 64));
      break;
    }
    carry += __shfl(incl, 63, 64);
  }
  bool fallback = pc < 0;
  if (fallback) pc = last;
  // level 2: the chunk's sub-chunks, in the row's reference
  const float fch = st[pc].x == kNegInf ? 0.f : fast_exp2(nm2 + st[pc].x * kLog2e);
  const float* subp = sub + ((int64_t)row * num_chunks + pc) * kSubs;
  const int si = lane >> 2, sw = lane & 3;  // lane s < 32 takes sub-chunk s = 4 i + w
  const float sm = lane < kSubs ? subp[sw * kLoads + si] * fch : 0.f;
  const float sincl = wave_incl_scan(sm);
  const uint64_t spos = __ballot(sm > 0.f);
  const uint64_t shit = fallback ? 0 : __ballot(sincl > rem);
  int ps;
  if (shit) {
    ps = __ffsll((long long)shit) - 1;
    rem -= __shfl(wave_shift_up(sincl), ps, 64);
  } else {
    fallback = true;
    ps = spos ? 63 - __clzll(spos) : 0;
  }
  // level 3: one 16-byte vector per lane of that sub-chunk
  const int e0 = pc * chunk + ((ps >> 2) * kThreads + (ps & 3) * 64 + lane) * VT::n;
  const char* rowp = reinterpret_cast<const char*>(logits) + (int64_t)row * ld * (kBf16 ? 2 : 4);
  const uint4 v = load_vec<kBf16>(rowp, e0, V);
  float w[VT::n];
  float seg = 0.f;
  int last_pos = -1;
#pragma unroll
  for (int e = 0; e < VT::n; ++e) {
    w[e] = fast_exp2(fmaf(VT::get(v, e), kLog2e, nm2));
    seg += w[e];
    if (w[e] > 0.f) last_pos = e0 + e;
  }
  const float lincl = wave_incl_scan(seg);
  const float lexcl = wave_shift_up(lincl);
  const uint64_t lhit = fallback ? 0 : __ballot(lincl > rem);
  if (lhit) {
    const int k = __ffsll((long long)lhit) - 1;
    if (lane == k) {
      float acc = lexcl;
      int got = last_pos;
#pragma unroll
      for (int e = 0; e < VT::n; ++e) {
        acc += w[e];
        if (acc > rem) {
          got = e0 + e;
          break;
        }
      }
      o.cand[row] = got;
    }
  } else {
    const int lp = wave_max_int(last_pos);
    if (lane == 0) o.cand[row] = lp;
  }
}

__global__ __launch_bounds__(kThreads) void sampler_select(ReqTable reqs, SelectParams sp, RowOut o) {
  select_request(blockIdx.x, reqs, sp, o);
}

// Start of a block: a uniform random canvas (Philox stream 2), state reset.
__global__ __launch_bounds__(kThreads) void sampler_init(ReqTable reqs, int vocab, RowOut o) {
  const int r = blockIdx.x, tid = threadIdx.x;
  const int n = reqs.num_rows[r], row0 = reqs.row_start[r];
  for (int j = tid; j < n; j += kThreads) {
    o.canvas[row0 + j] = renoise_token(reqs.seed[r], reqs.step[r], j, 2, vocab);
    o.prev_argmax[row0 + j] = -1;
    o.accept[row0 + j] = 0;
  }
  if (tid == 0) {
    if (reqs.step_dev) reqs.step_dev[r] = 0;
    o.stable_count[r] = 0;
    o.converged[r] = 0;
    o.num_accepted[r] = 0;
    o.mean_entropy[r] = 0.f;
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
  t.step_dev = a->step_counter;
  float4* stats = reinterpret_cast<float4*>(a->workspace);
  float* sub = reinterpret_cast<float*>(reinterpret_cast<char*>(a->workspace) + plan.sub_offset);
  RowOut o{a->entropy, a->conf, a->row_max, a->row_sum, a->argmax, a->cand, a->probs_scale, a->accept, a->canvas,
           a->prev_argmax, a->stable_count, a->num_accepted, a->converged, a->mean_entropy};
  if (a->flags & DG_INIT_CANVAS) {
    hipLaunchKernelGGL(sampler_init, dim3(a->num_reqs), dim3(kThreads), 0, s, t, a->vocab, o);
    return (int)hipGetLastError();
  }
  SelectParams sp{a->vocab, a->min_accept, a->conf_mode, a->renoise, a->stable_k, a->step_limit, a->combine,
                  a->budget, a->tau, a->flags};
  if (a->flags & DG_SELECT_ONLY) {
    hipLaunchKernelGGL(sampler_select, dim3(a->num_reqs), dim3(kThreads), 0, s, t, sp, o);
    return (int)hipGetLastError();
  }
  const int nfull = a->vocab / plan.chunk;
  const bool tail = nfull < plan.num_chunks;
  const dim3 gfull((unsigned)nfull * a->num_rows), gtail(a->num_rows), blk(kThreads);
  const dim3 gfin((unsigned)((a->num_rows + kWaves - 1) / kWaves));
#define DG_ROWPASS(BF, ST)                                                                                \
  do {                                                                                                    \
    if (nfull)                                                                                            \
      hipLaunchKernelGGL((sampler_rowpass<BF, ST, false>), gfull, blk, 0, s, a->logits, a->ld, a->vocab, \
                         plan.chunk, plan.num_chunks, nfull, stats, sub, a->probs, a->ldq);              \
    if (tail)                                                                                             \
      hipLaunchKernelGGL((sampler_rowpass<BF, ST, true>), gtail, blk, 0, s, a->logits, a->ld, a->vocab,  \
                         plan.chunk, plan.num_chunks, nfull, stats, sub, a->probs, a->ldq);              \
  } while (0)
  if (a->dtype == DG_BF16) {
    if (a->probs) DG_ROWPASS(true, true);
    else DG_ROWPASS(true, false);
    hipLaunchKernelGGL(sampler_finalize<true>, gfin, blk, 0, s, a->logits, a->ld, a->vocab, plan.chunk, plan.num_chunks,
                       a->num_rows, stats, sub, t, sp, o);
  } else {
    if (a->probs) DG_ROWPASS(false, true);
    else DG_ROWPASS(false, false);
    hipLaunchKernelGGL(sampler_finalize<false>, gfin, blk, 0, s, a->logits, a->ld, a->vocab, plan.chunk,
                       plan.num_chunks, a->num_rows, stats, sub, t, sp, o);
  }
#undef DG_ROWPASS
  if (!(a->flags & DG_SKIP_SELECT)) hipLaunchKernelGGL(sampler_select, dim3(a->num_reqs), blk, 0, s, t, sp, o);
  return (int)hipGetLastError();
}

const char* hip_error_name(int err) { return hipGetErrorString((hipError_t)err); }

// ---- dg_sampler_step_noalloc: the sampler's workspace in a static device array ----------
//
// `scratch` holds the row pass's chunk statistics and sub-chunk masses. Every byte a call
// reads there is written earlier in the same call (each (row, chunk) entry by the row
// pass, before the finalize reads it), so nothing has to start at zero. Each GPU holds its
// own copy at its own address, looked up once per device with hipGetSymbolAddress: in
// host code `scratch` names a host-side stand-in, never to be passed to a kernel.
namespace {
constexpr size_t kScratchBytes = (size_t)DG_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Device address of this device's scratch array (looked up on the first call on each
// device, with that device current), or null with *err set.
void* scratch_ptr(hipError_t* err) {
  int dev = -1;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (*err != hipSuccess || !p) {
      if (*err == hipSuccess) *err = hipErrorInvalidSymbol;
      return nullptr;
    }
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}
}  // namespace

}  // namespace dg

extern "C" dg_status dg_sampler_step_noalloc(const dg_sampler_args* a, void* stream) {
  using namespace dg;
  SamplerPlan plan;
  const char* msg = "";
  dg_status s = sampler_plan(a, &plan, &msg);
  if (s != DG_OK) return record_error(s, msg);
  if (plan.bytes > kScratchBytes)
    return record_error(DG_ERR_WORKSPACE, "dg_sampler_step_noalloc: the call needs more than the "
                                          "DG_NOALLOC_SCRATCH_BYTES of static scratch (see dg_sampler_workspace_size)");
  dg_sampler_args b = *a;
  b.workspace = nullptr;
  b.workspace_bytes = 0;
  if (plan.bytes) {
    hipError_t err = hipSuccess;
    void* p = scratch_ptr(&err);
    if (!p) return record_error(DG_ERR_HIP, hipGetErrorString(err));
    b.workspace = p;
    b.workspace_bytes = kScratchBytes;
  }
  const int e = launch_sampler(&b, plan, stream);
  if (e) return record_error(DG_ERR_HIP, hip_error_name(e));
  clear_error();
  return DG_OK;
}
