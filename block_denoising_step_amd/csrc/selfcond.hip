// Self-conditioning on gfx950: out[M, d] = P[M, V] . E[V, d], the probability-weighted
// average of the token embeddings ([P1] "DiffusionGemma: vLLM에서 네이티브로 처음 지원되는
// 첫 번째 Diffusion LLM", section "안정성을 위한 셀프 컨디셔닝"; [P3] "DiffusionGemma u vLLM:
// ...", section "Mehanizam odlučivanja o gotovim tokenima").
//
//   selfcond_gemm    128 x 128 output tile per work group (4 waves, 64 x 64 each, 2 x 2
//                    MFMA 32x32 blocks), K step of 128 bytes per row (64 bf16 / 32 fp32).
//                    The A tile (P, or logits turned into P on load from the sampler's
//                    row max and row sum) is staged row-major in LDS; the E tile is
//                    transposed on its way into LDS so both MFMA operands are single
//                    16-byte LDS reads. Global loads for step k+1 are in flight while
//                    step k runs on the matrix cores (double-buffered LDS, one barrier
//                    per step). Split-K over V; work groups that share an A slice and
//                    a B slice are placed on the same XCD so the re-reads hit its L2.
//   selfcond_reduce  sums the split-K partials in slice order (deterministic) and
//                    rounds to the output dtype.
#include "dg_common.cuh"
#include "dg_internal.h"

namespace dg {
namespace {

constexpr int kBM = 128, kBN = 128, kThreads = 256;
constexpr int kRowBytes = 128;             // bytes of one A row (or one E column) per K step
constexpr int kPitch = kRowBytes + 16;     // LDS row pitch: 16-byte pad keeps ds_read_b128 conflict-free

template <bool kBf16> struct Tr;
template <> struct Tr<true> {
  static constexpr int esz = 2, epv = 8, bk = 64;
};
template <> struct Tr<false> {
  static constexpr int esz = 4, epv = 4, bk = 32;
};

// One 32x32x16 MFMA step from 16 bytes (bf16) or 32 bytes (fp32) of A and B per lane.
// Lane half h = lane/32 supplies k = 8h..8h+7 of the step for both operands.
template <bool kBf16> struct Mfma;
template <> struct Mfma<true> {
  struct Frag { uint4 v; };
  __device__ static Frag load(const char* p) { return Frag{*reinterpret_cast<const uint4*>(p)}; }
  __device__ static void step(f32x16_t& acc, const Frag& a, const Frag& b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a.v), __builtin_bit_cast(bf16x8_t, b.v),
                                                  acc, 0, 0, 0);
  }
};
template <> struct Mfma<false> {
  struct Frag { float4 lo, hi; };
  __device__ static Frag load(const char* p) {
    return Frag{*reinterpret_cast<const float4*>(p), *reinterpret_cast<const float4*>(p + 16)};
  }
  __device__ static void step(f32x16_t& acc, const Frag& a, const Frag& b) {
    // k-element j of each half goes through one 32x32x2 MFMA: the pair {j, 8+j}
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.lo.x, b.lo.x, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.lo.y, b.lo.y, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.lo.z, b.lo.z, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.lo.w, b.lo.w, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.hi.x, b.hi.x, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.hi.y, b.hi.y, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.hi.z, b.hi.z, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.hi.w, b.hi.w, acc, 0, 0, 0);
  }
};

struct GemmArgs {
  const void* p;
  int64_t ldp;
  const float* row_max;
  const float* row_sum;
  const void* e;
  int64_t lde;
  void* out;
  int64_t ldo;
  float* part;  // [splits][M][d] fp32, or null when splits == 1
  int M, V, d;
  int m_tiles, n_tiles, splits, k_per_split;
};

// Turn 16 bytes of logits into probabilities p = 2^(l*log2e + c) with
// c = -row_max*log2e - log2(row_sum).
template <bool kBf16> __device__ __forceinline__ uint4 to_prob(uint4 v, float c);
template <> __device__ __forceinline__ uint4 to_prob<true>(uint4 v, float c) {
  uint4 r;
  uint32_t* o = &r.x;
  const uint32_t* w = &v.x;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    o[i] = pack_bf16(fast_exp2(fmaf(bf16lo(w[i]), kLog2e, c)), fast_exp2(fmaf(bf16hi(w[i]), kLog2e, c)));
  return r;
}
template <> __device__ __forceinline__ uint4 to_prob<false>(uint4 v, float c) {
  uint4 r;
  r.x = __float_as_uint(fast_exp2(fmaf(__uint_as_float(v.x), kLog2e, c)));
  r.y = __float_as_uint(fast_exp2(fmaf(__uint_as_float(v.y), kLog2e, c)));
  r.z = __float_as_uint(fast_exp2(fmaf(__uint_as_float(v.z), kLog2e, c)));
  r.w = __float_as_uint(fast_exp2(fmaf(__uint_as_float(v.w), kLog2e, c)));
  return r;
}

template <bool kBf16, bool kFused>
__global__ __launch_bounds__(kThreads) void selfcond_gemm(GemmArgs g) {
  using T = Tr<kBf16>;
  using MF = Mfma<kBf16>;
  constexpr int BK = T::bk, ESZ = T::esz, EPV = T::epv;
  __shared__ __attribute__((aligned(16))) char lds_a[2][kBM * kPitch];
  __shared__ __attribute__((aligned(16))) char lds_b[2][kBN * kPitch];

  // XCD-aware placement: consecutive work-group ids go round-robin over 8 XCDs; give
  // each XCD a contiguous block of (slice, m tile, n tile) work so the work groups
  // sharing a K slice run on one XCD.
  const int nwg = gridDim.x;
  int L = blockIdx.x;
  if ((nwg & 7) == 0) L = (blockIdx.x & 7) * (nwg >> 3) + (blockIdx.x >> 3);
  const int per_split = g.m_tiles * g.n_tiles;
  const int split = L / per_split;
  const int mt = (L % per_split) / g.n_tiles;
  const int nt = L % g.n_tiles;
  const int m0 = mt * kBM, n0 = nt * kBN;
  const int k_lo = split * g.k_per_split;
  const int k_hi = min(g.V, k_lo + g.k_per_split);
  const int nsteps = (k_hi - k_lo + BK - 1) / BK;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = (wave >> 1) * 64, wn = (wave & 1) * 64;

  // A loads: chunk q = i*256 + tid -> row q/8, 16-byte column q%8
  const char* pbase = reinterpret_cast<const char*>(g.p);
  float crow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = m0 + (i * kThreads + tid) / 8;
    crow[i] = 0.f;
    if (kFused && r < g.M) crow[i] = -g.row_max[r] * kLog2e - __builtin_amdgcn_logf(g.row_sum[r]);
  }
  // B loads: thread -> n group nq (EPV columns), k group kq (4 rows)
  constexpr int NG = kBN / EPV;
  const int nq = tid % NG, kq = tid / NG;
  const char* ebase = reinterpret_cast<const char*>(g.e);

  // Raw A values; out-of-range entries hold a neutral value (0, or -inf in the fused
  // mode so that 2^(-inf) = 0). The fused transform runs at LDS-store time, after the
  // current step's MFMAs, so the loads of the next step stay in flight meanwhile.
  const uint32_t neutral = kFused ? (kBf16 ? 0xFF80FF80u : 0xFF800000u) : 0u;
  uint4 ra[4], rb[4];
  auto load_step = [&](int s) {
    const int k0 = k_lo + s * BK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = i * kThreads + tid;
      const int r = m0 + q / 8, kc = k0 + (q % 8) * EPV;
      if (r < g.M && kc + EPV <= k_hi) {
        ra[i] = *reinterpret_cast<const uint4*>(pbase + ((int64_t)r * g.ldp + kc) * ESZ);
      } else {
        ra[i] = make_uint4(neutral, neutral, neutral, neutral);
        if (r < g.M)
          for (int e = 0; e < EPV; ++e)
            if (kc + e < k_hi) {
              if (kBf16)
                reinterpret_cast<uint16_t*>(&ra[i])[e] = reinterpret_cast<const uint16_t*>(pbase)[(int64_t)r * g.ldp + kc + e];
              else
                reinterpret_cast<float*>(&ra[i])[e] = reinterpret_cast<const float*>(pbase)[(int64_t)r * g.ldp + kc + e];
            }
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int k = k0 + kq * 4 + j;
      rb[j] = k < k_hi ? *reinterpret_cast<const uint4*>(ebase + ((int64_t)k * g.lde + n0 + nq * EPV) * ESZ)
                       : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_step = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = i * kThreads + tid;
      const uint4 v = kFused ? to_prob<kBf16>(ra[i], crow[i]) : ra[i];
      *reinterpret_cast<uint4*>(&lds_a[buf][(q / 8) * kPitch + (q % 8) * 16]) = v;
    }
    // transpose 4 (k) x EPV (n) into EPV rows of Bt[n][k]
    if (kBf16) {
#pragma unroll
      for (int c = 0; c < EPV; ++c) {
        const int w = c >> 1;
        const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;  // high or low bf16 of each word
        const uint32_t k01 = __builtin_amdgcn_perm((&rb[1].x)[w], (&rb[0].x)[w], sel);
        const uint32_t k23 = __builtin_amdgcn_perm((&rb[3].x)[w], (&rb[2].x)[w], sel);
        *reinterpret_cast<uint2*>(&lds_b[buf][(nq * EPV + c) * kPitch + kq * 4 * ESZ]) = make_uint2(k01, k23);
      }
    } else {
#pragma unroll
      for (int c = 0; c < EPV; ++c)
        *reinterpret_cast<uint4*>(&lds_b[buf][(nq * EPV + c) * kPitch + kq * 4 * ESZ]) =
            make_uint4((&rb[0].x)[c], (&rb[1].x)[c], (&rb[2].x)[c], (&rb[3].x)[c]);
    }
  };

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int h = lane >> 5, l32 = lane & 31;
  if (nsteps > 0) load_step(0);
  for (int s = 0; s < nsteps; ++s) {
    const int buf = s & 1;
    store_step(buf);
    __syncthreads();
    if (s + 1 < nsteps) load_step(s + 1);
    const char* A = lds_a[buf];
    const char* B = lds_b[buf];
#pragma unroll
    for (int ks = 0; ks < kRowBytes / (16 * ESZ); ++ks) {
      const int koff = (ks * 16 + 8 * h) * ESZ;
      typename MF::Frag fa[2], fb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) fa[i] = MF::load(A + (wm + i * 32 + l32) * kPitch + koff);
#pragma unroll
      for (int j = 0; j < 2; ++j) fb[j] = MF::load(B + (wn + j * 32 + l32) * kPitch + koff);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) MF::step(acc[i][j], fa[i], fb[j]);
    }
  }

  // epilogue: acc[i][j][e] holds C[wm + 32i + 8(e/4) + 4h + e%4][wn + 32j + l32]
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int r = m0 + wm + 32 * i + 8 * (e >> 2) + 4 * h + (e & 3);
        const int c = n0 + wn + 32 * j + l32;
        if (r >= g.M) continue;
        const float v = acc[i][j][e];
        if (g.part) {
          g.part[((int64_t)split * g.M + r) * g.d + c] = v;
        } else if (kBf16) {
          reinterpret_cast<__bf16*>(g.out)[(int64_t)r * g.ldo + c] = (__bf16)v;
        } else {
          reinterpret_cast<float*>(g.out)[(int64_t)r * g.ldo + c] = v;
        }
      }
}

// Sum split-K partials in slice order and store in the output dtype; 4 columns per thread.
template <bool kBf16>
__global__ __launch_bounds__(256) void selfcond_reduce(const float* __restrict__ part, int splits, int M, int d,
                                                       void* __restrict__ out, int64_t ldo) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)M * d / 4;
  if (i >= total) return;
  const int64_t e = i * 4;
  const int r = (int)(e / d), c = (int)(e % d);
  float4 s = *reinterpret_cast<const float4*>(part + e);
  for (int k = 1; k < splits; ++k) {
    const float4 v = *reinterpret_cast<const float4*>(part + (int64_t)k * M * d + e);
    s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
  }
  if (kBf16) {
    *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(out) + (int64_t)r * ldo + c) =
        make_uint2(pack_bf16(s.x, s.y), pack_bf16(s.z, s.w));
  } else {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(out) + (int64_t)r * ldo + c) = s;
  }
}

}  // namespace

int launch_selfcond(const dg_selfcond_args* a, const SelfcondPlan& plan, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  GemmArgs g;
  g.p = a->p;
  g.ldp = a->ldp;
  g.row_max = a->row_max;
  g.row_sum = a->row_sum;
  g.e = a->embed;
  g.lde = a->lde;
  g.out = a->out;
  g.ldo = a->ldo;
  g.part = plan.splits > 1 ? reinterpret_cast<float*>(a->workspace) : nullptr;
  g.M = a->M;
  g.V = a->V;
  g.d = a->d;
  g.m_tiles = plan.m_tiles;
  g.n_tiles = plan.n_tiles;
  g.splits = plan.splits;
  g.k_per_split = plan.k_per_split;
  const dim3 grid(plan.m_tiles * plan.n_tiles * plan.splits);
  const bool fused = a->row_max != nullptr;
  if (a->dtype == DG_BF16) {
    if (fused) hipLaunchKernelGGL((selfcond_gemm<true, true>), grid, dim3(kThreads), 0, s, g);
    else hipLaunchKernelGGL((selfcond_gemm<true, false>), grid, dim3(kThreads), 0, s, g);
  } else {
    if (fused) hipLaunchKernelGGL((selfcond_gemm<false, true>), grid, dim3(kThreads), 0, s, g);
    else hipLaunchKernelGGL((selfcond_gemm<false, false>), grid, dim3(kThreads), 0, s, g);
  }
  if (plan.splits > 1) {
    const int64_t n4 = (int64_t)a->M * a->d / 4;
    const dim3 rg((unsigned)((n4 + 255) / 256));
    if (a->dtype == DG_BF16)
      hipLaunchKernelGGL(selfcond_reduce<true>, rg, dim3(256), 0, s, g.part, plan.splits, a->M, a->d, a->out, a->ldo);
    else
      hipLaunchKernelGGL(selfcond_reduce<false>, rg, dim3(256), 0, s, g.part, plan.splits, a->M, a->d, a->out, a->ldo);
  }
  return (int)hipGetLastError();
}

}  // namespace dg
