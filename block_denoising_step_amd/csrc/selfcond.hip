// Self-conditioning on gfx950: out[M, d] = P[M, V] . E[V, d], the probability-weighted
// average of the token embeddings ([P1] "DiffusionGemma: vLLM에서 네이티브로 처음 지원되는
// 첫 번째 Diffusion LLM", section "안정성을 위한 셀프 컨디셔닝"; [P3] "DiffusionGemma u vLLM:
// ...", section "Mehanizam odlučivanja o gotovim tokenima").
//
// Both GEMM kernels compute a 256 x 256 output tile per work group, split-K over V
// with the work groups that share a K slice placed on one XCD so their re-reads of it
// hit that XCD's L2. LDS rows are XOR-swizzled in 16-byte chunks so staging writes and
// operand reads are free of bank conflicts.
//
//   selfcond_gemm_dma  bf16, V a multiple of 32; 8 waves, two per SIMD, each 64 x 128
//                      as 2 x 4 MFMA 32x32 blocks. The P and E tiles go straight from
//                      HBM to LDS (global_load_lds_dwordx4) through a 5-stage ring,
//                      so four K steps are in flight with no register staging. E
//                      stays row-major in LDS; its MFMA operand (8 consecutive k of one
//                      column per lane) comes from two ds_read_b64_tr_b16 transposing
//                      reads. One fence-free barrier per K step.
//   selfcond_gemm_reg  general case (fp32, any V); 4 waves, each 128 x 128 as 4 x 4
//                      blocks. Tiles are staged through registers
//                      one K step ahead, E transposed in registers on its way to LDS;
//                      in the logits mode P is rebuilt at LDS-store time.
//   selfcond_normalize bf16 logits + row statistics -> probabilities, so the logits
//                      mode can use the DMA kernel (the rebuild would otherwise be
//                      repeated once per 256-column tile).
//   selfcond_reduce    sums the split-K partials in slice order (deterministic) and
//                      rounds to the output dtype.
// With block-scaled P (w and per-row scales per DG_PROB_BLOCK vocabulary entries),
// every split lies inside one scale block and its rows are scaled in the epilogue.
#include "dg_common.cuh"
#include "dg_internal.h"

namespace dg {
namespace {

constexpr int kBM = 256, kBN = 256, kThreads = 256;
constexpr int kRow = 128;   // bytes per LDS row (one A row or one E column per K step)
constexpr int kStages = 1;  // K steps of global loads in flight in registers

template <bool kBf16> struct Tr;
template <> struct Tr<true> {
  static constexpr int esz = 2, epv = 8, bk = 64;
};
template <> struct Tr<false> {
  static constexpr int esz = 4, epv = 4, bk = 32;
};

// swizzled 16-byte chunk position inside a 128-byte LDS row
__device__ __forceinline__ int swz_a(int row, int chunk) { return chunk ^ (row & 7); }
__device__ __forceinline__ int swz_b(int n, int chunk) { return chunk ^ ((n & 7) ^ ((n >> 3) & 7)); }

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
  const float* p_scale;  // [M][nblocks] block scales, or null
  int nblocks;
  int M, V, d;
  int m_tiles, n_tiles, splits, k_per_split;
};

// Logits -> probabilities p = 2^(l*log2e + c), c = -row_max*log2e - log2(row_sum).
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

// Epilogue shared by both kernels: acc[i][j][e] = C[wm + 32i + 8(e/4) + 4h + e%4][wn + 32j + l32],
// for a BM x BN tile held as NI x NJ blocks of 32x32 per wave: the wave's rows start at
// 32-row block `rb0`, its columns at 32-column block `cb0`.
// Split-K partials are stored in the accumulators' native order (every store a coalesced
// wave write; selfcond_reduce maps them back to rows and columns), with kCh = BN / 128:
//   group index = (((rb * kCh + ch) * 4 + j) * 4 + e4) * 64 + lane, holding rows
//   32 rb + 8 e4 + 4 (lane / 32) + 0..3 of column 128 ch + 32 j + lane % 32;
// a group is a float4, or 4 bf16 in 8 bytes for bf16 products.
template <int BM, int BN, int NI, int NJ>
__device__ __forceinline__ void store_blocks(const GemmArgs& g, f32x16_t (&acc)[NI][NJ], int split, int k_lo, int mt,
                                             int nt, int rb0, int cb0, int lane, bool bf16) {
  // acc[i][j] is the 32x32 block at 32-row block rb0 + i, 32-column block cb0 + j
  constexpr int kCh = BN / 128;
  const int h = lane >> 5, l32 = lane & 31;
  const int m0 = mt * BM, n0 = nt * BN;
  const int blk = k_lo / DG_PROB_BLOCK;
  auto scale = [&](int r) { return g.p_scale ? g.p_scale[(int64_t)min(r, g.M - 1) * g.nblocks + blk] : 1.f; };
  if (g.part) {
    // partials in the output's precision class: bf16 for bf16 products (one rounding of
    // each slice sum), fp32 for fp32 ones; 4 values (rows r .. r+3 of a column) per lane
    const int64_t t0 = (((int64_t)split * g.m_tiles + mt) * g.n_tiles + nt) * (BM * BN / 4);
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int r = m0 + 32 * (rb0 + i) + 8 * e4 + 4 * h;  // rows r .. r+3
        const float s0 = scale(r), s1 = scale(r + 1), s2 = scale(r + 2), s3 = scale(r + 3);
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const int cb = cb0 + j, ch = cb >> 2, jj = cb & 3;
          const int64_t q = t0 + ((((rb0 + i) * kCh + ch) * 4 + jj) * 4 + e4) * 64 + lane;
          const float v0 = acc[i][j][4 * e4] * s0, v1 = acc[i][j][4 * e4 + 1] * s1;
          const float v2 = acc[i][j][4 * e4 + 2] * s2, v3 = acc[i][j][4 * e4 + 3] * s3;
          if (bf16) reinterpret_cast<uint2*>(g.part)[q] = make_uint2(pack_bf16(v0, v1), pack_bf16(v2, v3));
          else reinterpret_cast<float4*>(g.part)[q] = make_float4(v0, v1, v2, v3);
        }
      }
    return;
  }
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int r = m0 + 32 * (rb0 + i) + 8 * (e >> 2) + 4 * h + (e & 3);
      if (r >= g.M) continue;
      const float sr = scale(r);
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const int c = n0 + 32 * (cb0 + j) + l32;
        if (c >= g.d) continue;
        const float v = acc[i][j][e] * sr;
        if (bf16) reinterpret_cast<__bf16*>(g.out)[(int64_t)r * g.ldo + c] = (__bf16)v;
        else reinterpret_cast<float*>(g.out)[(int64_t)r * g.ldo + c] = v;
      }
    }
}

// Work placement shared by both kernels (XCD-aware, see the file comment).
struct TileIdx {
  int split, mt, nt, m0, n0, k_lo, k_hi;
};
template <int BM, int BN>
__device__ __forceinline__ TileIdx tile_index(const GemmArgs& g) {
  const int nwg = gridDim.x;
  int L = blockIdx.x;
  if ((nwg & 7) == 0) L = (blockIdx.x & 7) * (nwg >> 3) + (blockIdx.x >> 3);
  const int per_split = g.m_tiles * g.n_tiles;
  TileIdx t;
  t.split = L / per_split;
  t.mt = (L % per_split) / g.n_tiles;
  t.nt = L % g.n_tiles;
  t.m0 = t.mt * BM;
  t.n0 = t.nt * BN;
  t.k_lo = t.split * g.k_per_split;
  t.k_hi = min(g.V, t.k_lo + g.k_per_split);
  return t;
}

// BM x BN tile: 256 x 256, or 64 x 128 for small fp32 products (a 256 x 256 tile leaves
// them half the CUs idle, each work group a one-step slice with a 256 KB partial); 4 waves
// of (BM/2) x (BN/2). A staging: BM rows x 8 chunks of 16 bytes per K step, BM/32 chunks
// per thread; B staging (fp32): (BN/4) column blocks x 8 k blocks, BN/128 blocks per thread.
template <bool kBf16, bool kFused, int BM = 256, int BN = 256>
__global__ __launch_bounds__(kThreads) void selfcond_gemm_reg(GemmArgs g) {
  using T = Tr<kBf16>;
  constexpr int BK = T::bk, ESZ = T::esz, EPV = T::epv;
  constexpr int NI = BM / 64, NJ = BN / 64;     // 32 x 32 blocks per wave along rows, columns
  constexpr int kAC = BM * 8 / kThreads;        // A chunks per thread
  constexpr int kBB = BN / 128;                 // fp32 B blocks per thread
  static_assert((BM == 256 && BN == 256) || (BM == 64 && BN == 128 && !kBf16), "tile shapes");
  __shared__ __attribute__((aligned(16))) char lds_a[2][BM * kRow];
  __shared__ __attribute__((aligned(16))) char lds_b[2][BN * kRow];

  const TileIdx ti = tile_index<BM, BN>(g);
  const int m0 = ti.m0, n0 = ti.n0, k_lo = ti.k_lo, k_hi = ti.k_hi;
  const int nsteps = (k_hi - k_lo + BK - 1) / BK;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, l32 = lane & 31;
  const int wm = (wave >> 1) * (BM / 2), wn = (wave & 1) * (BN / 2);

  // A staging: chunk q = i*256 + tid (i < kAC) -> row q >> 3, 16-byte chunk q & 7
  const char* pbase = reinterpret_cast<const char*>(g.p);
  float crow[kAC];
#pragma unroll
  for (int i = 0; i < kAC; ++i) {
    const int r = m0 + ((i * kThreads + tid) >> 3);
    crow[i] = 0.f;
    if (kFused && r < g.M) crow[i] = -g.row_max[r] * kLog2e - __builtin_amdgcn_logf(g.row_sum[r]);
  }
  // B staging (E transposed): bf16 - one block of 8 k rows x 8 columns per thread;
  // fp32 - two blocks of 4 k rows x 4 columns.
  const char* ebase = reinterpret_cast<const char*>(g.e);
  const uint32_t neutral = kFused ? (kBf16 ? 0xFF80FF80u : 0xFF800000u) : 0u;  // p = 0 past the end

  uint4 ra[kStages][8], rb[kStages][8];

  auto load_step = [&](int s, uint4 (&a)[8], uint4 (&b)[8]) {
    const int k0 = k_lo + s * BK;
#pragma unroll
    for (int i = 0; i < kAC; ++i) {
      const int q = i * kThreads + tid;
      const int r = m0 + (q >> 3), kc = k0 + (q & 7) * EPV;
      if (r < g.M && kc + EPV <= k_hi) {
        a[i] = *reinterpret_cast<const uint4*>(pbase + ((int64_t)r * g.ldp + kc) * ESZ);
      } else {
        a[i] = make_uint4(neutral, neutral, neutral, neutral);
        if (r < g.M)
          for (int e = 0; e < EPV; ++e)
            if (kc + e < k_hi) {
              if (kBf16)
                reinterpret_cast<uint16_t*>(&a[i])[e] =
                    reinterpret_cast<const uint16_t*>(pbase)[(int64_t)r * g.ldp + kc + e];
              else
                reinterpret_cast<float*>(&a[i])[e] = reinterpret_cast<const float*>(pbase)[(int64_t)r * g.ldp + kc + e];
            }
      }
    }
    if constexpr (kBf16) {
      const int nb = tid & 31, kb = tid >> 5;  // 32 column blocks x 8 k blocks
      const int col = n0 + nb * 8;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int k = k0 + kb * 8 + j;
        b[j] = (k < k_hi && col < g.d) ? *reinterpret_cast<const uint4*>(ebase + ((int64_t)k * g.lde + col) * 2)
                                       : make_uint4(0, 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int blk = 0; blk < kBB; ++blk) {
        const int id = blk * kThreads + tid;
        const int nb = id % (BN / 4), kb = id / (BN / 4);  // BN/4 column blocks x 8 k blocks
        const int col = n0 + nb * 4;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int k = k0 + kb * 4 + j;
          b[blk * 4 + j] = (k < k_hi && col < g.d)
                               ? *reinterpret_cast<const uint4*>(ebase + ((int64_t)k * g.lde + col) * 4)
                               : make_uint4(0, 0, 0, 0);
        }
      }
    }
  };

  auto store_step = [&](int buf, const uint4 (&a)[8], const uint4 (&b)[8]) {
    char* A = lds_a[buf];
    char* B = lds_b[buf];
#pragma unroll
    for (int i = 0; i < kAC; ++i) {
      const int q = i * kThreads + tid;
      const int row = q >> 3;
      const uint4 v = kFused ? to_prob<kBf16>(a[i], crow[i]) : a[i];
      *reinterpret_cast<uint4*>(A + row * kRow + swz_a(row, q & 7) * 16) = v;
    }
    if constexpr (kBf16) {
      const int nb = tid & 31, kb = tid >> 5;
#pragma unroll
      for (int c = 0; c < 8; ++c) {  // column nb*8 + c gets k = kb*8 .. kb*8+7
        const int w = c >> 1;
        const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
        uint4 o;
        o.x = __builtin_amdgcn_perm((&b[1].x)[w], (&b[0].x)[w], sel);
        o.y = __builtin_amdgcn_perm((&b[3].x)[w], (&b[2].x)[w], sel);
        o.z = __builtin_amdgcn_perm((&b[5].x)[w], (&b[4].x)[w], sel);
        o.w = __builtin_amdgcn_perm((&b[7].x)[w], (&b[6].x)[w], sel);
        const int n = nb * 8 + c;
        *reinterpret_cast<uint4*>(B + n * kRow + swz_b(n, kb) * 16) = o;
      }
    } else {
#pragma unroll
      for (int blk = 0; blk < kBB; ++blk) {
        const int id = blk * kThreads + tid;
        const int nb = id % (BN / 4), kb = id / (BN / 4);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const int n = nb * 4 + c;
          const uint4 o = make_uint4((&b[blk * 4 + 0].x)[c], (&b[blk * 4 + 1].x)[c], (&b[blk * 4 + 2].x)[c],
                                     (&b[blk * 4 + 3].x)[c]);
          *reinterpret_cast<uint4*>(B + n * kRow + swz_b(n, kb) * 16) = o;
        }
      }
    }
  };

  f32x16_t acc[NI][NJ];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  auto compute_step = [&](int buf) {
    const char* A = lds_a[buf];
    const char* B = lds_b[buf];
    if constexpr (kBf16) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {  // 16 k per MFMA, lane half h holds chunk 2ks + h
        const int kc = 2 * ks + h;
        uint4 fa[4], fb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = wm + 32 * i + l32;
          fa[i] = *reinterpret_cast<const uint4*>(A + row * kRow + swz_a(row, kc) * 16);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int n = wn + 32 * j + l32;
          fb[j] = *reinterpret_cast<const uint4*>(B + n * kRow + swz_b(n, kc) * 16);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, fa[i]),
                                                                __builtin_bit_cast(bf16x8_t, fb[j]), acc[i][j], 0, 0,
                                                                0);
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {  // 16 k per step: lane half h holds chunks 4ks+2h, 4ks+2h+1
        float4 fa[NI][2], fb[NJ][2];
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          const int row = wm + 32 * i + l32;
#pragma unroll
          for (int c = 0; c < 2; ++c)
            fa[i][c] = *reinterpret_cast<const float4*>(A + row * kRow + swz_a(row, 4 * ks + 2 * h + c) * 16);
        }
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const int n = wn + 32 * j + l32;
#pragma unroll
          for (int c = 0; c < 2; ++c)
            fb[j][c] = *reinterpret_cast<const float4*>(B + n * kRow + swz_b(n, 4 * ks + 2 * h + c) * 16);
        }
#pragma unroll
        for (int i = 0; i < NI; ++i)
#pragma unroll
          for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int c = 0; c < 2; ++c) {
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[i][c].x, fb[j][c].x, acc[i][j], 0, 0, 0);
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[i][c].y, fb[j][c].y, acc[i][j], 0, 0, 0);
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[i][c].z, fb[j][c].z, acc[i][j], 0, 0, 0);
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(fa[i][c].w, fb[j][c].w, acc[i][j], 0, 0, 0);
            }
      }
    }
  };

  // prologue: the first kStages steps in flight
#pragma unroll
  for (int j = 0; j < kStages; ++j)
    if (j < nsteps) load_step(j, ra[j], rb[j]);
  // main loop, unrolled by kStages so every register buffer index is static
  for (int s0 = 0; s0 < nsteps; s0 += kStages) {
#pragma unroll
    for (int j = 0; j < kStages; ++j) {
      const int s = s0 + j;
      if (s < nsteps) {
        store_step(s & 1, ra[j], rb[j]);
        __syncthreads();
        if (s + kStages < nsteps) load_step(s + kStages, ra[j], rb[j]);
        compute_step(s & 1);
      }
    }
  }

  store_blocks<BM, BN, NI, NJ>(g, acc, ti.split, k_lo, ti.mt, ti.nt, wm >> 5, wn >> 5, lane, kBf16);
}


// ---- LDS-DMA kernel (bf16) -------------------------------------------------------

constexpr int kDmaBK = 32;  // k per step
// Cache policy of the E copies when E is larger than the last-level cache: non-temporal.
// Such an E is a once-per-call stream (its second reader, the other row tile, runs beside
// the first on the same XCD); marked this way it displaces less of P, which four column
// tiles read and the sampler has just written. Measured in the step loop: 268.9 -> 258.1
// us per call. A smaller E (a weight matrix) keeps the default policy: it is read again
// and stays cached (non-temporal there measured 45.5 -> 50.8 us for the injection's pair).
constexpr int kCpolStream = 2;
constexpr int64_t kStreamMinBytes = 256ll << 20;
// s_waitcnt with only the vector-memory counter limited (expcnt, lgkmcnt left open).
#define DG_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (7 << 4) | (15 << 8) | (((n) >> 4) << 14))
// s_waitcnt for all LDS reads of this wave (vmcnt left open).
#define DG_WAIT_LGKM0()                                              \
  do {                                                               \
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14)); \
    __builtin_amdgcn_sched_barrier(0);                               \
  } while (0)

// LDS operand reads as inline asm: the compiler's wait insertion would otherwise put a
// vmcnt(0) before every LDS read that follows an LDS DMA, serialising the ring. Each
// use of the results is preceded by an explicit DG_WAIT_LGKM0.
__device__ __forceinline__ uint4 lds_read_b128(uint32_t addr) {
  uint4 r;
  asm volatile("ds_read_b128 %0, %1" : "=v"(r) : "v"(addr) : "memory");
  return r;
}
__device__ __forceinline__ uint2 lds_read_tr16(uint32_t addr) {
  uint2 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(r) : "v"(addr) : "memory");
  return r;
}

// A stage: row r (0..BM-1) holds 32 bf16 = 4 chunks; chunk c sits at c ^ swa(r).
// B stage: k row kk (0..31) holds BN bf16 = BN/8 chunks; chunk c sits at c ^ swb(kk).
// The XOR masks keep the operand reads (ds_read_b128 over 32 rows; ds_read_b64_tr_b16
// over 4 k rows x 32 columns) free of bank conflicts with 64 banks of 4 bytes and with
// 32; the DMA writes are contiguous 1 KB runs either way.
__device__ __forceinline__ int swa(int r) { return ((r >> 1) & 3) ^ (((r >> 3) & 1) * 3); }
__device__ __forceinline__ int swb(int kk) { return ((kk & 1) * 4) ^ (((kk >> 1) & 1) * 10); }
__device__ __forceinline__ uint32_t a_off(int r, int c) { return r * 64 + ((c ^ swa(r)) << 4); }

// 8 waves (two per SIMD, so one wave's LDS waits and barriers overlap the other's
// MFMAs), each 64 x 128 as 2 x 4 MFMA blocks of 32x32 (128 accumulators), over a
// BM x BN tile: 256 x 256 (5-stage ring), or 128 x 512 (4-stage ring) whose stages
// hold 8 KB of P and 32 KB of E, so more of E - the stream from HBM - is in flight.
constexpr int kDmaThreads = 512;
constexpr int kDmaIssuers = 4;  // waves that refill the ring (one per SIMD)

template <int BM_, int BN_>
struct DmaTile {
  static constexpr int BM = BM_, BN = BN_;
  static constexpr int kWN = BN / 128;                 // waves along N (256 x 256 tile)
  static constexpr int kStageA = BM * 64;              // BM rows x 32 bf16
  static constexpr int kRowB = BN * 2;                 // bytes per B k row
  static constexpr int kStageB = kDmaBK * kRowB;
  static constexpr int kStageBytes = kStageA + kStageB;
  static constexpr int kStages = 163840 / kStageBytes;  // 4, 5 or 6
  // The ring is refilled by the first kDmaIssuers waves (one per SIMD): while one wave
  // of a SIMD issues its copies, the other keeps the matrix core busy.
  static constexpr int kSegA = kStageA / 1024 / kDmaIssuers;  // 1 KB DMA segments per issuing wave
  static constexpr int kSegB = kStageB / 1024 / kDmaIssuers;
  static constexpr int kRowsPerSegB = 1024 / kRowB;    // k rows per B segment (1, 2 or 4)
};

template <int BM_, int BN, bool kStreamE>
__global__ __launch_bounds__(kDmaThreads) void selfcond_gemm_dma(GemmArgs g) {
  using T = DmaTile<BM_, BN>;
  constexpr int BM = T::BM, kStages = T::kStages, kStageA = T::kStageA, kStageBytes = T::kStageBytes;
  constexpr int kSegA = T::kSegA, kSegB = T::kSegB;
  __shared__ __attribute__((aligned(1024))) char lds[kStages][kStageBytes];
  const TileIdx ti = tile_index<BM, BN>(g);
  const int nsteps = (ti.k_hi - ti.k_lo) / kDmaBK;  // K range is a multiple of 32
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5, l32 = lane & 31;
  // Wave placement. BN = 512: SIMD s (waves s and s + 4) owns rows 64 (s / 2) .. +63 and
  // columns 256 (s % 2) .. +255; the wave that refills the ring (s) takes the first 96
  // columns and the other the next 160, so the copies the first issues are balanced by
  // the second's extra MFMAs. BN = 256: every wave a 64 x 128 tile. BN = 128 (256 rows,
  // for small products): every wave a 64 x 64 tile.
  constexpr bool kSplit = BN == 512;
  constexpr bool kNarrow = BN == 128;
  const int s4 = wave % kDmaIssuers;
  const int wm = kSplit ? (s4 >> 1) * 64 : kNarrow ? (wave >> 1) * 64 : (wave / T::kWN) * 64;
  const int wn = kSplit ? (s4 & 1) * 256 + (wave < kDmaIssuers ? 0 : 96)
                        : kNarrow ? (wave & 1) * 64 : (wave % T::kWN) * 128;

  // Per-lane DMA sources. Issuing wave w fills A segments kSegA*w .. and B segments
  // kSegB*w .. (1 KB each, lane i -> bytes 16i .. 16i+15 of the segment); the lane
  // fetches the chunk that the swizzle puts in its slot. Rows past M and columns past d
  // are clamped to valid memory; their results are never stored. The other waves
  // compute the same pointers as wave w % kDmaIssuers and never use them.
  const int dw = wave % kDmaIssuers;
  const char* psrc[kSegA];
  const char* esrc[kSegB];
  const char* pb = reinterpret_cast<const char*>(g.p);
  const char* eb = reinterpret_cast<const char*>(g.e);
#pragma unroll
  for (int t = 0; t < kSegA; ++t) {
    const int seg = kSegA * dw + t;
    const int r = seg * 16 + (lane >> 2);         // A row within the tile
    const int ca = (lane & 3) ^ swa(r);           // logical chunk stored in this slot
    const int grow = min(ti.m0 + r, g.M - 1);
    psrc[t] = pb + ((int64_t)grow * g.ldp + ti.k_lo + ca * 8) * 2;
  }
#pragma unroll
  for (int t = 0; t < kSegB; ++t) {
    const int seg = kSegB * dw + t;
    constexpr int kLanesPerRow = 64 / T::kRowsPerSegB;  // one 16-byte chunk of a k row per lane
    const int kk = seg * T::kRowsPerSegB + lane / kLanesPerRow;  // B k row
    const int cb = (lane % kLanesPerRow) ^ swb(kk);
    const int gcol = min(ti.n0 + cb * 8, g.d - 8);
    esrc[t] = eb + ((int64_t)(ti.k_lo + kk) * g.lde + gcol) * 2;
  }
  const int64_t pstep = kDmaBK * 2;                 // bytes per K step along a P row
  const int64_t estep = (int64_t)kDmaBK * g.lde * 2;  // bytes per K step down E
  __attribute__((address_space(3))) char* lds0 = (__attribute__((address_space(3))) char*)lds[0];
  const uint32_t lbase = (uint32_t)(uintptr_t)lds0;

  auto issue = [&](int s) {
    if (wave >= kDmaIssuers) return;  // uniform
    __attribute__((address_space(3))) char* st = lds0 + (s % kStages) * kStageBytes;
#pragma unroll
    for (int t = 0; t < kSegA; ++t)
      __builtin_amdgcn_global_load_lds((const void*)(psrc[t] + s * pstep),
                                       (__attribute__((address_space(3))) void*)(st + (kSegA * dw + t) * 1024), 16, 0,
                                       0);
#pragma unroll
    for (int t = 0; t < kSegB; ++t)
      __builtin_amdgcn_global_load_lds((const void*)(esrc[t] + s * estep),
                                       (__attribute__((address_space(3))) void*)(st + kStageA + (kSegB * dw + t) * 1024),
                                       16, 0, kStreamE ? kCpolStream : 0);
  };
  constexpr int kGroup = kSegA + kSegB;  // DMA instructions per stage per issuing wave (0 for the others)


  // B operand addresses (tr16): lane group grp = lane/16 covers k rows 8*(grp/2) + 4q
  // + (lane%16)/4 and columns 16*(grp%2) + 4*(lane%4) of each 32-column block.
  const int grp = lane >> 4, s16 = lane & 15;
  const int brow = 8 * (grp >> 1) + (s16 >> 2);
  const int bcol = 16 * (grp & 1) + 4 * (s16 & 3);  // + wn + 32j

  // One half step = 16 k: A fragments of 2 row blocks, B fragments of NJ column blocks
  // (two transposing reads of 4 k rows each). The 2 NJ + 2 LDS reads of the next half
  // step are interleaved with the 2 NJ MFMAs of the current one (sched_barrier pins the
  // order). The loop is instantiated per NJ, so each wave keeps only its own registers.
  auto a_addr = [&](uint32_t st, int ks, int i) { return st + a_off(wm + 32 * i + l32, 2 * ks + h); };
  auto b_addr = [&](uint32_t st, int ks, int j, int q) {
    const int col = wn + 32 * j + bcol;
    const int kk = 16 * ks + brow + 4 * q;
    return st + kStageA + kk * T::kRowB + (((col >> 3) ^ swb(kk)) << 4) + ((col & 7) << 1);
  };
  auto run = [&](auto njc) {
    constexpr int NJ = decltype(njc)::value;
    f32x16_t acc[2][NJ];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
    uint4 fa[2][2], fb[2][NJ];
    auto read_half = [&](uint32_t st, int ks, int buf) {
#pragma unroll
      for (int i = 0; i < 2; ++i) fa[buf][i] = lds_read_b128(a_addr(st, ks, i));
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        const uint2 lo = lds_read_tr16(b_addr(st, ks, j, 0)), hi = lds_read_tr16(b_addr(st, ks, j, 1));
        fb[buf][j] = make_uint4(lo.x, lo.y, hi.x, hi.y);
      }
    };
    auto mma_half = [&](int buf, uint32_t next_st, int next_ks) {
      const int nb = buf ^ 1;
      uint2 lo[NJ], hi[NJ];
#pragma unroll
      for (int t = 0; t < 2 * NJ; ++t) {
        const int i = t / NJ, j = t % NJ;
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, fa[buf][i]),
                                                            __builtin_bit_cast(bf16x8_t, fb[buf][j]), acc[i][j], 0, 0, 0);
        if (next_st != ~0u) {
          if (t & 1) hi[t >> 1] = lds_read_tr16(b_addr(next_st, next_ks, t >> 1, 1));
          else lo[t >> 1] = lds_read_tr16(b_addr(next_st, next_ks, t >> 1, 0));
          if (t == NJ - 1) fa[nb][0] = lds_read_b128(a_addr(next_st, next_ks, 0));
          if (t == 2 * NJ - 1) fa[nb][1] = lds_read_b128(a_addr(next_st, next_ks, 1));
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (next_st != ~0u) {
#pragma unroll
        for (int j = 0; j < NJ; ++j) fb[nb][j] = make_uint4(lo[j].x, lo[j].y, hi[j].x, hi[j].y);
      }
    };

    // Pipeline: step s's fragments are all in registers once the reads issued during
    // its first half have landed, so its ring slot is refilled (with step s+kStages)
    // right after the barrier that follows; the same barrier publishes step s+1.
    // kStages-1 steps stay in flight while one is consumed.
    const int pro = min(nsteps, kStages);
    for (int t = 0; t < pro; ++t) issue(t);
    if (nsteps > 0) {
      // step 0 has landed once at most the pro-1 groups issued after it remain
      if (pro == 6) DG_WAIT_VM(kGroup * 5);
      else if (pro == 5) DG_WAIT_VM(kGroup * 4);
      else if (pro == 4) DG_WAIT_VM(kGroup * 3);
      else if (pro == 3) DG_WAIT_VM(kGroup * 2);
      else if (pro == 2) DG_WAIT_VM(kGroup * 1);
      else DG_WAIT_VM(0);
      __builtin_amdgcn_s_barrier();
      read_half(lbase, 0, 0);
    }
    for (int s = 0; s < nsteps; ++s) {
      const uint32_t st = lbase + (s % kStages) * kStageBytes;
      DG_WAIT_LGKM0();       // fragments of (s, 0) in buffer 0
      mma_half(0, st, 1);    // ... with the reads of (s, 1) into buffer 1
      DG_WAIT_LGKM0();       // fragments of (s, 1) in buffer 1: this wave is done with slot s
      if (s + 1 < nsteps) {
        // step s+1 has landed once at most the groups issued after it (steps s+2 ..
        // min(s+kStages-1, nsteps-1)) remain
        const int after = min(kStages - 2, nsteps - 2 - s);
        if (after >= 4) DG_WAIT_VM(kGroup * 4);
        else if (after == 3) DG_WAIT_VM(kGroup * 3);
        else if (after == 2) DG_WAIT_VM(kGroup * 2);
        else if (after == 1) DG_WAIT_VM(kGroup * 1);
        else DG_WAIT_VM(0);
        __builtin_amdgcn_s_barrier();
        if (s + kStages < nsteps) issue(s + kStages);  // into slot s
      }
      mma_half(1, s + 1 < nsteps ? lbase + ((s + 1) % kStages) * kStageBytes : ~0u, 0);
    }
    store_blocks<BM, BN, 2, NJ>(g, acc, ti.split, ti.k_lo, ti.mt, ti.nt, wm >> 5, wn >> 5, lane, true);
  };
  if constexpr (kSplit) {
    if (wave < kDmaIssuers) run(std::integral_constant<int, 3>{});
    else run(std::integral_constant<int, 5>{});
  } else if constexpr (kNarrow) {
    run(std::integral_constant<int, 2>{});
  } else {
    run(std::integral_constant<int, 4>{});
  }
}

// bf16 logits + row statistics -> probabilities p = 2^(l*log2e + c); 8 per thread.
__global__ __launch_bounds__(256) void selfcond_normalize(const uint16_t* __restrict__ l, int64_t ldl,
                                                          const float* __restrict__ row_max,
                                                          const float* __restrict__ row_sum, int M, int V,
                                                          uint16_t* __restrict__ p) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t per_row = V / 8;
  if (i >= (int64_t)M * per_row) return;
  const int r = (int)(i / per_row);
  const int64_t c = (i % per_row) * 8;
  const float cr = -row_max[r] * kLog2e - __builtin_amdgcn_logf(row_sum[r]);
  const uint4 v = *reinterpret_cast<const uint4*>(l + (int64_t)r * ldl + c);
  *reinterpret_cast<uint4*>(p + (int64_t)r * V + c) = to_prob<true>(v, cr);
}

// Sum split-K partials in slice order (deterministic) and store in the output dtype.
// Thread = one 4-value group of the MFMA-layout tile (4 consecutive rows of one column).
template <bool kBf16>
__global__ __launch_bounds__(256) void selfcond_reduce(const void* __restrict__ part_v, int splits, int m_tiles,
                                                       int n_tiles, int tile_m, int tile_n, int M, int d,
                                                       void* __restrict__ out, int64_t ldo) {
  const int kTile4 = tile_m * tile_n / 4;  // float4 groups per tile
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t per_split = (int64_t)m_tiles * n_tiles * kTile4;
  if (i >= per_split) return;
  // slices added in order; loads in batches of 8, all issued before the adds.
  // Partials are bf16 (4 values in 8 bytes) for bf16 products, else fp32.
  auto load = [&](int64_t idx) {
    if constexpr (kBf16) {
      const uint2 u = reinterpret_cast<const uint2*>(part_v)[idx];
      return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u), __uint_as_float(u.y << 16),
                         __uint_as_float(u.y & 0xffff0000u));
    } else {
      return reinterpret_cast<const float4*>(part_v)[idx];
    }
  };
  float4 s = load(i);
  int k = 1;
  for (; k + 8 <= splits; k += 8) {
    float4 v[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) v[t] = load((int64_t)(k + t) * per_split + i);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      s.x += v[t].x;
      s.y += v[t].y;
      s.z += v[t].z;
      s.w += v[t].w;
    }
  }
  for (; k < splits; ++k) {
    const float4 v = load((int64_t)k * per_split + i);
    s.x += v.x;
    s.y += v.y;
    s.z += v.z;
    s.w += v.w;
  }
  // decode [tile][32-row block][128-column group][j][e/4][lane] -> rows r..r+3 of column c
  const int q = (int)(i % kTile4);
  const int64_t tile = i / kTile4;
  const int mt = (int)(tile / n_tiles), nt = (int)(tile % n_tiles);
  const int chs = tile_n / 128;
  const int lane = q & 63, e4 = (q >> 6) & 3, jj = (q >> 8) & 3, ch = (q >> 10) % chs, rb = (q >> 10) / chs;
  const int r = mt * tile_m + 32 * rb + 8 * e4 + 4 * (lane >> 5);
  const int c = nt * tile_n + 128 * ch + 32 * jj + (lane & 31);
  if (c >= d) return;
  const float v[4] = {s.x, s.y, s.z, s.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if (r + e >= M) break;
    if (kBf16) reinterpret_cast<__bf16*>(out)[(int64_t)(r + e) * ldo + c] = (__bf16)v[e];
    else reinterpret_cast<float*>(out)[(int64_t)(r + e) * ldo + c] = v[e];
  }
}

// The reduce with an epilogue, for the self-conditioning injection's two bf16 products
// (bf16 partials). Same slice order and tile decode as selfcond_reduce.
//   kReduceGeglu:   the product is [gate | up], N = 2 hidden with hidden a multiple of the
//                   tile width; a thread sums a gate element and its partner hidden
//                   columns on (same rows, `half_tiles` column tiles on), rounds both to
//                   bf16, and stores h = bf16(gelu(g) * u) into out [M][hidden];
//   kReduceAddRows: out[r][c] = bf16(sum + embed[token r][c]), one rounding.
template <int kMode>
__global__ __launch_bounds__(256) void selfcond_reduce_epi(const uint2* __restrict__ part, int splits, int m_tiles,
                                                           int n_tiles, int tile_m, int tile_n, int M, int d,
                                                           uint16_t* __restrict__ out, int64_t ldo, int half_tiles,
                                                           const uint16_t* __restrict__ embed,
                                                           const int32_t* __restrict__ tokens, int vocab) {
  const int kTile4 = tile_m * tile_n / 4;  // float4 groups per tile
  const int64_t per_split = (int64_t)m_tiles * n_tiles * kTile4;
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  int64_t i = j;
  if constexpr (kMode == kReduceGeglu) {
    // j walks the gate tiles only: (mt, nt < half_tiles, q)
    const int64_t per_row_tiles = (int64_t)half_tiles * kTile4;
    if (j >= (int64_t)m_tiles * per_row_tiles) return;
    i = (j / per_row_tiles) * n_tiles * kTile4 + j % per_row_tiles;
  } else {
    if (j >= per_split) return;
  }
  auto sum = [&](int64_t idx) {
    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    int k = 0;
    for (; k + 8 <= splits; k += 8) {
      uint2 u[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) u[t] = part[(int64_t)(k + t) * per_split + idx];
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        s.x += bf16lo(u[t].x);
        s.y += bf16hi(u[t].x);
        s.z += bf16lo(u[t].y);
        s.w += bf16hi(u[t].y);
      }
    }
    for (; k < splits; ++k) {
      const uint2 u = part[(int64_t)k * per_split + idx];
      s.x += bf16lo(u.x);
      s.y += bf16hi(u.x);
      s.z += bf16lo(u.y);
      s.w += bf16hi(u.y);
    }
    return s;
  };
  const float4 s = sum(i);
  float4 s2 = make_float4(0.f, 0.f, 0.f, 0.f);
  if constexpr (kMode == kReduceGeglu) s2 = sum(i + (int64_t)half_tiles * kTile4);
  const int q = (int)(i % kTile4);
  const int64_t tile = i / kTile4;
  const int mt = (int)(tile / n_tiles), nt = (int)(tile % n_tiles);
  const int chs = tile_n / 128;
  const int lane = q & 63, e4 = (q >> 6) & 3, jj = (q >> 8) & 3, ch = (q >> 10) % chs, rb = (q >> 10) / chs;
  const int r = mt * tile_m + 32 * rb + 8 * e4 + 4 * (lane >> 5);
  const int c = nt * tile_n + 128 * ch + 32 * jj + (lane & 31);
  if (c >= d) return;
  const float v[4] = {s.x, s.y, s.z, s.w};
  const float w[4] = {s2.x, s2.y, s2.z, s2.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if (r + e >= M) break;
    float x;
    if constexpr (kMode == kReduceGeglu) {
      const float g = bf16lo(pack_bf16(v[e], 0.f)), u = bf16lo(pack_bf16(w[e], 0.f));
      x = gelu_tanh(g) * u;
    } else {
      const int tok = min(max(tokens[r + e], 0), vocab - 1);
      x = v[e] + bf16lo((uint32_t)embed[(int64_t)tok * d + c]);
    }
    out[(int64_t)(r + e) * ldo + c] = (uint16_t)(pack_bf16(x, 0.f) & 0xFFFFu);
  }
}

}  // namespace

int launch_selfcond(const dg_selfcond_args* a, const SelfcondPlan& plan, void* stream, const ReduceEpi* epi) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* ws = reinterpret_cast<char*>(a->workspace);
  GemmArgs g;
  g.p = a->p;
  g.ldp = a->ldp;
  g.row_max = a->row_max;
  g.row_sum = a->row_sum;
  g.e = a->embed;
  g.lde = a->lde;
  g.out = a->out;
  g.ldo = a->ldo;
  g.part = plan.splits > 1 ? reinterpret_cast<float*>(ws + plan.part_offset) : nullptr;
  g.p_scale = a->p_scale;
  g.nblocks = (a->V + DG_PROB_BLOCK - 1) / DG_PROB_BLOCK;
  g.M = a->M;
  g.V = a->V;
  g.d = a->d;
  g.m_tiles = plan.m_tiles;
  g.n_tiles = plan.n_tiles;
  g.splits = plan.splits;
  g.k_per_split = plan.k_per_split;
  const dim3 grid(plan.m_tiles * plan.n_tiles * plan.splits);
  const bool fused = a->row_max != nullptr;
  if (plan.dma) {
    if (fused) {  // rebuild P once into the workspace, then the plain DMA GEMM
      uint16_t* pn = reinterpret_cast<uint16_t*>(ws + plan.p_offset);
      const int64_t n8 = (int64_t)a->M * (a->V / 8);
      hipLaunchKernelGGL(selfcond_normalize, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s,
                         reinterpret_cast<const uint16_t*>(a->p), a->ldp, a->row_max, a->row_sum, a->M, a->V, pn);
      g.p = pn;
      g.ldp = a->V;
      g.row_max = g.row_sum = nullptr;
    }
    const bool stream_e = (int64_t)a->V * a->lde * 2 > kStreamMinBytes;
    if (plan.tile_n == 512) {
      if (stream_e) hipLaunchKernelGGL((selfcond_gemm_dma<128, 512, true>), grid, dim3(kDmaThreads), 0, s, g);
      else hipLaunchKernelGGL((selfcond_gemm_dma<128, 512, false>), grid, dim3(kDmaThreads), 0, s, g);
    } else if (plan.tile_n == 128) {  // small products: E (a weight matrix) stays cached
      hipLaunchKernelGGL((selfcond_gemm_dma<256, 128, false>), grid, dim3(kDmaThreads), 0, s, g);
    } else {
      if (stream_e) hipLaunchKernelGGL((selfcond_gemm_dma<256, 256, true>), grid, dim3(kDmaThreads), 0, s, g);
      else hipLaunchKernelGGL((selfcond_gemm_dma<256, 256, false>), grid, dim3(kDmaThreads), 0, s, g);
    }
  } else if (a->dtype == DG_BF16) {
    if (fused) hipLaunchKernelGGL((selfcond_gemm_reg<true, true>), grid, dim3(kThreads), 0, s, g);
    else hipLaunchKernelGGL((selfcond_gemm_reg<true, false>), grid, dim3(kThreads), 0, s, g);
  } else {
    if (plan.tile_m == 64) {
      if (fused) hipLaunchKernelGGL((selfcond_gemm_reg<false, true, 64, 128>), grid, dim3(kThreads), 0, s, g);
      else hipLaunchKernelGGL((selfcond_gemm_reg<false, false, 64, 128>), grid, dim3(kThreads), 0, s, g);
    } else {
      if (fused) hipLaunchKernelGGL((selfcond_gemm_reg<false, true>), grid, dim3(kThreads), 0, s, g);
      else hipLaunchKernelGGL((selfcond_gemm_reg<false, false>), grid, dim3(kThreads), 0, s, g);
    }
  }
  if (plan.splits > 1 && epi && epi->mode != kReducePlain) {
    const int64_t n4 = (int64_t)plan.m_tiles * (epi->mode == kReduceGeglu ? epi->half_tiles : plan.n_tiles) *
                       (plan.tile_m * plan.tile_n / 4);
    const dim3 rg((unsigned)((n4 + 255) / 256));
    const uint2* part = reinterpret_cast<const uint2*>(g.part);
    uint16_t* o = reinterpret_cast<uint16_t*>(a->out);
    const uint16_t* emb = reinterpret_cast<const uint16_t*>(epi->embed);
    if (epi->mode == kReduceGeglu)
      hipLaunchKernelGGL(selfcond_reduce_epi<kReduceGeglu>, rg, dim3(256), 0, s, part, plan.splits, plan.m_tiles,
                         plan.n_tiles, plan.tile_m, plan.tile_n, a->M, a->d, o, a->ldo, epi->half_tiles, emb,
                         epi->tokens, epi->vocab);
    else
      hipLaunchKernelGGL(selfcond_reduce_epi<kReduceAddRows>, rg, dim3(256), 0, s, part, plan.splits, plan.m_tiles,
                         plan.n_tiles, plan.tile_m, plan.tile_n, a->M, a->d, o, a->ldo, epi->half_tiles, emb,
                         epi->tokens, epi->vocab);
  } else if (plan.splits > 1) {
    const int64_t n4 = (int64_t)plan.m_tiles * plan.n_tiles * (plan.tile_m * plan.tile_n / 4);
    const dim3 rg((unsigned)((n4 + 255) / 256));
    const void* part = g.part;
    if (a->dtype == DG_BF16)
      hipLaunchKernelGGL(selfcond_reduce<true>, rg, dim3(256), 0, s, part, plan.splits, plan.m_tiles, plan.n_tiles,
                         plan.tile_m, plan.tile_n, a->M, a->d, a->out, a->ldo);
    else
      hipLaunchKernelGGL(selfcond_reduce<false>, rg, dim3(256), 0, s, part, plan.splits, plan.m_tiles, plan.n_tiles,
                         plan.tile_m, plan.tile_n, a->M, a->d, a->out, a->ldo);
  }
  return (int)hipGetLastError();
}

}  // namespace dg
