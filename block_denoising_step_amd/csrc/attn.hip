// Mixed-mode attention on gfx950: each request of a batch is causal (prefill/commit,
// "encoder mode") or bidirectional (denoising, "decoder mode"), optionally inside a
// sliding window that is one-sided for causal requests and symmetric (2W+1 keys)
// for bidirectional ones ([P1] "DiffusionGemma: vLLM에서 네이티브로 처음 지원되는 첫 번째
// Diffusion LLM", sections "듀얼 모드 운영", "동적 퍼-시퀀스 인과적 어텐션",
// "대칭 슬라이딩 윈도우 어텐션"; [P3] "DiffusionGemma u vLLM: ...", section
// "Zašto je difuzijsko generiranje teksta drugačije?").
//
// attn_fwd: one work group = 128 query rows (tokens x the G query heads of one KV
// head) of one request, over one chunk of its keys, in 64-key tiles. Each of the 4
// waves owns 32 rows. Per tile:
//   S^T = K . Q^T   (MFMA 32x32; K tile in LDS, Q^T fragments held in registers),
//   so lane l holds scores of query row l%32 only: the row max/sum need one
//   xor-32 shuffle, and the key bounds are per lane;
//   mask (only on tiles that cross some row's key bounds), online softmax in base 2;
//   O^T += V^T . P^T (MFMA 32x32; P^T taken straight from the S^T accumulators,
//   V transposed into LDS with the key order permuted to match them), so the
//   softmax rescale of O is a per-lane multiply.
// FP8 K/V (OCP E4M3 codes with per-tensor scales, the FP8 configuration of [P1]
// section "성능 및 양자화"): attn_fwd's <kFp8> instance loads 8 codes where it loaded
// 8 bf16 and widens them to bf16 while staging the tile, exactly (every E4M3 value
// is a bf16 value), so the LDS layout and the inner loop are the bf16 ones; the next
// tile's codes are loaded while the current tile is computed. k_scale is folded into
// the score scale and v_scale into the output normalisation.
// A request whose keys were split into several chunks writes partials: O of the
// chunk normalised by its own sum, in the input dtype, plus the chunk's (max, sum)
// in fp32; attn_merge combines them in chunk order.
#include "dg_common.cuh"
#include "dg_internal.h"

namespace dg {
namespace {

constexpr int kThreads = 256;
constexpr int kKT = kAttnKeyTile;  // keys per tile
constexpr int kRows = kAttnTileRows;

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* lse;
  void* part_o;  // [partial rows][D], input dtype
  float* part_ml;
  int hq, hkv, group, window, num_seqs;
  int work_offset;  // work index of this launch's block 0
  float scale_log2;  // scale * log2(e) (times k_scale for FP8 K/V)
  float v_scale;     // FP8 K/V: the value scale, applied with the output normalisation
  const int32_t* block_table;  // paged K/V: a request's table starts at its kv_start
  int64_t pool_blocks;         // blocks in the K and V pools
  int block_shift;             // log2(block_size)
  AttnSeqPlan seqs[DG_MAX_SEQS];
};

// Pool row of key `key` of request sp. Contiguous: kv_start + key. Paged: through the
// request's block table, read with a scalar load (the table is uniform and read-only).
// Blocks hold a power of two >= 64 rows and key tiles start at multiples of 32, so the
// rows of one 32-key sub-tile or 64-key tile are consecutive in the pool. An entry
// outside the pool is clamped to its last block, so no read leaves the pools.
template <bool kPaged>
__device__ __forceinline__ int64_t key_row(const AttnArgs& a, const AttnSeqPlan& sp, int key) {
  if constexpr (!kPaged) {
    return (int64_t)sp.kv_start + key;
  } else {
    typedef const __attribute__((address_space(4))) int32_t* const_i32p;
    const uint32_t e = (uint32_t)((const_i32p)a.block_table)[sp.kv_start + (key >> a.block_shift)];
    const int64_t blk = min((int64_t)e, a.pool_blocks - 1);
    return (blk << a.block_shift) + (key & ((1 << a.block_shift) - 1));
  }
}

__device__ __forceinline__ void key_bounds(int mode, int prefix, int num_q, int window, int i, int& lo, int& hi) {
  const int p = prefix + i;
  const int last = prefix + num_q - 1;
  lo = window < 0 ? 0 : max(0, p - window);
  hi = mode == DG_CAUSAL ? p : (window < 0 ? last : min(last, p + window));
}

// The request whose work (or merge) range holds index w (the ranges are disjoint, in
// any order).
__device__ __forceinline__ int find_seq(const AttnArgs& a, int w, bool merge) {
  int s = 0;
  for (int i = 0; i < a.num_seqs; ++i) {
    const int b = merge ? a.seqs[i].merge_begin : a.seqs[i].work_begin;
    const int n = merge ? a.seqs[i].merge_count : a.seqs[i].work_count;
    if (b <= w && w < b + n) s = i;
  }
  return s;
}

template <bool kBf16> struct Op;
// bf16: a "k16" fragment is 8 bf16 (16 bytes) per lane, one 32x32x16 MFMA.
template <> struct Op<true> {
  static constexpr int esz = 2;
  struct Frag { uint4 v; };
  __device__ static Frag lds(const char* p) { return Frag{*reinterpret_cast<const uint4*>(p)}; }
  __device__ static Frag gmem(const char* p) { return Frag{*reinterpret_cast<const uint4*>(p)}; }
  __device__ static Frag zero() { return Frag{make_uint4(0, 0, 0, 0)}; }
  __device__ static void mma(f32x16_t& acc, const Frag& a, const Frag& b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a.v), __builtin_bit_cast(bf16x8_t, b.v),
                                                  acc, 0, 0, 0);
  }
  __device__ static Frag from_f32(const float* x) {
    return Frag{make_uint4(pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3]), pack_bf16(x[4], x[5]), pack_bf16(x[6], x[7]))};
  }
};
// fp32: 8 floats (32 bytes) per lane, eight 32x32x2 MFMAs; element j of both halves
// forms the k pair of MFMA j, consistently for A and B.
template <> struct Op<false> {
  static constexpr int esz = 4;
  struct Frag { float4 lo, hi; };
  __device__ static Frag lds(const char* p) {
    return Frag{*reinterpret_cast<const float4*>(p), *reinterpret_cast<const float4*>(p + 16)};
  }
  __device__ static Frag gmem(const char* p) { return lds(p); }
  __device__ static Frag zero() { return Frag{make_float4(0, 0, 0, 0), make_float4(0, 0, 0, 0)}; }
  __device__ static void mma(f32x16_t& acc, const Frag& a, const Frag& b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.lo.x, b.lo.x, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.lo.y, b.lo.y, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.lo.z, b.lo.z, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.lo.w, b.lo.w, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.hi.x, b.hi.x, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.hi.y, b.hi.y, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.hi.z, b.hi.z, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a.hi.w, b.hi.w, acc, 0, 0, 0);
  }
  __device__ static Frag from_f32(const float* x) {
    return Frag{make_float4(x[0], x[1], x[2], x[3]), make_float4(x[4], x[5], x[6], x[7])};
  }
};

template <bool kBf16, int D>
struct Lds {
  static constexpr int esz = kBf16 ? 2 : 4;
  static constexpr int k_pitch = D * esz + 16;     // K tile: [64 keys][D]
  static constexpr int v_pitch = kKT * esz + 16;   // V^T tile: [D][64 keys, permuted]
  static constexpr int k_bytes = kKT * k_pitch;
  static constexpr int v_bytes = D * v_pitch;
};

// Two E4M3 codes (bytes 0-1, or 2-3 with kHi, of w) as two bf16 in one word. The
// conversion is to fp32 and exact, and an E4M3 value needs at most 4 significant
// bits, so the upper half of each fp32 is its bf16 value.
template <bool kHi>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w) {
  const auto f = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, kHi);
  return __builtin_amdgcn_perm(__float_as_uint(f[1]), __float_as_uint(f[0]), 0x07060302u);
}

// Stage one 64-key tile of K (row-major) and V (transposed) into LDS. Key rows at
// or past `nvalid` (request-local) are zero.
template <bool kBf16, int D>
__device__ __forceinline__ void stage_tile(char* lk, char* lv, const char* kg, const char* vg, int64_t row_stride,
                                           int nvalid) {
  using L = Lds<kBf16, D>;
  constexpr int esz = L::esz;
  constexpr int cpr = D * esz / 16;  // 16-byte chunks per key row
  const int tid = threadIdx.x;
  // K: chunk q -> key q / cpr, column q % cpr
#pragma unroll
  for (int q = tid; q < kKT * cpr; q += kThreads) {
    const int key = q / cpr, col = q % cpr;
    uint4 val = make_uint4(0, 0, 0, 0);
    if (key < nvalid) val = *reinterpret_cast<const uint4*>(kg + (int64_t)key * row_stride + col * 16);
    *reinterpret_cast<uint4*>(lk + key * L::k_pitch + col * 16) = val;
  }
  // V^T: within each 16-key group, key w sits at position w with bits 2 and 3 swapped
  if (kBf16) {
    // block = 8 keys {16a+4c+0..3, 16a+8+4c+0..3} (positions 16a+8c+0..7) x 8 dims
    constexpr int dgroups = D / 8;
    for (int b = tid; b < (kKT / 8) * dgroups; b += kThreads) {
      const int dgp = b % dgroups, kb = b / dgroups;  // kb = 2a + c
      const int a16 = kb >> 1, c = kb & 1;
      uint4 r[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int key = 16 * a16 + 4 * c + (j & 3) + ((j >> 2) << 3);
        r[j] = make_uint4(0, 0, 0, 0);
        if (key < nvalid) r[j] = *reinterpret_cast<const uint4*>(vg + (int64_t)key * row_stride + dgp * 16);
      }
#pragma unroll
      for (int dd = 0; dd < 8; ++dd) {
        const int w = dd >> 1;
        const uint32_t sel = (dd & 1) ? 0x07060302u : 0x05040100u;
        uint4 o;
        o.x = __builtin_amdgcn_perm((&r[1].x)[w], (&r[0].x)[w], sel);
        o.y = __builtin_amdgcn_perm((&r[3].x)[w], (&r[2].x)[w], sel);
        o.z = __builtin_amdgcn_perm((&r[5].x)[w], (&r[4].x)[w], sel);
        o.w = __builtin_amdgcn_perm((&r[7].x)[w], (&r[6].x)[w], sel);
        *reinterpret_cast<uint4*>(lv + (dgp * 8 + dd) * L::v_pitch + (16 * a16 + 8 * c) * esz) = o;
      }
    }
  } else {
    // block = 4 consecutive keys (one permuted quad of positions) x 4 dims
    constexpr int dgroups = D / 4;
    for (int b = tid; b < (kKT / 4) * dgroups; b += kThreads) {
      const int dgp = b % dgroups, kq = b / dgroups;  // key quad kq = 4a + qq
      const int a16 = kq >> 2, qq = kq & 3;
      const int key0 = 16 * a16 + 4 * qq;
      const int pos0 = 16 * a16 + 4 * (((qq & 1) << 1) | (qq >> 1));
      float4 r[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        r[j] = make_float4(0, 0, 0, 0);
        if (key0 + j < nvalid) r[j] = *reinterpret_cast<const float4*>(vg + (int64_t)(key0 + j) * row_stride + dgp * 16);
      }
      *reinterpret_cast<float4*>(lv + (dgp * 4 + 0) * L::v_pitch + pos0 * 4) = make_float4(r[0].x, r[1].x, r[2].x, r[3].x);
      *reinterpret_cast<float4*>(lv + (dgp * 4 + 1) * L::v_pitch + pos0 * 4) = make_float4(r[0].y, r[1].y, r[2].y, r[3].y);
      *reinterpret_cast<float4*>(lv + (dgp * 4 + 2) * L::v_pitch + pos0 * 4) = make_float4(r[0].z, r[1].z, r[2].z, r[3].z);
      *reinterpret_cast<float4*>(lv + (dgp * 4 + 3) * L::v_pitch + pos0 * 4) = make_float4(r[0].w, r[1].w, r[2].w, r[3].w);
    }
  }
}

// FP8 tiles are staged in two halves so that the next tile's loads are in flight while
// the current one is computed: fp8_load issues a tile's global loads (8 codes per load)
// into registers, fp8_store widens them and writes the same LDS layout as stage_tile.
template <int D>
struct Fp8Regs {
  static constexpr int kK = kKT * (D / 8) / kThreads;  // K loads per thread (8 codes each)
  static constexpr int kVBlocks = (kKT / 8) * (D / 8);  // V blocks of 8 keys x 8 dims (<= kThreads)
  uint2 k[kK];
  uint2 v[8];
};

template <int D>
__device__ __forceinline__ void fp8_load(Fp8Regs<D>& r, const char* kg, const char* vg, int64_t row_stride,
                                         int nvalid) {
  constexpr int cpr = D / 8;  // 8-code chunks per key row
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < Fp8Regs<D>::kK; ++i) {
    const int q = i * kThreads + tid;
    const int key = q / cpr, col = q % cpr;
    r.k[i] = key < nvalid ? *reinterpret_cast<const uint2*>(kg + (int64_t)key * row_stride + col * 8)
                          : make_uint2(0, 0);
  }
  if (tid < Fp8Regs<D>::kVBlocks) {
    constexpr int dgroups = D / 8;
    const int dgp = tid % dgroups, kb = tid / dgroups;
    const int a16 = kb >> 1, c = kb & 1;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int key = 16 * a16 + 4 * c + (j & 3) + ((j >> 2) << 3);
      r.v[j] = key < nvalid ? *reinterpret_cast<const uint2*>(vg + (int64_t)key * row_stride + dgp * 8)
                            : make_uint2(0, 0);
    }
  }
}

template <int D>
__device__ __forceinline__ void fp8_store(const Fp8Regs<D>& r, char* lk, char* lv) {
  using L = Lds<true, D>;
  constexpr int cpr = D / 8;
  const int tid = threadIdx.x;
  auto widen = [](uint2 w) {
    return make_uint4(e4m3x2_to_bf16x2<false>(w.x), e4m3x2_to_bf16x2<true>(w.x), e4m3x2_to_bf16x2<false>(w.y),
                      e4m3x2_to_bf16x2<true>(w.y));
  };
#pragma unroll
  for (int i = 0; i < Fp8Regs<D>::kK; ++i) {
    const int q = i * kThreads + tid;
    const int key = q / cpr, col = q % cpr;
    *reinterpret_cast<uint4*>(lk + key * L::k_pitch + col * 16) = widen(r.k[i]);
  }
  if (tid < Fp8Regs<D>::kVBlocks) {
    constexpr int dgroups = D / 8;
    const int dgp = tid % dgroups, kb = tid / dgroups;
    const int a16 = kb >> 1, c = kb & 1;
    uint4 x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = widen(r.v[j]);
#pragma unroll
    for (int dd = 0; dd < 8; ++dd) {
      const int w = dd >> 1;
      const uint32_t sel = (dd & 1) ? 0x07060302u : 0x05040100u;
      uint4 o;
      o.x = __builtin_amdgcn_perm((&x[1].x)[w], (&x[0].x)[w], sel);
      o.y = __builtin_amdgcn_perm((&x[3].x)[w], (&x[2].x)[w], sel);
      o.z = __builtin_amdgcn_perm((&x[5].x)[w], (&x[4].x)[w], sel);
      o.w = __builtin_amdgcn_perm((&x[7].x)[w], (&x[6].x)[w], sel);
      *reinterpret_cast<uint4*>(lv + (dgp * 8 + dd) * L::v_pitch + (16 * a16 + 8 * c) * 2) = o;
    }
  }
}

template <bool kBf16, int D, bool kPaged, bool kFp8 = false>
__global__ __launch_bounds__(kThreads) void attn_fwd(AttnArgs a) {
  using OP = Op<kBf16>;
  using L = Lds<kBf16, D>;
  constexpr int esz = L::esz;
  constexpr int kv_esz = kFp8 ? 1 : esz;  // bytes per K/V element in HBM
  constexpr int KS = D / 16;  // k16 steps over the head dimension
  constexpr int DB = D / 32;  // 32-wide output blocks
  // FP8: two tile buffers (the next tile is stored while no wave reads its buffer)
  constexpr int kBufs = kFp8 ? 2 : 1;
  __shared__ __attribute__((aligned(16))) char lk_s[kBufs][L::k_bytes];
  __shared__ __attribute__((aligned(16))) char lv_s[kBufs][L::v_bytes];

  const int w = a.work_offset + blockIdx.x;
  const int s = find_seq(a, w, false);
  const AttnSeqPlan sp = a.seqs[s];
  const int nqt = (sp.num_q + sp.tokens_per_tile - 1) / sp.tokens_per_tile;
  const int local = w - sp.work_begin;
  const int chunk = local % sp.num_chunks;
  const int rest = local / sp.num_chunks;
  const int qt = rest % nqt;
  const int g = rest / nqt;
  const int i0 = qt * sp.tokens_per_tile;
  const int nq = min(sp.tokens_per_tile, sp.num_q - i0);
  const int nkeys = sp.prefix_len + sp.num_q;

  int lo_first, hi_first, lo_last, hi_last;
  key_bounds(sp.mode, sp.prefix_len, sp.num_q, a.window, i0, lo_first, hi_first);
  key_bounds(sp.mode, sp.prefix_len, sp.num_q, a.window, i0 + nq - 1, lo_last, hi_last);
  const int kt_lo = lo_first / kKT, kt_hi = hi_last / kKT;
  const int t_begin = kt_lo + chunk * sp.chunk_tiles;
  const int t_end = min(kt_hi + 1, t_begin + sp.chunk_tiles);
  if (t_begin > kt_hi) return;  // empty chunk (uniform across the work group)

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int row = wave * 32 + l32;  // row within the tile
  const int tok = i0 + row / a.group;
  const int head = g * a.group + row % a.group;
  const bool valid = tok < sp.num_q;
  int lo = 0, hi = -1;
  if (valid) key_bounds(sp.mode, sp.prefix_len, sp.num_q, a.window, tok, lo, hi);

  // Q^T fragments: lane supplies q[row][16*ks + 8*hh .. +8]
  typename OP::Frag qf[KS];
  {
    const char* qrow = reinterpret_cast<const char*>(a.q) + ((int64_t)(sp.q_start + tok) * a.hq + head) * D * esz;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = valid ? OP::gmem(qrow + (16 * ks + 8 * hh) * esz) : OP::zero();
  }

  f32x16_t o[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b)
#pragma unroll
    for (int e = 0; e < 16; ++e) o[b][e] = 0.f;
  float m_run = kNegInf;  // running max of scale*log2e*score (base-2 units)
  float l_run = 0.f;      // this lane's share of the running sum

  const int64_t row_stride = (int64_t)a.hkv * D * kv_esz;
  const char* kg = reinterpret_cast<const char*>(a.k) + (int64_t)g * D * kv_esz;
  const char* vg = reinterpret_cast<const char*>(a.v) + (int64_t)g * D * kv_esz;

  // FP8: tile t_begin + i sits in buffer i % 2. Tile kt + 1 is stored into the other
  // buffer after tile kt's compute (that buffer's last reads, of tile kt - 1, ended at
  // the previous barrier), one barrier publishes it, and the loads of tile kt + 2 are
  // issued right after that barrier, so they are in flight during tile kt + 1.
  Fp8Regs<D> pre;
  auto fp8_fetch = [&](int kt) {
    const int64_t r = key_row<kPaged>(a, sp, kt * kKT) * row_stride;
    fp8_load<D>(pre, kg + r, vg + r, row_stride, nkeys - kt * kKT);
  };
  if constexpr (kFp8) {
    fp8_fetch(t_begin);
    fp8_store<D>(pre, lk_s[0], lv_s[0]);
    __syncthreads();
    if (t_begin + 1 < t_end) fp8_fetch(t_begin + 1);
  }
  for (int kt = t_begin; kt < t_end; ++kt) {
    const int k0 = kt * kKT;
    const char* lk = lk_s[kFp8 ? (kt - t_begin) & 1 : 0];
    const char* lv = lv_s[kFp8 ? (kt - t_begin) & 1 : 0];
    if constexpr (!kFp8) {
      __syncthreads();  // previous tile fully consumed
      const int64_t r0 = key_row<kPaged>(a, sp, k0) * row_stride;  // the tile's 64 rows are consecutive
      stage_tile<kBf16, D>(lk_s[0], lv_s[0], kg + r0, vg + r0, row_stride, nkeys - k0);
      __syncthreads();
    }

    // S^T blocks: sblk[kb][i] = score of key k0 + 32kb + 8(i/4) + 4hh + i%4 for this lane's row
    f32x16_t sblk[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int e = 0; e < 16; ++e) sblk[kb][e] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const typename OP::Frag kf = OP::lds(lk + (32 * kb + l32) * L::k_pitch + (16 * ks + 8 * hh) * esz);
        OP::mma(sblk[kb], kf, qf[ks]);
      }
    }
    // mask unless every row of the work group sees the whole tile
    const bool full = lo_last <= k0 && k0 + kKT - 1 <= hi_first;
    if (!full) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = k0 + 32 * kb + 8 * (e >> 2) + 4 * hh + (e & 3);
          if (key < lo || key > hi) sblk[kb][e] = kNegInf;
        }
    }
    float tmax = kNegInf;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) tmax = fmaxf(tmax, sblk[kb][e]);
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const float m_new = fmaxf(m_run, tmax * a.scale_log2);
    const float m_use = m_new == kNegInf ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);  // 0 when nothing was seen yet
    m_run = m_new;
    float p[2][16];
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        p[kb][e] = fast_exp2(fmaf(sblk[kb][e], a.scale_log2, -m_use));
        psum += p[kb][e];
      }
    l_run = fmaf(l_run, alpha, psum);
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[b][e] *= alpha;
    }
    // O^T += V^T . P^T over the 4 k16 steps of the tile
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const typename OP::Frag pf = OP::from_f32(&p[u >> 1][8 * (u & 1)]);
#pragma unroll
      for (int b = 0; b < DB; ++b) {
        const typename OP::Frag vf = OP::lds(lv + (32 * b + l32) * L::v_pitch + (16 * u + 8 * hh) * esz);
        OP::mma(o[b], vf, pf);
      }
    }
    if constexpr (kFp8) {
      if (kt + 1 < t_end) fp8_store<D>(pre, lk_s[(kt + 1 - t_begin) & 1], lv_s[(kt + 1 - t_begin) & 1]);
      __syncthreads();
      if (kt + 2 < t_end) fp8_fetch(kt + 2);
    }
  }

  // epilogue: o[b][e] = O^T[d = 32b + 8(e/4) + 4hh + e%4][this lane's row]; a row
  // with no key in this chunk (l = 0) stores zeros
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (!valid) return;
  {
    float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if constexpr (kFp8) inv *= a.v_scale;
    const int64_t prow = sp.part_begin + (int64_t)local * kRows + row;
    char* orow = sp.num_chunks == 1
                     ? reinterpret_cast<char*>(a.out) + ((int64_t)(sp.q_start + tok) * a.hq + head) * D * esz
                     : reinterpret_cast<char*>(a.part_o) + prow * D * esz;
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        const int d = 32 * b + 8 * e4 + 4 * hh;
        const float x0 = o[b][4 * e4] * inv, x1 = o[b][4 * e4 + 1] * inv;
        const float x2 = o[b][4 * e4 + 2] * inv, x3 = o[b][4 * e4 + 3] * inv;
        if (kBf16) *reinterpret_cast<uint2*>(orow + d * 2) = make_uint2(pack_bf16(x0, x1), pack_bf16(x2, x3));
        else *reinterpret_cast<float4*>(orow + d * 4) = make_float4(x0, x1, x2, x3);
      }
    if (hh == 0) {
      if (sp.num_chunks > 1)
        *reinterpret_cast<float2*>(a.part_ml + prow * 2) = make_float2(m_run, l_tot);
      else if (a.lse)
        a.lse[(int64_t)(sp.q_start + tok) * a.hq + head] = m_run * kLn2 + __builtin_amdgcn_logf(l_tot) * kLn2;
    }
  }
}

// Combine the chunk partials of one (request, KV head, q tile) in chunk order:
// with w_j = 2^(m_j - M) l_j (M a running max over the chunks), O = sum_j w_j O_j / sum_j w_j,
// where O_j is chunk j's output normalised by its own sum l_j.
// One thread per 16 bytes of partial row (8 bf16 or 4 fp32 columns), so that one
// (q tile, kv head) unit spreads over several work groups and every load is an
// independent, coalesced 16-byte load.
template <bool kBf16>
constexpr int merge_cols() { return kBf16 ? 8 : 4; }
template <bool kBf16, int D>
constexpr int merge_rows_per_group() { return kThreads / (D / merge_cols<kBf16>()); }

template <bool kBf16, int D>
__global__ __launch_bounds__(kThreads) void attn_merge(AttnArgs a) {
  constexpr int esz = kBf16 ? 2 : 4;
  constexpr int kC = merge_cols<kBf16>();
  constexpr int kTpr = D / kC;            // threads per row
  constexpr int kRpw = merge_rows_per_group<kBf16, D>();  // rows per work group
  static_assert(kRpw == attn_merge_rows_per_group(kBf16, D), "merge geometry");
  const int s = find_seq(a, blockIdx.x, true);
  const AttnSeqPlan sp = a.seqs[s];
  const int gpu = sp.tile_rows / kRpw;  // work groups per (q tile, kv head) unit
  const int lg = blockIdx.x - sp.merge_begin;
  const int nqt = (sp.num_q + sp.tokens_per_tile - 1) / sp.tokens_per_tile;
  const int unit = lg / gpu;
  const int qt = unit % nqt, g = unit / nqt;
  const int i0 = qt * sp.tokens_per_tile;
  const int nq = min(sp.tokens_per_tile, sp.num_q - i0);
  int lo_first, hi_first, lo_last, hi_last;
  key_bounds(sp.mode, sp.prefix_len, sp.num_q, a.window, i0, lo_first, hi_first);
  key_bounds(sp.mode, sp.prefix_len, sp.num_q, a.window, i0 + nq - 1, lo_last, hi_last);
  const int kt_lo = lo_first / kKT, kt_hi = hi_last / kKT;
  const int nonempty = min(sp.num_chunks, (kt_hi - kt_lo) / sp.chunk_tiles + 1);
  const int64_t prow0 = sp.part_begin + (int64_t)(g * nqt + qt) * sp.num_chunks * sp.tile_rows;

  const int row = (lg % gpu) * kRpw + threadIdx.x / kTpr;
  const int c = (threadIdx.x % kTpr) * kC;
  const int tok = i0 + row / a.group;
  const int head = g * a.group + row % a.group;
  if (tok >= sp.num_q) return;
  // batches of up to 8 chunks, all loads of a batch issued before first use; the
  // running reference mmax moves up between batches (acc and wsum are rescaled)
  constexpr int kB = 8;
  float mmax = kNegInf, wsum = 0.f;
  float acc[kC];
#pragma unroll
  for (int i = 0; i < kC; ++i) acc[i] = 0.f;
  const char* pbase = reinterpret_cast<const char*>(a.part_o);
  for (int j0 = 0; j0 < nonempty; j0 += kB) {
    float2 ml[kB];
    uint4 x[kB];
#pragma unroll
    for (int t = 0; t < kB; ++t) {
      const int64_t pr = prow0 + (int64_t)min(j0 + t, nonempty - 1) * sp.tile_rows + row;
      ml[t] = *reinterpret_cast<const float2*>(a.part_ml + pr * 2);
      x[t] = *reinterpret_cast<const uint4*>(pbase + (pr * D + c) * esz);
    }
    float bmax = mmax;
#pragma unroll
    for (int t = 0; t < kB; ++t)
      if (j0 + t < nonempty) bmax = fmaxf(bmax, ml[t].x);
    if (bmax != mmax) {  // mmax = -inf only before the first finite chunk (acc and wsum are 0)
      const float r = mmax == kNegInf ? 0.f : fast_exp2(mmax - bmax);
      wsum *= r;
#pragma unroll
      for (int i = 0; i < kC; ++i) acc[i] *= r;
      mmax = bmax;
    }
#pragma unroll
    for (int t = 0; t < kB; ++t) {
      const float f = (j0 + t >= nonempty || ml[t].x == kNegInf) ? 0.f : fast_exp2(ml[t].x - mmax) * ml[t].y;
      wsum += f;
      const uint32_t xw[4] = {x[t].x, x[t].y, x[t].z, x[t].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (kBf16) {
          acc[2 * i] = fmaf(f, __uint_as_float(xw[i] << 16), acc[2 * i]);
          acc[2 * i + 1] = fmaf(f, __uint_as_float(xw[i] & 0xffff0000u), acc[2 * i + 1]);
        } else {
          acc[i] = fmaf(f, __uint_as_float(xw[i]), acc[i]);
        }
      }
    }
  }
  const float inv = 1.f / wsum;
  char* orow = reinterpret_cast<char*>(a.out) + ((int64_t)(sp.q_start + tok) * a.hq + head) * D * esz + c * esz;
  uint32_t ow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (kBf16) ow[i] = pack_bf16(acc[2 * i] * inv, acc[2 * i + 1] * inv);
    else ow[i] = __float_as_uint(acc[i] * inv);
  }
  *reinterpret_cast<uint4*>(orow) = make_uint4(ow[0], ow[1], ow[2], ow[3]);
  if (a.lse && c == 0) a.lse[(int64_t)(sp.q_start + tok) * a.hq + head] = (mmax + __builtin_amdgcn_logf(wsum)) * kLn2;
}

// ---- bf16, head_dim 256: LDS-DMA ring kernel -------------------------------------
//
// The same work unit as attn_fwd (128 query rows x one key chunk), in 32-key
// sub-tiles, software-pipelined by one sub-tile: while the matrix cores compute
// S(j+1) = K(j+1) . Q^T, the vector units turn S(j) into P(j), and then
// O^T += V(j)^T . P(j)^T. K and V rows go from HBM straight to LDS
// through a 4-deep ring whose stage j holds K(j+1) and V(j), so every iteration reads
// exactly one stage while the next three are in flight. The copies are
// global_load_lds_dwordx4 (uniform 64-bit base, per-lane 32-bit offset).
//
// LDS layout: one DMA instruction writes 1 KB = 2 key rows; inside it, 16-byte chunk
// c of the row with parity p sits at slot 2c + p, and 2-row pairs are 1056 B (K) and
// 1152 B (V) apart. With these pitches the S^T operand reads (ds_read_b128, 32 rows x
// one chunk) and the V^T operand reads (ds_read_b64_tr_b16, 4 rows x 32 columns) hit
// 64 distinct banks, and every read address is a per-lane base plus an immediate.
// The V^T reads take keys 4h+0..3 and 8+4h+0..3 of each 16, the order in which the
// S^T accumulator holds P^T.
//
// Softmax: base 2 against a fixed reference per row, the max of the first sub-tile
// in which the row has a finite score (until then the row's O and sum are exactly
// zero). Later scores may exceed it: P = 2^(s - ref) then grows, which bf16 and the
// fp32 accumulators represent with the same relative precision, so O is never
// rescaled and its 128 accumulators stay in AGPRs, touched only by MFMAs. Should a
// score exceed the reference by more than 2^64 (beyond any practical attention
// logit spread, but possible for adversarial inputs), the work group recomputes the
// chunk with the largest score it saw as the new reference.

constexpr int kSub = 32;                         // keys per sub-tile
constexpr int kAttStages = 4;
constexpr int kKPitch = 1056;                    // bytes between K row pairs
constexpr int kVPitch = 1152;                    // bytes between V row pairs
constexpr int kKRegion = (kSub / 2) * kKPitch;   // 16896
constexpr int kVRegion = (kSub / 2) * kVPitch;   // 18432
constexpr int kAttStage = kKRegion + kVRegion;   // 35328; 4 stages = 138 KB
constexpr float kOverflow = 64.f;             // log2 headroom of the fixed reference

#define DG_ATT_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (7 << 4) | (15 << 8) | (((n) >> 4) << 14))
// The LDS reads are inline asm, whose results the compiler takes as ready at once:
// the fence keeps every use of them below the wait.
#define DG_ATT_WAIT_LGKM0()                                          \
  do {                                                               \
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14)); \
    __builtin_amdgcn_sched_barrier(0);                               \
  } while (0)

// Empty asm that takes a value: everything computing it stays above this point, so the
// compiler cannot sink the exps and sums that run under one phase's MFMAs into the next
// block (past a branch), where they would run with no MFMA beside them.
#define DG_ATT_ANCHOR(val) asm volatile("" ::"v"(val))
#define DG_ATT_ANCHOR4(u4) asm volatile("" ::"v"((u4).x), "v"((u4).y), "v"((u4).z), "v"((u4).w))

template <int I, int N>
struct StaticFor {
  template <class F>
  static __device__ __forceinline__ void run(F&& f) {
    f(std::integral_constant<int, I>{});
    StaticFor<I + 1, N>::run(f);
  }
};
template <int N>
struct StaticFor<N, N> {
  template <class F>
  static __device__ __forceinline__ void run(F&&) {}
};

template <int kOff>
__device__ __forceinline__ uint4 att_b128(uint32_t addr) {
  uint4 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(kOff) : "memory");
  return r;
}
template <int kOff>
__device__ __forceinline__ uint2 att_tr16(uint32_t addr) {
  uint2 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(kOff) : "memory");
  return r;
}

// max(a, b, c) in one instruction. fmaxf would also quiet signalling NaNs, which costs
// an extra instruction per operand on scores the compiler cannot prove canonical.
__device__ __forceinline__ float att_max3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
// max of the 16 entries and m
__device__ __forceinline__ float att_max16(const f32x16_t& sv, float m) {
  const float t0 = att_max3(sv[0], sv[1], sv[2]), t1 = att_max3(sv[3], sv[4], sv[5]);
  const float t2 = att_max3(sv[6], sv[7], sv[8]), t3 = att_max3(sv[9], sv[10], sv[11]);
  const float t4 = att_max3(sv[12], sv[13], sv[14]);
  return att_max3(att_max3(t0, t1, t2), att_max3(t3, t4, sv[15]), m);
}

// Both halves of the wave get f(x[lane % 32], x[lane % 32 + 32]).
__device__ __forceinline__ float half_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Work groups are dealt round-robin to the 8 XCDs. Renumber them so that each XCD takes
// runs of kXcdRun consecutive work items (the q tiles of one key chunk read the same K/V,
// which its L2 then serves once), while all XCDs walk the work list together from its
// start: long and short requests spread evenly over the XCDs. Blocks of the last partial
// round keep their launch order.
constexpr int kXcdRun = 4;
__device__ __forceinline__ int xcd_order(int b, int n) {
  constexpr int kRound = 8 * kXcdRun;
  if (b >= n / kRound * kRound) return b;
  return b / kRound * kRound + (b & 7) * kXcdRun + (b >> 3) % kXcdRun;
}

template <bool kPaged>
__global__ __launch_bounds__(kThreads) void attn_fwd_bf16_d256(AttnArgs a) {
  constexpr int D = 256, KS = 16, DB = 8;
  __shared__ __attribute__((aligned(1024))) char lds[kAttStages * kAttStage];
  __shared__ int redo_flag[1];  // set by a wave that saw a score past the reference

  const int w = a.work_offset + xcd_order(blockIdx.x, gridDim.x);
  const int s_ = find_seq(a, w, false);
  const AttnSeqPlan sp = a.seqs[s_];
  const int nqt = (sp.num_q + sp.tokens_per_tile - 1) / sp.tokens_per_tile;
  const int local = w - sp.work_begin;
  // items [key chunk][kv head][q tile]: the q tiles of one (chunk, head) are consecutive,
  // and a run of xcd_order's deal covers one head, so an XCD keeps to few heads' Q. A
  // causal request's later q tiles see more keys: they come first, so that the long
  // items of every chunk start early and short ones fill in behind them.
  const int qt = sp.mode == DG_CAUSAL ? nqt - 1 - local % nqt : local % nqt;
  const int rest = local / nqt;
  const int g = rest % a.hkv;
  const int chunk = rest / a.hkv;
  const int i0 = qt * sp.tokens_per_tile;
  const int nq = min(sp.tokens_per_tile, sp.num_q - i0);
  const int nkeys = sp.prefix_len + sp.num_q;
  int lo_first, hi_first, lo_last, hi_last;
  key_bounds(sp.mode, sp.prefix_len, sp.num_q, a.window, i0, lo_first, hi_first);
  key_bounds(sp.mode, sp.prefix_len, sp.num_q, a.window, i0 + nq - 1, lo_last, hi_last);
  const int kt_lo = lo_first / kKT, kt_hi = hi_last / kKT;
  const int t_begin = kt_lo + chunk * sp.chunk_tiles;
  const int t_end = min(kt_hi + 1, t_begin + sp.chunk_tiles);
  if (t_begin > kt_hi) return;  // empty chunk (uniform across the work group)
  const int key0 = t_begin * kKT;
  const int kend = min(t_end * kKT, hi_last + 1);  // <= nkeys
  const int nsub = (kend - key0 + kSub - 1) / kSub;  // >= 1

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  const int row = wave * 32 + l32;
  const int tok = i0 + row / a.group;
  const int head = g * a.group + row % a.group;
  const bool valid = tok < sp.num_q;
  int lo = 0, hi = -1;
  if (valid) key_bounds(sp.mode, sp.prefix_len, sp.num_q, a.window, tok, lo, hi);

  uint4 qf[KS];
  {
    const char* qrow = reinterpret_cast<const char*>(a.q) + ((int64_t)(sp.q_start + tok) * a.hq + head) * D * 2;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[ks] = valid ? *reinterpret_cast<const uint4*>(qrow + (16 * ks + 8 * hh) * 2) : make_uint4(0, 0, 0, 0);
  }

  // ---- DMA: wave w fills pairs 4w..4w+3 of the K and V regions; lane i loads
  // chunk i/2 of key row 2*pair + i%2 (per-request byte offsets fit in 32 bits).
  const int rs = a.hkv * D * 2;  // bytes between consecutive keys
  const int64_t head_off = (int64_t)g * D * 2;
  const char* kb = reinterpret_cast<const char*>(a.k) + head_off;
  const char* vb = reinterpret_cast<const char*>(a.v) + head_off;
  uint32_t vo[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) vo[t] = (2 * (4 * wave + t) + (lane & 1)) * rs + (lane >> 1) * 16;
  typedef __attribute__((address_space(3))) char lds_char;
  lds_char* lds0 = (lds_char*)lds;
  // rows kbase .. kbase+31 into the K or V region at `dst` (uniform base + per-lane
  // 32-bit offset); rows past the request's last key repeat that key (they are masked)
  auto dma_rows = [&](const char* base, lds_char* dst, int pitch, int kbase) {
    const char* src = base + key_row<kPaged>(a, sp, kbase) * rs;
    if (kbase + kSub <= nkeys) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
        __builtin_amdgcn_global_load_lds((const void*)(src + vo[t]),
                                         (__attribute__((address_space(3))) void*)(dst + (4 * wave + t) * pitch), 16, 0, 0);
    } else {
      const int last = nkeys - 1 - kbase;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint32_t r = min(2 * (4 * wave + t) + (lane & 1), last);
        __builtin_amdgcn_global_load_lds((const void*)(src + (r * rs + (lane >> 1) * 16)),
                                         (__attribute__((address_space(3))) void*)(dst + (4 * wave + t) * pitch), 16, 0, 0);
      }
    }
  };
  // stage j: K of sub-tile j+1 and V of j; stages past the chunk's last sub-tile repeat
  // it (never read: they keep every iteration's count of copies the same)
  auto issue = [&](int j) {
    lds_char* st = lds0 + (j & 3) * kAttStage;
    dma_rows(kb, st, kKPitch, key0 + kSub * min(j + 1, nsub - 1));
    dma_rows(vb, st + kKRegion, kVPitch, key0 + kSub * min(j, nsub - 1));
  };

  // ---- LDS read addresses: per-lane base + immediates
  const uint32_t lbase = (uint32_t)(uintptr_t)lds0;
  const uint32_t k_lane = (l32 >> 1) * kKPitch + 16 * (l32 & 1) + 32 * hh;  // + 64*ks
  const int grp = lane >> 4, s16 = lane & 15;
  const int vrow = 4 * (grp >> 1) + (s16 >> 2);  // + 8q + 16 half
  const int vcol = 16 * (grp & 1) + 4 * (s16 & 3);  // + 32 b
  const uint32_t v_lane = kKRegion + (vrow >> 1) * kVPitch + 16 * (vrow & 1) + 32 * (vcol >> 3) + 2 * (vcol & 7);

  // mask S(j) where some row's bounds cut sub-tile j
  auto mask = [&](f32x16_t& sv, int kbase) {
    if (!(lo_last <= kbase && kbase + kSub - 1 <= hi_first)) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = kbase + 8 * (e >> 2) + 4 * hh + (e & 3);
        if (key < lo || key > hi) sv[e] = kNegInf;
      }
    }
  };
  // ... and its row max (scaled)
  auto front = [&](f32x16_t& sv, int kbase) {
    mask(sv, kbase);
    float t = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])), fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
    t = fmaxf(t, fmaxf(fmaxf(fmaxf(sv[8], sv[9]), fmaxf(sv[10], sv[11])), fmaxf(fmaxf(sv[12], sv[13]), fmaxf(sv[14], sv[15]))));
    return half_max(t) * a.scale_log2;
  };

  f32x16_t o[DB];
  float l_run;
  float m_ref = kNegInf;  // fixed reference (scaled log2 units) of this lane's row
  for (;;) {
    if (tid == 0) redo_flag[0] = 0;
    // ---- prologue: K(0) into the K region of slot 3, stages 0..2, then S(0)
    dma_rows(kb, lds0 + 3 * kAttStage, kKPitch, key0);
    issue(0);
    issue(1);
    issue(2);
    DG_ATT_WAIT_VM(24);  // K(0) landed
    DG_ATT_WAIT_LGKM0();
    __builtin_amdgcn_s_barrier();
    f32x16_t scur;
    {
      const uint32_t ka = lbase + 3 * kAttStage + k_lane;
      uint4 kf[KS];
      StaticFor<0, KS>::run([&](auto ks) { kf[ks] = att_b128<64 * decltype(ks)::value>(ka); });
      DG_ATT_WAIT_LGKM0();
#pragma unroll
      for (int e = 0; e < 16; ++e) scur[e] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        scur = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, kf[ks]),
                                                       __builtin_bit_cast(bf16x8_t, qf[ks]), scur, 0, 0, 0);
    }
    float m_seen = front(scur, key0);
    if (m_ref == kNegInf) m_ref = m_seen;  // on a retry m_ref already covers this sub-tile
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[b][e] = 0.f;
    l_run = 0.f;

    bool overflow = false;
    for (int sub = 0; sub < nsub; ++sub) {
      // every iteration (and the prologue, per stage) issues one stage of copies, so two
      // stages are younger than stage sub here
      DG_ATT_WAIT_VM(16);
      __builtin_amdgcn_s_barrier();  // stage sub landed for every wave; slot of sub-1 is free
      __builtin_amdgcn_sched_barrier(0);
      const uint32_t ka = lbase + (sub & 3) * kAttStage + k_lane;
      const uint32_t va = lbase + (sub & 3) * kAttStage + v_lane;
      const float mu = m_ref == kNegInf ? 0.f : m_ref;
      const bool has_next = sub + 1 < nsub;  // uniform
      // The refill below (stage sub+3 into the slot of sub-1; past the last sub-tile it
      // repeats that sub-tile's rows into the slot, which nothing reads again), addressed
      // once here: row bases (the K reads' wait also covers a table load), the LDS slot
      // and per-lane 32-bit offsets, which are vo except in a request's last sub-tile,
      // whose rows past the last key repeat it.
      const int kkb = key0 + kSub * min(sub + 4, nsub - 1), vkb = key0 + kSub * min(sub + 3, nsub - 1);
      const char* rk = kb + key_row<kPaged>(a, sp, kkb) * rs;
      const char* rv = vb + key_row<kPaged>(a, sp, vkb) * rs;
      lds_char* rst = lds0 + ((sub + 3) & 3) * kAttStage;
      uint32_t ko[4], vv[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) ko[t] = vv[t] = vo[t];
      if (kkb + kSub > nkeys || vkb + kSub > nkeys) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int r = 2 * (4 * wave + t) + (lane & 1);
          ko[t] = (uint32_t)min(r, nkeys - 1 - kkb) * rs + (lane >> 1) * 16;
          vv[t] = (uint32_t)min(r, nkeys - 1 - vkb) * rs + (lane >> 1) * 16;
        }
      }

      uint4 kf[KS];
      uint2 v0[DB][2], v1[DB][2];
      StaticFor<0, 8>::run([&](auto ks) { kf[ks] = att_b128<64 * decltype(ks)::value>(ka); });
      DG_ATT_WAIT_LGKM0();

      // S(sub+1) k-steps 0..7 with K reads 8..15, the V^T reads of keys 0..15 and the
      // probabilities P(sub) of keys 0..15
      f32x16_t snxt;
#pragma unroll
      for (int e = 0; e < 16; ++e) snxt[e] = 0.f;
      float p[16];
      StaticFor<0, 8>::run([&](auto ic) {
        constexpr int ks = decltype(ic)::value;
        snxt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, kf[ks]),
                                                       __builtin_bit_cast(bf16x8_t, qf[ks]), snxt, 0, 0, 0);
        kf[ks + 8] = att_b128<64 * (ks + 8)>(ka);
        v0[ks][0] = att_tr16<128 * ks>(va);
        v0[ks][1] = att_tr16<128 * ks + 4 * kVPitch>(va);
        p[ks] = fast_exp2(fmaf(scur[ks], a.scale_log2, -mu));
        l_run += p[ks];
        __builtin_amdgcn_sched_barrier(0);
      });
      uint4 pf[2];
      pf[0] = make_uint4(pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3]), pack_bf16(p[4], p[5]), pack_bf16(p[6], p[7]));
      DG_ATT_ANCHOR(l_run);
      DG_ATT_WAIT_LGKM0();

      // O^T += V^T(keys 0..15) . P^T and S(sub+1) k-steps 8..15, with the V^T reads of
      // keys 16..31, P(sub) of keys 16..31, and the refill of the ring slot of sub-1
      {
        StaticFor<0, DB>::run([&](auto ic) {
          constexpr int b = decltype(ic)::value;
          o[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8_t, make_uint4(v0[b][0].x, v0[b][0].y, v0[b][1].x, v0[b][1].y)),
              __builtin_bit_cast(bf16x8_t, pf[0]), o[b], 0, 0, 0);
          snxt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, kf[8 + b]),
                                                         __builtin_bit_cast(bf16x8_t, qf[8 + b]), snxt, 0, 0, 0);
          v1[b][0] = att_tr16<128 * b + 8 * kVPitch>(va);
          v1[b][1] = att_tr16<128 * b + 12 * kVPitch>(va);
          {  // DMA b: K pairs 0..3, then V pairs 0..3
            if constexpr (b < 4)
              __builtin_amdgcn_global_load_lds((const void*)(rk + ko[b]),
                                               (__attribute__((address_space(3))) void*)(rst + (4 * wave + b) * kKPitch),
                                               16, 0, 0);
            else
              __builtin_amdgcn_global_load_lds(
                  (const void*)(rv + vv[b - 4]),
                  (__attribute__((address_space(3))) void*)(rst + kKRegion + (4 * wave + b - 4) * kVPitch), 16, 0, 0);
          }
          p[8 + b] = fast_exp2(fmaf(scur[8 + b], a.scale_log2, -mu));
          l_run += p[8 + b];
          __builtin_amdgcn_sched_barrier(0);
        });
      }
      pf[1] = make_uint4(pack_bf16(p[8], p[9]), pack_bf16(p[10], p[11]), pack_bf16(p[12], p[13]),
                         pack_bf16(p[14], p[15]));
      DG_ATT_ANCHOR4(pf[1]);
      DG_ATT_ANCHOR(l_run);
      DG_ATT_WAIT_LGKM0();

      // O^T += V^T(keys 16..31) . P^T, with the next sub-tile's mask, row max and
      // reference (S(sub+1) is complete) between the MFMAs
      if (has_next) mask(snxt, key0 + kSub * (sub + 1));
      float t4[4], tmax = kNegInf;
      StaticFor<0, DB>::run([&](auto ic) {
        constexpr int b = decltype(ic)::value;
        o[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8_t, make_uint4(v1[b][0].x, v1[b][0].y, v1[b][1].x, v1[b][1].y)),
            __builtin_bit_cast(bf16x8_t, pf[1]), o[b], 0, 0, 0);
        if constexpr (b < 4) t4[b] = fmaxf(fmaxf(snxt[4 * b], snxt[4 * b + 1]), fmaxf(snxt[4 * b + 2], snxt[4 * b + 3]));
        if (b == 4) tmax = fmaxf(fmaxf(t4[0], t4[1]), fmaxf(t4[2], t4[3]));
        if (b == 5) tmax = half_max(tmax) * a.scale_log2;
        if (b == 6 && has_next) {
          m_seen = fmaxf(m_seen, tmax);
          if (m_ref == kNegInf) m_ref = tmax;
          overflow |= tmax > m_ref + kOverflow;
        }
        __builtin_amdgcn_sched_barrier(0);
      });
      scur = snxt;
    }
    // the ring drains (the last stages' repeated copies too) before the barrier below,
    // after which the LDS is free; a rare overflow anywhere redoes the chunk
    DG_ATT_WAIT_VM(0);
    if (__any(overflow) && lane == 0) redo_flag[0] = 1;
    __syncthreads();
    const int redo = redo_flag[0];
    if (!redo) break;
    __syncthreads();  // every wave has read the flag before it is cleared
    m_ref = fmaxf(m_ref, m_seen);
  }

  // ---- epilogue: O (normalised, bf16) goes through LDS, the ring being free after the
  // loop's final barrier, so that the global stores are whole rows: each wave stages its
  // 32 rows at a 528-byte pitch, then writes 2 rows (1 KB) per store.
  // o[b][e] = O^T[d = 32b + 8(e/4) + 4hh + e%4][this lane's row]
  constexpr int kOPitch = 528;
  char* ost = lds + wave * 32 * kOPitch;
  const float l_tot = half_sum(l_run);
  {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    char* orow = ost + l32 * kOPitch;
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4)
        *reinterpret_cast<uint2*>(orow + (32 * b + 8 * e4 + 4 * hh) * 2) =
            make_uint2(pack_bf16(o[b][4 * e4] * inv, o[b][4 * e4 + 1] * inv),
                       pack_bf16(o[b][4 * e4 + 2] * inv, o[b][4 * e4 + 3] * inv));
  }
  const int64_t prow0 = sp.part_begin + ((int64_t)(g * nqt + qt) * sp.num_chunks + chunk) * kRows;
  if (valid && hh == 0) {
    if (sp.num_chunks > 1)
      *reinterpret_cast<float2*>(a.part_ml + (prow0 + row) * 2) = make_float2(m_ref, l_tot);
    else if (a.lse)
      a.lse[(int64_t)(sp.q_start + tok) * a.hq + head] = (m_ref + __builtin_amdgcn_logf(l_tot)) * kLn2;
  }
  DG_ATT_WAIT_LGKM0();  // this wave's rows are in LDS (each wave reads only its own)
  // store r covers rows 2r, 2r+1 of this wave: lane i takes 16 bytes i%32 of row 2r + i/32
#pragma unroll 4
  for (int r = 0; r < 16; ++r) {
    const int lr = 2 * r + hh;  // local row 0..31
    const int srow = wave * 32 + lr, stok = i0 + srow / a.group, shead = g * a.group + srow % a.group;
    const uint4 x = *reinterpret_cast<const uint4*>(ost + lr * kOPitch + l32 * 16);
    if (stok >= sp.num_q) continue;
    char* dst = sp.num_chunks == 1
                    ? reinterpret_cast<char*>(a.out) + ((int64_t)(sp.q_start + stok) * a.hq + shead) * D * 2
                    : reinterpret_cast<char*>(a.part_o) + (prow0 + srow) * D * 2;
    *reinterpret_cast<uint4*>(dst + l32 * 16) = x;
  }
}

// ---- FP8 (E4M3) K/V, head_dim 256: the 128-row LDS-DMA kernel over codes ---------
//
// attn_fwd_bf16_d256 with the K/V ring holding E4M3 codes: a stage is half the bytes,
// the copies and the LDS fragment reads halve, and each fragment is widened to bf16
// after its read (v_cvt_scalef32_pk_bf16_fp8 at scale 1: every E4M3 value is a bf16
// value, so the widening is exact), feeding the same bf16 MFMAs. k_scale is folded
// into the score scale and v_scale into the output normalisation.
//
// LDS layout: one copy instruction writes 1 KB = 4 key rows of 256 codes, 16-byte chunk
// c of row r at slot 4c + r; blocks of 4 rows are 1088 B (K) and 1056 B (V) apart.
// - K operand: one ds_read_b128 per lane and pair of k-steps (16 codes of its key). So
//   that it feeds both steps, the contraction runs over the head dims in a permuted
//   order: k-step 2j + u takes dims 32j + 16h + 8u .. +7 in the lane half h (Q's
//   fragments are loaded in the same order). 8 lanes of a read hit 8 distinct 16-byte
//   bank groups.
// - V^T operand: one ds_read_b64_tr_b8 per fragment. In each 16-lane group the read
//   returns to lane j byte j % 8 of the 8 bytes that lane 2r + j / 8 addressed, as byte
//   r (r = 0..7). A lane of group g (half h = g / 2) addresses 8 codes of key
//   (4h + r', then 8 + 4h + r' - 4) at dims 32b + 16 (g % 2) + 8 (lane % 2), which gives
//   lane (row, h) the codes of its P^T keys in order, at dim 32b + row. The two blocks a
//   group touches are 2 apart, 64 bytes apart in the banks: no conflicts.

constexpr int kF8KPitch = 1088;                     // bytes between K blocks of 4 rows
constexpr int kF8VPitch = 1056;                     // bytes between V blocks
constexpr int kF8KRegion = (kSub / 4) * kF8KPitch;  // 8704
constexpr int kF8VRegion = (kSub / 4) * kF8VPitch;  // 8448
constexpr int kF8Stage = kF8KRegion + kF8VRegion;   // 17152; 4 stages = 67 KB

template <int kOff>
__device__ __forceinline__ uint2 att_tr8(uint32_t addr) {
  uint2 r;
  asm volatile("ds_read_b64_tr_b8 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(kOff) : "memory");
  return r;
}
// 8 E4M3 codes (bytes of lo, then hi) -> 8 bf16, in order
__device__ __forceinline__ uint4 widen_e4m3(uint32_t lo, uint32_t hi) {
  return make_uint4(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true)));
}

template <bool kPaged>
__global__ __launch_bounds__(kThreads) void attn_fwd_fp8_d256(AttnArgs a) {
  constexpr int D = 256, KS = 16, DB = 8;
  __shared__ __attribute__((aligned(1024))) char lds[kAttStages * kF8Stage];
  __shared__ int redo_flag[1];

  const int w = a.work_offset + xcd_order(blockIdx.x, gridDim.x);
  const int s_ = find_seq(a, w, false);
  const AttnSeqPlan sp = a.seqs[s_];
  const int nqt = (sp.num_q + sp.tokens_per_tile - 1) / sp.tokens_per_tile;
  const int local = w - sp.work_begin;
  const int qt = sp.mode == DG_CAUSAL ? nqt - 1 - local % nqt : local % nqt;
  const int rest = local / nqt;
  const int g = rest % a.hkv;
  const int chunk = rest / a.hkv;
  const int i0 = qt * sp.tokens_per_tile;
  const int nq = min(sp.tokens_per_tile, sp.num_q - i0);
  const int nkeys = sp.prefix_len + sp.num_q;
  int lo_first, hi_first, lo_last, hi_last;
  key_bounds(sp.mode, sp.prefix_len, sp.num_q, a.window, i0, lo_first, hi_first);
  key_bounds(sp.mode, sp.prefix_len, sp.num_q, a.window, i0 + nq - 1, lo_last, hi_last);
  const int kt_lo = lo_first / kKT, kt_hi = hi_last / kKT;
  const int t_begin = kt_lo + chunk * sp.chunk_tiles;
  const int t_end = min(kt_hi + 1, t_begin + sp.chunk_tiles);
  if (t_begin > kt_hi) return;  // empty chunk (uniform across the work group)
  const int key0 = t_begin * kKT;
  const int kend = min(t_end * kKT, hi_last + 1);
  const int nsub = (kend - key0 + kSub - 1) / kSub;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  const int row = wave * 32 + l32;
  const int tok = i0 + row / a.group;
  const int head = g * a.group + row % a.group;
  const bool valid = tok < sp.num_q;
  int lo = 0, hi = -1;
  if (valid) key_bounds(sp.mode, sp.prefix_len, sp.num_q, a.window, tok, lo, hi);

  // Q^T fragments in the permuted dim order of the K reads
  uint4 qf[KS];
  {
    const char* qrow = reinterpret_cast<const char*>(a.q) + ((int64_t)(sp.q_start + tok) * a.hq + head) * D * 2;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[ks] = valid ? *reinterpret_cast<const uint4*>(qrow + (32 * (ks >> 1) + 16 * hh + 8 * (ks & 1)) * 2)
                     : make_uint4(0, 0, 0, 0);
  }

  // ---- DMA: wave w fills blocks 2w, 2w+1 of the K and V regions; lane i loads chunk
  // i/4 of key row 4*block + i%4
  const int rs = a.hkv * D;  // bytes between consecutive keys
  const int64_t head_off = (int64_t)g * D;
  const char* kb = reinterpret_cast<const char*>(a.k) + head_off;
  const char* vb = reinterpret_cast<const char*>(a.v) + head_off;
  uint32_t vo[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) vo[u] = (4 * (2 * wave + u) + (lane & 3)) * rs + (lane >> 2) * 16;
  typedef __attribute__((address_space(3))) char lds_char;
  lds_char* lds0 = (lds_char*)lds;
  auto dma_rows = [&](const char* base, lds_char* dst, int pitch, int kbase) {
    const char* src = base + key_row<kPaged>(a, sp, kbase) * rs;
    const int last = nkeys - 1 - kbase;  // rows past the request's last key repeat it (masked)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const uint32_t off =
          kbase + kSub <= nkeys ? vo[u] : (uint32_t)min(4 * (2 * wave + u) + (lane & 3), last) * rs + (lane >> 2) * 16;
      __builtin_amdgcn_global_load_lds((const void*)(src + off),
                                       (__attribute__((address_space(3))) void*)(dst + (2 * wave + u) * pitch), 16, 0, 0);
    }
  };
  // stage j: K of sub-tile j+1 and V of j (past the chunk's last sub-tile: repeats)
  auto issue = [&](int j) {
    lds_char* st = lds0 + (j & 3) * kF8Stage;
    dma_rows(kb, st, kF8KPitch, key0 + kSub * min(j + 1, nsub - 1));
    dma_rows(vb, st + kF8KRegion, kF8VPitch, key0 + kSub * min(j, nsub - 1));
  };

  // ---- LDS read addresses: per-lane base + immediates
  const uint32_t lbase = (uint32_t)(uintptr_t)lds0;
  const uint32_t k_lane = (l32 >> 2) * kF8KPitch + 16 * (l32 & 3) + 64 * hh;  // + 128 j
  const int grp = lane >> 4, s16 = lane & 15;
  const int kr = (s16 >> 1) < 4 ? 4 * (grp >> 1) + (s16 >> 1) : 8 + 4 * (grp >> 1) + (s16 >> 1) - 4;  // key 0..15
  const uint32_t v_lane =
      kF8KRegion + (kr >> 2) * kF8VPitch + 16 * (kr & 3) + 64 * (grp & 1) + 8 * (s16 & 1);  // + 128 b + 4 kh V blocks

  auto mask = [&](f32x16_t& sv, int kbase) {
    if (!(lo_last <= kbase && kbase + kSub - 1 <= hi_first)) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = kbase + 8 * (e >> 2) + 4 * hh + (e & 3);
        if (key < lo || key > hi) sv[e] = kNegInf;
      }
    }
  };
  auto front = [&](f32x16_t& sv, int kbase) {
    mask(sv, kbase);
    float t = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])), fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
    t = fmaxf(t, fmaxf(fmaxf(fmaxf(sv[8], sv[9]), fmaxf(sv[10], sv[11])), fmaxf(fmaxf(sv[12], sv[13]), fmaxf(sv[14], sv[15]))));
    return half_max(t) * a.scale_log2;
  };
  // bf16 operand of k-step ks from the K read of its pair
  auto kop = [](const uint4& k, int u) { return u == 0 ? widen_e4m3(k.x, k.y) : widen_e4m3(k.z, k.w); };

  f32x16_t o[DB];
  float l_run;
  float m_ref = kNegInf;
  for (;;) {
    if (tid == 0) redo_flag[0] = 0;
    // ---- prologue: K(0) into the K region of slot 3, stages 0..2, then S(0)
    dma_rows(kb, lds0 + 3 * kF8Stage, kF8KPitch, key0);
    issue(0);
    issue(1);
    issue(2);
    DG_ATT_WAIT_VM(12);  // K(0) landed
    DG_ATT_WAIT_LGKM0();
    __builtin_amdgcn_s_barrier();
    f32x16_t scur;
    {
      const uint32_t ka = lbase + 3 * kF8Stage + k_lane;
      uint4 k8[KS / 2];
      StaticFor<0, KS / 2>::run([&](auto j) { k8[j] = att_b128<128 * decltype(j)::value>(ka); });
      DG_ATT_WAIT_LGKM0();
#pragma unroll
      for (int e = 0; e < 16; ++e) scur[e] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        scur = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, kop(k8[ks >> 1], ks & 1)),
                                                       __builtin_bit_cast(bf16x8_t, qf[ks]), scur, 0, 0, 0);
    }
    float m_seen = front(scur, key0);
    if (m_ref == kNegInf) m_ref = m_seen;  // on a retry m_ref already covers this sub-tile
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[b][e] = 0.f;
    l_run = 0.f;

    bool overflow = false;
    for (int sub = 0; sub < nsub; ++sub) {
      // one stage of copies per iteration (and per prologue stage): two stages are
      // younger than stage sub here
      DG_ATT_WAIT_VM(8);
      __builtin_amdgcn_s_barrier();  // stage sub landed for every wave; slot of sub-1 is free
      __builtin_amdgcn_sched_barrier(0);
      const uint32_t ka = lbase + (sub & 3) * kF8Stage + k_lane;
      const uint32_t va = lbase + (sub & 3) * kF8Stage + v_lane;
      const float mu = m_ref == kNegInf ? 0.f : m_ref;
      const bool has_next = sub + 1 < nsub;  // uniform
      // refill of stage sub+3 into the slot of sub-1, addressed once here
      const int kkb = key0 + kSub * min(sub + 4, nsub - 1), vkb = key0 + kSub * min(sub + 3, nsub - 1);
      const char* rk = kb + key_row<kPaged>(a, sp, kkb) * rs;
      const char* rv = vb + key_row<kPaged>(a, sp, vkb) * rs;
      lds_char* rst = lds0 + ((sub + 3) & 3) * kF8Stage;
      uint32_t ko[2], vv[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) ko[u] = vv[u] = vo[u];
      if (kkb + kSub > nkeys || vkb + kSub > nkeys) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int r = 4 * (2 * wave + u) + (lane & 3);
          ko[u] = (uint32_t)min(r, nkeys - 1 - kkb) * rs + (lane >> 2) * 16;
          vv[u] = (uint32_t)min(r, nkeys - 1 - vkb) * rs + (lane >> 2) * 16;
        }
      }

      uint4 k8[KS / 2];
      uint2 v0[DB], v1[DB];
      StaticFor<0, 4>::run([&](auto j) { k8[j] = att_b128<128 * decltype(j)::value>(ka); });
      DG_ATT_WAIT_LGKM0();

      // S(sub+1) k-steps 0..7 with K reads of pairs 4..7, the V^T reads of keys 0..15
      // and P(sub) of keys 0..15
      f32x16_t snxt;
#pragma unroll
      for (int e = 0; e < 16; ++e) snxt[e] = 0.f;
      float p[16];
      StaticFor<0, 8>::run([&](auto ic) {
        constexpr int ks = decltype(ic)::value;
        snxt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, kop(k8[ks >> 1], ks & 1)),
                                                       __builtin_bit_cast(bf16x8_t, qf[ks]), snxt, 0, 0, 0);
        if constexpr ((ks & 1) == 0) k8[4 + (ks >> 1)] = att_b128<128 * (4 + (ks >> 1))>(ka);
        v0[ks] = att_tr8<128 * ks>(va);
        p[ks] = fast_exp2(fmaf(scur[ks], a.scale_log2, -mu));
        l_run += p[ks];
        __builtin_amdgcn_sched_barrier(0);
      });
      uint4 pf[2];
      pf[0] = make_uint4(pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3]), pack_bf16(p[4], p[5]), pack_bf16(p[6], p[7]));
      DG_ATT_ANCHOR(l_run);
      DG_ATT_WAIT_LGKM0();

      // O^T += V^T(keys 0..15) . P^T and S(sub+1) k-steps 8..15, with the V^T reads of
      // keys 16..31, P(sub) of keys 16..31, and the refill of the ring slot of sub-1
      StaticFor<0, DB>::run([&](auto ic) {
        constexpr int b = decltype(ic)::value;
        o[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, widen_e4m3(v0[b].x, v0[b].y)),
                                                       __builtin_bit_cast(bf16x8_t, pf[0]), o[b], 0, 0, 0);
        snxt = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8_t, kop(k8[4 + (b >> 1)], b & 1)), __builtin_bit_cast(bf16x8_t, qf[8 + b]), snxt,
            0, 0, 0);
        v1[b] = att_tr8<128 * b + 4 * kF8VPitch>(va);
        if constexpr (b < 2)
          __builtin_amdgcn_global_load_lds((const void*)(rk + ko[b]),
                                           (__attribute__((address_space(3))) void*)(rst + (2 * wave + b) * kF8KPitch),
                                           16, 0, 0);
        else if constexpr (b < 4)
          __builtin_amdgcn_global_load_lds(
              (const void*)(rv + vv[b - 2]),
              (__attribute__((address_space(3))) void*)(rst + kF8KRegion + (2 * wave + b - 2) * kF8VPitch), 16, 0, 0);
        p[8 + b] = fast_exp2(fmaf(scur[8 + b], a.scale_log2, -mu));
        l_run += p[8 + b];
        __builtin_amdgcn_sched_barrier(0);
      });
      pf[1] = make_uint4(pack_bf16(p[8], p[9]), pack_bf16(p[10], p[11]), pack_bf16(p[12], p[13]),
                         pack_bf16(p[14], p[15]));
      DG_ATT_ANCHOR4(pf[1]);
      DG_ATT_ANCHOR(l_run);
      DG_ATT_WAIT_LGKM0();

      // O^T += V^T(keys 16..31) . P^T, with the next sub-tile's mask, row max and
      // reference between the MFMAs
      if (has_next) mask(snxt, key0 + kSub * (sub + 1));
      float t4[4], tmax = kNegInf;
      StaticFor<0, DB>::run([&](auto ic) {
        constexpr int b = decltype(ic)::value;
        o[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, widen_e4m3(v1[b].x, v1[b].y)),
                                                       __builtin_bit_cast(bf16x8_t, pf[1]), o[b], 0, 0, 0);
        if constexpr (b < 4) t4[b] = fmaxf(fmaxf(snxt[4 * b], snxt[4 * b + 1]), fmaxf(snxt[4 * b + 2], snxt[4 * b + 3]));
        if (b == 4) tmax = fmaxf(fmaxf(t4[0], t4[1]), fmaxf(t4[2], t4[3]));
        if (b == 5) tmax = half_max(tmax) * a.scale_log2;
        if (b == 6 && has_next) {
          m_seen = fmaxf(m_seen, tmax);
          if (m_ref == kNegInf) m_ref = tmax;
          overflow |= tmax > m_ref + kOverflow;
        }
        __builtin_amdgcn_sched_barrier(0);
      });
      scur = snxt;
    }
    DG_ATT_WAIT_VM(0);
    if (__any(overflow) && lane == 0) redo_flag[0] = 1;
    __syncthreads();
    const int redo = redo_flag[0];
    if (!redo) break;
    __syncthreads();  // every wave has read the flag before it is cleared
    m_ref = fmaxf(m_ref, m_seen);
  }

  // ---- epilogue (as attn_fwd_bf16_d256, with v_scale in the normalisation)
  constexpr int kOPitch = 528;
  char* ost = lds + wave * 32 * kOPitch;
  const float l_tot = half_sum(l_run);
  {
    const float inv = (l_tot > 0.f ? 1.f / l_tot : 0.f) * a.v_scale;
    char* orow = ost + l32 * kOPitch;
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4)
        *reinterpret_cast<uint2*>(orow + (32 * b + 8 * e4 + 4 * hh) * 2) =
            make_uint2(pack_bf16(o[b][4 * e4] * inv, o[b][4 * e4 + 1] * inv),
                       pack_bf16(o[b][4 * e4 + 2] * inv, o[b][4 * e4 + 3] * inv));
  }
  const int64_t prow0 = sp.part_begin + ((int64_t)(g * nqt + qt) * sp.num_chunks + chunk) * kRows;
  if (valid && hh == 0) {
    if (sp.num_chunks > 1)
      *reinterpret_cast<float2*>(a.part_ml + (prow0 + row) * 2) = make_float2(m_ref, l_tot);
    else if (a.lse)
      a.lse[(int64_t)(sp.q_start + tok) * a.hq + head] = (m_ref + __builtin_amdgcn_logf(l_tot)) * kLn2;
  }
  DG_ATT_WAIT_LGKM0();
#pragma unroll 4
  for (int r = 0; r < 16; ++r) {
    const int lr = 2 * r + hh;
    const int srow = wave * 32 + lr, stok = i0 + srow / a.group, shead = g * a.group + srow % a.group;
    const uint4 x = *reinterpret_cast<const uint4*>(ost + lr * kOPitch + l32 * 16);
    if (stok >= sp.num_q) continue;
    char* dst = sp.num_chunks == 1
                    ? reinterpret_cast<char*>(a.out) + ((int64_t)(sp.q_start + stok) * a.hq + shead) * D * 2
                    : reinterpret_cast<char*>(a.part_o) + (prow0 + srow) * D * 2;
    *reinterpret_cast<uint4*>(dst + l32 * 16) = x;
  }
}

// ---- bf16, head_dim 256, 64 query rows per wave ---------------------------------
//
// The ring, LDS layout and copies of attn_fwd_bf16_d256, with each wave owning 64
// query rows (two 32-row halves), so that every K and V^T fragment read from LDS feeds
// two MFMAs; a work group covers 256 rows. Per 32-key sub-tile j a wave computes
// S(j+1) = K(j+1) . Q^T for both halves (32 MFMAs, K fragments streamed from LDS four
// ahead, the ring refill interleaved), then O^T += V(j)^T . P(j)^T (32 MFMAs, V^T
// fragments two ahead) while the vector units turn S(j+1) into P(j+1). O (2 x 128
// accumulators) fills the AGPRs; Q^T (128), S (32) and the two P buffers (32) stay in
// VGPRs. Softmax, reference and overflow handling are those of attn_fwd_bf16_d256,
// per row half.

// S^T MFMA in its VGPR form (accumulator in VGPRs): O fills the AGPRs, so S must not
// go there. As inline asm, its hazards are handled here: a chain starts from the inline
// zero (no vector write feeds it), each step accumulates into exactly the registers its
// previous step wrote, and the last step (mfma_v_last2) carries the wait states the
// vector units need before they read the result.
__device__ __forceinline__ void mfma_v(f32x16_t& c, const uint4& a, const uint4& b, bool first) {
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  const u32x4_t av = __builtin_bit_cast(u32x4_t, a), bv = __builtin_bit_cast(u32x4_t, b);
  if (first) asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(c) : "v"(av), "v"(bv));
  else asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c) : "v"(av), "v"(bv));
}
// The last step of two chains, with the wait states in the same statement so that no
// read of the results can be placed before them.
__device__ __forceinline__ void mfma_v_last2(f32x16_t& c0, f32x16_t& c1, const uint4& a, const uint4& b0,
                                             const uint4& b1) {
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  const u32x4_t av = __builtin_bit_cast(u32x4_t, a), b0v = __builtin_bit_cast(u32x4_t, b0),
                b1v = __builtin_bit_cast(u32x4_t, b1);
  asm volatile(
      "v_mfma_f32_32x32x16_bf16 %0, %2, %3, %0\n\t"
      "v_mfma_f32_32x32x16_bf16 %1, %2, %4, %1\n\t"
      "s_nop 15\n\ts_nop 15\n\ts_nop 7"
      : "+v"(c0), "+v"(c1)
      : "v"(av), "v"(b0v), "v"(b1v));
}

#define DG_ATT_WAIT_LGKM(n)                                                   \
  do {                                                                        \
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | ((n) << 8) | (3 << 14));       \
    __builtin_amdgcn_sched_barrier(0);                                        \
  } while (0)

template <bool kPaged>
__global__ __launch_bounds__(kThreads) void attn_fwd_bf16_d256_w64(AttnArgs a) {
  constexpr int D = 256, KS = 16, DB = 8, kTile = 256;
  __shared__ __attribute__((aligned(1024))) char lds[kAttStages * kAttStage];
  __shared__ int redo_flag[1];
  // Q^T fragments of the second row half, k-steps kQL..15, kept in LDS (per wave, lane order)
  // instead of VGPRs: with O filling the AGPRs, the registers are short by about that much
  constexpr int kQL = 11;
  __shared__ __attribute__((aligned(16))) char qlds[4 * (KS - kQL) * 1024];

  const int w = a.work_offset + xcd_order(blockIdx.x, gridDim.x);
  const int s_ = find_seq(a, w, false);
  const AttnSeqPlan sp = a.seqs[s_];
  const int nqt = (sp.num_q + sp.tokens_per_tile - 1) / sp.tokens_per_tile;
  const int local = w - sp.work_begin;
  // items [key chunk][kv head][q tile], causal q tiles longest first, as in attn_fwd_bf16_d256
  const int qt = sp.mode == DG_CAUSAL ? nqt - 1 - local % nqt : local % nqt;
  const int rest = local / nqt;
  const int g = rest % a.hkv;
  const int chunk = rest / a.hkv;
  const int i0 = qt * sp.tokens_per_tile;
  const int nq = min(sp.tokens_per_tile, sp.num_q - i0);
  const int nkeys = sp.prefix_len + sp.num_q;
  int lo_first, hi_first, lo_last, hi_last;
  key_bounds(sp.mode, sp.prefix_len, sp.num_q, a.window, i0, lo_first, hi_first);
  key_bounds(sp.mode, sp.prefix_len, sp.num_q, a.window, i0 + nq - 1, lo_last, hi_last);
  const int kt_lo = lo_first / kKT, kt_hi = hi_last / kKT;
  const int t_begin = kt_lo + chunk * sp.chunk_tiles;
  const int t_end = min(kt_hi + 1, t_begin + sp.chunk_tiles);
  if (t_begin > kt_hi) return;
  const int key0 = t_begin * kKT;
  const int kend = min(t_end * kKT, hi_last + 1);
  const int nsub = (kend - key0 + kSub - 1) / kSub;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  // row (h) = wave*64 + 32h + l32 holds token i0 + row/G, head g*G + row%G
  auto row_of = [&](int h) { return wave * 64 + 32 * h + l32; };
  int lo[2], hi[2];
  uint4 qf[2][KS];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int tok = i0 + row_of(h) / a.group, head = g * a.group + row_of(h) % a.group;
    lo[h] = 0;
    hi[h] = -1;
    if (tok < sp.num_q) key_bounds(sp.mode, sp.prefix_len, sp.num_q, a.window, tok, lo[h], hi[h]);
    // rows past the request read its last token (their outputs are never stored)
    const char* qrow = reinterpret_cast<const char*>(a.q) +
                       ((int64_t)(sp.q_start + min(tok, sp.num_q - 1)) * a.hq + head) * D * 2;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[h][ks] = *reinterpret_cast<const uint4*>(qrow + (16 * ks + 8 * hh) * 2);
  }

  {
    const uint32_t qa = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)qlds + wave * (KS - kQL) * 1024 + lane * 16;
#pragma unroll
    for (int ks = kQL; ks < KS; ++ks) {
      typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
      const u32x4_t x = {qf[1][ks].x, qf[1][ks].y, qf[1][ks].z, qf[1][ks].w};
      asm volatile("ds_write_b128 %0, %1 offset:%2" : : "v"(qa), "v"(x), "i"((ks - kQL) * 1024) : "memory");
    }
  }
  const uint32_t q_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)qlds + wave * (KS - kQL) * 1024 + lane * 16;
  const int rs = a.hkv * D * 2;
  const int64_t head_off = (int64_t)g * D * 2;
  const char* kb = reinterpret_cast<const char*>(a.k) + head_off;
  const char* vb = reinterpret_cast<const char*>(a.v) + head_off;
  // lane offset of DMA pair t (recomputed at each use: it is cheap, and registers are not)
  auto vo = [&](int t) { return (uint32_t)((2 * (4 * wave + t) + (lane & 1)) * rs + (lane >> 1) * 16); };
  typedef __attribute__((address_space(3))) char lds_char;
  lds_char* lds0 = (lds_char*)lds;
  // rows kbase .. kbase+31 from pool row `row` on (row < 0: look it up)
  auto dma_rows = [&](const char* base, lds_char* dst, int pitch, int kbase, int64_t row) {
    const char* src = base + (row < 0 ? key_row<kPaged>(a, sp, kbase) : row) * rs;
    if (kbase + kSub <= nkeys) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
        __builtin_amdgcn_global_load_lds((const void*)(src + vo(t)),
                                         (__attribute__((address_space(3))) void*)(dst + (4 * wave + t) * pitch), 16, 0, 0);
    } else {
      const int last = nkeys - 1 - kbase;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint32_t r = min(2 * (4 * wave + t) + (lane & 1), last);
        __builtin_amdgcn_global_load_lds((const void*)(src + (r * rs + (lane >> 1) * 16)),
                                         (__attribute__((address_space(3))) void*)(dst + (4 * wave + t) * pitch), 16, 0, 0);
      }
    }
  };
  // stage j: K of sub-tile j+1 and V of sub-tile j, from pool rows krow / vrow (< 0: look up)
  auto issue = [&](int j, int64_t krow = -1, int64_t vrow = -1) {
    lds_char* st = lds0 + (j & 3) * kAttStage;
    dma_rows(kb, st, kKPitch, key0 + kSub * min(j + 1, nsub - 1), krow);
    dma_rows(vb, st + kKRegion, kVPitch, key0 + kSub * j, vrow);
  };
  // pool rows of stage j's K and V keys; in the loop they are looked up one sub-tile
  // ahead, so that the softmax's LDS waits also cover the table loads
  auto stage_rows = [&](int j, int64_t& krow, int64_t& vrow) {
    krow = key_row<kPaged>(a, sp, key0 + kSub * min(j + 1, nsub - 1));
    vrow = key_row<kPaged>(a, sp, key0 + kSub * min(j, nsub - 1));
  };

  const uint32_t lbase = (uint32_t)(uintptr_t)lds0;
  const uint32_t k_lane = (l32 >> 1) * kKPitch + 16 * (l32 & 1) + 32 * hh;
  const int grp = lane >> 4, s16 = lane & 15;
  const int vrow = 4 * (grp >> 1) + (s16 >> 2);
  const int vcol = 16 * (grp & 1) + 4 * (s16 & 3);
  const uint32_t v_lane = kKRegion + (vrow >> 1) * kVPitch + 16 * (vrow & 1) + 32 * (vcol >> 3) + 2 * (vcol & 7);

  auto mask = [&](f32x16_t& sv, int kbase, int h) {
    if (!(lo_last <= kbase && kbase + kSub - 1 <= hi_first)) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = kbase + 8 * (e >> 2) + 4 * hh + (e & 3);
        if (key < lo[h] || key > hi[h]) sv[e] = kNegInf;
      }
    }
  };

  // S = K(slot) . Q^T for both halves: K fragments four ahead in a 5-slot ring, the
  // half-1 Q fragments kQL..15 from LDS with them; dma(i) runs after step i
  f32x16_t sc[2];
  auto compute_s = [&](uint32_t ka, auto&& dma) {
    uint4 kf[5], ql[5];
    auto kread = [&](auto jc) {  // read j: K fragment j, and Q fragment j of half 1 when j >= kQL
      constexpr int j = decltype(jc)::value;
      kf[j % 5] = att_b128<64 * j>(ka);
      if constexpr (j >= kQL) ql[j % 5] = att_b128<1024 * (j - kQL)>(q_lds);
    };
    StaticFor<0, 4>::run(kread);
    StaticFor<0, KS>::run([&](auto ic) {
      constexpr int ks = decltype(ic)::value;
      constexpr int last = ks + 3 < KS - 1 ? ks + 3 : KS - 1;  // last read issued so far
      constexpr int ops_last = last + 1 + (last >= kQL ? last - kQL + 1 : 0);
      constexpr int ops_ks = ks + 1 + (ks >= kQL ? ks - kQL + 1 : 0);
      DG_ATT_WAIT_LGKM(ops_last - ops_ks);
      if constexpr (ks < KS - 1) {
        mfma_v(sc[0], kf[ks % 5], qf[0][ks], ks == 0);
        mfma_v(sc[1], kf[ks % 5], ks < kQL ? qf[1][ks] : ql[ks % 5], ks == 0);
      } else {
        mfma_v_last2(sc[0], sc[1], kf[ks % 5], qf[0][ks], ql[ks % 5]);
      }
      if constexpr (ks + 4 < KS) kread(std::integral_constant<int, ks + 4>{});
      if constexpr (ks < 8) dma(ks);
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  f32x16_t o[2][DB];
  float l_run[2];
  float m_ref[2] = {kNegInf, kNegInf};
  for (;;) {
    if (tid == 0) redo_flag[0] = 0;
    dma_rows(kb, lds0 + 3 * kAttStage, kKPitch, key0, -1);
    issue(0);
    if (nsub > 1) issue(1);
    if (nsub > 2) issue(2);
    if (nsub > 2) DG_ATT_WAIT_VM(24);
    else if (nsub > 1) DG_ATT_WAIT_VM(16);
    else DG_ATT_WAIT_VM(8);
    DG_ATT_WAIT_LGKM0();
    __builtin_amdgcn_s_barrier();
    compute_s(lbase + 3 * kAttStage + k_lane, [](int) {});
    // Once every row has its reference, the reference no longer changes, so the overflow
    // test only needs the chunk's largest score: each lane keeps a running max of its raw
    // scores (m_lane), and the row max, scale and test run once, after the loop.
    float m_seen[2] = {kNegInf, kNegInf}, m_lane[2] = {kNegInf, kNegInf};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      l_run[h] = 0.f;
#pragma unroll
      for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[h][b][e] = 0.f;
    }

    bool overflow = false;
    int64_t krow, vrow;
    stage_rows(3, krow, vrow);
    for (int sub = 0; sub < nsub; ++sub) {
      const int left = nsub - 1 - sub;
      if (left >= 2) DG_ATT_WAIT_VM(16);
      else if (left == 1) DG_ATT_WAIT_VM(8);
      else DG_ATT_WAIT_VM(0);
      __builtin_amdgcn_s_barrier();  // stage sub landed for every wave; slot of sub-1 is free
      __builtin_amdgcn_sched_barrier(0);
      const uint32_t ka = lbase + (sub & 3) * kAttStage + k_lane;
      const uint32_t va = lbase + (sub & 3) * kAttStage + v_lane;
      if (sub + 3 < nsub) issue(sub + 3, krow, vrow);  // into the slot of sub-1, free since the barrier
      stage_rows(sub + 4, krow, vrow);
      __builtin_amdgcn_sched_barrier(0);

      // ---- softmax of S(sub), keys 0..15 (elements 0..7). Once every row has its
      // reference, only the lanes' running max is kept, under the MFMAs below.
      uint2 vf[3][2];
      auto vread = [&](auto fc) {  // fragment f = 8 kh + b: d block b, key half kh
        constexpr int f = decltype(fc)::value;
        constexpr int b = f & 7, kh = f >> 3;
        vf[f % 3][0] = att_tr16<128 * b + 8 * kh * kVPitch>(va);
        vf[f % 3][1] = att_tr16<128 * b + (8 * kh + 4) * kVPitch>(va);
      };
      vread(std::integral_constant<int, 0>{});
      vread(std::integral_constant<int, 1>{});
      mask(sc[0], key0 + kSub * sub, 0);
      mask(sc[1], key0 + kSub * sub, 1);
      auto row_max = [&](int h) {
        const float t = half_max(att_max16(sc[h], kNegInf)) * a.scale_log2;
        m_seen[h] = fmaxf(m_seen[h], t);
        if (m_ref[h] == kNegInf) m_ref[h] = t;  // on a retry m_ref already covers this sub-tile
        overflow |= t > m_ref[h] + kOverflow;
      };
      const bool late_max = !__any(m_ref[0] == kNegInf || m_ref[1] == kNegInf);  // uniform
      if (!late_max) {
        row_max(0);
        row_max(1);
      }
      float mu[2];
      uint4 pc[2][2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        mu[h] = m_ref[h] == kNegInf ? 0.f : m_ref[h];
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          p[e] = fast_exp2(fmaf(sc[h][e], a.scale_log2, -mu[h]));
          l_run[h] += p[e];
        }
        asm volatile("" : "+v"(l_run[h]));  // keep the sums here
        pc[h][0] = make_uint4(pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3]), pack_bf16(p[4], p[5]), pack_bf16(p[6], p[7]));
      }
      __builtin_amdgcn_sched_barrier(0);

      // ---- O^T += V(sub)^T . P(sub)^T: 16 fragments (two V^T reads each, two ahead), each
      // feeding both halves; P of keys 16..31 during the first eight, the running max next
      float pv[2][8];
      StaticFor<0, 2 * DB>::run([&](auto fc) {
        constexpr int f = decltype(fc)::value;
        constexpr int b = f & 7, kh = f >> 3;
        DG_ATT_WAIT_LGKM(f < 2 * DB - 1 ? 2 : 0);
        const bf16x8_t va8 = __builtin_bit_cast(
            bf16x8_t, make_uint4(vf[f % 3][0].x, vf[f % 3][0].y, vf[f % 3][1].x, vf[f % 3][1].y));
        o[0][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va8, __builtin_bit_cast(bf16x8_t, pc[0][kh]), o[0][b], 0, 0, 0);
        o[1][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va8, __builtin_bit_cast(bf16x8_t, pc[1][kh]), o[1][b], 0, 0, 0);
        if constexpr (f + 2 < 2 * DB) vread(std::integral_constant<int, f + 2>{});
        if constexpr (f < 8) {
          constexpr int h = f >> 2, e0 = 8 + 2 * (f & 3);
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            pv[h][e0 - 8 + i] = fast_exp2(fmaf(sc[h][e0 + i], a.scale_log2, -mu[h]));
            l_run[h] += pv[h][e0 - 8 + i];
          }
          asm volatile("" : "+v"(l_run[h]));
          if constexpr ((f & 3) == 3)
            pc[h][1] = make_uint4(pack_bf16(pv[h][0], pv[h][1]), pack_bf16(pv[h][2], pv[h][3]),
                                  pack_bf16(pv[h][4], pv[h][5]), pack_bf16(pv[h][6], pv[h][7]));
        }
        if constexpr (f == 8 || f == 9) {
          if (late_max) m_lane[f - 8] = att_max16(sc[f - 8], m_lane[f - 8]);
        }
        __builtin_amdgcn_sched_barrier(0);
      });

      // ---- S(sub+1) = K(sub+1) . Q^T (the ring refill was issued at the top of the
      // sub-tile: spreading it over these steps measured no faster, with more spills)
      if (sub + 1 < nsub) {
        compute_s(ka, [](int) {});
      }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float t = half_max(m_lane[h]) * a.scale_log2;
      m_seen[h] = fmaxf(m_seen[h], t);
      overflow |= t > m_ref[h] + kOverflow;
    }
    if (__any(overflow) && lane == 0) redo_flag[0] = 1;
    __syncthreads();
    const int redo = redo_flag[0];
    if (!redo) break;
    __syncthreads();
    m_ref[0] = fmaxf(m_ref[0], m_seen[0]);
    m_ref[1] = fmaxf(m_ref[1], m_seen[1]);
  }

  // ---- epilogue: O (normalised, bf16) goes through LDS, the ring being free after the
  // loop's final barrier, so that the global stores are whole rows: each wave stages
  // its 64 rows at a 528-byte pitch, then writes 2 rows (1 KB) per store.
  // o[h][b][e] = O^T[d = 32b + 8(e/4) + 4hh + e%4][row h].
  constexpr int kOPitch = 528;
  char* ost = lds + wave * 64 * kOPitch;
  float ltot[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    ltot[h] = half_sum(l_run[h]);
    const float inv = ltot[h] > 0.f ? 1.f / ltot[h] : 0.f;
    char* orow = ost + (32 * h + l32) * kOPitch;
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4)
        *reinterpret_cast<uint2*>(orow + (32 * b + 8 * e4 + 4 * hh) * 2) =
            make_uint2(pack_bf16(o[h][b][4 * e4] * inv, o[h][b][4 * e4 + 1] * inv),
                       pack_bf16(o[h][b][4 * e4 + 2] * inv, o[h][b][4 * e4 + 3] * inv));
  }
  const int64_t prow0 = sp.part_begin + ((int64_t)(g * nqt + qt) * sp.num_chunks + chunk) * kTile;
  if (hh == 0) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = row_of(h), tok = i0 + row / a.group, head = g * a.group + row % a.group;
      if (tok >= sp.num_q) continue;
      if (sp.num_chunks > 1)
        *reinterpret_cast<float2*>(a.part_ml + (prow0 + row) * 2) = make_float2(m_ref[h], ltot[h]);
      else if (a.lse)
        a.lse[(int64_t)(sp.q_start + tok) * a.hq + head] = (m_ref[h] + __builtin_amdgcn_logf(ltot[h])) * kLn2;
    }
  }
  DG_ATT_WAIT_LGKM0();  // this wave's rows are in LDS (each wave reads only its own)
  // store r covers rows 2r, 2r+1 of this wave: lane i takes 16 bytes i%32 of row 2r + i/32
#pragma unroll 4
  for (int r = 0; r < 32; ++r) {
    const int lr = 2 * r + (lane >> 5);  // local row 0..63
    const int row = wave * 64 + lr, tok = i0 + row / a.group, head = g * a.group + row % a.group;
    const uint4 x = *reinterpret_cast<const uint4*>(ost + lr * kOPitch + l32 * 16);
    if (tok >= sp.num_q) continue;
    char* dst = sp.num_chunks == 1
                    ? reinterpret_cast<char*>(a.out) + ((int64_t)(sp.q_start + tok) * a.hq + head) * D * 2
                    : reinterpret_cast<char*>(a.part_o) + (prow0 + row) * D * 2;
    *reinterpret_cast<uint4*>(dst + l32 * 16) = x;
  }
}

// ---- FP8 (E4M3) K/V, head_dim 256, 64 query rows per wave -------------------------
//
// attn_fwd_bf16_d256_w64 over the code ring of attn_fwd_fp8_d256 (same layout, copies
// and fragment reads, same permuted contraction order). The smaller ring leaves room in
// LDS for k-steps kF8QL..15 of the second half's Q^T fragments. S's K operands are
// widened one k-step ahead, so that no vector write of an asm MFMA's operand comes right
// before it. The epilogue stages O one 32-row half at a time (the ring is smaller than
// the 64 rows per wave).

constexpr int kF8QL = 8;  // second-half Q^T k-steps kept in VGPRs; the rest in LDS

// lgkmcnt of k-step ks in the S phase below. Reads are issued in this order: K pairs 0, 1
// and 2 before step 0; after step i, the second half's Q fragment of step i + 4 when it
// comes from LDS (i + 4 >= kF8QL), and after odd i, K pair (i + 5) / 2. Step ks waits for
// its Q fragment (from LDS) and for the K pair of step ks + 2, which is widened after its
// MFMAs.
constexpr int f8w_wait(int ks) {
  int pos_k[8] = {}, pos_q[16] = {}, before[16] = {};
  int n = 0;
  pos_k[0] = n++;
  pos_k[1] = n++;
  pos_k[2] = n++;
  for (int i = 0; i < 16; ++i) {
    before[i] = n;
    if (i + 4 < 16 && i + 4 >= kF8QL) pos_q[i + 4] = n++;
    if ((i & 1) && (i + 5) / 2 <= 7) pos_k[(i + 5) / 2] = n++;
  }
  int need = -1;
  if (ks >= kF8QL) need = pos_q[ks];
  if (ks + 2 < 16 && pos_k[(ks + 2) / 2] > need) need = pos_k[(ks + 2) / 2];
  return before[ks] - 1 - need;
}
static_assert(f8w_wait(0) == 1 && f8w_wait(6) == 3 && f8w_wait(7) == 4 && f8w_wait(15) == 0, "read schedule");

template <bool kPaged>
__global__ __launch_bounds__(kThreads) void attn_fwd_fp8_d256_w64(AttnArgs a) {
  constexpr int D = 256, KS = 16, DB = 8, kTile = 256;
  __shared__ __attribute__((aligned(1024))) char lds[kAttStages * kF8Stage];
  __shared__ int redo_flag[1];
  __shared__ __attribute__((aligned(16))) char qlds[4 * (KS - kF8QL) * 1024];

  const int w = a.work_offset + xcd_order(blockIdx.x, gridDim.x);
  const int s_ = find_seq(a, w, false);
  const AttnSeqPlan sp = a.seqs[s_];
  const int nqt = (sp.num_q + sp.tokens_per_tile - 1) / sp.tokens_per_tile;
  const int local = w - sp.work_begin;
  const int qt = sp.mode == DG_CAUSAL ? nqt - 1 - local % nqt : local % nqt;
  const int rest = local / nqt;
  const int g = rest % a.hkv;
  const int chunk = rest / a.hkv;
  const int i0 = qt * sp.tokens_per_tile;
  const int nq = min(sp.tokens_per_tile, sp.num_q - i0);
  const int nkeys = sp.prefix_len + sp.num_q;
  int lo_first, hi_first, lo_last, hi_last;
  key_bounds(sp.mode, sp.prefix_len, sp.num_q, a.window, i0, lo_first, hi_first);
  key_bounds(sp.mode, sp.prefix_len, sp.num_q, a.window, i0 + nq - 1, lo_last, hi_last);
  const int kt_lo = lo_first / kKT, kt_hi = hi_last / kKT;
  const int t_begin = kt_lo + chunk * sp.chunk_tiles;
  const int t_end = min(kt_hi + 1, t_begin + sp.chunk_tiles);
  if (t_begin > kt_hi) return;
  const int key0 = t_begin * kKT;
  const int kend = min(t_end * kKT, hi_last + 1);
  const int nsub = (kend - key0 + kSub - 1) / kSub;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hh = lane >> 5;
  auto row_of = [&](int h) { return wave * 64 + 32 * h + l32; };
  int lo[2], hi[2];
  uint4 qf0[KS], qf1[kF8QL];  // Q^T fragments in the permuted dim order of the K reads
  const uint32_t q_lds =
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char*)qlds + wave * (KS - kF8QL) * 1024 + lane * 16;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int tok = i0 + row_of(h) / a.group, head = g * a.group + row_of(h) % a.group;
    lo[h] = 0;
    hi[h] = -1;
    if (tok < sp.num_q) key_bounds(sp.mode, sp.prefix_len, sp.num_q, a.window, tok, lo[h], hi[h]);
    // rows past the request read its last token (their outputs are never stored)
    const char* qrow = reinterpret_cast<const char*>(a.q) +
                       ((int64_t)(sp.q_start + min(tok, sp.num_q - 1)) * a.hq + head) * D * 2;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint4 x = *reinterpret_cast<const uint4*>(qrow + (32 * (ks >> 1) + 16 * hh + 8 * (ks & 1)) * 2);
      if (h == 0) {
        qf0[ks] = x;
      } else if (ks < kF8QL) {
        qf1[ks] = x;
      } else {
        typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
        const u32x4_t xv = {x.x, x.y, x.z, x.w};
        asm volatile("ds_write_b128 %0, %1 offset:%2" : : "v"(q_lds), "v"(xv), "i"((ks - kF8QL) * 1024) : "memory");
      }
    }
  }

  const int rs = a.hkv * D;  // bytes between consecutive keys
  const int64_t head_off = (int64_t)g * D;
  const char* kb = reinterpret_cast<const char*>(a.k) + head_off;
  const char* vb = reinterpret_cast<const char*>(a.v) + head_off;
  auto vo = [&](int u) { return (uint32_t)((4 * (2 * wave + u) + (lane & 3)) * rs + (lane >> 2) * 16); };
  typedef __attribute__((address_space(3))) char lds_char;
  lds_char* lds0 = (lds_char*)lds;
  // rows kbase .. kbase+31 from pool row `row` on (row < 0: look it up); rows past the
  // request's last key repeat it (masked)
  auto dma_rows = [&](const char* base, lds_char* dst, int pitch, int kbase, int64_t row) {
    const char* src = base + (row < 0 ? key_row<kPaged>(a, sp, kbase) : row) * rs;
    const int last = nkeys - 1 - kbase;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const uint32_t off =
          kbase + kSub <= nkeys ? vo(u) : (uint32_t)min(4 * (2 * wave + u) + (lane & 3), last) * rs + (lane >> 2) * 16;
      __builtin_amdgcn_global_load_lds((const void*)(src + off),
                                       (__attribute__((address_space(3))) void*)(dst + (2 * wave + u) * pitch), 16, 0, 0);
    }
  };
  auto issue = [&](int j, int64_t krow = -1, int64_t vrow = -1) {
    lds_char* st = lds0 + (j & 3) * kF8Stage;
    dma_rows(kb, st, kF8KPitch, key0 + kSub * min(j + 1, nsub - 1), krow);
    dma_rows(vb, st + kF8KRegion, kF8VPitch, key0 + kSub * j, vrow);
  };
  auto stage_rows = [&](int j, int64_t& krow, int64_t& vrow) {
    krow = key_row<kPaged>(a, sp, key0 + kSub * min(j + 1, nsub - 1));
    vrow = key_row<kPaged>(a, sp, key0 + kSub * min(j, nsub - 1));
  };

  const uint32_t lbase = (uint32_t)(uintptr_t)lds0;
  const uint32_t k_lane = (l32 >> 2) * kF8KPitch + 16 * (l32 & 3) + 64 * hh;  // + 128 j
  const int grp = lane >> 4, s16 = lane & 15;
  const int kr = (s16 >> 1) < 4 ? 4 * (grp >> 1) + (s16 >> 1) : 8 + 4 * (grp >> 1) + (s16 >> 1) - 4;
  const uint32_t v_lane = kF8KRegion + (kr >> 2) * kF8VPitch + 16 * (kr & 3) + 64 * (grp & 1) + 8 * (s16 & 1);

  auto mask = [&](f32x16_t& sv, int kbase, int h) {
    if (!(lo_last <= kbase && kbase + kSub - 1 <= hi_first)) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = kbase + 8 * (e >> 2) + 4 * hh + (e & 3);
        if (key < lo[h] || key > hi[h]) sv[e] = kNegInf;
      }
    }
  };

  // S = K(slot) . Q^T for both halves. K pairs (16 codes, two k-steps) are read three
  // pairs ahead into a 4-slot ring, the second half's Q fragments kF8QL..15 four steps
  // ahead into a 5-slot ring. The K operand of step ks + 2 is widened after step ks's
  // MFMAs (a 3-slot ring), so its conversions sit two MFMA steps before the asm MFMA
  // that reads it.
  f32x16_t sc[2];
  auto compute_s = [&](uint32_t ka) {
    uint4 k8[4], ql[5], kw[3];
    auto kpair = [&](auto pc) {
      constexpr int p = decltype(pc)::value;
      k8[p % 4] = att_b128<128 * p>(ka);
    };
    auto qread = [&](auto ic) {
      constexpr int i = decltype(ic)::value;
      ql[i % 5] = att_b128<1024 * (i - kF8QL)>(q_lds);
    };
    auto widen_k = [&](int u, const uint4& k) { return u == 0 ? widen_e4m3(k.x, k.y) : widen_e4m3(k.z, k.w); };
    static_assert(kF8QL >= 4, "the first four steps take Q from VGPRs");
    kpair(std::integral_constant<int, 0>{});
    kpair(std::integral_constant<int, 1>{});
    kpair(std::integral_constant<int, 2>{});
    DG_ATT_WAIT_LGKM(2);  // K pair 0
    kw[0] = widen_k(0, k8[0]);
    kw[1] = widen_k(1, k8[0]);
    StaticFor<0, KS>::run([&](auto ic) {
      constexpr int ks = decltype(ic)::value;
      DG_ATT_WAIT_LGKM(f8w_wait(ks));
      const uint4& qb1 = ks < kF8QL ? qf1[ks < kF8QL ? ks : 0] : ql[ks % 5];
      if constexpr (ks < KS - 1) {
        mfma_v(sc[0], kw[ks % 3], qf0[ks], ks == 0);
        mfma_v(sc[1], kw[ks % 3], qb1, ks == 0);
      } else {
        mfma_v_last2(sc[0], sc[1], kw[ks % 3], qf0[ks], qb1);
      }
      if constexpr (ks + 4 < KS && ks + 4 >= kF8QL) qread(std::integral_constant<int, ks + 4>{});
      if constexpr ((ks & 1) && (ks + 5) / 2 <= 7) kpair(std::integral_constant<int, (ks + 5) / 2>{});
      if constexpr (ks + 2 < KS) kw[(ks + 2) % 3] = widen_k((ks + 2) & 1, k8[((ks + 2) >> 1) % 4]);
      __builtin_amdgcn_sched_barrier(0);
    });
  };

  f32x16_t o[2][DB];
  float l_run[2];
  float m_ref[2] = {kNegInf, kNegInf};
  for (;;) {
    if (tid == 0) redo_flag[0] = 0;
    dma_rows(kb, lds0 + 3 * kF8Stage, kF8KPitch, key0, -1);
    issue(0);
    if (nsub > 1) issue(1);
    if (nsub > 2) issue(2);
    if (nsub > 2) DG_ATT_WAIT_VM(12);
    else if (nsub > 1) DG_ATT_WAIT_VM(8);
    else DG_ATT_WAIT_VM(4);
    DG_ATT_WAIT_LGKM0();  // also the Q writes into LDS
    __builtin_amdgcn_s_barrier();
    compute_s(lbase + 3 * kF8Stage + k_lane);
    // as in attn_fwd_bf16_d256_w64: once every row has its reference, a running max per
    // lane, and the overflow test once, after the loop
    float m_seen[2] = {kNegInf, kNegInf}, m_lane[2] = {kNegInf, kNegInf};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      l_run[h] = 0.f;
#pragma unroll
      for (int b = 0; b < DB; ++b)
#pragma unroll
        for (int e = 0; e < 16; ++e) o[h][b][e] = 0.f;
    }

    bool overflow = false;
    int64_t krow, vrow;
    stage_rows(3, krow, vrow);
    for (int sub = 0; sub < nsub; ++sub) {
      const int left = nsub - 1 - sub;
      if (left >= 2) DG_ATT_WAIT_VM(8);
      else if (left == 1) DG_ATT_WAIT_VM(4);
      else DG_ATT_WAIT_VM(0);
      __builtin_amdgcn_s_barrier();  // stage sub landed for every wave; slot of sub-1 is free
      __builtin_amdgcn_sched_barrier(0);
      const uint32_t ka = lbase + (sub & 3) * kF8Stage + k_lane;
      const uint32_t va = lbase + (sub & 3) * kF8Stage + v_lane;
      if (sub + 3 < nsub) issue(sub + 3, krow, vrow);  // into the slot of sub-1, free since the barrier
      stage_rows(sub + 4, krow, vrow);
      __builtin_amdgcn_sched_barrier(0);

      // ---- softmax of S(sub), keys 0..15 (elements 0..7)
      uint2 vf[3];
      auto vread = [&](auto fc) {  // fragment f = 8 kh + b: d block b, key half kh
        constexpr int f = decltype(fc)::value;
        vf[f % 3] = att_tr8<128 * (f & 7) + 4 * kF8VPitch * (f >> 3)>(va);
      };
      vread(std::integral_constant<int, 0>{});
      vread(std::integral_constant<int, 1>{});
      mask(sc[0], key0 + kSub * sub, 0);
      mask(sc[1], key0 + kSub * sub, 1);
      auto row_max = [&](int h) {
        const float t = half_max(att_max16(sc[h], kNegInf)) * a.scale_log2;
        m_seen[h] = fmaxf(m_seen[h], t);
        if (m_ref[h] == kNegInf) m_ref[h] = t;  // on a retry m_ref already covers this sub-tile
        overflow |= t > m_ref[h] + kOverflow;
      };
      const bool late_max = !__any(m_ref[0] == kNegInf || m_ref[1] == kNegInf);  // uniform
      if (!late_max) {
        row_max(0);
        row_max(1);
      }
      float mu[2];
      uint4 pc[2][2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        mu[h] = m_ref[h] == kNegInf ? 0.f : m_ref[h];
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          p[e] = fast_exp2(fmaf(sc[h][e], a.scale_log2, -mu[h]));
          l_run[h] += p[e];
        }
        asm volatile("" : "+v"(l_run[h]));  // keep the sums here
        pc[h][0] = make_uint4(pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3]), pack_bf16(p[4], p[5]), pack_bf16(p[6], p[7]));
      }
      __builtin_amdgcn_sched_barrier(0);

      // ---- O^T += V(sub)^T . P(sub)^T: 16 fragments (one transposing read each, two
      // ahead, widened at their step), each feeding both halves
      float pv[2][8];
      StaticFor<0, 2 * DB>::run([&](auto fc) {
        constexpr int f = decltype(fc)::value;
        constexpr int b = f & 7, kh = f >> 3;
        DG_ATT_WAIT_LGKM(f < 2 * DB - 1 ? 1 : 0);
        const bf16x8_t va8 = __builtin_bit_cast(bf16x8_t, widen_e4m3(vf[f % 3].x, vf[f % 3].y));
        o[0][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va8, __builtin_bit_cast(bf16x8_t, pc[0][kh]), o[0][b], 0, 0, 0);
        o[1][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va8, __builtin_bit_cast(bf16x8_t, pc[1][kh]), o[1][b], 0, 0, 0);
        if constexpr (f + 2 < 2 * DB) vread(std::integral_constant<int, f + 2>{});
        if constexpr (f < 8) {
          constexpr int h = f >> 2, e0 = 8 + 2 * (f & 3);
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            pv[h][e0 - 8 + i] = fast_exp2(fmaf(sc[h][e0 + i], a.scale_log2, -mu[h]));
            l_run[h] += pv[h][e0 - 8 + i];
          }
          asm volatile("" : "+v"(l_run[h]));
          if constexpr ((f & 3) == 3)
            pc[h][1] = make_uint4(pack_bf16(pv[h][0], pv[h][1]), pack_bf16(pv[h][2], pv[h][3]),
                                  pack_bf16(pv[h][4], pv[h][5]), pack_bf16(pv[h][6], pv[h][7]));
        }
        if constexpr (f == 8 || f == 9) {
          if (late_max) m_lane[f - 8] = att_max16(sc[f - 8], m_lane[f - 8]);
        }
        __builtin_amdgcn_sched_barrier(0);
      });

      // ---- S(sub+1) = K(sub+1) . Q^T
      if (sub + 1 < nsub) compute_s(ka);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float t = half_max(m_lane[h]) * a.scale_log2;
      m_seen[h] = fmaxf(m_seen[h], t);
      overflow |= t > m_ref[h] + kOverflow;
    }
    if (__any(overflow) && lane == 0) redo_flag[0] = 1;
    __syncthreads();
    const int redo = redo_flag[0];
    if (!redo) break;
    __syncthreads();
    m_ref[0] = fmaxf(m_ref[0], m_seen[0]);
    m_ref[1] = fmaxf(m_ref[1], m_seen[1]);
  }

  // ---- epilogue: as attn_fwd_bf16_d256_w64, with v_scale in the normalisation and O
  // staged one 32-row half at a time (each wave reads back only its own rows)
  constexpr int kOPitch = 528;
  char* ost = lds + wave * 32 * kOPitch;
  float ltot[2];
  const int64_t prow0 = sp.part_begin + ((int64_t)(g * nqt + qt) * sp.num_chunks + chunk) * kTile;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    ltot[h] = half_sum(l_run[h]);
    const float inv = (ltot[h] > 0.f ? 1.f / ltot[h] : 0.f) * a.v_scale;
    char* orow = ost + l32 * kOPitch;
    DG_ATT_WAIT_LGKM0();  // the previous half's rows have been read back
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4)
        *reinterpret_cast<uint2*>(orow + (32 * b + 8 * e4 + 4 * hh) * 2) =
            make_uint2(pack_bf16(o[h][b][4 * e4] * inv, o[h][b][4 * e4 + 1] * inv),
                       pack_bf16(o[h][b][4 * e4 + 2] * inv, o[h][b][4 * e4 + 3] * inv));
    if (hh == 0) {
      const int row = row_of(h), tok = i0 + row / a.group, head = g * a.group + row % a.group;
      if (tok < sp.num_q) {
        if (sp.num_chunks > 1)
          *reinterpret_cast<float2*>(a.part_ml + (prow0 + row) * 2) = make_float2(m_ref[h], ltot[h]);
        else if (a.lse)
          a.lse[(int64_t)(sp.q_start + tok) * a.hq + head] = (m_ref[h] + __builtin_amdgcn_logf(ltot[h])) * kLn2;
      }
    }
    DG_ATT_WAIT_LGKM0();  // this half's rows are in LDS
    // store r covers local rows 2r, 2r+1 of the half: lane i takes 16 bytes i%32 of row 2r + i/32
#pragma unroll 4
    for (int r = 0; r < 16; ++r) {
      const int lr = 2 * r + (lane >> 5);  // row 0..31 of the half
      const int row = wave * 64 + 32 * h + lr, tok = i0 + row / a.group, head = g * a.group + row % a.group;
      const uint4 x = *reinterpret_cast<const uint4*>(ost + lr * kOPitch + l32 * 16);
      if (tok >= sp.num_q) continue;
      char* dst = sp.num_chunks == 1
                      ? reinterpret_cast<char*>(a.out) + ((int64_t)(sp.q_start + tok) * a.hq + head) * D * 2
                      : reinterpret_cast<char*>(a.part_o) + (prow0 + row) * D * 2;
      *reinterpret_cast<uint4*>(dst + l32 * 16) = x;
    }
  }
}

template <bool kBf16, int D, bool kPaged>
int launch_typed(AttnArgs args, const AttnPlan& plan, hipStream_t s) {
  // work [0, num_wide): 64-rows-per-wave kernel; [num_wide, num_dma): 128-row LDS-DMA
  // kernel; [num_dma, num_work): register-staged kernel (each request on one of them)
  if constexpr (kBf16 && D == 256) {
    if (plan.num_wide > 0) {
      args.work_offset = 0;
      hipLaunchKernelGGL(attn_fwd_bf16_d256_w64<kPaged>, dim3(plan.num_wide), dim3(kThreads), 0, s, args);
    }
    if (plan.num_dma > plan.num_wide) {
      args.work_offset = plan.num_wide;
      hipLaunchKernelGGL(attn_fwd_bf16_d256<kPaged>, dim3(plan.num_dma - plan.num_wide), dim3(kThreads), 0, s, args);
    }
  }
  if (plan.num_work > plan.num_dma) {
    args.work_offset = plan.num_dma;
    hipLaunchKernelGGL((attn_fwd<kBf16, D, kPaged>), dim3(plan.num_work - plan.num_dma), dim3(kThreads), 0, s, args);
  }
  if (plan.num_merge > 0) hipLaunchKernelGGL((attn_merge<kBf16, D>), dim3(plan.num_merge), dim3(kThreads), 0, s, args);
  return (int)hipGetLastError();
}

// FP8 K/V: work [0, num_wide) on the 64-rows-per-wave kernel over codes, [num_wide,
// num_dma) on the 128-row one (head_dim 256), the rest on the register-staged kernel at
// bf16, then the merge of bf16 partials
template <int D, bool kPaged>
int launch_fp8(AttnArgs args, const AttnPlan& plan, hipStream_t s) {
  if constexpr (D == 256) {
    if (plan.num_wide > 0) {
      args.work_offset = 0;
      hipLaunchKernelGGL(attn_fwd_fp8_d256_w64<kPaged>, dim3(plan.num_wide), dim3(kThreads), 0, s, args);
    }
    if (plan.num_dma > plan.num_wide) {
      args.work_offset = plan.num_wide;
      hipLaunchKernelGGL(attn_fwd_fp8_d256<kPaged>, dim3(plan.num_dma - plan.num_wide), dim3(kThreads), 0, s, args);
    }
  }
  if (plan.num_work > plan.num_dma) {
    args.work_offset = plan.num_dma;
    hipLaunchKernelGGL((attn_fwd<true, D, kPaged, true>), dim3(plan.num_work - plan.num_dma), dim3(kThreads), 0, s,
                       args);
  }
  if (plan.num_merge > 0) hipLaunchKernelGGL((attn_merge<true, D>), dim3(plan.num_merge), dim3(kThreads), 0, s, args);
  return (int)hipGetLastError();
}

}  // namespace

int launch_attn(const dg_attn_args* a, const AttnPlan& plan, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  AttnArgs args;
  args.q = a->q;
  args.k = a->k;
  args.v = a->v;
  args.out = a->out;
  args.lse = a->lse;
  char* ws = reinterpret_cast<char*>(a->workspace);
  args.part_o = plan.part_rows ? reinterpret_cast<void*>(ws + plan.part_o_offset) : nullptr;
  args.part_ml = plan.part_rows ? reinterpret_cast<float*>(ws + plan.part_ml_offset) : nullptr;
  args.hq = a->num_q_heads;
  args.hkv = a->num_kv_heads;
  args.group = plan.group;
  args.window = a->window;
  args.work_offset = 0;
  args.num_seqs = plan.num_seqs;
  const float scale = a->scale > 0.f ? a->scale : 1.f / sqrtf((float)a->head_dim);
  args.scale_log2 = scale * kLog2e;
  args.block_table = a->block_size > 0 ? a->block_table : nullptr;
  args.pool_blocks = a->block_size > 0 ? a->total_kv / a->block_size : 0;
  args.block_shift = plan.block_shift;
  for (int i = 0; i < plan.num_seqs; ++i) args.seqs[i] = plan.seqs[i];
  for (int i = plan.num_seqs; i < DG_MAX_SEQS; ++i) args.seqs[i] = AttnSeqPlan{};
  args.v_scale = 1.f;
  const bool paged = plan.block_shift >= 0;
  if (plan.kv_fp8) {
    args.scale_log2 = scale * a->k_scale * kLog2e;
    args.v_scale = a->v_scale;
    switch (a->head_dim) {
      case 64: return paged ? launch_fp8<64, true>(args, plan, s) : launch_fp8<64, false>(args, plan, s);
      case 128: return paged ? launch_fp8<128, true>(args, plan, s) : launch_fp8<128, false>(args, plan, s);
      default: return paged ? launch_fp8<256, true>(args, plan, s) : launch_fp8<256, false>(args, plan, s);
    }
  }
  if (a->dtype == DG_BF16) {
    switch (a->head_dim) {
      case 64: return paged ? launch_typed<true, 64, true>(args, plan, s) : launch_typed<true, 64, false>(args, plan, s);
      case 128: return paged ? launch_typed<true, 128, true>(args, plan, s) : launch_typed<true, 128, false>(args, plan, s);
      default: return paged ? launch_typed<true, 256, true>(args, plan, s) : launch_typed<true, 256, false>(args, plan, s);
    }
  }
  switch (a->head_dim) {
    case 64: return paged ? launch_typed<false, 64, true>(args, plan, s) : launch_typed<false, 64, false>(args, plan, s);
    default: return paged ? launch_typed<false, 128, true>(args, plan, s) : launch_typed<false, 128, false>(args, plan, s);
  }
}

}  // namespace dg
