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
// A request whose keys were split into several chunks writes fp32 partials
// (unnormalised O, running max and sum); attn_merge combines them in chunk order.
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
  float* part_o;
  float* part_ml;
  int hq, hkv, group, window, tokens_per_tile, num_seqs;
  float scale_log2;  // scale * log2(e)
  AttnSeqPlan seqs[DG_MAX_SEQS];
};

__device__ __forceinline__ void key_bounds(int mode, int prefix, int num_q, int window, int i, int& lo, int& hi) {
  const int p = prefix + i;
  const int last = prefix + num_q - 1;
  lo = window < 0 ? 0 : max(0, p - window);
  hi = mode == DG_CAUSAL ? p : (window < 0 ? last : min(last, p + window));
}

// The request owning a global work (or merge) index: the last one whose first index
// is <= w. Requests without work share their first index with the next request, so
// the last of a tie is the one that has work.
__device__ __forceinline__ int find_seq(const AttnArgs& a, int w, bool merge) {
  int s = 0;
  for (int i = 1; i < a.num_seqs; ++i) {
    const int b = merge ? a.seqs[i].merge_begin : a.seqs[i].work_begin;
    if (b <= w) s = i;
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

// Stage one 64-key tile of K (row-major) and V (transposed) into LDS. Key rows at
// or past `nkeys` (request-local) are zero.
template <bool kBf16, int D>
__device__ __forceinline__ void stage_tile(char* lk, char* lv, const char* kg, const char* vg, int64_t row_stride,
                                           int k0, int nkeys) {
  using L = Lds<kBf16, D>;
  constexpr int esz = L::esz;
  constexpr int cpr = D * esz / 16;  // 16-byte chunks per key row
  const int tid = threadIdx.x;
  // K: chunk q -> key q / cpr, column q % cpr
#pragma unroll
  for (int q = tid; q < kKT * cpr; q += kThreads) {
    const int key = q / cpr, col = q % cpr;
    uint4 val = make_uint4(0, 0, 0, 0);
    if (k0 + key < nkeys) val = *reinterpret_cast<const uint4*>(kg + (int64_t)(k0 + key) * row_stride + col * 16);
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
        if (k0 + key < nkeys) r[j] = *reinterpret_cast<const uint4*>(vg + (int64_t)(k0 + key) * row_stride + dgp * 16);
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
        if (k0 + key0 + j < nkeys) r[j] = *reinterpret_cast<const float4*>(vg + (int64_t)(k0 + key0 + j) * row_stride + dgp * 16);
      }
      *reinterpret_cast<float4*>(lv + (dgp * 4 + 0) * L::v_pitch + pos0 * 4) = make_float4(r[0].x, r[1].x, r[2].x, r[3].x);
      *reinterpret_cast<float4*>(lv + (dgp * 4 + 1) * L::v_pitch + pos0 * 4) = make_float4(r[0].y, r[1].y, r[2].y, r[3].y);
      *reinterpret_cast<float4*>(lv + (dgp * 4 + 2) * L::v_pitch + pos0 * 4) = make_float4(r[0].z, r[1].z, r[2].z, r[3].z);
      *reinterpret_cast<float4*>(lv + (dgp * 4 + 3) * L::v_pitch + pos0 * 4) = make_float4(r[0].w, r[1].w, r[2].w, r[3].w);
    }
  }
}

template <bool kBf16, int D>
__global__ __launch_bounds__(kThreads) void attn_fwd(AttnArgs a) {
  using OP = Op<kBf16>;
  using L = Lds<kBf16, D>;
  constexpr int esz = L::esz;
  constexpr int KS = D / 16;  // k16 steps over the head dimension
  constexpr int DB = D / 32;  // 32-wide output blocks
  __shared__ __attribute__((aligned(16))) char lk[L::k_bytes];
  __shared__ __attribute__((aligned(16))) char lv[L::v_bytes];

  const int w = blockIdx.x;
  const int s = find_seq(a, w, false);
  const AttnSeqPlan sp = a.seqs[s];
  const int nqt = (sp.num_q + a.tokens_per_tile - 1) / a.tokens_per_tile;
  const int local = w - sp.work_begin;
  const int chunk = local % sp.num_chunks;
  const int rest = local / sp.num_chunks;
  const int qt = rest % nqt;
  const int g = rest / nqt;
  const int i0 = qt * a.tokens_per_tile;
  const int nq = min(a.tokens_per_tile, sp.num_q - i0);
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

  const int64_t row_stride = (int64_t)a.hkv * D * esz;
  const char* kg = reinterpret_cast<const char*>(a.k) + ((int64_t)sp.kv_start * a.hkv + g) * D * esz;
  const char* vg = reinterpret_cast<const char*>(a.v) + ((int64_t)sp.kv_start * a.hkv + g) * D * esz;

  for (int kt = t_begin; kt < t_end; ++kt) {
    const int k0 = kt * kKT;
    __syncthreads();  // previous tile fully consumed
    stage_tile<kBf16, D>(lk, lv, kg, vg, row_stride, k0, nkeys);
    __syncthreads();

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
  }

  // epilogue: o[b][e] = O^T[d = 32b + 8(e/4) + 4hh + e%4][this lane's row]
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (!valid) return;
  if (sp.num_chunks == 1) {
    const float inv = 1.f / l_tot;
    char* orow = reinterpret_cast<char*>(a.out) + ((int64_t)(sp.q_start + tok) * a.hq + head) * D * esz;
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
    if (a.lse && hh == 0) a.lse[(int64_t)(sp.q_start + tok) * a.hq + head] = m_run * kLn2 + __builtin_amdgcn_logf(l_tot) * kLn2;
  } else {
    const int part = sp.part_begin + local;
    float* po = a.part_o + ((int64_t)part * kRows + row) * D;
#pragma unroll
    for (int b = 0; b < DB; ++b)
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4)
        *reinterpret_cast<float4*>(po + 32 * b + 8 * e4 + 4 * hh) =
            make_float4(o[b][4 * e4], o[b][4 * e4 + 1], o[b][4 * e4 + 2], o[b][4 * e4 + 3]);
    if (hh == 0) *reinterpret_cast<float2*>(a.part_ml + ((int64_t)part * kRows + row) * 2) = make_float2(m_run, l_tot);
  }
}

// Combine the chunk partials of one (request, KV head, q tile) in chunk order:
// O = sum_j 2^(m_j - M) O_j / sum_j 2^(m_j - M) l_j.
template <bool kBf16, int D>
__global__ __launch_bounds__(kThreads) void attn_merge(AttnArgs a) {
  constexpr int esz = kBf16 ? 2 : 4;
  const int w = blockIdx.x;
  const int s = find_seq(a, w, true);
  const AttnSeqPlan sp = a.seqs[s];
  const int nqt = (sp.num_q + a.tokens_per_tile - 1) / a.tokens_per_tile;
  const int local = w - sp.merge_begin;
  const int qt = local % nqt, g = local / nqt;
  const int i0 = qt * a.tokens_per_tile;
  const int nq = min(a.tokens_per_tile, sp.num_q - i0);
  int lo_first, hi_first, lo_last, hi_last;
  key_bounds(sp.mode, sp.prefix_len, sp.num_q, a.window, i0, lo_first, hi_first);
  key_bounds(sp.mode, sp.prefix_len, sp.num_q, a.window, i0 + nq - 1, lo_last, hi_last);
  const int kt_lo = lo_first / kKT, kt_hi = hi_last / kKT;
  const int nonempty = min(sp.num_chunks, (kt_hi - kt_lo) / sp.chunk_tiles + 1);
  const int part0 = sp.part_begin + (g * nqt + qt) * sp.num_chunks;

  // two threads per row, each half of D
  const int row = threadIdx.x >> 1, half = threadIdx.x & 1;
  const int tok = i0 + row / a.group;
  const int head = g * a.group + row % a.group;
  if (tok >= sp.num_q) return;
  float mmax = kNegInf;
  for (int j = 0; j < nonempty; ++j) mmax = fmaxf(mmax, a.part_ml[((int64_t)(part0 + j) * kRows + row) * 2]);
  float wsum = 0.f;
  float acc[D / 2];
#pragma unroll
  for (int d = 0; d < D / 2; ++d) acc[d] = 0.f;
  for (int j = 0; j < nonempty; ++j) {
    const float2 ml = *reinterpret_cast<const float2*>(a.part_ml + ((int64_t)(part0 + j) * kRows + row) * 2);
    const float f = fast_exp2(ml.x - mmax);
    if (f == 0.f) continue;
    wsum = fmaf(f, ml.y, wsum);
    const float* po = a.part_o + ((int64_t)(part0 + j) * kRows + row) * D + half * (D / 2);
#pragma unroll
    for (int d = 0; d < D / 2; d += 4) {
      const float4 x = *reinterpret_cast<const float4*>(po + d);
      acc[d] = fmaf(f, x.x, acc[d]);
      acc[d + 1] = fmaf(f, x.y, acc[d + 1]);
      acc[d + 2] = fmaf(f, x.z, acc[d + 2]);
      acc[d + 3] = fmaf(f, x.w, acc[d + 3]);
    }
  }
  const float inv = 1.f / wsum;
  char* orow = reinterpret_cast<char*>(a.out) + ((int64_t)(sp.q_start + tok) * a.hq + head) * D * esz + half * (D / 2) * esz;
#pragma unroll
  for (int d = 0; d < D / 2; d += 4) {
    if (kBf16)
      *reinterpret_cast<uint2*>(orow + d * 2) =
          make_uint2(pack_bf16(acc[d] * inv, acc[d + 1] * inv), pack_bf16(acc[d + 2] * inv, acc[d + 3] * inv));
    else
      *reinterpret_cast<float4*>(orow + d * 4) = make_float4(acc[d] * inv, acc[d + 1] * inv, acc[d + 2] * inv, acc[d + 3] * inv);
  }
  if (a.lse && half == 0) a.lse[(int64_t)(sp.q_start + tok) * a.hq + head] = (mmax + __builtin_amdgcn_logf(wsum)) * kLn2;
}

template <bool kBf16, int D>
int launch_typed(const AttnArgs& args, const AttnPlan& plan, hipStream_t s) {
  hipLaunchKernelGGL((attn_fwd<kBf16, D>), dim3(plan.num_work), dim3(kThreads), 0, s, args);
  if (plan.num_merge > 0) hipLaunchKernelGGL((attn_merge<kBf16, D>), dim3(plan.num_merge), dim3(kThreads), 0, s, args);
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
  args.part_o = plan.num_parts ? reinterpret_cast<float*>(ws + plan.part_o_offset) : nullptr;
  args.part_ml = plan.num_parts ? reinterpret_cast<float*>(ws + plan.part_ml_offset) : nullptr;
  args.hq = a->num_q_heads;
  args.hkv = a->num_kv_heads;
  args.group = plan.group;
  args.window = a->window;
  args.tokens_per_tile = plan.tokens_per_tile;
  args.num_seqs = plan.num_seqs;
  const float scale = a->scale > 0.f ? a->scale : 1.f / sqrtf((float)a->head_dim);
  args.scale_log2 = scale * kLog2e;
  for (int i = 0; i < plan.num_seqs; ++i) args.seqs[i] = plan.seqs[i];
  for (int i = plan.num_seqs; i < DG_MAX_SEQS; ++i) args.seqs[i] = AttnSeqPlan{};
  if (a->dtype == DG_BF16) {
    switch (a->head_dim) {
      case 64: return launch_typed<true, 64>(args, plan, s);
      case 128: return launch_typed<true, 128>(args, plan, s);
      default: return launch_typed<true, 256>(args, plan, s);
    }
  }
  switch (a->head_dim) {
    case 64: return launch_typed<false, 64>(args, plan, s);
    default: return launch_typed<false, 128>(args, plan, s);
  }
}

}  // namespace dg
