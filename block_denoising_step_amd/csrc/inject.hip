// Self-conditioning injection on gfx950: the canvas embedding plus the
// self-conditioning vector passed through a gated MLP ([P1] ("DiffusionGemma:
// vLLM에서 네이티브로 처음 지원되는 첫 번째 Diffusion LLM") sections "안정성을 위한
// 셀프 컨디셔닝" and "ModelState 인터페이스"). The gated MLP is read as a GeGLU with
// the tanh GELU, no bias.
//
//   gu  = s . w_gate_up            MFMA GEMM (the self-conditioning GEMM, [M, d] x [d, 2h])
//   h   = gelu(gu[:, :h]) * gu[:, h:]   inject_geglu (elementwise, 8 values per thread)
//   out = h . w_down               MFMA GEMM ([M, h] x [h, d])
//   out += embed[tokens]           inject_add_rows (gather and add, 8 values per thread)
// For bf16 products split over K, the GeGLU and the gather run in the split-K reduce's
// epilogue instead (no gu tensor, two launches fewer).
//
// The two contractions are dense GEMMs on the matrix cores; the two elementwise
// passes touch M x (3h + 2d) values, a few MB at the canvas sizes.
#include <cmath>

#include "dg_common.cuh"
#include "dg_internal.h"

namespace dg {
namespace {

constexpr int kThreads = 256;

// 8 consecutive values as fp32, from bf16 or fp32 storage
template <bool kBf16>
__device__ __forceinline__ void load8(const void* base, int64_t i, float (&x)[8]) {
  if constexpr (kBf16) {
    const uint4 v = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(base) + i);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[2 * k] = bf16lo(w[k]);
      x[2 * k + 1] = bf16hi(w[k]);
    }
  } else {
    const float4 a = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + i);
    const float4 b = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + i + 4);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
}

template <bool kBf16>
__device__ __forceinline__ void store8(void* base, int64_t i, const float (&x)[8]) {
  if constexpr (kBf16) {
    *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(base) + i) =
        make_uint4(pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3]), pack_bf16(x[4], x[5]), pack_bf16(x[6], x[7]));
  } else {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(base) + i) = make_float4(x[0], x[1], x[2], x[3]);
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(base) + i + 4) = make_float4(x[4], x[5], x[6], x[7]);
  }
}

template <bool kBf16>
__global__ __launch_bounds__(kThreads) void inject_geglu(const void* __restrict__ gu, void* __restrict__ h, int M,
                                                         int hidden) {
  const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int per_row = hidden / 8;
  if (t >= (int64_t)M * per_row) return;
  const int i = (int)(t / per_row), c = (int)(t % per_row) * 8;
  float g[8], u[8], y[8];
  load8<kBf16>(gu, (int64_t)i * 2 * hidden + c, g);
  load8<kBf16>(gu, (int64_t)i * 2 * hidden + hidden + c, u);
#pragma unroll
  for (int k = 0; k < 8; ++k) y[k] = gelu_tanh(g[k]) * u[k];
  store8<kBf16>(h, (int64_t)i * hidden + c, y);
}

template <bool kBf16>
__global__ __launch_bounds__(kThreads) void inject_add_rows(void* __restrict__ out, const void* __restrict__ embed,
                                                            const int32_t* __restrict__ tokens, int M, int d,
                                                            int vocab) {
  const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int per_row = d / 8;
  if (t >= (int64_t)M * per_row) return;
  const int i = (int)(t / per_row), c = (int)(t % per_row) * 8;
  const int tok = min(max(tokens[i], 0), vocab - 1);
  float o[8], e[8];
  load8<kBf16>(out, (int64_t)i * d + c, o);
  load8<kBf16>(embed, (int64_t)tok * d + c, e);
#pragma unroll
  for (int k = 0; k < 8; ++k) o[k] += e[k];
  store8<kBf16>(out, (int64_t)i * d + c, o);
}

}  // namespace

int launch_inject(const dg_inject_args* a, InjectPlan& plan, void* stream) {
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* ws = reinterpret_cast<char*>(a->workspace);
  void* gu = ws + plan.gu_offset;
  void* h = ws + plan.h_offset;
  void* gemm_ws = ws + plan.gemm_ws_offset;
  plan.gemm1.out = gu;
  plan.gemm1.workspace = gemm_ws;
  plan.gemm1.workspace_bytes = plan.plan1.bytes;
  plan.gemm2.p = h;
  plan.gemm2.workspace = gemm_ws;
  plan.gemm2.workspace_bytes = plan.plan2.bytes;
  const bool bf = a->dtype == DG_BF16;
  // bf16 products split over K: the GeGLU and the embedding gather run in the reduce's
  // epilogue (the gate half must be whole column tiles of the product)
  const bool fuse1 = bf && plan.plan1.splits > 1 && a->hidden % plan.plan1.tile_n == 0;
  const bool fuse2 = bf && plan.plan2.splits > 1;
  int e;
  if (fuse1) {
    dg_selfcond_args g1 = plan.gemm1;
    g1.out = h;
    g1.ldo = a->hidden;
    const ReduceEpi epi{kReduceGeglu, a->hidden / plan.plan1.tile_n, nullptr, nullptr, 0};
    e = launch_selfcond(&g1, plan.plan1, stream, &epi);
    if (e) return e;
  } else {
    e = launch_selfcond(&plan.gemm1, plan.plan1, stream);
    if (e) return e;
    const int64_t n1 = (int64_t)a->M * (a->hidden / 8);
    const dim3 g1((unsigned)((n1 + kThreads - 1) / kThreads));
    if (bf) hipLaunchKernelGGL(inject_geglu<true>, g1, dim3(kThreads), 0, s, gu, h, a->M, a->hidden);
    else hipLaunchKernelGGL(inject_geglu<false>, g1, dim3(kThreads), 0, s, gu, h, a->M, a->hidden);
    e = (int)hipGetLastError();
    if (e) return e;
  }
  if (fuse2) {
    const ReduceEpi epi{kReduceAddRows, 0, a->embed, a->tokens, a->vocab};
    return launch_selfcond(&plan.gemm2, plan.plan2, stream, &epi);
  }
  e = launch_selfcond(&plan.gemm2, plan.plan2, stream);
  if (e) return e;
  const int64_t n2 = (int64_t)a->M * (a->d / 8);
  const dim3 g2((unsigned)((n2 + kThreads - 1) / kThreads));
  if (bf) hipLaunchKernelGGL(inject_add_rows<true>, g2, dim3(kThreads), 0, s, a->out, a->embed, a->tokens, a->M, a->d, a->vocab);
  else hipLaunchKernelGGL(inject_add_rows<false>, g2, dim3(kThreads), 0, s, a->out, a->embed, a->tokens, a->M, a->d, a->vocab);
  return (int)hipGetLastError();
}

}  // namespace dg
