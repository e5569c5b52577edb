// Decode-shaped grouped GEMM: few rows per expert, bound by streaming each
// touched expert's weights from HBM once.
//
// Same contraction and epilogues as the prefill kernel (Linear -> GELU ->
// Linear per expert, yunthe.com "MoE混合专家模型实战" reference forward).
// With a handful of tokens per expert the work is a weight stream: every
// weight byte is used for only rows_e multiply-adds.  The weights of each
// touched expert are therefore split over many workgroups along the output
// dimension, and each wavefront streams 16 weight rows through
// v_mfma_f32_16x16x32_bf16 with the expert's (up to 16) token rows as the
// other operand, eight 16-byte loads per lane in flight per step.
// Workgroup (bx, e): outputs [64*bx, 64*bx + 64) of expert e, one wavefront
// per 16 outputs; experts with no rows exit at once.  Expert index E stands
// for the dense shared problem when one is present.
#include "gemm_common.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int NTHR = 256;
constexpr int NPW = 16;                 // output features per wavefront
constexpr int NPB = NPW * NTHR / 64;    // per workgroup
constexpr int U = 8;                    // k-steps of 32 in flight

template <bool GELU>
__global__ __launch_bounds__(NTHR) void gemm_skinny_kernel(GemmArgs a) {
  const int e = blockIdx.y;
  const int Kd = a.Kd, Nd = a.Nd;
  const uint16_t* A;
  const uint16_t* W;
  const uint16_t* bias = nullptr;
  uint16_t* C;
  int r0, r1;
  if (e == a.E) {
    A = static_cast<const uint16_t*>(a.As);
    W = static_cast<const uint16_t*>(a.Ws);
    C = static_cast<uint16_t*>(a.Cs);
    r0 = 0;
    r1 = a.Ts;
  } else {
    A = static_cast<const uint16_t*>(a.A);
    W = static_cast<const uint16_t*>(a.W) + (int64_t)e * Nd * Kd;
    if (a.bias) bias = static_cast<const uint16_t*>(a.bias) + (int64_t)e * Nd;
    C = static_cast<uint16_t*>(a.C);
    r0 = a.offsets[e];
    r1 = a.offsets[e + 1];
  }
  if (r1 <= r0) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n0 = blockIdx.x * NPB + wave * NPW;
  if (n0 >= Nd) return;
  const int kq = (lane >> 4) * 8;      // this lane's 8-element slice of each 32-wide k-step
  const uint16_t* wrow = W + (int64_t)(n0 + (lane & 15)) * Kd + kq;
  const float bv = bias ? bf16_to_f32(bias[n0 + (lane & 15)]) : 0.f;

  for (int g0 = r0; g0 < r1; g0 += 16) {
    const int ar = g0 + (lane & 15);
    const bool arow_ok = ar < r1;
    const uint16_t* arow = A + (int64_t)(arow_ok ? ar : r0) * Kd + kq;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    int k0 = 0;
    for (; k0 + 32 * U <= Kd; k0 += 32 * U) {
      uint4 wv[U], av[U];
#pragma unroll
      for (int u = 0; u < U; ++u) wv[u] = *reinterpret_cast<const uint4*>(wrow + k0 + u * 32);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        av[u] = *reinterpret_cast<const uint4*>(arow + k0 + u * 32);
        if (!arow_ok) av[u] = make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av[u]),
                                                      __builtin_bit_cast(bf16x8, wv[u]), acc, 0,
                                                      0, 0);
    }
    for (; k0 < Kd; k0 += 32) {
      uint4 wv = *reinterpret_cast<const uint4*>(wrow + k0);
      uint4 av = *reinterpret_cast<const uint4*>(arow + k0);
      if (!arow_ok) av = make_uint4(0, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av),
                                                    __builtin_bit_cast(bf16x8, wv), acc, 0, 0, 0);
    }
    // 16x16 accumulator layout: element v of lane l holds row (l/16)*4 + v, column l%16.
    const int col = n0 + (lane & 15);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int r = g0 + (lane >> 4) * 4 + v;
      if (r < r1) {
        float z = acc[v] + bv;
        if (GELU) z = gelu_erf(z);
        C[(int64_t)r * Nd + col] = f32_to_bf16(z);
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm_skinny_bf16(const GemmArgs& a, bool gelu, int /*max_rows_per_expert*/,
                                   hipStream_t s) {
  const int E = a.E + (a.As ? 1 : 0);
  if (E == 0) return hipSuccess;
  dim3 grid((a.Nd + NPB - 1) / NPB, E);
  if (gelu)
    hipLaunchKernelGGL(gemm_skinny_kernel<true>, grid, dim3(NTHR), 0, s, a);
  else
    hipLaunchKernelGGL(gemm_skinny_kernel<false>, grid, dim3(NTHR), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
