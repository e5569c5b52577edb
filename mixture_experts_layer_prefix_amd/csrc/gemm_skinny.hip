// Decode-shaped grouped GEMM: few rows per expert, bound by streaming each
// touched expert's weights from HBM once.
//
// Same contraction and epilogues as the prefill kernel (Linear -> GELU ->
// Linear per expert, yunthe.com "MoE混合专家模型实战" reference forward).
// With a handful of tokens per expert the work is a weight stream: every
// weight byte is used for only rows_e multiply-adds.  The weights of each
// touched expert are therefore split over many workgroups along the output
// dimension, and each wavefront streams 16 NR weight rows (NR = 1 for bf16,
// 2 for INT8 weights) through v_mfma_f32_16x16x32_bf16 with the expert's
// (up to 16) token rows as the other operand, eight 16-byte loads per lane
// and row tile in flight per step (four per tile for INT8: 128 codes each).
// Workgroup (bx, e): outputs [64 NR bx, 64 NR (bx + 1)) of expert e, one
// wavefront per 16 NR outputs; experts with no rows exit at once.  Expert
// index E stands for the dense shared problem when one is present (its
// weights are always in the activation dtype; launches with INT8 routed
// weights carry none).
// KS = 4 (long reductions, Kd > Nd): a workgroup takes 16 NR outputs and its
// four wavefronts split the model dimension in quarters; the four partial
// sums are added in wavefront order through LDS.  Four times as many,
// shorter workgroups keep every CU streaming: with one wavefront per 16
// outputs the decode shape's second GEMM has about 4 workgroups per CU of
// the 5 that fit, so some CUs idle while the rest run their long loops.
#include "gemm_common.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int NTHR = 256;
constexpr int U = 8;                    // k-steps of 32 in flight (bf16 weights)
// NR 16-row MFMA tiles per wavefront: 16 * NR output features per
// wavefront, 4x that per workgroup (KS = 1).  The tiles share each
// activation fragment: INT8 weights take NR = 2, since a wavefront's
// activation loads are two thirds of its load instructions there (same-GPU:
// the decode-shaped INT8 stage 10% faster); with bf16 weights NR = 2
// measured 5% slower and NR = 1 stays.
template <bool QW>
constexpr int skinny_nr() { return QW ? 2 : 1; }

// INT8 weights (QW): a lane loads 16 codes = one 16-byte load per 64-wide
// k-block (its slice is k = 64j + 16*(lane/16) .. +16) and feeds two MFMAs
// with the first and second 8; the activations use the same permutation of
// k inside the block (the dot product does not depend on it).  The row
// scale multiplies the result before the bias.
template <bool GELU, bool QW, int KS>
__global__ __launch_bounds__(NTHR) void gemm_skinny_kernel(GemmArgs a) {
  constexpr int NR = skinny_nr<QW>();
  constexpr int NPW = 16 * NR, NPB = NPW * NTHR / 64;
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
  // KS > 1: one n0 for the whole workgroup, so the exit below is uniform
  // and every wavefront reaches the barriers of the reduction.  Nd is a
  // multiple of 64, so the NR row tiles of a wavefront lie inside it.
  const int n0 = KS == 1 ? blockIdx.x * NPB + wave * NPW : blockIdx.x * NPW;
  if (n0 >= Nd) return;
  int kb = 0, ke = Kd;   // this wavefront's part of the model dimension
  if constexpr (KS > 1) {
    const int kq = ((Kd + KS - 1) / KS + 63) / 64 * 64;
    kb = min(Kd, wave * kq);
    ke = min(Kd, kb + kq);
  }
  __shared__ f32x4 red[KS][NR][64];
  // the KS partial sums of a row group in wavefront order; wavefront 0
  // stores the result
  auto reduce = [&](f32x4 (&acc)[NR]) -> bool {
    if constexpr (KS == 1) {
      return true;
    } else {
#pragma unroll
      for (int j = 0; j < NR; ++j) red[wave][j][lane] = acc[j];
      __syncthreads();
      if (wave == 0) {
#pragma unroll
        for (int j = 0; j < NR; ++j) {
          acc[j] = red[0][j][lane];
#pragma unroll
          for (int w = 1; w < KS; ++w) acc[j] += red[w][j][lane];
        }
      }
      __syncthreads();
      return wave == 0;
    }
  };
  // 16x16 accumulator layout: element v of lane l holds row (l/16)*4 + v,
  // column l%16 of its row tile
  auto store = [&](const f32x4 (&acc)[NR], int g0, const float* sc, const float* bv) {
#pragma unroll
    for (int j = 0; j < NR; ++j) {
      const int col = n0 + 16 * j + (lane & 15);
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = g0 + (lane >> 4) * 4 + v;
        if (r < r1) {
          float z = QW ? fmaf(acc[j][v], sc[j], bv[j]) : acc[j][v] + bv[j];
          if (GELU) z = gelu_erf(z);
          C[(int64_t)r * Nd + col] = f32_to_bf16(z);
        }
      }
    }
  };
  float bv[NR], sc[NR];
#pragma unroll
  for (int j = 0; j < NR; ++j) {
    bv[j] = bias ? bf16_to_f32(bias[n0 + 16 * j + (lane & 15)]) : 0.f;
    sc[j] = QW ? a.wscale[(int64_t)e * Nd + n0 + 16 * j + (lane & 15)] : 1.f;
  }
  if constexpr (QW) {
    const int8_t* w8 = static_cast<const int8_t*>(a.W) + (int64_t)e * Nd * Kd +
                       (int64_t)(n0 + (lane & 15)) * Kd + (lane >> 4) * 16;
    constexpr int U8 = 8 / NR;        // 64-wide k-blocks in flight
    for (int g0 = r0; g0 < r1; g0 += 16) {
      const int ar = g0 + (lane & 15);
      const bool arow_ok = ar < r1;
      const uint16_t* arow = A + (int64_t)(arow_ok ? ar : r0) * Kd + (lane >> 4) * 16;
      f32x4 acc[NR];
#pragma unroll
      for (int j = 0; j < NR; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int k0 = kb; k0 < ke; k0 += 64 * U8) {
        const int nb = min(U8, (ke - k0) / 64);
        uint4 wv[NR][U8], av[U8][2];
#pragma unroll
        for (int u = 0; u < U8; ++u)
          if (u < nb) {
#pragma unroll
            for (int j = 0; j < NR; ++j)
              wv[j][u] = *reinterpret_cast<const uint4*>(w8 + (int64_t)16 * j * Kd + k0 + u * 64);
          }
#pragma unroll
        for (int u = 0; u < U8; ++u)
          if (u < nb) {
            av[u][0] = *reinterpret_cast<const uint4*>(arow + k0 + u * 64);
            av[u][1] = *reinterpret_cast<const uint4*>(arow + k0 + u * 64 + 8);
            if (!arow_ok) av[u][0] = av[u][1] = make_uint4(0, 0, 0, 0);
          }
#pragma unroll
        for (int u = 0; u < U8; ++u)
          if (u < nb) {
#pragma unroll
            for (int j = 0; j < NR; ++j) {
              const bf16x8 w0 =
                  __builtin_bit_cast(bf16x8, int8x8_to_bf16x8(make_uint2(wv[j][u].x, wv[j][u].y)));
              const bf16x8 w1 =
                  __builtin_bit_cast(bf16x8, int8x8_to_bf16x8(make_uint2(wv[j][u].z, wv[j][u].w)));
              acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av[u][0]),
                                                               w0, acc[j], 0, 0, 0);
              acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av[u][1]),
                                                               w1, acc[j], 0, 0, 0);
            }
          }
      }
      if (!reduce(acc)) continue;
      store(acc, g0, sc, bv);
    }
    return;
  }

  const int kq = (lane >> 4) * 8;      // this lane's 8-element slice of each 32-wide k-step
  const uint16_t* wrow = W + (int64_t)(n0 + (lane & 15)) * Kd + kq;
  for (int g0 = r0; g0 < r1; g0 += 16) {
    const int ar = g0 + (lane & 15);
    const bool arow_ok = ar < r1;
    const uint16_t* arow = A + (int64_t)(arow_ok ? ar : r0) * Kd + kq;
    f32x4 acc[NR];
#pragma unroll
    for (int j = 0; j < NR; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    int k0 = kb;
    for (; k0 + 32 * U <= ke; k0 += 32 * U) {
      uint4 wv[NR][U], av[U];
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int j = 0; j < NR; ++j)
          wv[j][u] = *reinterpret_cast<const uint4*>(wrow + (int64_t)16 * j * Kd + k0 + u * 32);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        av[u] = *reinterpret_cast<const uint4*>(arow + k0 + u * 32);
        if (!arow_ok) av[u] = make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int j = 0; j < NR; ++j)
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av[u]),
                                                           __builtin_bit_cast(bf16x8, wv[j][u]),
                                                           acc[j], 0, 0, 0);
    }
    for (; k0 < ke; k0 += 32) {
      uint4 av = *reinterpret_cast<const uint4*>(arow + k0);
      if (!arow_ok) av = make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int j = 0; j < NR; ++j) {
        const uint4 wv = *reinterpret_cast<const uint4*>(wrow + (int64_t)16 * j * Kd + k0);
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av),
                                                         __builtin_bit_cast(bf16x8, wv), acc[j], 0,
                                                         0, 0);
      }
    }
    if (!reduce(acc)) continue;
    store(acc, g0, sc, bv);
  }
}

}  // namespace

hipError_t launch_gemm_skinny_bf16(const GemmArgs& a, bool gelu, int /*max_rows_per_expert*/,
                                   hipStream_t s) {
  const int E = a.E + (a.As ? 1 : 0);
  if (E == 0) return hipSuccess;
  // long reductions: the four wavefronts of a workgroup split the model dimension
  const bool ks = a.Kd > a.Nd && a.Kd >= 4096;
  const int npw = 16 * (a.wscale ? skinny_nr<true>() : skinny_nr<false>());   // per wavefront
  const int per_wg = ks ? npw : npw * NTHR / 64;
  const dim3 grid((a.Nd + per_wg - 1) / per_wg, E);
  if (ks) {
    if (a.wscale && gelu)
      hipLaunchKernelGGL((gemm_skinny_kernel<true, true, 4>), grid, dim3(NTHR), 0, s, a);
    else if (a.wscale)
      hipLaunchKernelGGL((gemm_skinny_kernel<false, true, 4>), grid, dim3(NTHR), 0, s, a);
    else if (gelu)
      hipLaunchKernelGGL((gemm_skinny_kernel<true, false, 4>), grid, dim3(NTHR), 0, s, a);
    else
      hipLaunchKernelGGL((gemm_skinny_kernel<false, false, 4>), grid, dim3(NTHR), 0, s, a);
  } else if (a.wscale) {
    if (gelu)
      hipLaunchKernelGGL((gemm_skinny_kernel<true, true, 1>), grid, dim3(NTHR), 0, s, a);
    else
      hipLaunchKernelGGL((gemm_skinny_kernel<false, true, 1>), grid, dim3(NTHR), 0, s, a);
  } else {
    if (gelu)
      hipLaunchKernelGGL((gemm_skinny_kernel<true, false, 1>), grid, dim3(NTHR), 0, s, a);
    else
      hipLaunchKernelGGL((gemm_skinny_kernel<false, false, 1>), grid, dim3(NTHR), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace moe
