// Decode-shaped grouped GEMM: few rows per expert, bound by streaming each
// touched expert's weights from HBM once.
//
// Same contraction and epilogues as the prefill kernel (Linear -> GELU ->
// Linear per expert, yunthe.com "MoE混合专家模型实战" reference forward).
// With a handful of tokens per expert the work is a weight stream: every
// weight byte is used for only rows_e multiply-adds.  The weights of each
// touched expert are therefore split over many workgroups along the output
// dimension, and each wavefront streams 16 NR weight rows (NR = 2 for bf16
// and INT8, 4 for INT4 weights) through v_mfma_f32_16x16x32_bf16 with the
// expert's (up to 16) token rows as the other operand, four 16-byte loads
// per lane and row tile in flight per step (two per tile for INT8: 128 codes
// each, one for INT4).
// Workgroup (bx, e): outputs [64 NR bx, 64 NR (bx + 1)) of expert e, one
// wavefront per 16 NR outputs; experts with no rows exit at once.  Expert
// index E stands for the dense shared problem when one is present (its
// weights are always in the activation dtype; launches with INT8 routed
// weights carry none).
// KS = 4 (long reductions, Kd >= 2048): a
// workgroup takes 16 NR outputs and its
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
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int NTHR = 256;
constexpr int U = 4;                    // k-steps of 32 in flight (bf16 weights)
// NR 16-row MFMA tiles per wavefront: 16 * NR output features per
// wavefront, 4x that per workgroup (KS = 1).  The tiles share each
// activation fragment: INT8 weights take NR = 2, since a wavefront's
// activation loads are two thirds of its load instructions there (same-GPU:
// the decode-shaped INT8 stage 10% faster).  With the k-split of every
// Kd >= 2048 (below), bf16 weights take NR = 2 too and 4 k-steps in flight,
// INT8 codes 2 k-blocks (same-GPU A/B, two runs each: bf16 0.564 -> 0.537
// ms, INT8 0.378 -> 0.356 ms; bf16 with NR = 1 and 8 k-steps had been the
// better choice before the k-split).
template <bool QW, bool Q4 = false>
constexpr int skinny_nr() { return Q4 ? 4 : 2; }

// INT8 weights (QW): a lane loads 16 codes = one 16-byte load per 64-wide
// k-block (its slice is k = 64j + 16*(lane/16) .. +16) and feeds two MFMAs
// with the first and second 8; the activations use the same permutation of
// k inside the block (the dot product does not depend on it).  The row
// scale multiplies the result before the bias.
// INT4 weights (Q4, with QW): a lane loads 16 bytes = 32 codes per 128-wide
// k-block (its slice is k = 128j + 32*(lane/16) .. +32) and feeds four MFMAs
// with 8 codes each, activations in the same order of k; four 16-row tiles
// per wavefront share each activation load (64 outputs per wavefront).  The
// codes are widened as bf16(136 + q) (int4x8_to_bf16x8_o136), and one more
// MFMA per 32 k multiplies the activations by a constant -136 into a
// separate accumulator that is added to every tile: sum x (q + 136) -
// 136 sum x = sum x q, with an fp32 cancellation error near 2e-5 of the
// result for unit-scale activations (bf16 output rounding: 4e-3).
template <bool GELU, bool QW, int KS, bool Q4 = false>
__global__ __launch_bounds__(NTHR) void gemm_skinny_kernel(GemmArgs a) {
  constexpr int NR = skinny_nr<QW, Q4>();
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
    constexpr int KA = Q4 ? 128 : 64;   // k-block of one load step
    const int kq = ((Kd + KS - 1) / KS + KA - 1) / KA * KA;
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
          if (GELU) z = gelu_as(z);
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
  if constexpr (Q4) {
    const int Kb = Kd / 2;             // bytes per row of codes
    const uint8_t* w4 = static_cast<const uint8_t*>(a.W) + (int64_t)e * Nd * Kb +
                        (int64_t)(n0 + (lane & 15)) * Kb + (lane >> 4) * 16;
    // one 128-wide k-block per step: more registers for a deeper stream
    // measured slower (two blocks 0.24 ms, three 0.26, four 0.29, and with
    // the next block's codes loaded a step ahead 0.27-0.28, against 0.22 for
    // one: the wavefronts per SIMD, not the loads in flight, set the rate)
    // codes widened with the +136 offset; kM136 carries the correction
    const bf16x8 kM136 = __builtin_bit_cast(
        bf16x8, make_uint4(0xC308C308u, 0xC308C308u, 0xC308C308u, 0xC308C308u));   // -136
    for (int g0 = r0; g0 < r1; g0 += 16) {
      const int ar = g0 + (lane & 15);
      const bool arow_ok = ar < r1;
      const uint16_t* arow = A + (int64_t)(arow_ok ? ar : r0) * Kd + (lane >> 4) * 32;
      f32x4 acc[NR], accm = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < NR; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
      for (int k0 = kb; k0 < ke; k0 += 128) {
        uint4 wv[NR], av[4];
#pragma unroll
        for (int j = 0; j < NR; ++j)
          wv[j] = *reinterpret_cast<const uint4*>(w4 + (int64_t)16 * j * Kb + k0 / 2);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          av[m] = *reinterpret_cast<const uint4*>(arow + k0 + 8 * m);
          if (!arow_ok) av[m] = make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const bf16x8 am = __builtin_bit_cast(bf16x8, av[m]);
#pragma unroll
          for (int j = 0; j < NR; ++j) {
            const uint32_t wd = m == 0 ? wv[j].x : m == 1 ? wv[j].y : m == 2 ? wv[j].z : wv[j].w;
            acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                am, __builtin_bit_cast(bf16x8, int4x8_to_bf16x8_o136(wd)), acc[j], 0, 0, 0);
          }
          accm = __builtin_amdgcn_mfma_f32_16x16x32_bf16(am, kM136, accm, 0, 0, 0);
        }
      }
      // every column of accm holds -136 * sum_k x[row, k] over this
      // wavefront's k-range: the same element layout as acc[j]
#pragma unroll
      for (int j = 0; j < NR; ++j) acc[j] += accm;
      if (!reduce(acc)) continue;
      store(acc, g0, sc, bv);
    }
    return;
  } else if constexpr (QW) {
    const int8_t* w8 = static_cast<const int8_t*>(a.W) + (int64_t)e * Nd * Kd +
                       (int64_t)(n0 + (lane & 15)) * Kd + (lane >> 4) * 16;
    constexpr int U8 = 2;             // 64-wide k-blocks in flight
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
            // rows past the expert's block issue no loads (most of the 16 on
            // decode shapes; same-GPU, the INT8 stage 0.356 -> 0.340 ms,
            // while the bf16 and INT4 loops measured no gain or a loss)
            av[u][0] = av[u][1] = make_uint4(0, 0, 0, 0);
            if (arow_ok) {
              av[u][0] = *reinterpret_cast<const uint4*>(arow + k0 + u * 64);
              av[u][1] = *reinterpret_cast<const uint4*>(arow + k0 + u * 64 + 8);
            }
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

// k-major weights: the backward's input gradients (d_h = d_y W2_e, d_x_perm =
// d_z W1_e) read the forward's weights as W_e [Kd, Nd] with Nd contiguous,
// so a 16-byte load holds one k of several output columns while the MFMA
// wants 8 consecutive k of one column in a lane.  Each lane loads 8 rows of
// W (k = 8 (lane/16) + t of the 32-wide k-step, t = 0..7) at its 4 columns
// n0 + 4 (lane%16) .. +3, 8 bytes each (16 lanes read 128 contiguous bytes
// of a row), and transposes the 8 x 4 block in registers: one v_perm_b32 per
// output dword, joining the same half of two rows.  MFMA c (c = 0..3) then
// produces columns n0 + 4 (lane%16) + c, so a lane's 4 results of an output
// row are adjacent: 8-byte stores, 128 contiguous bytes per row and lane
// group.  Up to 32 rows (two 16-row groups sharing each weight fragment) per
// pass over the weights.  A wavefront covers 64 columns; workgroups split
// long reductions over their 4 wavefronts as above (KS = 4).
template <int RG, int UK>
__device__ __forceinline__ void kmaj_pass(const uint16_t* __restrict__ A,
                                          __amdgpu_buffer_rsrc_t wr, uint32_t loff, int Kd, int Nd,
                                          int g0, int r0, int r1, int kb, int ke, int lane,
                                          f32x4 (&acc)[2][4]) {
  // buffer loads of W_e: row k's byte offset k * rb is wave-uniform (the
  // scalar offset), this lane's place in the row the vector offset loff, so
  // every load shares one address register
  const uint32_t rb = (uint32_t)Nd * 2u;
  auto wload = [&](int k) -> uint2 {
    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(wr, loff, (int)((uint32_t)k * rb), 0);
    return make_uint2(v.x, v.y);
  };
  const uint16_t* arow[RG];
  bool aok[RG];
#pragma unroll
  for (int q = 0; q < RG; ++q) {
    const int ar = g0 + 16 * q + (lane & 15);
    aok[q] = ar < r1;
    arow[q] = A + (int64_t)(aok[q] ? ar : r0) * Kd + (lane >> 4) * 8;
  }
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[q][c] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto step = [&](const uint2 (&wv)[8], const uint4 (&av)[RG]) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
      uint32_t dw[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const uint32_t lo = (c >> 1) ? wv[2 * m].y : wv[2 * m].x;
        const uint32_t hi = (c >> 1) ? wv[2 * m + 1].y : wv[2 * m + 1].x;
        dw[m] = __builtin_amdgcn_perm(hi, lo, sel);
      }
      const bf16x8 b = __builtin_bit_cast(bf16x8, make_uint4(dw[0], dw[1], dw[2], dw[3]));
#pragma unroll
      for (int q = 0; q < RG; ++q)
        acc[q][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av[q]), b,
                                                            acc[q][c], 0, 0, 0);
    }
  };
  int k0 = kb;
  for (; k0 + 32 * UK <= ke; k0 += 32 * UK) {
    uint2 wv[UK][8];
    uint4 av[UK][RG];
#pragma unroll
    for (int u = 0; u < UK; ++u)
#pragma unroll
      for (int t = 0; t < 8; ++t) wv[u][t] = wload(k0 + 32 * u + t);
#pragma unroll
    for (int u = 0; u < UK; ++u)
#pragma unroll
      for (int q = 0; q < RG; ++q) {
        av[u][q] = *reinterpret_cast<const uint4*>(arow[q] + k0 + 32 * u);
        if (!aok[q]) av[u][q] = make_uint4(0, 0, 0, 0);
      }
#pragma unroll
    for (int u = 0; u < UK; ++u) step(wv[u], av[u]);
  }
  for (; k0 < ke; k0 += 32) {
    uint2 wv[8];
    uint4 av[RG];
#pragma unroll
    for (int t = 0; t < 8; ++t) wv[t] = wload(k0 + t);
#pragma unroll
    for (int q = 0; q < RG; ++q) {
      av[q] = *reinterpret_cast<const uint4*>(arow[q] + k0);
      if (!aok[q]) av[q] = make_uint4(0, 0, 0, 0);
    }
    step(wv, av);
  }
}

// k-steps of 32 in flight: 4 with one 16-row group, 2 with two (the same
// registers)
#ifndef KMAJ_UK1
#define KMAJ_UK1 4
#endif
#ifndef KMAJ_UK2
#define KMAJ_UK2 2
#endif
template <int KS>
__global__ __launch_bounds__(NTHR) void gemm_skinny_kmaj_kernel(GemmArgs a) {
  constexpr int NPW = 64, NPB = NPW * NTHR / 64;
  const int e = blockIdx.y;
  const int Kd = a.Kd, Nd = a.Nd;
  const uint16_t* A;
  const uint16_t* W;
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
    C = static_cast<uint16_t*>(a.C);
    r0 = a.offsets[e];
    r1 = a.offsets[e + 1];
  }
  if (r1 <= r0) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // KS > 1: one n0 for the whole workgroup (uniform exit, every wavefront
  // reaches the reduction's barriers); Nd is a multiple of 64
  const int n0 = KS == 1 ? blockIdx.x * NPB + wave * NPW : blockIdx.x * NPW;
  if (n0 >= Nd) return;
  int kb = 0, ke = Kd;
  if constexpr (KS > 1) {
    const int kq = ((Kd + KS - 1) / KS + 31) / 32 * 32;
    kb = min(Kd, __builtin_amdgcn_readfirstlane(wave) * kq);
    ke = min(Kd, kb + kq);
  }
  // this lane's rows 8 (lane/16) + t of every k-step, columns n0 + 4 (lane%16)
  // .. +3, as a byte offset from the row's start
  // Kd * Nd * 2 < 2^32 bytes (d_model * d_ff < 2^31)
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(W), (short)0, (int)((uint32_t)Kd * (uint32_t)Nd * 2u), 0x00020000);
  const uint32_t loff = (uint32_t)((8 * (lane >> 4)) * Nd + n0 + 4 * (lane & 15)) * 2u;
  __shared__ f32x4 red[KS][2][4][64];
  for (int g0 = r0; g0 < r1; g0 += 32) {
    f32x4 acc[2][4];
    // the row count is uniform over the workgroup: every wavefront takes the
    // same branch and reaches the barriers below
    const int ng = r1 - g0 > 16 ? 2 : 1;
    if (ng == 2)
      kmaj_pass<2, KMAJ_UK2>(A, wr, loff, Kd, Nd, g0, r0, r1, kb, ke, lane, acc);
    else
      kmaj_pass<1, KMAJ_UK1>(A, wr, loff, Kd, Nd, g0, r0, r1, kb, ke, lane, acc);
    if constexpr (KS > 1) {
#pragma unroll
      for (int q = 0; q < 2; ++q)
        if (q < ng) {
#pragma unroll
          for (int c = 0; c < 4; ++c) red[wave][q][c][lane] = acc[q][c];
        }
      __syncthreads();
      if (wave == 0) {
#pragma unroll
        for (int q = 0; q < 2; ++q)
          if (q < ng) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              acc[q][c] = red[0][q][c][lane];
#pragma unroll
              for (int w = 1; w < KS; ++w) acc[q][c] += red[w][q][c][lane];
            }
          }
      }
      __syncthreads();
      if (wave != 0) continue;
    }
    // 16x16 accumulator layout: element v of lane l holds row (l/16)*4 + v of
    // its group, column l%16 of the MFMA, i.e. output column n0 + 4 (l%16) + c
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int r = g0 + 16 * q + (lane >> 4) * 4 + v;
        if (q < ng && r < r1) {
          const uint32_t lo = (uint32_t)f32_to_bf16(acc[q][0][v]) |
                              ((uint32_t)f32_to_bf16(acc[q][1][v]) << 16);
          const uint32_t hi = (uint32_t)f32_to_bf16(acc[q][2][v]) |
                              ((uint32_t)f32_to_bf16(acc[q][3][v]) << 16);
          *reinterpret_cast<uint2*>(C + (int64_t)r * Nd + n0 + 4 * (lane & 15)) = make_uint2(lo, hi);
        }
      }
  }
}

}  // namespace

hipError_t launch_gemm_skinny_bf16(const GemmArgs& a, bool gelu, int /*max_rows_per_expert*/,
                                   hipStream_t s) {
  const int E = a.E + (a.As ? 1 : 0);
  if (E == 0) return hipSuccess;
  // long reductions: the four wavefronts of a workgroup split the model
  // dimension whenever it is at least 2048 (four times as many, shorter
  // workgroups; same-GPU A/B of the decode-shaped stage, whose first GEMM
  // has Kd = 4096 < Nd: INT4 0.248 -> 0.235 ms, INT8 0.393 -> 0.379 ms,
  // bf16 0.577 -> 0.564 ms)
  const bool q4 = a.wscale && a.w4;
  const bool ks = a.Kd >= 2048;
  const int npw = 16 * (q4 ? skinny_nr<true, true>()
                           : (a.wscale ? skinny_nr<true>() : skinny_nr<false>()));   // per wavefront
  const int per_wg = ks ? npw : npw * NTHR / 64;
  const dim3 grid((a.Nd + per_wg - 1) / per_wg, E);
  if (q4) {
    if (ks && gelu)
      hipLaunchKernelGGL((gemm_skinny_kernel<true, true, 4, true>), grid, dim3(NTHR), 0, s, a);
    else if (ks)
      hipLaunchKernelGGL((gemm_skinny_kernel<false, true, 4, true>), grid, dim3(NTHR), 0, s, a);
    else if (gelu)
      hipLaunchKernelGGL((gemm_skinny_kernel<true, true, 1, true>), grid, dim3(NTHR), 0, s, a);
    else
      hipLaunchKernelGGL((gemm_skinny_kernel<false, true, 1, true>), grid, dim3(NTHR), 0, s, a);
  } else if (ks) {
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

hipError_t launch_gemm_skinny_kmaj_bf16(const GemmArgs& a, hipStream_t s) {
  const int E = a.E + (a.As ? 1 : 0);
  if (E == 0) return hipSuccess;
  // the same k-split rule as the n-major kernel
  const bool ks = a.Kd >= 2048;
  const int per_wg = ks ? 64 : 64 * NTHR / 64;
  const dim3 grid((a.Nd + per_wg - 1) / per_wg, E);
  if (ks)
    hipLaunchKernelGGL((gemm_skinny_kmaj_kernel<4>), grid, dim3(NTHR), 0, s, a);
  else
    hipLaunchKernelGGL((gemm_skinny_kmaj_kernel<1>), grid, dim3(NTHR), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
