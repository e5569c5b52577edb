// Router scoring, then Top-K selection and the softmax over the K chosen
// logits.
//
// What it computes (lmnt.cn MoE walkthrough §2.1, gate scoring equation
// score = Softmax(TopK(W_g . x)), TopK taken before the softmax so the K
// weights are normalised within the candidate set; yunthe.com "MoE混合专家
// 模型实战", reference forward: Linear router, topk, softmax over the K
// values; yunthe.com aux-loss section: a per-expert bias b_i that steers the
// routing score):
//   logit[t,e] = fp32( (sum_j x[t,j] W_r[e,j]) + b_r[e] + off[e] ), the dot
//                product accumulated in fp64 (bf16*bf16 and fp32*fp32
//                products are exact in fp64), one rounding at the end;
//   s[t,e]     = fp32(logit[t,e] + sel_bias[e]);
//   idx[t,:]   = the K experts of largest s, ordered by (s desc, e asc),
//                NaN ordering as -inf;
//   w[t,k]     = exp(logit[idx_k] - max) / sum over the K chosen, in fp64.
//
// Two kernels:
//   1. router GEMM on the fp64 matrix cores (v_mfma_f64_16x16x4f64): each
//      workgroup takes a tile of tokens x experts and one slice of the model
//      dimension, and writes fp64 partial dot products.  The slice count S
//      is chosen so that there are about four workgroups per CU.  Each lane
//      feeds the MFMA from 16 consecutive elements of its row (one 32- or
//      64-byte load), so the k order inside a 64-wide chunk is permuted
//      identically for x and W_r -- the dot product does not depend on it;
//   2. select: one wavefront per token sums the S partials in slice order,
//      adds the router bias and offset in fp64, rounds once to fp32, writes
//      the logits, and picks the Top-K with a 64-lane arg-max reduction;
//      optionally it also writes the per-block routing partials of the aux
//      loss (lmnt.cn §5.1-5.2), the router z-loss (§5.3) and the routing
//      statistics (§8.2) from the row it holds.
//
// Certified path for bf16 routers (the same Top-K, order and weights'
// inputs for the K chosen experts, far fewer fp64 operations):
//   1'. router GEMM on the bf16 matrix cores (v_mfma_f32_16x16x32_bf16):
//      each MFMA sums 32 exact products in fp32 from zero, its result is
//      added to an fp64 accumulator, and each slice of the model dimension
//      is written as one fp32 partial; the same workgroups also write
//      per-slice fp32 sums of squares of the x rows and of the W_r rows;
//   2'. select, with a prologue: the fp32 slices are added in fp64 to an
//      approximation z' of each dot product z, with |z' - z| <= B[t,e] =
//      c0 * ||x_t|| * ||W_r[e]|| + c1 * (||x_t|| + ||W_r[e]|| + 1)
//      (the accumulation error bound with Cauchy-Schwarz for sum |x||w|; c0
//      and c1 at the launcher).  Each expert's selection
//      score then lies in [lo, hi] = score(z' - B), score(z' + B) (every
//      step from z to the score -- fp64 adds, the fp32 rounding, the fp32
//      add of the selection bias -- is monotone).  With theta the K-th
//      largest lo, the experts with hi >= theta (the candidates) contain
//      the exact Top-K, and every other expert's score, approximate or
//      exact, is below the K-th exact score.  A candidate whose interval
//      is disjoint from every other candidate's has a certain rank among
//      them; the candidates whose intervals meet another's get their dot
//      products recomputed in fp64 (lanes across the model dimension)
//      before the selection, which then compares exact values wherever the
//      order is open.  With exactly K candidates and no meeting intervals
//      the token is certified as it is.  A row with any non-finite value is
//      recomputed whole.
//   The logits the certified path writes are exact (as in path 1-2) for the
//   recomputed experts and within B of the exact dot product elsewhere.
#include <math.h>

#include "moe_internal.h"

namespace moe {
namespace {

typedef double f64x4 __attribute__((ext_vector_type(4)));

constexpr int KC = 64;   // model-dimension chunk per iteration (16 per lane group)

template <typename T>
struct Row16;
// 16 consecutive bf16 (8 dwords)
template <>
struct Row16<uint16_t> {
  uint4 v[2];
  __device__ __forceinline__ void load(const uint16_t* p) {
    v[0] = reinterpret_cast<const uint4*>(p)[0];
    v[1] = reinterpret_cast<const uint4*>(p)[1];
  }
  __device__ __forceinline__ double get(int i) const {
    const uint32_t w = (i < 8 ? (&v[0].x)[i >> 1] : (&v[1].x)[(i - 8) >> 1]);
    const uint32_t b = (i & 1) ? (w & 0xffff0000u) : (w << 16);
    return (double)__uint_as_float(b);
  }
};
// 16 consecutive fp32 (16 dwords)
template <>
struct Row16<float> {
  uint4 v[4];
  __device__ __forceinline__ void load(const float* p) {
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = reinterpret_cast<const uint4*>(p)[i];
  }
  __device__ __forceinline__ double get(int i) const {
    return (double)__uint_as_float((&v[i >> 2].x)[i & 3]);
  }
};

// Workgroup: 4 wavefronts stacked along tokens; wavefront tile = (WT*16)
// tokens x (WE*16) experts.  grid = (token tiles, expert tiles, slices).
template <typename T, int WT, int WE>
__global__ __launch_bounds__(256) void router_gemm_kernel(const T* __restrict__ x,
                                                          const T* __restrict__ wr,
                                                          double* __restrict__ part, int Ttok,
                                                          int d, int N, int klen) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t0 = (blockIdx.x * 4 + wave) * WT * 16;
  const int e0 = blockIdx.y * WE * 16;
  const int kb = blockIdx.z * klen, ke = min(d, kb + klen);
  if (t0 >= Ttok) return;
  const int g = lane >> 4;        // lane group: k offset 16*g inside a chunk
  const int r = lane & 15;        // row inside a 16-row MFMA tile

  const T* xrow[WT];
  const T* wrow[WE];
#pragma unroll
  for (int i = 0; i < WT; ++i) xrow[i] = x + (int64_t)min(t0 + i * 16 + r, Ttok - 1) * d + g * 16;
#pragma unroll
  for (int j = 0; j < WE; ++j) wrow[j] = wr + (int64_t)min(e0 + j * 16 + r, N - 1) * d + g * 16;

  f64x4 acc[WT][WE];
#pragma unroll
  for (int i = 0; i < WT; ++i)
#pragma unroll
    for (int j = 0; j < WE; ++j) acc[i][j] = f64x4{0.0, 0.0, 0.0, 0.0};

  // chunk c of the slice; the loads of chunk c+1 are in flight during the
  // products of chunk c (a chunk past the slice re-reads its last one)
  const int nch = (ke - kb) / KC;
  auto load = [&](int c, Row16<T>* xa, Row16<T>* wb) {
    const int k0 = kb + min(c, nch - 1) * KC;
#pragma unroll
    for (int i = 0; i < WT; ++i) xa[i].load(xrow[i] + k0);
#pragma unroll
    for (int j = 0; j < WE; ++j) wb[j].load(wrow[j] + k0);
  };
  auto mma = [&](const Row16<T>* xa, const Row16<T>* wb) {
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      double a[WT], b[WE];
#pragma unroll
      for (int i = 0; i < WT; ++i) a[i] = xa[i].get(s);
#pragma unroll
      for (int j = 0; j < WE; ++j) b[j] = wb[j].get(s);
#pragma unroll
      for (int i = 0; i < WT; ++i)
#pragma unroll
        for (int j = 0; j < WE; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  };
  Row16<T> xa0[WT], wb0[WE], xa1[WT], wb1[WE];
  load(0, xa0, wb0);
  int c = 0;
  for (; c + 1 < nch; c += 2) {
    load(c + 1, xa1, wb1);
    __builtin_amdgcn_sched_barrier(0);
    mma(xa0, wb0);
    __builtin_amdgcn_sched_barrier(0);
    load(c + 2, xa0, wb0);
    __builtin_amdgcn_sched_barrier(0);
    mma(xa1, wb1);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (c < nch) mma(xa0, wb0);
  // 16x16 fp64 accumulator: element v of lane l is row 4*v + l/16, column l%16.
  double* out = part + (int64_t)blockIdx.z * Ttok * N;
#pragma unroll
  for (int i = 0; i < WT; ++i)
#pragma unroll
    for (int j = 0; j < WE; ++j) {
      const int e = e0 + j * 16 + r;
      if (e >= N) continue;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int t = t0 + i * 16 + v * 4 + g;
        if (t < Ttok) out[(int64_t)t * N + e] = acc[i][j][v];
      }
    }
}

// ---------------------------------------------------------------- certified path
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

typedef double f64x4v __attribute__((ext_vector_type(4)));

// Sum of squares of 8 bf16 (exact squares, one rounding per add).
__device__ __forceinline__ float sq8(u32x4 v, float acc) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float a = __uint_as_float(v[q] << 16), b = __uint_as_float(v[q] & 0xffff0000u);
    acc = fmaf(a, a, acc);
    acc = fmaf(b, b, acc);
  }
  return acc;
}

// Wavefront tile of the certified path: FI x FJ blocks of 16 x 16 (64 tokens x
// 32 experts); its fp64 accumulators take 64 registers.
constexpr int FI = 4, FJ = 2;

// Workgroup: 4 wavefronts as TW = 4 / EW token groups x EW expert groups.
// grid = (token tiles, expert tiles, slices).  Per 32-wide step of the model
// dimension the workgroup's 64 TW x rows go through LDS (each thread moves
// TW 16-byte pieces; two stages, loads two steps ahead), so the EW
// wavefronts of a token group share them; row r's piece p sits at piece
// p ^ ((r >> 2) & 3), so the 16 rows one read instruction touches fall in
// distinct banks.  Each lane loads its W_r pieces (8 consecutive elements
// of row l % 16 at offset 8 (l / 16)) straight into registers, also two
// steps ahead.  Every MFMA starts from zero and its fp32 result -- 32 exact
// bf16 products summed -- is added at once to an fp64 accumulator, so the
// fp32 error of each block stays that of one 32-term sum.  Wavefronts of
// expert group 0 also add up the squares of their x rows and those of token
// group 0 the squares of their W_r rows (fp32, per slice).
template <int EW>
__global__ __launch_bounds__(256) void router_mfma_kernel(const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ wr,
                                                          float* __restrict__ part,
                                                          float* __restrict__ nx2,
                                                          float* __restrict__ nw2, int Ttok,
                                                          int d, int N, int klen) {
  constexpr int TW = 4 / EW, XR = 16 * FI * TW;     // x rows per workgroup
  __shared__ __align__(16) uint16_t xs[2][XR * 32];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tt = wave / EW;
  const int tg = blockIdx.x * TW + tt, eg = blockIdx.y * EW + wave % EW;
  const int tw0 = blockIdx.x * XR, t0 = tg * 16 * FI, e0 = eg * 16 * FJ;
  const bool active = t0 < Ttok && e0 < N;     // (inactive wavefronts still move x)
  const int kb = blockIdx.z * klen, ke = min(d, kb + klen);
  const int r = lane & 15, g = lane >> 4;
  const bool do_x = eg == 0, do_w = tg == 0;
  const uint16_t* xsrc[TW];
  int xdst[TW];
#pragma unroll
  for (int h = 0; h < TW; ++h) {
    const int q = tid + 256 * h, row = q >> 2, pc = q & 3;
    xsrc[h] = x + (int64_t)min(tw0 + row, Ttok - 1) * d + 8 * pc;
    xdst[h] = row * 32 + ((pc ^ ((row >> 2) & 3)) * 8);
  }
  int xrd[FI];
#pragma unroll
  for (int i = 0; i < FI; ++i) xrd[i] = (tt * 16 * FI + 16 * i + r) * 32 + ((g ^ ((r >> 2) & 3)) * 8);
  const uint16_t* wrow[FJ];
#pragma unroll
  for (int j = 0; j < FJ; ++j) wrow[j] = wr + (int64_t)min(e0 + 16 * j + r, N - 1) * d + 8 * g;
  f64x4v acc[FI][FJ];
#pragma unroll
  for (int i = 0; i < FI; ++i)
#pragma unroll
    for (int j = 0; j < FJ; ++j) acc[i][j] = f64x4v{0.0, 0.0, 0.0, 0.0};
  float sx[FI], sw[FJ];
#pragma unroll
  for (int i = 0; i < FI; ++i) sx[i] = 0.f;
#pragma unroll
  for (int j = 0; j < FJ; ++j) sw[j] = 0.f;

  const int nst = (ke - kb) / 32;
  auto kof = [&](int c) { return kb + min(c, nst - 1) * 32; };
  auto gx = [&](int c, u32x4 (&xq)[TW]) {
#pragma unroll
    for (int h = 0; h < TW; ++h) xq[h] = *reinterpret_cast<const u32x4*>(xsrc[h] + kof(c));
  };
  auto sxs = [&](int st, const u32x4 (&xq)[TW]) {
#pragma unroll
    for (int h = 0; h < TW; ++h) *reinterpret_cast<u32x4*>(&xs[st][xdst[h]]) = xq[h];
  };
  auto gw = [&](int c, u32x4 (&wq)[FJ]) {
#pragma unroll
    for (int j = 0; j < FJ; ++j) wq[j] = *reinterpret_cast<const u32x4*>(wrow[j] + kof(c));
  };
  auto step = [&](int st, const u32x4 (&wb)[FJ]) {
    if (!active) return;
    u32x4 xa[FI];
#pragma unroll
    for (int i = 0; i < FI; ++i) xa[i] = *reinterpret_cast<const u32x4*>(&xs[st][xrd[i]]);
#pragma unroll
    for (int i = 0; i < FI; ++i)
#pragma unroll
      for (int j = 0; j < FJ; ++j) {
        const f32x4 p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, xa[i]), __builtin_bit_cast(bf16x8, wb[j]),
            f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[i][j][v] += (double)p[v];
      }
    if (do_x)
#pragma unroll
      for (int i = 0; i < FI; ++i) sx[i] = sq8(xa[i], sx[i]);
    if (do_w)
#pragma unroll
      for (int j = 0; j < FJ; ++j) sw[j] = sq8(wb[j], sw[j]);
  };
  // stage 0 holds x(c) and wA = W(c) at the top of each iteration; xB = x(c+1),
  // wB = W(c+1) loaded; xA = x(c+2) in flight (steps past the slice re-read
  // its last one)
  u32x4 xA[TW], xB[TW], wA[FJ], wB[FJ];
  gx(0, xA);
  gw(0, wA);
  gx(1, xB);
  gw(1, wB);
  sxs(0, xA);
  __syncthreads();
  gx(2, xA);
  for (int c = 0; c < nst; c += 2) {
    step(0, wA);
    sxs(1, xB);
    gw(c + 2, wA);
    gx(c + 3, xB);
    __syncthreads();
    if (c + 1 >= nst) break;
    step(1, wB);
    sxs(0, xA);
    gw(c + 3, wB);
    gx(c + 4, xA);
    __syncthreads();
  }
  if (!active) return;

  // 16x16 accumulator: element v of lane l is row 4 (l / 16) + v, column l % 16.
  float* out = part + (int64_t)blockIdx.z * Ttok * N;
#pragma unroll
  for (int i = 0; i < FI; ++i)
#pragma unroll
    for (int j = 0; j < FJ; ++j) {
      const int e = e0 + 16 * j + r;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int t = t0 + 16 * i + 4 * g + v;
        if (t < Ttok && e < N) out[(int64_t)t * N + e] = (float)acc[i][j][v];
      }
    }
  // row sums of squares: the four lanes holding a row's pieces, fixed pairing
  if (do_x)
#pragma unroll
    for (int i = 0; i < FI; ++i) {
      float q = sx[i];
      q += __shfl_xor(q, 16, 64);
      q += __shfl_xor(q, 32, 64);
      const int t = t0 + 16 * i + r;
      if (g == 0 && t < Ttok) nx2[(int64_t)blockIdx.z * Ttok + t] = q;
    }
  if (do_w)
#pragma unroll
    for (int j = 0; j < FJ; ++j) {
      float q = sw[j];
      q += __shfl_xor(q, 16, 64);
      q += __shfl_xor(q, 32, 64);
      const int e = e0 + 16 * j + r;
      if (g == 0 && e < N) nw2[(int64_t)blockIdx.z * N + e] = q;
    }
}

__device__ __forceinline__ bool better(float sa, int ea, float sb, int eb) {
  return sa > sb || (sa == sb && ea < eb);
}

// Inputs of the certified select prologue.
struct CertIn {
  const float* part;     // [S, T, N] fp32 slice partials of the dot products
  const float* nx2;      // [S, T] slice sums of squares of the x rows
  const float* nw2;      // [S, N] slice sums of squares of the W_r rows
  const uint16_t* x;     // [T, d] bf16, for the recomputation
  const uint16_t* wr;    // [N, d] bf16
  int S, d;
  double c0, c1;         // error bound coefficients
};

// sum_j x[j] w[j] in fp64 (exact products), lanes across 8-element pieces,
// eight pieces' loads in flight together and four independent accumulators
// (added in a fixed order), then a fixed butterfly: every lane returns the
// same value.
__device__ __forceinline__ double dot_f64(const uint16_t* xr, const uint16_t* wrow, int d,
                                          int lane) {
  constexpr int U = 8;
  double a[4] = {0.0, 0.0, 0.0, 0.0};
  const int nc = d / 8;
  for (int c0 = lane; c0 < nc; c0 += 64 * U) {
    u32x4 xv[U], wv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + 64 * u;
      if (c < nc) {
        xv[u] = *reinterpret_cast<const u32x4*>(xr + 8 * c);
        wv[u] = *reinterpret_cast<const u32x4*>(wrow + 8 * c);
      } else {
        xv[u] = u32x4{0u, 0u, 0u, 0u};
        wv[u] = u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        a[q] = fma((double)__uint_as_float(xv[u][q] << 16), (double)__uint_as_float(wv[u][q] << 16),
                   a[q]);
        a[q] = fma((double)__uint_as_float(xv[u][q] & 0xffff0000u),
                   (double)__uint_as_float(wv[u][q] & 0xffff0000u), a[q]);
      }
  }
  double r = (a[0] + a[1]) + (a[2] + a[3]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) r += __shfl_xor(r, off, 64);
  return r;
}

// CERT: the dot products come from the bf16 matrix-core kernel's fp32 slices
// and are certified or recomputed first (the prologue below; the rest of the
// kernel is the same for both paths).
template <bool PART, bool CERT>
__global__ __launch_bounds__(256) void select_kernel(
    const double* __restrict__ part, int S, const float* __restrict__ b_router,
    const float* __restrict__ logit_offset, const float* __restrict__ sel_bias,
    float* __restrict__ logits, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    int Ttok, int N, int K, RoutePartials rp, CertIn ci) {
  const int wave = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wave;
  const bool valid = t < Ttok;
  if (!PART && !valid) return;   // (with partials every wavefront reaches the barrier)
  const int lane = threadIdx.x & 63;
  // z -> logit -> selection score, each step monotone in z
  auto logit_of = [&](double z, int e) -> float {
    if (b_router) z += (double)b_router[e];
    if (logit_offset) z += (double)logit_offset[e];
    return (float)z;
  };
  auto score_of = [&](float l, int e) -> float {
    return sel_bias ? __fadd_rn(l, sel_bias[e]) : l;
  };
  double zs[4] = {0.0, 0.0, 0.0, 0.0};
  if constexpr (!CERT) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int e = lane + 64 * v;
      if (valid && e < N) {
        // the slices in order; eight loads in flight before their adds
        double z = part[(int64_t)t * N + e];
        int s = 1;
        for (; s + 8 <= S; s += 8) {
          double q[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) q[u] = part[((int64_t)(s + u) * Ttok + t) * N + e];
#pragma unroll
          for (int u = 0; u < 8; ++u) z += q[u];
        }
        for (; s < S; ++s) z += part[((int64_t)s * Ttok + t) * N + e];
        zs[v] = z;
      }
    }
  } else if (valid) {
    // approximate dot products z' (slices in order) and the bound B of |z' - z|
    double nx = 0.0;
    for (int s = 0; s < ci.S; ++s) nx += (double)ci.nx2[(int64_t)s * Ttok + t];
    nx = sqrt(nx);
    float lo[4], hi[4];
    bool ok = true;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int e = lane + 64 * v;
      lo[v] = hi[v] = -INFINITY;
      if (e < N) {
        double z = 0.0, nw = 0.0;
        for (int s0 = 0; s0 < ci.S; s0 += 8) {
          float q[8], qw[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int s = min(s0 + u, ci.S - 1);
            q[u] = ci.part[((int64_t)s * Ttok + t) * N + e];
            qw[u] = ci.nw2[(int64_t)s * N + e];
          }
#pragma unroll
          for (int u = 0; u < 8; ++u)
            if (s0 + u < ci.S) {
              z += (double)q[u];
              nw += (double)qw[u];
            }
        }
        nw = sqrt(nw);
        const double B = ci.c0 * nx * nw + ci.c1 * (nx + nw + 1.0);
        zs[v] = z;
        lo[v] = score_of(logit_of(z - B, e), e);
        hi[v] = score_of(logit_of(z + B, e), e);
        ok = ok && isfinite(z) && isfinite(B) && isfinite(lo[v]) && isfinite(hi[v]);
      }
    }
    uint64_t redo[4];
    if (__ballot(!ok) == 0) {
      // theta = K-th largest lo (K rounds of the arg-max, index order on ties)
      bool tk[4] = {false, false, false, false};
      float theta = -INFINITY;
      for (int k = 0; k < K; ++k) {
        float bl = -INFINITY;
        int be = 0x7fffffff;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int e = lane + 64 * v;
          if (e < N && !tk[v] && better(lo[v], e, bl, be)) {
            bl = lo[v];
            be = e;
          }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
          const float ol = __shfl_xor(bl, off, 64);
          const int oe = __shfl_xor(be, off, 64);
          if (better(ol, oe, bl, be)) {
            bl = ol;
            be = oe;
          }
        }
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (lane + 64 * v == be) tk[v] = true;
        theta = bl;
      }
      // candidates: every expert whose interval reaches theta (they contain
      // the exact Top-K); a candidate whose interval meets another
      // candidate's is recomputed, the others already have their exact rank
      bool cand[4], meet[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        cand[v] = lane + 64 * v < N && hi[v] >= theta;
        meet[v] = false;
      }
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        uint64_t m = __ballot(cand[w]);
        while (m) {
          const int l = __ffsll((unsigned long long)m) - 1;
          m &= m - 1;
          const float cl = __shfl(lo[w], l, 64), ch = __shfl(hi[w], l, 64);
          const int ce = l + 64 * w;
#pragma unroll
          for (int v = 0; v < 4; ++v)
            if (cand[v] && lane + 64 * v != ce && lo[v] <= ch && cl <= hi[v]) meet[v] = true;
        }
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) redo[v] = __ballot(meet[v]);
    } else {
#pragma unroll
      for (int v = 0; v < 4; ++v) redo[v] = __ballot(lane + 64 * v < N);
    }
    // recompute the open dot products in fp64
    const uint16_t* xr = ci.x + (int64_t)t * ci.d;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      uint64_t m = redo[v];
      while (m) {
        const int l = __ffsll((unsigned long long)m) - 1;
        m &= m - 1;
        const double z = dot_f64(xr, ci.wr + (int64_t)(l + 64 * v) * ci.d, ci.d, lane);
        if (lane == l) zs[v] = z;
      }
    }
  }
  float lg[4], sc[4];
  bool taken[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int e = lane + 64 * v;
    lg[v] = -INFINITY;
    sc[v] = -INFINITY;
    taken[v] = false;
    if (valid && e < N) {
      lg[v] = logit_of(zs[v], e);
      if (logits) logits[(int64_t)t * N + e] = lg[v];
      const float sv = score_of(lg[v], e);
      sc[v] = isnan(sv) ? -INFINITY : sv;
    }
  }
  int my_e = 0;
  float my_logit = 0.f;
  for (int k = 0; k < K; ++k) {
    float bs = -INFINITY, bl = 0.f;
    int be = 0x7fffffff;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int e = lane + 64 * v;
      if (e < N && !taken[v] && better(sc[v], e, bs, be)) {
        bs = sc[v];
        be = e;
        bl = lg[v];
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float os = __shfl_xor(bs, off, 64);
      const int oe = __shfl_xor(be, off, 64);
      const float ol = __shfl_xor(bl, off, 64);
      if (better(os, oe, bs, be)) {
        bs = os;
        be = oe;
        bl = ol;
      }
    }
#pragma unroll
    for (int v = 0; v < 4; ++v)
      if (lane + 64 * v == be) taken[v] = true;
    if (lane == k) {
      my_e = be;
      my_logit = bl;
    }
  }
  double m = (lane < K) ? (double)my_logit : -INFINITY;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmax(m, __shfl_xor(m, off, 64));
  const double ex = (lane < K) ? exp((double)my_logit - m) : 0.0;
  double sum = ex;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off, 64);
  const float wk = (float)(ex / sum);
  if (valid && lane < K) {
    topk_idx[(int64_t)t * K + lane] = my_e;
    topk_w[(int64_t)t * K + lane] = wk;
  }
  if constexpr (PART) {
    __shared__ double sp[4][256];
    __shared__ double sz[4];
    __shared__ int32_t pe[4][64];
    __shared__ float pw[4][64];
    if (valid) {
      double px[4];
      float rm;
      const double s = row_softmax_terms(lg, lane, N, px, rm);
      const double inv = 1.0 / s;
#pragma unroll
      for (int v = 0; v < 4; ++v) sp[wave][lane + 64 * v] = px[v] * inv;
      if (lane == 0) {
        const double lse = (double)rm + log(s);
        sz[wave] = lse * lse;
      }
      if (lane < K) {
        pe[wave][lane] = my_e;
        pw[wave][lane] = wk;
      }
    } else {
      // tokens past T add nothing (+0.0 leaves the non-negative sums as they are)
#pragma unroll
      for (int v = 0; v < 4; ++v) sp[wave][lane + 64 * v] = 0.0;
      if (lane == 0) sz[wave] = 0.0;
      if (lane < K) pe[wave][lane] = -1;
    }
    __syncthreads();
    const int e = threadIdx.x;
    const int64_t blk = blockIdx.x;
    if (e < N) {
      rp.ppart[blk * N + e] = ((sp[0][e] + sp[1][e]) + sp[2][e]) + sp[3][e];
      int c = 0;
      double sw = 0.0;
      for (int w = 0; w < 4; ++w)
        for (int k = 0; k < K; ++k)
          if (pe[w][k] == e) {
            ++c;
            sw += (double)pw[w][k];
          }
      rp.spcnt[blk * N + e] = c;
      rp.spw[blk * N + e] = sw;
    }
    if (threadIdx.x == 0) rp.zpart[blk] = ((sz[0] + sz[1]) + sz[2]) + sz[3];
  }
}

struct Shape {
  int wt, we, tiles_t, tiles_e;
};
Shape shape_for(int T, int N) {
  Shape s;
  if (N <= 16) {
    s.wt = 2;
    s.we = 1;
  } else {
    s.wt = 1;
    s.we = 4;
  }
  s.tiles_t = (T + 4 * s.wt * 16 - 1) / (4 * s.wt * 16);
  s.tiles_e = (N + s.we * 16 - 1) / (s.we * 16);
  return s;
}

template <typename T>
hipError_t launch_gemm_t(const Shape& sh, int S, int klen, const void* x, const void* wr,
                         double* part, int Ttok, int d, int N, hipStream_t s) {
  dim3 grid(sh.tiles_t, sh.tiles_e, S);
  if (sh.we == 1)
    hipLaunchKernelGGL((router_gemm_kernel<T, 2, 1>), grid, dim3(256), 0, s,
                       static_cast<const T*>(x), static_cast<const T*>(wr), part, Ttok, d, N,
                       klen);
  else
    hipLaunchKernelGGL((router_gemm_kernel<T, 1, 4>), grid, dim3(256), 0, s,
                       static_cast<const T*>(x), static_cast<const T*>(wr), part, Ttok, d, N,
                       klen);
  return hipGetLastError();
}

// Certified path: up to four expert groups of 32 per workgroup, and slices
// of whole 32-wide steps for about two workgroups per CU.
struct CertShape {
  int ew, tiles_t, tiles_e, S, klen;
};
CertShape cert_shape(int T, int d, int N) {
  CertShape c;
  const int ge = 16 * FJ, gt = 16 * FI;
  c.ew = N <= ge ? 1 : (N <= 2 * ge ? 2 : 4);
  const int tw = 4 / c.ew;
  c.tiles_t = (T + gt * tw - 1) / (gt * tw);
  c.tiles_e = (N + ge * c.ew - 1) / (ge * c.ew);
  const int steps = d / 32, tiles = c.tiles_t * c.tiles_e;
  int S = (512 + tiles - 1) / tiles;
  if (S > steps) S = steps;
  if (S < 1) S = 1;
  const int per = (steps + S - 1) / S;
  c.S = (steps + per - 1) / per;
  c.klen = per * 32;
  return c;
}

size_t a256(size_t v) { return (v + 255) / 256 * 256; }

}  // namespace

// Slices of the model dimension: about four workgroups per CU, so each CU
// has several wavefronts per SIMD to cover the latency of the operand loads
// (they go straight from L2 to registers); each slice a whole number of
// 64-wide chunks, no empty slice.
int route_splits(int T, int d, int N) {
  const Shape sh = shape_for(T, N);
  const int tiles = sh.tiles_t * sh.tiles_e;
  const int chunks = d / KC;
  int S = (1024 + tiles - 1) / tiles;
  if (S > chunks) S = chunks;
  if (S < 1) S = 1;
  const int per = (chunks + S - 1) / S;
  return (chunks + per - 1) / per;
}

size_t route_ws_bytes(int T, int d, int N, bool certified) {
  if (!certified) return (size_t)route_splits(T, d, N) * T * N * sizeof(double);
  const CertShape c = cert_shape(T, d, N);
  return a256((size_t)c.S * T * N * 4) + a256((size_t)c.S * T * 4) + (size_t)c.S * N * 4;
}

// Error bound of the certified path, |z' - z| <= c0 |x||w| + c1 (|x| + |w| + 1)
// with |x|, |w| the norms formed from the slice sums of squares:
//  - an MFMA result (32 exact bf16 products added from zero in fp32) is
//    taken to be within 33 * 2^-23 * sum|p| of the exact sum: at most one
//    rounding of relative size 2^-23 (round-to-nearest or truncation) per
//    addition, in any order or with aligned, truncated addends;
//  - the fp64 accumulation of the steps, the fp32 rounding of each slice
//    (2^-23 of its sum|p|) and the fp64 sum of the slices;
//  - a margin of d * 2^-52 sum|p| that contains both the recomputed fp64
//    dot product and any other fp64 evaluation of it;
//  - sum|p| <= |x||w| (Cauchy-Schwarz), the norms' own fp32 sums of squares
//    (klen / 4 + 2 roundings each) inflating the product by (1 + (klen/4 + 3)
//    2^-22); flushed subnormal squares and products in c1.
void cert_coeffs(int d, int S, int klen, double* c0, double* c1) {
  const double u = 0x1p-23;
  const double steps = d / 32.0;
  const double acc = 33.0 * u + u + (steps + S + 2.0) * 0x1p-53 + d * 0x1p-52;
  const double infl = 1.0 + (klen / 4.0 + 3.0) * 0x1p-22;
  *c0 = acc * infl * (1.0 + 0x1p-30);
  *c1 = *c0 * sqrt((double)d) * 0x1p-62 + d * 0x1p-120;
}

hipError_t launch_route(int dtype, bool certified, const void* x, const void* w_router,
                        const float* b_router, const float* logit_offset, const float* sel_bias,
                        float* logits, int32_t* topk_idx, float* topk_w, void* ws, int T, int d,
                        int N, int K, const RoutePartials* parts, hipStream_t s) {
  static_assert(kAuxTokensPerBlock == 4, "one routing-partial block per select workgroup");
  const RoutePartials rp = parts ? *parts : RoutePartials{};
  const dim3 sgrid((T + 3) / 4);
  if (!certified) {
    double* part = static_cast<double*>(ws);
    const Shape sh = shape_for(T, N);
    const int S = route_splits(T, d, N);
    const int chunks = d / KC;
    const int klen = ((chunks + S - 1) / S) * KC;
    hipError_t e = (dtype == 0)
                       ? launch_gemm_t<float>(sh, S, klen, x, w_router, part, T, d, N, s)
                       : launch_gemm_t<uint16_t>(sh, S, klen, x, w_router, part, T, d, N, s);
    if (e != hipSuccess) return e;
    if (parts)
      hipLaunchKernelGGL((select_kernel<true, false>), sgrid, dim3(256), 0, s, part, S, b_router,
                         logit_offset, sel_bias, logits, topk_idx, topk_w, T, N, K, rp, CertIn{});
    else
      hipLaunchKernelGGL((select_kernel<false, false>), sgrid, dim3(256), 0, s, part, S, b_router,
                         logit_offset, sel_bias, logits, topk_idx, topk_w, T, N, K, rp, CertIn{});
    return hipGetLastError();
  }
  if (dtype != 1) return hipErrorInvalidValue;
  const CertShape c = cert_shape(T, d, N);
  char* base = static_cast<char*>(ws);
  CertIn ci;
  ci.part = reinterpret_cast<float*>(base);
  ci.nx2 = reinterpret_cast<float*>(base + a256((size_t)c.S * T * N * 4));
  ci.nw2 = reinterpret_cast<float*>(base + a256((size_t)c.S * T * N * 4) + a256((size_t)c.S * T * 4));
  ci.x = static_cast<const uint16_t*>(x);
  ci.wr = static_cast<const uint16_t*>(w_router);
  ci.S = c.S;
  ci.d = d;
  cert_coeffs(d, c.S, c.klen, &ci.c0, &ci.c1);
  const dim3 grid(c.tiles_t, c.tiles_e, c.S);
  float* pf = const_cast<float*>(ci.part);
  float* px = const_cast<float*>(ci.nx2);
  float* pw = const_cast<float*>(ci.nw2);
  if (c.ew == 1)
    hipLaunchKernelGGL(router_mfma_kernel<1>, grid, dim3(256), 0, s, ci.x, ci.wr, pf, px, pw, T, d,
                       N, c.klen);
  else if (c.ew == 2)
    hipLaunchKernelGGL(router_mfma_kernel<2>, grid, dim3(256), 0, s, ci.x, ci.wr, pf, px, pw, T, d,
                       N, c.klen);
  else
    hipLaunchKernelGGL(router_mfma_kernel<4>, grid, dim3(256), 0, s, ci.x, ci.wr, pf, px, pw, T, d,
                       N, c.klen);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (parts)
    hipLaunchKernelGGL((select_kernel<true, true>), sgrid, dim3(256), 0, s, nullptr, 0, b_router,
                       logit_offset, sel_bias, logits, topk_idx, topk_w, T, N, K, rp, ci);
  else
    hipLaunchKernelGGL((select_kernel<false, true>), sgrid, dim3(256), 0, s, nullptr, 0, b_router,
                       logit_offset, sel_bias, logits, topk_idx, topk_w, T, N, K, rp, ci);
  return hipGetLastError();
}

}  // namespace moe
