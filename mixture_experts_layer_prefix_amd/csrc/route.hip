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

__device__ __forceinline__ bool better(float sa, int ea, float sb, int eb) {
  return sa > sb || (sa == sb && ea < eb);
}

// One wavefront per token (4 per workgroup); lane = expert (4 per lane, N <= 256).
// PART: the workgroup's four tokens are one block of the routing partials
// (kAuxTokensPerBlock = 4): while the row is in registers, the wavefront
// forms its softmax_N probabilities and lse^2 with row_softmax_terms, the
// same routine and order as the aux-loss and z-loss kernels, and the
// workgroup adds the four tokens in token order; the K (expert, weight)
// picks give the block's per-expert counts and weight sums in (token, slot)
// order.  The loss and statistics kernels then never read the logits again.
template <bool PART>
__global__ __launch_bounds__(256) void select_kernel(
    const double* __restrict__ part, int S, const float* __restrict__ b_router,
    const float* __restrict__ logit_offset, const float* __restrict__ sel_bias,
    float* __restrict__ logits, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    int Ttok, int N, int K, RoutePartials rp) {
  const int wave = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wave;
  const bool valid = t < Ttok;
  if (!PART && !valid) return;   // (with partials every wavefront reaches the barrier)
  const int lane = threadIdx.x & 63;
  float lg[4], sc[4];
  bool taken[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int e = lane + 64 * v;
    lg[v] = -INFINITY;
    sc[v] = -INFINITY;
    taken[v] = false;
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
      if (b_router) z += (double)b_router[e];
      if (logit_offset) z += (double)logit_offset[e];
      lg[v] = (float)z;
      if (logits) logits[(int64_t)t * N + e] = lg[v];
      float sv = lg[v];
      if (sel_bias) sv = __fadd_rn(sv, sel_bias[e]);
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

hipError_t launch_route(int dtype, const void* x, const void* w_router, const float* b_router,
                        const float* logit_offset, const float* sel_bias, float* logits,
                        int32_t* topk_idx, float* topk_w, double* part, int T, int d, int N,
                        int K, const RoutePartials* parts, hipStream_t s) {
  const Shape sh = shape_for(T, N);
  const int S = route_splits(T, d, N);
  const int chunks = d / KC;
  const int klen = ((chunks + S - 1) / S) * KC;
  hipError_t e = (dtype == 0)
                     ? launch_gemm_t<float>(sh, S, klen, x, w_router, part, T, d, N, s)
                     : launch_gemm_t<uint16_t>(sh, S, klen, x, w_router, part, T, d, N, s);
  if (e != hipSuccess) return e;
  static_assert(kAuxTokensPerBlock == 4, "one routing-partial block per select workgroup");
  if (parts)
    hipLaunchKernelGGL(select_kernel<true>, dim3((T + 3) / 4), dim3(256), 0, s, part, S, b_router,
                       logit_offset, sel_bias, logits, topk_idx, topk_w, T, N, K, *parts);
  else
    hipLaunchKernelGGL(select_kernel<false>, dim3((T + 3) / 4), dim3(256), 0, s, part, S,
                       b_router, logit_offset, sel_bias, logits, topk_idx, topk_w, T, N, K,
                       RoutePartials{});
  return hipGetLastError();
}

}  // namespace moe
