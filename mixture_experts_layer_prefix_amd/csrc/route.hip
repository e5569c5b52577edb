// Router scoring fused with Top-K selection and the softmax over the K chosen
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
// Layout: one workgroup of 256 threads owns RT = 16 tokens and all N <= 256
// experts.  The logits tile [16, NPAD] is accumulated in fp64 registers
// (each thread 4x4 outputs, split-K across threads when N is small), reduced
// in a fixed order through LDS, and kept in LDS; then each wavefront selects
// the Top-K of one token row at a time with a 64-lane arg-max reduction.
#include <math.h>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int RT = 16;     // tokens per workgroup
constexpr int KC = 16;     // reduction chunk staged in LDS
constexpr int NTHR = 256;

__device__ __forceinline__ bool better(float sa, int ea, float sb, int eb) {
  return sa > sb || (sa == sb && ea < eb);
}

template <typename T, int NPAD, int TI, int TJ>
__global__ __launch_bounds__(NTHR) void route_kernel(
    const T* __restrict__ x, const T* __restrict__ wr, const float* __restrict__ b_router,
    const float* __restrict__ logit_offset, const float* __restrict__ sel_bias,
    float* __restrict__ logits, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
    int Ttok, int d, int N, int K) {
  constexpr int TG = RT / TI;             // token groups
  constexpr int EG = NPAD / TJ;           // expert groups
  constexpr int S = NTHR / (TG * EG);     // split of each chunk across threads
  static_assert(TG * EG * S == NTHR, "thread tiling");
  static_assert(KC % S == 0, "split must divide the chunk");

  struct Tiles {
    double xs[RT][KC + 1];
    double ws[NPAD][KC + 1];
  };
  __shared__ union {
    Tiles t;
    double part[S][RT * NPAD];
  } sm;
  __shared__ float lg[RT][NPAD];

  const int tid = threadIdx.x;
  const int sidx = tid / (TG * EG);
  const int rem = tid % (TG * EG);
  const int tg = rem / EG;
  const int eg = rem % EG;
  const int t0 = blockIdx.x * RT;

  double acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) acc[i][j] = 0.0;

  for (int k0 = 0; k0 < d; k0 += KC) {
    for (int i = tid; i < RT * KC; i += NTHR) {
      const int tt = i / KC, kk = i % KC, t = t0 + tt;
      sm.t.xs[tt][kk] = (t < Ttok) ? (double)Elem<T>::load(x, (int64_t)t * d + k0 + kk) : 0.0;
    }
    for (int i = tid; i < NPAD * KC; i += NTHR) {
      const int e = i / KC, kk = i % KC;
      sm.t.ws[e][kk] = (e < N) ? (double)Elem<T>::load(wr, (int64_t)e * d + k0 + kk) : 0.0;
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < KC / S; ++q) {
      const int kk = sidx + q * S;
      double xv[TI], wv[TJ];
#pragma unroll
      for (int i = 0; i < TI; ++i) xv[i] = sm.t.xs[tg + TG * i][kk];
#pragma unroll
      for (int j = 0; j < TJ; ++j) wv[j] = sm.t.ws[eg + EG * j][kk];
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) acc[i][j] = fma(xv[i], wv[j], acc[i][j]);
    }
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) sm.part[sidx][(tg + TG * i) * NPAD + eg + EG * j] = acc[i][j];
  __syncthreads();

  for (int o = tid; o < RT * NPAD; o += NTHR) {
    const int tt = o / NPAD, e = o % NPAD, t = t0 + tt;
    float v = -INFINITY;
    if (e < N) {
      double z = sm.part[0][o];
      for (int q = 1; q < S; ++q) z += sm.part[q][o];
      if (b_router) z += (double)b_router[e];
      if (logit_offset) z += (double)logit_offset[e];
      v = (float)z;
      if (logits && t < Ttok) logits[(int64_t)t * N + e] = v;
    }
    lg[tt][e] = v;
  }
  __syncthreads();

  // ---- Top-K + softmax over the K chosen: one wavefront per token row.
  constexpr int VPL = (NPAD + 63) / 64;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  for (int tt = wave; tt < RT; tt += NTHR / 64) {
    const int t = t0 + tt;
    if (t >= Ttok) break;
    float sc[VPL];
    bool taken[VPL];
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      const int e = lane + 64 * v;
      float s = -INFINITY;
      if (e < N) {
        s = lg[tt][e];
        if (sel_bias) s = __fadd_rn(s, sel_bias[e]);
        if (isnan(s)) s = -INFINITY;
      }
      sc[v] = s;
      taken[v] = false;
    }
    int my_e = 0;
    float my_logit = 0.f;
    for (int k = 0; k < K; ++k) {
      float bs = -INFINITY;
      int be = 0x7fffffff;
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        const int e = lane + 64 * v;
        if (!taken[v] && better(sc[v], e, bs, be)) {
          bs = sc[v];
          be = e;
        }
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const float os = __shfl_xor(bs, off, 64);
        const int oe = __shfl_xor(be, off, 64);
        if (better(os, oe, bs, be)) {
          bs = os;
          be = oe;
        }
      }
#pragma unroll
      for (int v = 0; v < VPL; ++v)
        if (lane + 64 * v == be) taken[v] = true;
      if (lane == k) {
        my_e = be;
        my_logit = lg[tt][min(be, NPAD - 1)];
      }
    }
    double m = (lane < K) ? (double)my_logit : -INFINITY;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmax(m, __shfl_xor(m, off, 64));
    double ex = (lane < K) ? exp((double)my_logit - m) : 0.0;
    double sum = ex;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off, 64);
    if (lane < K) {
      topk_idx[(int64_t)t * K + lane] = my_e;
      topk_w[(int64_t)t * K + lane] = (float)(ex / sum);
    }
  }
}

template <typename E, int NPAD, int TI, int TJ>
hipError_t launch_t(const void* x, const void* wr, const float* br, const float* off,
                    const float* sb, float* logits, int32_t* idx, float* w, int T, int d, int N,
                    int K, hipStream_t s) {
  dim3 grid((T + RT - 1) / RT);
  hipLaunchKernelGGL((route_kernel<E, NPAD, TI, TJ>), grid, dim3(NTHR), 0, s,
                     static_cast<const E*>(x), static_cast<const E*>(wr), br, off, sb, logits,
                     idx, w, T, d, N, K);
  return hipGetLastError();
}

template <typename E>
hipError_t launch_dt(const void* x, const void* wr, const float* br, const float* off,
                     const float* sb, float* logits, int32_t* idx, float* w, int T, int d, int N,
                     int K, hipStream_t s) {
  if (N <= 8) return launch_t<E, 8, 4, 2>(x, wr, br, off, sb, logits, idx, w, T, d, N, K, s);
  if (N <= 16) return launch_t<E, 16, 4, 4>(x, wr, br, off, sb, logits, idx, w, T, d, N, K, s);
  if (N <= 32) return launch_t<E, 32, 4, 4>(x, wr, br, off, sb, logits, idx, w, T, d, N, K, s);
  if (N <= 64) return launch_t<E, 64, 4, 4>(x, wr, br, off, sb, logits, idx, w, T, d, N, K, s);
  if (N <= 128) return launch_t<E, 128, 4, 4>(x, wr, br, off, sb, logits, idx, w, T, d, N, K, s);
  return launch_t<E, 256, 4, 4>(x, wr, br, off, sb, logits, idx, w, T, d, N, K, s);
}

}  // namespace

hipError_t launch_route(int dtype, const void* x, const void* w_router, const float* b_router,
                        const float* logit_offset, const float* sel_bias, float* logits,
                        int32_t* topk_idx, float* topk_w, int T, int d, int N, int K,
                        hipStream_t s) {
  if (dtype == 0)
    return launch_dt<float>(x, w_router, b_router, logit_offset, sel_bias, logits, topk_idx,
                            topk_w, T, d, N, K, s);
  return launch_dt<uint16_t>(x, w_router, b_router, logit_offset, sel_bias, logits, topk_idx,
                             topk_w, T, d, N, K, s);
}

}  // namespace moe
