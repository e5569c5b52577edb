// Switch auxiliary load-balance loss, router z-loss, routing statistics.
//
// Aux loss (yunthe.com "MoE混合专家模型实战", section "专家负载均衡与辅助损失函数设计":
// alpha * num_experts * sum(f * P) with f the per-expert mean of the 0/1
// selection mask and P the per-expert mean of the softmax router
// probabilities; lmnt.cn MoE walkthrough §5.1, same product):
//   P_e  = (1/T) sum_t softmax_N(logits[t])_e
//   f_e  = counts[e] / T          (pre-drop selections, sum_e f_e = K)
//   loss = alpha * N * sum_e f_e * P_e
// Router z-loss (lmnt.cn MoE walkthrough §5.3): beta * mean_t lse_t^2 with
// lse_t = logsumexp_e logits[t, e].
// Routing statistics (lmnt.cn MoE walkthrough §8.2: tokens per expert and
// mean routing weight).
//
// All three reduce per-block routing partials (RoutePartials, blocks of
// kAuxTokensPerBlock = 4 tokens): the select kernel of the router writes them
// from the rows it already holds, or the partial kernels below write the same
// bits from the logits / routing.  Fixed reduction orders throughout, so the
// results are deterministic: row max and exponentials in fp32 (relative
// error ~1e-7 per term, each in (0, 1]), every sum, logarithm, normalisation
// and product in fp64.
//
// Partials from the logits: one wavefront per block, its 4 rows loaded
// together, each row's softmax and lse^2 added to per-lane sums in token
// order.  Partials from the routing: one workgroup per 4 blocks stages their
// (expert, weight) pairs in LDS; thread e walks each block's pairs in
// token-major order.  Final passes: a wavefront per expert adds column e of
// a partial array (lanes stride over the blocks, then a fixed butterfly); the
// aux loss then reduces the experts' terms with a fixed tree.
#include <math.h>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int TB = kAuxTokensPerBlock;

// ppart [nblk, N] and zpart [nblk] from the logits: wavefront w of
// workgroup b takes block 4 b + w.
__global__ __launch_bounds__(256) void logit_partials_kernel(const float* __restrict__ logits,
                                                             int T, int N, int nblk,
                                                             double* __restrict__ ppart,
                                                             double* __restrict__ zpart) {
  const int lane = threadIdx.x & 63;
  const int blk = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (blk >= nblk) return;
  const int t0 = blk * TB;
  float l[TB][4];
  // the block's rows, loaded before any arithmetic so the loads are in flight
  // together; entries past T or N read as -inf
#pragma unroll
  for (int r = 0; r < TB; ++r) {
    const int t = t0 + r;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int e = lane + 64 * v;
      l[r][v] = (t < T && e < N) ? logits[(int64_t)t * N + e] : -INFINITY;
    }
  }
  double ps[4] = {0.0, 0.0, 0.0, 0.0};
  double zs = 0.0;
#pragma unroll
  for (int r = 0; r < TB; ++r) {
    if (t0 + r >= T) break;
    double ex[4];
    float m;
    const double s = row_softmax_terms(l[r], lane, N, ex, m);
    const double inv = 1.0 / s;
#pragma unroll
    for (int v = 0; v < 4; ++v) ps[v] += ex[v] * inv;
    const double lse = (double)m + log(s);
    zs += lse * lse;
  }
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int e = lane + 64 * v;
    if (e < N) ppart[(int64_t)blk * N + e] = ps[v];
  }
  if (lane == 0) zpart[blk] = zs;
}

// spcnt, spw [nblk, N] from the routing: workgroup b takes blocks 4 b .. 4 b + 3.
__global__ __launch_bounds__(256) void routing_partials_kernel(const int32_t* __restrict__ idx,
                                                               const float* __restrict__ w,
                                                               int T, int K, int N, int nblk,
                                                               int32_t* __restrict__ pcnt,
                                                               double* __restrict__ pw) {
  __shared__ int32_t s_idx[4 * TB * 64];
  __shared__ float s_w[4 * TB * 64];
  const int b0 = blockIdx.x * 4;
  const int64_t p0 = (int64_t)b0 * TB * K;
  const int np = (int)(min((int64_t)(b0 + 4) * TB, (int64_t)T) * K - p0);
  for (int i = threadIdx.x; i < np; i += 256) {
    s_idx[i] = idx[p0 + i];
    s_w[i] = w[p0 + i];
  }
  __syncthreads();
  const int e = threadIdx.x;
  if (e >= N) return;
  for (int b = 0; b < 4 && b0 + b < nblk; ++b) {
    const int i0 = b * TB * K, i1 = min(np, (b + 1) * TB * K);
    int c = 0;
    double sw = 0.0;
    for (int i = i0; i < i1; ++i)
      if (s_idx[i] == e) {
        ++c;
        sw += (double)s_w[i];
      }
    pcnt[(int64_t)(b0 + b) * N + e] = c;
    pw[(int64_t)(b0 + b) * N + e] = sw;
  }
}

// One wavefront per expert e: lanes stride over the blocks (their loads are
// independent and unrolled so they are in flight together), a fixed butterfly
// adds the lanes; term[e] = f_e * P_e.
__global__ __launch_bounds__(64) void aux_column_kernel(const double* __restrict__ ppart, int nblk,
                                                        const int32_t* __restrict__ counts, int T,
                                                        int N, double* __restrict__ term) {
  const int e = blockIdx.x, lane = threadIdx.x;
  double P = 0.0;
#pragma unroll 8
  for (int b = lane; b < nblk; b += 64) P += ppart[(int64_t)b * N + e];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) P += __shfl_xor(P, off, 64);
  if (lane == 0) term[e] = ((double)counts[e] / (double)T) * (P / (double)T);
}

// The experts' terms in a fixed tree.
__global__ __launch_bounds__(256) void aux_final_kernel(const double* __restrict__ term, int N,
                                                        float alpha, float* __restrict__ loss) {
  __shared__ double t[256];
  const int e = threadIdx.x;
  t[e] = e < N ? term[e] : 0.0;
  __syncthreads();
  for (int h = 128; h >= 1; h >>= 1) {
    if (e < h) t[e] += t[e + h];
    __syncthreads();
  }
  if (e == 0) loss[0] = (float)((double)alpha * (double)N * t[0]);
}

__global__ __launch_bounds__(64) void zloss_final_kernel(const double* __restrict__ zpart, int nblk,
                                                         int T, float beta,
                                                         float* __restrict__ loss) {
  double z = 0.0;
#pragma unroll 8
  for (int b = threadIdx.x; b < nblk; b += 64) z += zpart[b];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) z += __shfl_xor(z, off, 64);
  if (threadIdx.x == 0) loss[0] = (float)((double)beta * (z / (double)T));
}

__global__ __launch_bounds__(64) void stats_final_kernel(const int32_t* __restrict__ pcnt,
                                                         const double* __restrict__ pw, int nblk,
                                                         int N, int32_t* __restrict__ counts,
                                                         float* __restrict__ wmean) {
  const int e = blockIdx.x, lane = threadIdx.x;
  int c = 0;
  double sw = 0.0;
#pragma unroll 4
  for (int b = lane; b < nblk; b += 64) {
    c += pcnt[(int64_t)b * N + e];
    sw += pw[(int64_t)b * N + e];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    c += __shfl_xor(c, off, 64);
    sw += __shfl_xor(sw, off, 64);
  }
  if (lane == 0) {
    if (counts) counts[e] = c;
    wmean[e] = c > 0 ? (float)(sw / (double)c) : 0.0f;
  }
}

}  // namespace

hipError_t launch_logit_partials(const float* logits, int T, int N, const RoutePartials& rp,
                                 hipStream_t s) {
  const int nblk = aux_blocks(T);
  hipLaunchKernelGGL(logit_partials_kernel, dim3((nblk + 3) / 4), dim3(256), 0, s, logits, T, N,
                     nblk, rp.ppart, rp.zpart);
  return hipGetLastError();
}

hipError_t launch_routing_partials(const int32_t* topk_idx, const float* topk_w, int T, int K,
                                   int N, const RoutePartials& rp, hipStream_t s) {
  const int nblk = aux_blocks(T);
  hipLaunchKernelGGL(routing_partials_kernel, dim3((nblk + 3) / 4), dim3(256), 0, s, topk_idx,
                     topk_w, T, K, N, nblk, rp.spcnt, rp.spw);
  return hipGetLastError();
}

hipError_t launch_aux_final(const RoutePartials& rp, const int32_t* counts, int T, int N,
                            float alpha, double* term, float* loss_out, hipStream_t s) {
  const int nblk = aux_blocks(T);
  hipLaunchKernelGGL(aux_column_kernel, dim3(N), dim3(64), 0, s, rp.ppart, nblk, counts, T, N,
                     term);
  hipLaunchKernelGGL(aux_final_kernel, dim3(1), dim3(256), 0, s, term, N, alpha, loss_out);
  return hipGetLastError();
}

hipError_t launch_zloss_final(const RoutePartials& rp, int T, float beta, float* loss_out,
                              hipStream_t s) {
  hipLaunchKernelGGL(zloss_final_kernel, dim3(1), dim3(64), 0, s, rp.zpart, aux_blocks(T), T, beta,
                     loss_out);
  return hipGetLastError();
}

hipError_t launch_stats_final(const RoutePartials& rp, int T, int N, int32_t* counts, float* wmean,
                              hipStream_t s) {
  hipLaunchKernelGGL(stats_final_kernel, dim3(N), dim3(64), 0, s, rp.spcnt, rp.spw, aux_blocks(T),
                     N, counts, wmean);
  return hipGetLastError();
}

}  // namespace moe
