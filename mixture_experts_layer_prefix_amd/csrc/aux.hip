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
//
// Both use a fixed reduction order, so the results are deterministic: the row
// max and the exponentials in fp32 (relative error ~1e-7 per term, each in
// (0, 1]), every sum, logarithm, normalisation and product in fp64.
//
// Pass 1: a workgroup of 4 wavefronts takes TB = 16 tokens; a wavefront loads
// its 4 token rows at once (lane = expert, up to 4 experts per lane), then
// forms each row's softmax (or logsumexp) and adds it to per-lane sums in
// token order; the 4 wavefronts' sums are added in wavefront order into
// ppart[block, e] (or zpart[block]).
// Pass 2, aux: a wavefront per expert adds column e of ppart (lanes stride
// over the blocks, then a fixed butterfly) and multiplies by f_e; pass 3, one
// workgroup reduces the experts' terms with a fixed tree.  Z-loss: one
// wavefront adds zpart (lanes stride over the blocks, then a fixed
// butterfly).
#include <math.h>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int TB = kAuxTokensPerBlock;
constexpr int RPW = TB / 4;            // token rows per wavefront

// Row max and fp32 exponentials of one token row (lane = expert e, e + 64,
// e + 128, e + 192); returns the row's sum of exponentials in fp64.
__device__ __forceinline__ double row_exp(const float (&l)[4], int lane, int N, double (&ex)[4],
                                          float& m) {
  m = -INFINITY;
#pragma unroll
  for (int v = 0; v < 4; ++v) m = fmaxf(m, l[v]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  double s = 0.0;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    ex[v] = (lane + 64 * v < N) ? (double)expf(l[v] - m) : 0.0;
    s += ex[v];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
  return s;
}

// The wavefront's RPW rows, loaded before any arithmetic so their loads are
// in flight together; entries past T or N read as -inf (rows past T are
// skipped by the callers).
__device__ __forceinline__ void load_rows(const float* __restrict__ logits, int T, int N, int t0,
                                          int lane, float (&l)[RPW][4]) {
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    const int t = t0 + r;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int e = lane + 64 * v;
      l[r][v] = (t < T && e < N) ? logits[(int64_t)t * N + e] : -INFINITY;
    }
  }
}

__global__ __launch_bounds__(256) void aux_partial_kernel(const float* __restrict__ logits, int T,
                                                          int N, double* __restrict__ ppart) {
  __shared__ double part[4][256];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * TB + wave * RPW;
  float l[RPW][4];
  load_rows(logits, T, N, t0, lane, l);
  double ps[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    if (t0 + r >= T) break;
    double ex[4];
    float m;
    const double inv = 1.0 / row_exp(l[r], lane, N, ex, m);
#pragma unroll
    for (int v = 0; v < 4; ++v) ps[v] += ex[v] * inv;
  }
#pragma unroll
  for (int v = 0; v < 4; ++v) part[wave][lane + 64 * v] = ps[v];
  __syncthreads();
  for (int e = threadIdx.x; e < N; e += 256)
    ppart[(int64_t)blockIdx.x * N + e] = ((part[0][e] + part[1][e]) + part[2][e]) + part[3][e];
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

__global__ __launch_bounds__(256) void zloss_partial_kernel(const float* __restrict__ logits, int T,
                                                            int N, double* __restrict__ zpart) {
  __shared__ double part[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t0 = blockIdx.x * TB + wave * RPW;
  float l[RPW][4];
  load_rows(logits, T, N, t0, lane, l);
  double acc = 0.0;
#pragma unroll
  for (int r = 0; r < RPW; ++r) {
    if (t0 + r >= T) break;
    double ex[4];
    float m;
    const double s = row_exp(l[r], lane, N, ex, m);
    const double lse = (double)m + log(s);
    acc += lse * lse;
  }
  if (lane == 0) part[wave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) zpart[blockIdx.x] = ((part[0] + part[1]) + part[2]) + part[3];
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

// Routing statistics (lmnt.cn MoE walkthrough §8.2: tokens per expert and
// mean routing weight).  Pass 1: a workgroup stages the (expert, weight) pairs
// of STB tokens in LDS; thread e walks them in token-major order and counts
// the pairs routed to expert e and adds their weights (fp64).  Pass 2: a
// wavefront per expert adds the blocks' partials (lanes stride over the
// blocks, then a fixed butterfly).
constexpr int STB = kStatsTokensPerBlock;

__global__ __launch_bounds__(256) void stats_partial_kernel(const int32_t* __restrict__ idx,
                                                            const float* __restrict__ w, int T,
                                                            int K, int N,
                                                            int32_t* __restrict__ pcnt,
                                                            double* __restrict__ pw) {
  __shared__ int32_t s_idx[STB * 64];
  __shared__ float s_w[STB * 64];
  const int64_t p0 = (int64_t)blockIdx.x * STB * K;
  const int np = (int)(min((int64_t)(blockIdx.x + 1) * STB, (int64_t)T) * K - p0);
  for (int i = threadIdx.x; i < np; i += 256) {
    s_idx[i] = idx[p0 + i];
    s_w[i] = w[p0 + i];
  }
  __syncthreads();
  for (int e = threadIdx.x; e < N; e += 256) {
    int c = 0;
    double sw = 0.0;
    for (int i = 0; i < np; ++i)
      if (s_idx[i] == e) {
        ++c;
        sw += (double)s_w[i];
      }
    pcnt[(int64_t)blockIdx.x * N + e] = c;
    pw[(int64_t)blockIdx.x * N + e] = sw;
  }
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

hipError_t launch_stats(const int32_t* topk_idx, const float* topk_w, int T, int K, int N,
                        int32_t* pcnt, double* pw, int32_t* counts, float* wmean, hipStream_t s) {
  const int nblk = stats_blocks(T);
  hipLaunchKernelGGL(stats_partial_kernel, dim3(nblk), dim3(256), 0, s, topk_idx, topk_w, T, K, N,
                     pcnt, pw);
  hipLaunchKernelGGL(stats_final_kernel, dim3(N), dim3(64), 0, s, pcnt, pw, nblk, N, counts, wmean);
  return hipGetLastError();
}

hipError_t launch_zloss(const float* logits, int T, int N, float beta, double* zpart,
                        float* loss_out, hipStream_t s) {
  const int nblk = aux_blocks(T);
  hipLaunchKernelGGL(zloss_partial_kernel, dim3(nblk), dim3(256), 0, s, logits, T, N, zpart);
  hipLaunchKernelGGL(zloss_final_kernel, dim3(1), dim3(64), 0, s, zpart, nblk, T, beta, loss_out);
  return hipGetLastError();
}

hipError_t launch_aux(const float* logits, const int32_t* counts, int T, int N, float alpha,
                      double* ppart, double* term, float* loss_out, hipStream_t s) {
  const int nblk = aux_blocks(T);
  hipLaunchKernelGGL(aux_partial_kernel, dim3(nblk), dim3(256), 0, s, logits, T, N, ppart);
  hipLaunchKernelGGL(aux_column_kernel, dim3(N), dim3(64), 0, s, ppart, nblk, counts, T, N, term);
  hipLaunchKernelGGL(aux_final_kernel, dim3(1), dim3(256), 0, s, term, N, alpha, loss_out);
  return hipGetLastError();
}

}  // namespace moe
