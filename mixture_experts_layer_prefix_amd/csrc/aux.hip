// Switch auxiliary load-balance loss.
//
// What it computes (yunthe.com "MoE混合专家模型实战", section
// "专家负载均衡与辅助损失函数设计": alpha * num_experts * sum(f * P) with f the
// per-expert mean of the 0/1 selection mask and P the per-expert mean of the
// softmax router probabilities; lmnt.cn MoE walkthrough §5.1, same product):
//   P_e  = (1/T) sum_t softmax_N(logits[t])_e
//   f_e  = counts[e] / T          (pre-drop selections, sum_e f_e = K)
//   loss = alpha * N * sum_e f_e * P_e
// in fp64 with a fixed reduction order, so the result is deterministic.
//
// Pass 1: each workgroup of 4 wavefronts takes 64 tokens; a wavefront takes
// one token row at a time (lane = expert, up to 4 experts per lane), forms
// the row's softmax and adds it to per-lane sums; the 4 wavefronts' sums are
// added in wavefront order into ppart[block, e].
// Pass 2: one workgroup; a wavefront per expert adds ppart over the blocks
// (lanes stride over blocks, then a fixed butterfly), multiplies by f_e, and
// the experts' terms are reduced with a fixed tree.
#include <math.h>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int TB = kAuxTokensPerBlock;

__global__ __launch_bounds__(256) void aux_partial_kernel(const float* __restrict__ logits, int T,
                                                          int N, double* __restrict__ ppart) {
  __shared__ double part[4][256];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  double ps[4] = {0.0, 0.0, 0.0, 0.0};
  const int t0 = blockIdx.x * TB;
  for (int tt = wave; tt < TB; tt += 4) {
    const int t = t0 + tt;
    if (t >= T) break;
    const float* row = logits + (int64_t)t * N;
    double l[4];
    double m = -INFINITY;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int e = lane + 64 * v;
      l[v] = (e < N) ? (double)row[e] : -INFINITY;
      m = fmax(m, l[v]);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmax(m, __shfl_xor(m, off, 64));
    double ex[4], s = 0.0;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      ex[v] = (lane + 64 * v < N) ? exp(l[v] - m) : 0.0;
      s += ex[v];
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
#pragma unroll
    for (int v = 0; v < 4; ++v) ps[v] += ex[v] / s;
  }
#pragma unroll
  for (int v = 0; v < 4; ++v) part[wave][lane + 64 * v] = ps[v];
  __syncthreads();
  for (int e = threadIdx.x; e < N; e += 256)
    ppart[(int64_t)blockIdx.x * N + e] = ((part[0][e] + part[1][e]) + part[2][e]) + part[3][e];
}

__global__ __launch_bounds__(256) void aux_final_kernel(const double* __restrict__ ppart, int nblk,
                                                        const int32_t* __restrict__ counts, int T,
                                                        int N, float alpha,
                                                        float* __restrict__ loss) {
  __shared__ double term[256];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // wavefront w takes experts w, w+4, ...; its lanes stride over the blocks
  // (each lane sums its blocks in order, then a fixed butterfly)
  for (int e = wave; e < N; e += 4) {
    double P = 0.0;
    for (int b = lane; b < nblk; b += 64) P += ppart[(int64_t)b * N + e];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) P += __shfl_xor(P, off, 64);
    if (lane == 0) term[e] = ((double)counts[e] / (double)T) * (P / (double)T);
  }
  __syncthreads();
  if (threadIdx.x >= N) term[threadIdx.x] = 0.0;
  __syncthreads();
  for (int h = 128; h >= 1; h >>= 1) {
    if (threadIdx.x < h) term[threadIdx.x] += term[threadIdx.x + h];
    __syncthreads();
  }
  if (threadIdx.x == 0) loss[0] = (float)((double)alpha * (double)N * term[0]);
}

// Router z-loss (lmnt.cn MoE walkthrough §5.3): beta * mean_t lse_t^2 with
// lse_t = logsumexp_e logits[t, e], in fp64.  Pass 1: a wavefront per token
// row (lane = expert) forms lse = m + log(sum exp(l - m)); each wavefront adds
// its rows' lse^2 in token order, the 4 wavefronts' sums are added in order
// into zpart[block].  Pass 2: one wavefront adds zpart over the blocks (lanes
// stride, then a fixed butterfly).
__global__ __launch_bounds__(256) void zloss_partial_kernel(const float* __restrict__ logits, int T,
                                                            int N, double* __restrict__ zpart) {
  __shared__ double part[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  double acc = 0.0;
  const int t0 = blockIdx.x * TB;
  for (int tt = wave; tt < TB; tt += 4) {
    const int t = t0 + tt;
    if (t >= T) break;
    const float* row = logits + (int64_t)t * N;
    double l[4];
    double m = -INFINITY;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int e = lane + 64 * v;
      l[v] = (e < N) ? (double)row[e] : -INFINITY;
      m = fmax(m, l[v]);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmax(m, __shfl_xor(m, off, 64));
    double sum = 0.0;
#pragma unroll
    for (int v = 0; v < 4; ++v) sum += (lane + 64 * v < N) ? exp(l[v] - m) : 0.0;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off, 64);
    const double lse = m + log(sum);
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
  for (int b = threadIdx.x; b < nblk; b += 64) z += zpart[b];
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) z += __shfl_xor(z, off, 64);
  if (threadIdx.x == 0) loss[0] = (float)((double)beta * (z / (double)T));
}

}  // namespace

hipError_t launch_zloss(const float* logits, int T, int N, float beta, double* zpart,
                        float* loss_out, hipStream_t s) {
  const int nblk = aux_blocks(T);
  hipLaunchKernelGGL(zloss_partial_kernel, dim3(nblk), dim3(256), 0, s, logits, T, N, zpart);
  hipLaunchKernelGGL(zloss_final_kernel, dim3(1), dim3(64), 0, s, zpart, nblk, T, beta, loss_out);
  return hipGetLastError();
}

hipError_t launch_aux(const float* logits, const int32_t* counts, int T, int N, float alpha,
                      double* ppart, float* loss_out, hipStream_t s) {
  const int nblk = aux_blocks(T);
  hipLaunchKernelGGL(aux_partial_kernel, dim3(nblk), dim3(256), 0, s, logits, T, N, ppart);
  hipLaunchKernelGGL(aux_final_kernel, dim3(1), dim3(256), 0, s, ppart, nblk, counts, T, N, alpha,
                     loss_out);
  return hipGetLastError();
}

}  // namespace moe
