// Combine: restore token order and sum the K expert outputs of each token,
// weighted by its routing weights.
//
// What it computes (lmnt.cn MoE walkthrough §3.2 combine equation,
// output[t] = sum over the selected experts of weight[t,e] * expert_output_e,
// with the index table of the dispatch deciding where each output sits;
// yunthe.com "MoE混合专家模型实战" output equation y = sum_i g_i(x) E_i(x);
// wiblog.cn shared expert: always added):
//   out[t] = (sum_{k : slot_row[t,k] >= 0} w[t,k] * y_perm[slot_row[t,k]]) + y_shared[t]
// in slot order k = 0..K-1 with fp32 fma accumulation, rounded once to the
// output dtype.  Dropped slots contribute nothing.
//
// One wavefront per token; each lane moves 16-byte pieces of the rows, so a
// wavefront reads 1 KiB of a row per instruction; no atomics, every output
// element written exactly once.
#include "moe_internal.h"

namespace moe {
namespace {

template <typename T>
struct Vec;
template <>
struct Vec<float> {
  static constexpr int N = 4;
  static __device__ __forceinline__ void unpack(const uint4& v, float* f) {
    f[0] = __uint_as_float(v.x);
    f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z);
    f[3] = __uint_as_float(v.w);
  }
  static __device__ __forceinline__ uint4 pack(const float* f) {
    return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                      __float_as_uint(f[3]));
  }
};
template <>
struct Vec<uint16_t> {
  static constexpr int N = 8;
  static __device__ __forceinline__ void unpack(const uint4& v, float* f) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  static __device__ __forceinline__ uint4 pack(const float* f) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = (uint32_t)f32_to_bf16(f[2 * i]) | ((uint32_t)f32_to_bf16(f[2 * i + 1]) << 16);
    return make_uint4(w[0], w[1], w[2], w[3]);
  }
};

template <typename T>
__global__ __launch_bounds__(256) void combine_kernel(const uint4* __restrict__ y_perm,
                                                      const int32_t* __restrict__ slot_row,
                                                      const float* __restrict__ topk_w,
                                                      const uint4* __restrict__ y_shared,
                                                      uint4* __restrict__ out, int Ttok,
                                                      int nvec, int K) {
  constexpr int EV = Vec<T>::N;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= Ttok) return;
  const int lane = threadIdx.x & 63;
  const int32_t* sr = slot_row + (int64_t)t * K;
  const float* wt = topk_w + (int64_t)t * K;
  for (int c = lane; c < nvec; c += 64) {
    float acc[EV];
#pragma unroll
    for (int i = 0; i < EV; ++i) acc[i] = 0.f;
    for (int k = 0; k < K; ++k) {
      const int r = sr[k];
      if (r < 0) continue;
      const float w = wt[k];
      float y[EV];
      Vec<T>::unpack(y_perm[(int64_t)r * nvec + c], y);
#pragma unroll
      for (int i = 0; i < EV; ++i) acc[i] = fmaf(w, y[i], acc[i]);
    }
    if (y_shared) {
      float y[EV];
      Vec<T>::unpack(y_shared[(int64_t)t * nvec + c], y);
#pragma unroll
      for (int i = 0; i < EV; ++i) acc[i] += y[i];
    }
    out[(int64_t)t * nvec + c] = Vec<T>::pack(acc);
  }
}

}  // namespace

hipError_t launch_combine(int dtype, const void* y_perm, const int32_t* slot_row,
                          const float* topk_w, const void* y_shared, void* out, int T, int d,
                          int K, hipStream_t s) {
  const int nvec = d * (dtype == 0 ? 4 : 2) / 16;
  dim3 grid((T + 3) / 4);
  if (dtype == 0)
    hipLaunchKernelGGL(combine_kernel<float>, grid, dim3(256), 0, s,
                       static_cast<const uint4*>(y_perm), slot_row, topk_w,
                       static_cast<const uint4*>(y_shared), static_cast<uint4*>(out), T, nvec, K);
  else
    hipLaunchKernelGGL(combine_kernel<uint16_t>, grid, dim3(256), 0, s,
                       static_cast<const uint4*>(y_perm), slot_row, topk_w,
                       static_cast<const uint4*>(y_shared), static_cast<uint4*>(out), T, nvec, K);
  return hipGetLastError();
}

}  // namespace moe
