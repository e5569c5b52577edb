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
// wavefront reads 1 KiB of a row per instruction, and many such loads are in
// flight per lane; no atomics, every output element written exactly once.
#include <stdlib.h>

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
  static __device__ __forceinline__ uint4 pack(const float* f) { return pack_bf16x8(f); }
};

// One wavefront per token (its index made wave-uniform, so the slot rows and
// weights are scalar loads).  The slots are taken in groups of KB; for each
// group a lane first issues the loads of all the group's kept rows for U
// 16-byte pieces, then adds them in slot order, so KB * U loads per lane are in
// flight together instead of one row at a time.  NT: the expert rows, each
// read once, are loaded non-temporally (chosen when they are too large for
// the MALL to hold: the DeepSeek-shaped layer's 470 MB combine ran 10%
// faster; where they fit, as on the Switch shape, cached loads are better).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <typename T, int KB, int U, bool NT>
__global__ __launch_bounds__(256) void combine_kernel(const uint4* __restrict__ y_perm,
                                                      const int32_t* __restrict__ slot_row,
                                                      const float* __restrict__ topk_w,
                                                      const uint4* __restrict__ y_shared,
                                                      uint4* __restrict__ out, int Ttok,
                                                      int nvec, int K) {
  constexpr int EV = Vec<T>::N;
  const int t = __builtin_amdgcn_readfirstlane((int)(blockIdx.x * 4 + (threadIdx.x >> 6)));
  if (t >= Ttok) return;
  const int lane = threadIdx.x & 63;
  const int32_t* sr = slot_row + (int64_t)t * K;
  const float* wt = topk_w + (int64_t)t * K;
  for (int c0 = lane; c0 < nvec; c0 += 64 * U) {
    // the shared expert's pieces are loaded with the first group of rows
    uint4 vs[U];
    if (y_shared) {
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (c0 + 64 * u < nvec) vs[u] = y_shared[(int64_t)t * nvec + c0 + 64 * u];
    }
    float acc[U][EV];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < EV; ++i) acc[u][i] = 0.f;
    for (int k0 = 0; k0 < K; k0 += KB) {
      int r[KB];
      float w[KB];
#pragma unroll
      for (int j = 0; j < KB; ++j) {
        r[j] = (k0 + j < K) ? sr[k0 + j] : -1;
        w[j] = (r[j] >= 0) ? wt[k0 + j] : 0.f;
      }
      uint4 v[KB][U];
#pragma unroll
      for (int j = 0; j < KB; ++j)
        if (r[j] >= 0) {
          const uint4* yr = y_perm + (int64_t)r[j] * nvec;
#pragma unroll
          for (int u = 0; u < U; ++u)
            if (c0 + 64 * u < nvec) {
              if constexpr (NT) {
                const u32x4 q = __builtin_nontemporal_load(
                    reinterpret_cast<const u32x4*>(yr + c0 + 64 * u));
                v[j][u] = make_uint4(q[0], q[1], q[2], q[3]);
              } else {
                v[j][u] = yr[c0 + 64 * u];
              }
            }
        }
#pragma unroll
      for (int j = 0; j < KB; ++j)
        if (r[j] >= 0) {
#pragma unroll
          for (int u = 0; u < U; ++u) {
            float y[EV];
            Vec<T>::unpack(v[j][u], y);
#pragma unroll
            for (int i = 0; i < EV; ++i) acc[u][i] = fmaf(w[j], y[i], acc[u][i]);
          }
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + 64 * u;
      if (c >= nvec) break;
      if (y_shared) {
        float y[EV];
        Vec<T>::unpack(vs[u], y);
#pragma unroll
        for (int i = 0; i < EV; ++i) acc[u][i] += y[i];
      }
      out[(int64_t)t * nvec + c] = Vec<T>::pack(acc[u]);
    }
  }
}

template <typename T, bool NT>
void launch_combine_t(const void* y_perm, const int32_t* slot_row, const float* topk_w,
                      const void* y_shared, void* out, int Ttok, int nvec, int K, hipStream_t s) {
  const dim3 grid((Ttok + 3) / 4), block(256);
  const uint4* y = static_cast<const uint4*>(y_perm);
  const uint4* ys = static_cast<const uint4*>(y_shared);
  uint4* o = static_cast<uint4*>(out);
  if (K == 1)
    hipLaunchKernelGGL((combine_kernel<T, 1, 2, NT>), grid, block, 0, s, y, slot_row, topk_w, ys, o, Ttok,
                       nvec, K);
  else if (K <= 2)
    hipLaunchKernelGGL((combine_kernel<T, 2, 4, NT>), grid, block, 0, s, y, slot_row, topk_w, ys, o, Ttok,
                       nvec, K);
  else if (K <= 4)
    hipLaunchKernelGGL((combine_kernel<T, 4, 4, NT>), grid, block, 0, s, y, slot_row, topk_w, ys, o, Ttok,
                       nvec, K);
  else
    hipLaunchKernelGGL((combine_kernel<T, 8, 2, NT>), grid, block, 0, s, y, slot_row, topk_w, ys, o, Ttok,
                       nvec, K);
}

}  // namespace

int64_t nontemporal_rows_bytes() {
  const char* e = getenv("MOE_NONTEMPORAL_ROWS_BYTES");
  if (e && *e) {
    char* end = nullptr;
    const long long v = strtoll(e, &end, 10);
    if (end && *end == 0 && v >= 0) return (int64_t)v;
  }
  return int64_t(128) << 20;
}

hipError_t launch_combine(int dtype, const void* y_perm, const int32_t* slot_row,
                          const float* topk_w, const void* y_shared, void* out, int T, int d,
                          int K, hipStream_t s) {
  const int nvec = d * (dtype == 0 ? 4 : 2) / 16;
  // expert rows beyond half of the 256 MB MALL: non-temporal loads
  const bool nt = (int64_t)T * K * nvec * 16 > nontemporal_rows_bytes();
  if (dtype == 0)
    nt ? launch_combine_t<float, true>(y_perm, slot_row, topk_w, y_shared, out, T, nvec, K, s)
       : launch_combine_t<float, false>(y_perm, slot_row, topk_w, y_shared, out, T, nvec, K, s);
  else
    nt ? launch_combine_t<uint16_t, true>(y_perm, slot_row, topk_w, y_shared, out, T, nvec, K, s)
       : launch_combine_t<uint16_t, false>(y_perm, slot_row, topk_w, y_shared, out, T, nvec, K, s);
  return hipGetLastError();
}

}  // namespace moe
