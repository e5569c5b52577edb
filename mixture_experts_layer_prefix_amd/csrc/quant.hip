// Weight-only INT8 and INT4 quantisation, one fp32 scale per row.
//
// What it computes (lmnt.cn MoE walkthrough §4.3: expert weights compressed
// from 16-bit to INT8 for inference, memory and bandwidth halved; the pages
// fix no scheme, this is the symmetric per-output-channel one):
//   scale[r] = fp32(max_c |w[r, c]| / 127)
//   q[r, c]  = clamp(round_half_even(fp32(w[r, c] / scale[r])), -127, 127)
// Both divisions are IEEE round-to-nearest (__fdiv_rn) and the rounding to
// an integer is v_rndne (half to even), so every code is reproducible; a row
// of zeros gets scale 0 and codes 0.
//
// INT4 (lmnt.cn §4.3 names INT4 beside INT8): the same with 7 for 127, codes
// in [-7, 7] stored two per byte, element 2i in the low nibble of byte i
// (4-bit two's complement).
//
// One wavefront per row: a pass for the row's max |w| (exact in any order),
// then a pass writing the codes, 8 per lane per step (8-byte stores; 4-byte
// stores for INT4).
#include <math.h>

#include "moe_internal.h"

namespace moe {
namespace {

template <typename T>
struct Row8;
template <>
struct Row8<uint16_t> {   // 8 bf16 (16 bytes)
  static __device__ __forceinline__ void load(const uint16_t* p, float (&v)[8]) {
    const uint4 u = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};
template <>
struct Row8<float> {      // 8 fp32 (two 16-byte loads)
  static __device__ __forceinline__ void load(const float* p, float (&v)[8]) {
    const float4 a = reinterpret_cast<const float4*>(p)[0];
    const float4 b = reinterpret_cast<const float4*>(p)[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
};

template <typename T>
__global__ __launch_bounds__(256) void quantize_int8_kernel(const T* __restrict__ w, int64_t rows,
                                                            int cols, int8_t* __restrict__ q,
                                                            float* __restrict__ scale) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const T* row = w + r * cols;
  float m = 0.f;
  for (int c = lane * 8; c < cols; c += 512) {
    float v[8];
    Row8<T>::load(row + c, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  const float s = __fdiv_rn(m, 127.0f);
  if (lane == 0) scale[r] = s;
  int8_t* qrow = q + r * cols;
  for (int c = lane * 8; c < cols; c += 512) {
    float v[8];
    Row8<T>::load(row + c, v);
    uint32_t b[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float t = (s > 0.f) ? __builtin_rintf(__fdiv_rn(v[i], s)) : 0.f;
      t = fminf(fmaxf(t, -127.f), 127.f);
      b[i >> 2] |= ((uint32_t)(int32_t)t & 0xffu) << (8 * (i & 3));
    }
    *reinterpret_cast<uint2*>(qrow + c) = make_uint2(b[0], b[1]);
  }
}

// INT4: the same with 7 for 127 (codes in [-7, 7]); a lane's 8 codes of a
// step go out as one 4-byte store, element 2i in the low nibble of byte i.
template <typename T>
__global__ __launch_bounds__(256) void quantize_int4_kernel(const T* __restrict__ w, int64_t rows,
                                                            int cols, uint8_t* __restrict__ q,
                                                            float* __restrict__ scale) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const T* row = w + r * cols;
  float m = 0.f;
  for (int c = lane * 8; c < cols; c += 512) {
    float v[8];
    Row8<T>::load(row + c, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  const float s = __fdiv_rn(m, 7.0f);
  if (lane == 0) scale[r] = s;
  uint8_t* qrow = q + r * (cols / 2);
  for (int c = lane * 8; c < cols; c += 512) {
    float v[8];
    Row8<T>::load(row + c, v);
    uint32_t b = 0u;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float t = (s > 0.f) ? __builtin_rintf(__fdiv_rn(v[i], s)) : 0.f;
      t = fminf(fmaxf(t, -7.f), 7.f);
      b |= ((uint32_t)(int32_t)t & 0xfu) << (4 * i);
    }
    *reinterpret_cast<uint32_t*>(qrow + c / 2) = b;
  }
}

}  // namespace

hipError_t launch_quantize_int4(const void* w, int dtype, int64_t rows, int cols, uint8_t* q,
                                float* scale, hipStream_t s) {
  const int64_t blocks = (rows + 3) / 4;
  if (dtype == 0)
    hipLaunchKernelGGL(quantize_int4_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, s,
                       static_cast<const float*>(w), rows, cols, q, scale);
  else
    hipLaunchKernelGGL(quantize_int4_kernel<uint16_t>, dim3((unsigned)blocks), dim3(256), 0, s,
                       static_cast<const uint16_t*>(w), rows, cols, q, scale);
  return hipGetLastError();
}

hipError_t launch_quantize_int8(const void* w, int dtype, int64_t rows, int cols, int8_t* q,
                                float* scale, hipStream_t s) {
  const int64_t blocks = (rows + 3) / 4;
  if (dtype == 0)
    hipLaunchKernelGGL(quantize_int8_kernel<float>, dim3((unsigned)blocks), dim3(256), 0, s,
                       static_cast<const float*>(w), rows, cols, q, scale);
  else
    hipLaunchKernelGGL(quantize_int8_kernel<uint16_t>, dim3((unsigned)blocks), dim3(256), 0, s,
                       static_cast<const uint16_t*>(w), rows, cols, q, scale);
  return hipGetLastError();
}

}  // namespace moe
