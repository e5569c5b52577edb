// Backward pass of the layer: the bandwidth-bound kernels.
//
// What is computed (lmnt.cn MoE walkthrough §2.2: in training the K routing
// weights take part in back-propagation, which is how the gate learns;
// §5.1-5.3: the balance loss and the z-loss reach the gate through its
// probabilities and logits; §4.1: gradients are kept in 16 bits like the
// weights under mixed precision): the gradient of the forward with the Top-K
// choice and the capacity drops held at their forward values.  With
// g = d out (the upstream gradient of the layer output):
//   combine:   d_y_perm[row(t,k)] = w[t,k] * g[t];  d_w[t,k] = <g[t], y_perm[row(t,k)]>
//              (0 for a dropped slot)
//   GELU:      d_z = d_h * GELU'(z),  GELU'(z) = Phi(z) + z phi(z)
//   unpermute: d_x[t] = sum_{kept k} d_x_perm[row(t,k)] + d_x_shared[t] + d_x_router[t]
//   router:    d_l[t, sel_k] += w_k (d_w_k - sum_j w_j d_w_j)
//              d_l[t, e]     += g_aux * alpha N / T * p_te (f_e - sum_e' f_e' p_te')
//              d_l[t, e]     += g_z * 2 beta / T * lse_t * p_te
//              d_W_r = d_l^T x,  d_b_r = sum_t d_l,  d_x_router = d_l W_r
// The grouped GEMMs of the expert backward run on the forward's GEMM kernels:
// the input gradients read the forward's weights k-major, the weight
// gradients run in their k-segment mode on activations transposed per expert
// into zero-padded segments (transpose_segments below, which also forms the
// bias gradients as column sums).
//
// Every reduction has a fixed order, so results are deterministic.
#include <math.h>

#include "moe_internal.h"

namespace moe {
namespace {

// 16 bytes of T: 8 bf16 or 4 fp32
template <typename T>
struct V16;
template <>
struct V16<uint16_t> {
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
  static __device__ __forceinline__ float gelu(float z) { return gelu_as(z); }
  static __device__ __forceinline__ float gelu_grad(float z) { return gelu_grad_as(z); }
};
template <>
struct V16<float> {
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
  static __device__ __forceinline__ float gelu(float z) { return gelu_erf(z); }
  static __device__ __forceinline__ float gelu_grad(float z) { return gelu_grad_erf(z); }
};

// ---------------------------------------------------------------- elementwise
// Rows [0, *nrows) of a [*, width] matrix, as 16-byte pieces.  The GELU has
// the form the forward's fused epilogue uses for the dtype.
template <typename T>
__global__ __launch_bounds__(256) void gelu_fwd_kernel(const uint4* __restrict__ z,
                                                       uint4* __restrict__ h,
                                                       const int32_t* __restrict__ nrows,
                                                       int rows_const, int width) {
  const int rows = nrows ? *nrows : rows_const;
  const int64_t n = (int64_t)rows * width / V16<T>::N;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    float v[V16<T>::N];
    V16<T>::unpack(z[i], v);
#pragma unroll
    for (int q = 0; q < V16<T>::N; ++q) v[q] = V16<T>::gelu(v[q]);
    h[i] = V16<T>::pack(v);
  }
}

// d_z = d_h * GELU'(z), written over d_h.
template <typename T>
__global__ __launch_bounds__(256) void gelu_bwd_kernel(const uint4* __restrict__ z,
                                                       uint4* __restrict__ dh,
                                                       const int32_t* __restrict__ nrows,
                                                       int rows_const, int width) {
  const int rows = nrows ? *nrows : rows_const;
  const int64_t n = (int64_t)rows * width / V16<T>::N;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    float zv[V16<T>::N], g[V16<T>::N];
    V16<T>::unpack(z[i], zv);
    V16<T>::unpack(dh[i], g);
#pragma unroll
    for (int q = 0; q < V16<T>::N; ++q) g[q] *= V16<T>::gelu_grad(zv[q]);
    dh[i] = V16<T>::pack(g);
  }
}

// ---------------------------------------------------------------- combine backward
// A 16-byte piece of a permuted row; NT: a non-temporal load, for rows read
// once from arrays too large for the MALL (the per-slot rows of the
// DeepSeek-shaped layer, 470 MB), where cached loads only evict each other.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
template <bool NT>
__device__ __forceinline__ uint4 ld_row16(const uint4* p) {
  if constexpr (NT) {
    const u32x4 q = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(q[0], q[1], q[2], q[3]);
  } else {
    return *p;
  }
}
// Per-slot rows of T*K rows x nvec pieces: non-temporal beyond half the MALL.
inline bool rows_nt(int64_t rows, int nvec) { return rows * nvec * 16 > nontemporal_rows_bytes(); }

// One wavefront per token (wave-uniform index, so the slot rows and weights
// are scalar loads); slots in groups of KB.  For each group, a lane walks its
// 16-byte pieces of the row: it loads g[t] and the group's kept y_perm rows,
// adds the products into one fp32 partial dot per slot and stores w * g to
// each kept row of d_y_perm; the partials are then added across the lanes
// by a fixed butterfly.
template <typename T, int KB, int U, bool NT>
__global__ __launch_bounds__(256) void combine_bwd_kernel(
    const uint4* __restrict__ d_out, const uint4* __restrict__ y_perm,
    const int32_t* __restrict__ slot_row, const float* __restrict__ topk_w,
    uint4* __restrict__ d_y_perm, float* __restrict__ d_topk_w, int Ttok, int nvec, int K) {
  constexpr int EV = V16<T>::N;
  const int t = __builtin_amdgcn_readfirstlane((int)(blockIdx.x * 4 + (threadIdx.x >> 6)));
  if (t >= Ttok) return;
  const int lane = threadIdx.x & 63;
  const int32_t* sr = slot_row + (int64_t)t * K;
  const float* wt = topk_w + (int64_t)t * K;
  const uint4* g_row = d_out + (int64_t)t * nvec;
  for (int k0 = 0; k0 < K; k0 += KB) {
    int r[KB];
    float w[KB], dot[KB];
#pragma unroll
    for (int j = 0; j < KB; ++j) {
      r[j] = (k0 + j < K) ? sr[k0 + j] : -1;
      w[j] = (r[j] >= 0) ? wt[k0 + j] : 0.f;
      dot[j] = 0.f;
    }
    for (int c0 = lane; c0 < nvec; c0 += 64 * U) {
      uint4 gv[U];
      uint4 v[KB][U];
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (c0 + 64 * u < nvec) gv[u] = g_row[c0 + 64 * u];
#pragma unroll
      for (int j = 0; j < KB; ++j)
        if (r[j] >= 0) {
          const uint4* yr = y_perm + (int64_t)r[j] * nvec;
#pragma unroll
          for (int u = 0; u < U; ++u)
            if (c0 + 64 * u < nvec) v[j][u] = ld_row16<NT>(yr + c0 + 64 * u);
        }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int c = c0 + 64 * u;
        if (c >= nvec) break;
        float g[EV];
        V16<T>::unpack(gv[u], g);
#pragma unroll
        for (int j = 0; j < KB; ++j)
          if (r[j] >= 0) {
            float y[EV], o[EV];
            V16<T>::unpack(v[j][u], y);
#pragma unroll
            for (int q = 0; q < EV; ++q) {
              dot[j] = fmaf(g[q], y[q], dot[j]);
              o[q] = w[j] * g[q];
            }
            d_y_perm[(int64_t)r[j] * nvec + c] = V16<T>::pack(o);
          }
      }
    }
#pragma unroll
    for (int j = 0; j < KB; ++j) {
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) dot[j] += __shfl_xor(dot[j], off, 64);
      if (lane == 0 && k0 + j < K) d_topk_w[(int64_t)t * K + k0 + j] = r[j] >= 0 ? dot[j] : 0.f;
    }
  }
}

// ---------------------------------------------------------------- unpermute
// d_x[t] = (sum over kept slots, in slot order, of d_x_perm[row]) + d_x_shared[t]
// + d_x_router[t]; fp32 sums, one rounding.  Layout as the combine kernel.
template <typename T, int KB, int U, bool NT>
__global__ __launch_bounds__(256) void unpermute_kernel(
    const uint4* __restrict__ d_x_perm, const int32_t* __restrict__ slot_row,
    const uint4* __restrict__ d_x_shared, const float4* __restrict__ d_x_router,
    uint4* __restrict__ d_x, int Ttok, int nvec, int K) {
  constexpr int EV = V16<T>::N;
  const int t = __builtin_amdgcn_readfirstlane((int)(blockIdx.x * 4 + (threadIdx.x >> 6)));
  if (t >= Ttok) return;
  const int lane = threadIdx.x & 63;
  const int32_t* sr = slot_row + (int64_t)t * K;
  for (int c0 = lane; c0 < nvec; c0 += 64 * U) {
    float acc[U][EV];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < EV; ++i) acc[u][i] = 0.f;
    for (int k0 = 0; k0 < K; k0 += KB) {
      int r[KB];
#pragma unroll
      for (int j = 0; j < KB; ++j) r[j] = (k0 + j < K) ? sr[k0 + j] : -1;
      uint4 v[KB][U];
#pragma unroll
      for (int j = 0; j < KB; ++j)
        if (r[j] >= 0) {
          const uint4* src = d_x_perm + (int64_t)r[j] * nvec;
#pragma unroll
          for (int u = 0; u < U; ++u)
            if (c0 + 64 * u < nvec) v[j][u] = ld_row16<NT>(src + c0 + 64 * u);
        }
#pragma unroll
      for (int j = 0; j < KB; ++j)
        if (r[j] >= 0) {
#pragma unroll
          for (int u = 0; u < U; ++u) {
            float y[EV];
            V16<T>::unpack(v[j][u], y);
#pragma unroll
            for (int i = 0; i < EV; ++i) acc[u][i] += y[i];
          }
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + 64 * u;
      if (c >= nvec) break;
      if (d_x_shared) {
        float y[EV];
        V16<T>::unpack(d_x_shared[(int64_t)t * nvec + c], y);
#pragma unroll
        for (int i = 0; i < EV; ++i) acc[u][i] += y[i];
      }
      if (d_x_router) {
        // the EV fp32 values of this piece: EV / 4 float4 at element c * EV
        const float4* rr = d_x_router + ((int64_t)t * nvec + c) * (EV / 4);
#pragma unroll
        for (int i = 0; i < EV / 4; ++i) {
          const float4 q = rr[i];
          acc[u][4 * i] += q.x;
          acc[u][4 * i + 1] += q.y;
          acc[u][4 * i + 2] += q.z;
          acc[u][4 * i + 3] += q.w;
        }
      }
      d_x[(int64_t)t * nvec + c] = V16<T>::pack(acc[u]);
    }
  }
}

// ---------------------------------------------------------------- transposes
// 64 x 64 tiles through LDS: 16-byte loads of tile rows, 16-byte stores of
// transposed rows (each gathers VEC elements down a column of the tile).
constexpr int TD = 64;

template <typename T>
struct TileT {
  static constexpr int VEC = 16 / (int)sizeof(T);
  static constexpr int CPR = TD / VEC;               // 16-byte pieces per tile row
  // bf16: unpadded 128-byte rows, piece p of row r stored at p ^ ((r / 8) mod 8).
  // A read-phase instruction has its 64 lanes read element q of 8 rows r0 + 8i
  // (one per lane group) in 8 columns of one piece: the XOR puts the 8 rows'
  // pieces in 8 different 16-byte bank groups of the same 128-byte half, and
  // the 8 columns of a piece fall on 4 dwords, so no bank serves two dwords.
  // fp32: rows padded by one piece.
  static constexpr bool SWZ = sizeof(T) == 2;
  static constexpr int LD = SWZ ? TD : TD + VEC;     // LDS row (16-byte aligned)
  static __device__ __forceinline__ int at(int r, int c) {   // element (r, c) of the tile
    return SWZ ? r * LD + ((((c / VEC) ^ ((r >> 3) & (CPR - 1)))) * VEC) + c % VEC : r * LD + c;
  }
};

// Expert e's rows [off[e], off[e+1]) of in [*, C] become columns
// [kseg[e], kseg[e+1]) of out [C, ldo]: out[c][kseg[e] + j] = in[off[e] + j][c]
// for j < R_e and 0 in the padding up to kseg[e+1]; colsum[e][c] (if not null)
// = sum over the expert's rows of in[.][c] (fp32, fixed order, stored as T).
// grid (C/64, number of segments, row split); a workgroup walks every
// gridDim.z-th 64-row tile of its segment (the shared expert's single
// segment of T rows is split so that its launch fills the chip; with
// colsum the row split is 1).
template <typename T>
__global__ __launch_bounds__(256) void transpose_segments_kernel(
    const T* __restrict__ in, const int32_t* __restrict__ off, const int32_t* __restrict__ kseg,
    int C, int ldo, T* __restrict__ out, T* __restrict__ colsum) {
  using TT = TileT<T>;
  constexpr int PER = TD * TT::CPR / 256;            // read-phase items per thread
  __shared__ __attribute__((aligned(16))) T tile[TD * TT::LD];
  const int e = blockIdx.y, c0 = blockIdx.x * TD;
  const int row0 = off[e], R = off[e + 1] - row0;
  const int k0 = kseg[e], KP = kseg[e + 1] - k0;
  float part[PER];
#pragma unroll
  for (int p = 0; p < PER; ++p) part[p] = 0.f;
  for (int j0 = blockIdx.z * TD; j0 < KP; j0 += gridDim.z * TD) {
    for (int i = threadIdx.x; i < TD * TT::CPR; i += 256) {
      const int r = i / TT::CPR, cc = (i % TT::CPR) * TT::VEC;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (j0 + r < R) v = *reinterpret_cast<const uint4*>(in + (int64_t)(row0 + j0 + r) * C + c0 + cc);
      *reinterpret_cast<uint4*>(tile + TT::at(r, cc)) = v;
    }
    __syncthreads();
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      const int i = threadIdx.x + 256 * p;
      const int oc = i / TT::CPR, rr = (i % TT::CPR) * TT::VEC;
      alignas(16) T v[TT::VEC];
#pragma unroll
      for (int q = 0; q < TT::VEC; ++q) {
        v[q] = tile[TT::at(rr + q, oc)];
        part[p] += Elem<T>::load(v, q);
      }
      if (j0 + rr < KP)
        *reinterpret_cast<uint4*>(out + (int64_t)(c0 + oc) * ldo + k0 + j0 + rr) =
            *reinterpret_cast<const uint4*>(v);
    }
    __syncthreads();
  }
  if (colsum) {
#pragma unroll
    for (int p = 0; p < PER; ++p) {
      // the CPR threads of one column are consecutive lanes
#pragma unroll
      for (int o = 1; o < TT::CPR; o <<= 1) part[p] += __shfl_xor(part[p], o, 64);
      const int i = threadIdx.x + 256 * p;
      if (i % TT::CPR == 0) Elem<T>::store(colsum, (int64_t)e * C + c0 + i / TT::CPR, part[p]);
    }
  }
}

// kseg[e] = sum over e' < e of round_up(off[e'+1] - off[e'], 32), e = 0..N;
// wa[e] = e * ra, wb[e] = e * rb.  One workgroup of 256 threads (N <= 256).
__global__ __launch_bounds__(256) void seg_offsets_kernel(const int32_t* __restrict__ off, int N,
                                                          int ra, int rb,
                                                          int32_t* __restrict__ kseg,
                                                          int32_t* __restrict__ wa,
                                                          int32_t* __restrict__ wb) {
  __shared__ int wsum[4];
  const int e = threadIdx.x;
  const int n = e < N ? ((off[e + 1] - off[e] + 31) / 32) * 32 : 0;
  const int lane = e & 63, wave = e >> 6;
  int v = n;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(v, o, 64);
    if (lane >= o) v += u;
  }
  if (lane == 63) wsum[wave] = v;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += wsum[w];
  if (e < N) {
    kseg[e] = base + v - n;
    wa[e] = e * ra;
    wb[e] = e * rb;
  }
  if (e == N - 1) {
    kseg[N] = base + v;
    wa[N] = N * ra;
    wb[N] = N * rb;
  }
}

// One dense segment of T rows: off = {0, T}, kseg = {0, round_up(T, 32)},
// wa = {0, ra}, wb = {0, rb}.
__global__ void dense_offsets_kernel(int T, int ra, int rb, int32_t* __restrict__ off,
                                     int32_t* __restrict__ kseg, int32_t* __restrict__ wa,
                                     int32_t* __restrict__ wb) {
  if (threadIdx.x == 0) {
    off[0] = 0;
    off[1] = T;
    kseg[0] = 0;
    kseg[1] = ((T + 31) / 32) * 32;
    wa[0] = 0;
    wa[1] = ra;
    wb[0] = 0;
    wb[1] = rb;
  }
}

// ---------------------------------------------------------------- router backward
// d_l for one token per wavefront; lane = expert (e, e + 64, e + 128, e + 192).
// The softmax over all N (for the aux loss and the z-loss) in fp32.
__global__ __launch_bounds__(256) void route_bwd_logits_kernel(
    const float* __restrict__ logits, const int32_t* __restrict__ idx,
    const float* __restrict__ w, const float* __restrict__ dw,
    const int32_t* __restrict__ counts, int Ttok, int N, int K, float aux_coef, float z_coef,
    float* __restrict__ dl) {
  const int t = __builtin_amdgcn_readfirstlane((int)(blockIdx.x * 4 + (threadIdx.x >> 6)));
  if (t >= Ttok) return;
  const int lane = threadIdx.x & 63;
  const int32_t* it = idx + (int64_t)t * K;
  const float* wtt = w + (int64_t)t * K;
  const float* dwt = dw + (int64_t)t * K;
  float s = 0.f;
  for (int k = lane; k < K; k += 64) s = fmaf(wtt[k], dwt[k], s);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) s += __shfl_xor(s, o, 64);
  float l[4], p[4];
  float lse = 0.f, fp = 0.f;
  const bool smx = aux_coef != 0.f || z_coef != 0.f;
  if (smx) {
    float m = -INFINITY;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int e = lane + 64 * v;
      l[v] = e < N ? logits[(int64_t)t * N + e] : -INFINITY;
      m = fmaxf(m, l[v]);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    float S = 0.f;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      p[v] = (lane + 64 * v < N) ? expf(l[v] - m) : 0.f;
      S += p[v];
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) S += __shfl_xor(S, o, 64);
    const float inv = 1.0f / S;
    lse = m + logf(S);
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      p[v] *= inv;
      const int e = lane + 64 * v;
      if (aux_coef != 0.f && e < N) fp = fmaf((float)counts[e] / (float)Ttok, p[v], fp);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) fp += __shfl_xor(fp, o, 64);
  }
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int e = lane + 64 * v;
    if (e >= N) continue;
    float g = 0.f;
    for (int k = 0; k < K; ++k)
      if (it[k] == e) g = wtt[k] * (dwt[k] - s);
    if (aux_coef != 0.f) g = fmaf(aux_coef * p[v], (float)counts[e] / (float)Ttok - fp, g);
    if (z_coef != 0.f) g = fmaf(z_coef * lse, p[v], g);
    dl[(int64_t)t * N + e] = g;
  }
}

// Four consecutive elements of a bf16 or fp32 row (aligned to four
// elements), kept packed until each is widened to fp32 (at).
template <typename T>
struct R4;
template <>
struct R4<uint16_t> {
  uint2 v;
  __device__ __forceinline__ void load(const uint16_t* p) { v = *reinterpret_cast<const uint2*>(p); }
  __device__ __forceinline__ float at(int q) const {
    const uint32_t w = q < 2 ? v.x : v.y;
    return __uint_as_float((q & 1) ? (w & 0xffff0000u) : (w << 16));
  }
};
template <>
struct R4<float> {
  float4 v;
  __device__ __forceinline__ void load(const float* p) { v = *reinterpret_cast<const float4*>(p); }
  __device__ __forceinline__ float at(int q) const {
    return q == 0 ? v.x : (q == 1 ? v.y : (q == 2 ? v.z : v.w));
  }
};

typedef float f32x16 __attribute__((ext_vector_type(16)));

// The router's two gradient products run on the fp32 matrix cores
// (v_mfma_f32_32x32x2f32: a 32x32 block, two k per instruction; the bf16
// operands widen to fp32 exactly).  A workgroup tile is 32 rows x 512
// columns; wavefront w owns columns [128w, 128w + 128) as four 32-column
// blocks, column n of block q being tile column 4n + q, so each lane loads
// and stores four consecutive columns.  In the instruction's layout lane l
// supplies row l%32 and column l%32 of the two operands at k = l/32, and its
// result register v holds row (v/4)*8 + (l/32)*4 + v%4, column l%32.
//
// Workgroup b runs on XCD b mod 8; it takes the b/8-th tile of that XCD's
// contiguous share of the tile space, so workgroups running together on one
// XCD take neighbouring tiles and share their operands in its L2.
__device__ __forceinline__ int xcd_tile(int b, int total) {
  const int xcd = b & 7, slot = b >> 3, per = total >> 3, extra = total & 7;
  return xcd * per + min(xcd, extra) + slot;
}

// Partial router weight gradient over a slice of tokens:
// part[s][e][j] = sum_{t in slice s} d_l[t][e] * x[t][j].  Tile: 32 experts x
// 512 columns x one slice, ordered expert block fastest (the tiles an XCD runs
// together read the same x panel), then column block, then slice.  The k-loop
// runs 16 tokens (8 instructions per block) at a time, the loads of the next
// 16 in flight during the products of these.
template <typename T>
__global__ __launch_bounds__(256) void router_dw_kernel(const float* __restrict__ dl,
                                                        const T* __restrict__ x, int Ttok, int N,
                                                        int d, int tslice, int nS,
                                                        float* __restrict__ part) {
  const int nE = (N + 31) / 32, nC = (d + 511) / 512;
  const int L = xcd_tile(blockIdx.x, nE * nC * nS);
  const int eb = (L % nE) * 32, cb = (L / nE) % nC, s = L / (nE * nC);
  const int lane = threadIdx.x & 63, n = lane & 31, kh = lane >> 5;
  const int j = cb * 512 + (threadIdx.x >> 6) * 128 + 4 * n;
  const bool jv = j < d;
  const int jc = jv ? j : 0, ec = min(eb + n, N - 1);
  const int tlo = s * tslice, thi = min(Ttok, tlo + tslice);
  f32x16 acc[4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[q][v] = 0.f;
  // a token past the slice reads the last token's row and weighs it 0; rows
  // and columns past N and d are computed from clamped addresses and not stored
  auto load = [&](int t0, float* a, R4<T>* b) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int tc = min(t0 + 2 * u + kh, thi - 1);
      a[u] = dl[(int64_t)tc * N + ec];
      b[u].load(x + (int64_t)tc * d + jc);
    }
  };
  auto mma = [&](int t0, const float* a, const R4<T>* b) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float av = a[u] * (t0 + 2 * u + kh < thi ? 1.f : 0.f);
#pragma unroll
      for (int q = 0; q < 4; ++q)
        acc[q] = __builtin_amdgcn_mfma_f32_32x32x2f32(av, b[u].at(q), acc[q], 0, 0, 0);
    }
  };
  const int nch = (thi - tlo + 15) / 16;
  float a0[8], a1[8];
  R4<T> b0[8], b1[8];
  load(tlo, a0, b0);
  int c = 0;
  for (; c + 1 < nch; c += 2) {
    load(tlo + 16 * (c + 1), a1, b1);
    __builtin_amdgcn_sched_barrier(0);
    mma(tlo + 16 * c, a0, b0);
    __builtin_amdgcn_sched_barrier(0);
    load(tlo + 16 * (c + 2), a0, b0);
    __builtin_amdgcn_sched_barrier(0);
    mma(tlo + 16 * (c + 1), a1, b1);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (c < nch) mma(tlo + 16 * c, a0, b0);
  if (!jv) return;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int e = eb + (v >> 2) * 8 + kh * 4 + (v & 3);
    if (e < N)
      *reinterpret_cast<float4*>(part + ((int64_t)s * N + e) * d + j) =
          make_float4(acc[0][v], acc[1][v], acc[2][v], acc[3][v]);
  }
}

// d_W_r[e][j] = sum over slices, in slice order, of part[s][e][j].
__global__ __launch_bounds__(256) void router_dw_reduce_kernel(const float* __restrict__ part,
                                                               int S, int64_t n,
                                                               float* __restrict__ dwr) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    float a = 0.f;
    for (int s = 0; s < S; ++s) a += part[(int64_t)s * n + i];
    dwr[i] = a;
  }
}

// d_b_r[e] = sum_t d_l[t][e]: one wavefront per expert, lanes stride over the
// tokens, then a fixed butterfly.
__global__ __launch_bounds__(64) void router_db_kernel(const float* __restrict__ dl, int Ttok,
                                                       int N, float* __restrict__ dbr) {
  const int e = blockIdx.x, lane = threadIdx.x;
  float a = 0.f;
  for (int t = lane; t < Ttok; t += 64) a += dl[(int64_t)t * N + e];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) a += __shfl_xor(a, o, 64);
  if (lane == 0) dbr[e] = a;
}

// d_x_router[t][j] = sum_e d_l[t][e] * W_r[e][j] (fp32).  Tile: 32 tokens x
// 512 columns, ordered token block fastest (the tiles an XCD runs together
// read the same W_r panel).  d_l of the 32 tokens is staged in LDS whole
// (N <= 256, zero-padded to a multiple of 16 experts); W_r is read straight
// from memory, 16 experts at a time with the next 16 in flight.
template <typename T>
__global__ __launch_bounds__(256) void router_dx_kernel(const float* __restrict__ dl,
                                                        const T* __restrict__ wr, int Ttok, int N,
                                                        int d, float* __restrict__ dxr) {
  __shared__ float sdl[32][257];
  const int nT = (Ttok + 31) / 32, nC = (d + 511) / 512;
  const int L = xcd_tile(blockIdx.x, nT * nC);
  const int tb = (L % nT) * 32, cb = L / nT;
  const int lane = threadIdx.x & 63, n = lane & 31, kh = lane >> 5;
  const int j = cb * 512 + (threadIdx.x >> 6) * 128 + 4 * n;
  const bool jv = j < d;
  const int jc = jv ? j : 0;
  const int Np = (N + 15) / 16 * 16;
  for (int i = threadIdx.x; i < 32 * Np; i += 256) {
    const int tt = i / Np, ee = i % Np;
    sdl[tt][ee] = (tb + tt < Ttok && ee < N) ? dl[(int64_t)(tb + tt) * N + ee] : 0.f;
  }
  __syncthreads();
  f32x16 acc[4];
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[q][v] = 0.f;
  // an expert past N reads W_r's last row against a staged 0; columns past d
  // are computed from clamped addresses and not stored
  auto load = [&](int k0, R4<T>* b) {
#pragma unroll
    for (int u = 0; u < 8; ++u)
      b[u].load(wr + (int64_t)min(k0 + 2 * u + kh, N - 1) * d + jc);
  };
  auto mma = [&](int k0, const R4<T>* b) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float a = sdl[n][k0 + 2 * u + kh];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        acc[q] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b[u].at(q), acc[q], 0, 0, 0);
    }
  };
  const int nch = Np / 16;
  R4<T> b0[8], b1[8];
  load(0, b0);
  int c = 0;
  for (; c + 1 < nch; c += 2) {
    load(16 * (c + 1), b1);
    __builtin_amdgcn_sched_barrier(0);
    mma(16 * c, b0);
    __builtin_amdgcn_sched_barrier(0);
    load(16 * (c + 2), b0);
    __builtin_amdgcn_sched_barrier(0);
    mma(16 * (c + 1), b1);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (c < nch) mma(16 * c, b0);
  if (!jv) return;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int t = tb + (v >> 2) * 8 + kh * 4 + (v & 3);
    if (t < Ttok)
      *reinterpret_cast<float4*>(dxr + (int64_t)t * d + j) =
          make_float4(acc[0][v], acc[1][v], acc[2][v], acc[3][v]);
  }
}

inline unsigned ew_blocks(int64_t rows, int width, int vec) {
  const int64_t n = rows * width / vec;
  const int64_t b = (n + 255) / 256;
  return (unsigned)(b < 1 ? 1 : (b > 65536 ? 65536 : b));
}

}  // namespace

hipError_t launch_gelu_fwd(int dtype, const void* z, void* h, const int32_t* nrows, int rows_max,
                           int width, hipStream_t s) {
  if (dtype == 0)
    hipLaunchKernelGGL(gelu_fwd_kernel<float>, dim3(ew_blocks(rows_max, width, 4)), dim3(256), 0,
                       s, static_cast<const uint4*>(z), static_cast<uint4*>(h), nrows, rows_max,
                       width);
  else
    hipLaunchKernelGGL(gelu_fwd_kernel<uint16_t>, dim3(ew_blocks(rows_max, width, 8)), dim3(256),
                       0, s, static_cast<const uint4*>(z), static_cast<uint4*>(h), nrows,
                       rows_max, width);
  return hipGetLastError();
}

hipError_t launch_gelu_bwd(int dtype, const void* z, void* dh, const int32_t* nrows, int rows_max,
                           int width, hipStream_t s) {
  if (dtype == 0)
    hipLaunchKernelGGL(gelu_bwd_kernel<float>, dim3(ew_blocks(rows_max, width, 4)), dim3(256), 0,
                       s, static_cast<const uint4*>(z), static_cast<uint4*>(dh), nrows, rows_max,
                       width);
  else
    hipLaunchKernelGGL(gelu_bwd_kernel<uint16_t>, dim3(ew_blocks(rows_max, width, 8)), dim3(256),
                       0, s, static_cast<const uint4*>(z), static_cast<uint4*>(dh), nrows,
                       rows_max, width);
  return hipGetLastError();
}

template <typename T>
static void combine_bwd_t(const void* d_out, const void* y_perm, const int32_t* slot_row,
                          const float* topk_w, void* d_y_perm, float* d_topk_w, int Ttok,
                          int nvec, int K, hipStream_t s) {
  const dim3 grid((Ttok + 3) / 4), block(256);
  const uint4* g = static_cast<const uint4*>(d_out);
  const uint4* y = static_cast<const uint4*>(y_perm);
  uint4* dy = static_cast<uint4*>(d_y_perm);
  const bool nt = rows_nt((int64_t)Ttok * K, nvec);
  if (K <= 2)
    hipLaunchKernelGGL((combine_bwd_kernel<T, 2, 2, false>), grid, block, 0, s, g, y, slot_row,
                       topk_w, dy, d_topk_w, Ttok, nvec, K);
  else if (nt)
    hipLaunchKernelGGL((combine_bwd_kernel<T, 8, 1, true>), grid, block, 0, s, g, y, slot_row,
                       topk_w, dy, d_topk_w, Ttok, nvec, K);
  else
    hipLaunchKernelGGL((combine_bwd_kernel<T, 8, 1, false>), grid, block, 0, s, g, y, slot_row,
                       topk_w, dy, d_topk_w, Ttok, nvec, K);
}

hipError_t launch_combine_bwd(int dtype, const void* d_out, const void* y_perm,
                              const int32_t* slot_row, const float* topk_w, void* d_y_perm,
                              float* d_topk_w, int T, int d, int K, hipStream_t s) {
  const int nvec = d * (dtype == 0 ? 4 : 2) / 16;
  if (dtype == 0)
    combine_bwd_t<float>(d_out, y_perm, slot_row, topk_w, d_y_perm, d_topk_w, T, nvec, K, s);
  else
    combine_bwd_t<uint16_t>(d_out, y_perm, slot_row, topk_w, d_y_perm, d_topk_w, T, nvec, K, s);
  return hipGetLastError();
}

template <typename T>
static void unpermute_t(const void* d_x_perm, const int32_t* slot_row, const void* d_x_shared,
                        const float* d_x_router, void* d_x, int Ttok, int nvec, int K,
                        hipStream_t s) {
  const dim3 grid((Ttok + 3) / 4), block(256);
  const uint4* a = static_cast<const uint4*>(d_x_perm);
  const uint4* sh = static_cast<const uint4*>(d_x_shared);
  const float4* rt = reinterpret_cast<const float4*>(d_x_router);
  uint4* o = static_cast<uint4*>(d_x);
  const bool nt = rows_nt((int64_t)Ttok * K, nvec);
  if (K <= 2)
    hipLaunchKernelGGL((unpermute_kernel<T, 2, 4, false>), grid, block, 0, s, a, slot_row, sh, rt,
                       o, Ttok, nvec, K);
  else if (nt)
    hipLaunchKernelGGL((unpermute_kernel<T, 8, 2, true>), grid, block, 0, s, a, slot_row, sh, rt,
                       o, Ttok, nvec, K);
  else
    hipLaunchKernelGGL((unpermute_kernel<T, 8, 2, false>), grid, block, 0, s, a, slot_row, sh, rt,
                       o, Ttok, nvec, K);
}

hipError_t launch_unpermute(int dtype, const void* d_x_perm, const int32_t* slot_row,
                            const void* d_x_shared, const float* d_x_router, void* d_x, int T,
                            int d, int K, hipStream_t s) {
  const int nvec = d * (dtype == 0 ? 4 : 2) / 16;
  if (dtype == 0)
    unpermute_t<float>(d_x_perm, slot_row, d_x_shared, d_x_router, d_x, T, nvec, K, s);
  else
    unpermute_t<uint16_t>(d_x_perm, slot_row, d_x_shared, d_x_router, d_x, T, nvec, K, s);
  return hipGetLastError();
}

hipError_t launch_transpose_segments(int dtype, const void* in, const int32_t* off,
                                     const int32_t* kseg, int nseg, int C, int ldo, void* out,
                                     void* colsum, hipStream_t s, int max_rows) {
  // a single segment of max_rows rows: split its 64-row tiles over enough
  // workgroups for about eight per CU (column sums need one walk per column)
  int rs = 1;
  if (nseg == 1 && !colsum && max_rows > TD) {
    const int tiles = (max_rows + TD - 1) / TD, cols = C / TD;
    rs = max(1, min(tiles, (2048 + cols - 1) / cols));
  }
  const dim3 grid(C / TD, nseg, rs);
  if (dtype == 0)
    hipLaunchKernelGGL(transpose_segments_kernel<float>, grid, dim3(256), 0, s,
                       static_cast<const float*>(in), off, kseg, C, ldo, static_cast<float*>(out),
                       static_cast<float*>(colsum));
  else
    hipLaunchKernelGGL(transpose_segments_kernel<uint16_t>, grid, dim3(256), 0, s,
                       static_cast<const uint16_t*>(in), off, kseg, C, ldo,
                       static_cast<uint16_t*>(out), static_cast<uint16_t*>(colsum));
  return hipGetLastError();
}

hipError_t launch_seg_offsets(const int32_t* off, int N, int ra, int rb, int32_t* kseg,
                              int32_t* wa, int32_t* wb, hipStream_t s) {
  hipLaunchKernelGGL(seg_offsets_kernel, dim3(1), dim3(256), 0, s, off, N, ra, rb, kseg, wa, wb);
  return hipGetLastError();
}

hipError_t launch_dense_offsets(int T, int ra, int rb, int32_t* off, int32_t* kseg, int32_t* wa,
                                int32_t* wb, hipStream_t s) {
  hipLaunchKernelGGL(dense_offsets_kernel, dim3(1), dim3(64), 0, s, T, ra, rb, off, kseg, wa, wb);
  return hipGetLastError();
}

// Token slices of the router weight gradient: about 2048 wavefronts in all
// (4 per tile and slice), at least 64 tokens a slice, each slice a multiple
// of 16 tokens.  Returns the slice count; *tslice gets the slice length.
int router_dw_split(int T, int N, int d, int* tslice) {
  const int tiles = ((N + 31) / 32) * ((d + 511) / 512);
  int S = (512 + tiles - 1) / tiles;
  const int maxS = (T + 63) / 64;
  if (S > maxS) S = maxS;
  if (S < 1) S = 1;
  const int ts = ((T + S - 1) / S + 15) / 16 * 16;
  if (tslice) *tslice = ts;
  return (T + ts - 1) / ts;
}

int router_dw_slices(int T, int N, int d) { return router_dw_split(T, N, d, nullptr); }

hipError_t launch_route_bwd(int dtype, const void* x, const void* w_router, const float* logits,
                            const int32_t* topk_idx, const float* topk_w, const float* d_topk_w,
                            const int32_t* counts, float aux_coef, float z_coef, float* dl,
                            float* part, float* d_w_router, float* d_b_router, float* d_x_router,
                            int T, int d, int N, int K, hipStream_t s) {
  // the d_x share stages a token block's d_l (at most 256 experts) in LDS
  if (N > 256 || d % 64 != 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(route_bwd_logits_kernel, dim3((T + 3) / 4), dim3(256), 0, s, logits,
                     topk_idx, topk_w, d_topk_w, counts, T, N, K, aux_coef, z_coef, dl);
  int tslice = 0;
  const int S = router_dw_split(T, N, d, &tslice);
  const int nC = (d + 511) / 512;
  const dim3 g1((unsigned)(((N + 31) / 32) * nC * S));
  if (dtype == 0)
    hipLaunchKernelGGL(router_dw_kernel<float>, g1, dim3(256), 0, s, dl,
                       static_cast<const float*>(x), T, N, d, tslice, S, part);
  else
    hipLaunchKernelGGL(router_dw_kernel<uint16_t>, g1, dim3(256), 0, s, dl,
                       static_cast<const uint16_t*>(x), T, N, d, tslice, S, part);
  const int64_t n = (int64_t)N * d;
  hipLaunchKernelGGL(router_dw_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                     part, S, n, d_w_router);
  if (d_b_router)
    hipLaunchKernelGGL(router_db_kernel, dim3(N), dim3(64), 0, s, dl, T, N, d_b_router);
  if (d_x_router) {
    const dim3 g2((unsigned)(((T + 31) / 32) * nC));
    if (dtype == 0)
      hipLaunchKernelGGL(router_dx_kernel<float>, g2, dim3(256), 0, s, dl,
                         static_cast<const float*>(w_router), T, N, d, d_x_router);
    else
      hipLaunchKernelGGL(router_dx_kernel<uint16_t>, g2, dim3(256), 0, s, dl,
                         static_cast<const uint16_t*>(w_router), T, N, d, d_x_router);
  }
  return hipGetLastError();
}

}  // namespace moe
