// Internal declarations shared by the HIP translation units of libmoe.so.
// Device helpers for bf16 storage and the launchers each kernel file exports
// to the host API (moe_api.hip).  Nothing here is part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// ---------------------------------------------------------------- bf16 storage
// bf16 values travel as raw uint16 bit patterns; widening is exact.
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// fp32 -> bf16, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

// Eight fp32 values rounded to bf16 and packed into 16 bytes: v_cvt_pk_bf16_f32
// rounds to nearest even like f32_to_bf16 (equal on every finite input,
// ties included), two values per instruction.
__device__ __forceinline__ uint4 pack_bf16x8(const float* f) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    w[i] = __builtin_bit_cast(uint32_t,
                              __builtin_convertvector((f32x2_t){f[2 * i], f[2 * i + 1]}, bf16x2_t));
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// Exact GELU, z/2 * (1 + erf(z / sqrt(2))).
__device__ __forceinline__ float gelu_erf(float z) {
  return 0.5f * z * (1.0f + erff(z * 0.70710678118654752440f));
}

// GELU with erf from Abramowitz & Stegun, Handbook of Mathematical Functions,
// formula 7.1.26: for x >= 0, erf(x) = 1 - P(t) exp(-x^2), P(t) = a1 t + ... +
// a5 t^5, t = 1 / (1 + p x), |error| <= 1.5e-7; odd symmetry for x < 0.
// With x = |z| / sqrt(2) both signs of z collapse to
//   GELU(z) = max(z, 0) - |z|/2 * P(t) * exp(-z^2 / 2),
// which the code evaluates with the -1/2 folded into the coefficients: one
// reciprocal, one exp2 and ten other VALU operations (this runs on every
// element of the first GEMM's output, at a quarter of the MFMA tile's time
// budget when it was written naively).  Against the exact GELU (a CPU sweep
// of z in [-9, 9]): absolute error <= 2.2e-7 everywhere, i.e. <= 0.013 bf16
// ulp of the result for |z| < 3 and <= 0.4 ulp for -5 < z < -3; below -5,
// where |GELU(z)| < 1.5e-6, the relative error grows (a few ulp, and more
// far out) while the absolute error stays below 2.3e-9.  Every bf16 path
// (prefill and decode GEMMs, training forward and backward) uses this form;
// the fp32 layer uses the library erff.
__device__ __forceinline__ float gelu_as(float z) {
  const float az = fabsf(z);
  const float t = __builtin_amdgcn_rcpf(fmaf(0.23164189f, az, 1.0f));   // p / sqrt(2)
  float q = fmaf(-0.5307027145f, t, 0.7265760135f);   // -a5/2, -a4/2
  q = fmaf(q, t, -0.7107068705f);                      // -a3/2
  q = fmaf(q, t, 0.1422483680f);                       // -a2/2
  q = fmaf(q, t, -0.1274147960f);                      // -a1/2
  const float e = __builtin_amdgcn_exp2f(z * z * -0.72134752044448170368f);   // exp(-z^2/2)
  // max(z, 0) as one v_max_f32 (fmaxf adds a NaN-quieting max in front)
  float relu;
  asm("v_max_f32 %0, 0, %1" : "=v"(relu) : "v"(z));
  return fmaf(az * t, q * e, relu);
}

// d/dz GELU(z) = Phi(z) + z phi(z), with the erf of gelu_as: for x = |z|/sqrt(2),
// t q e = -erfc(x) / 2, so Phi(z) = 1 + t q e for z >= 0 and -t q e for z < 0.
__device__ __forceinline__ float gelu_grad_as(float z) {
  const float az = fabsf(z);
  const float t = __builtin_amdgcn_rcpf(fmaf(0.23164189f, az, 1.0f));
  float q = fmaf(-0.5307027145f, t, 0.7265760135f);
  q = fmaf(q, t, -0.7107068705f);
  q = fmaf(q, t, 0.1422483680f);
  q = fmaf(q, t, -0.1274147960f);
  const float e = __builtin_amdgcn_exp2f(z * z * -0.72134752044448170368f);
  const float tqe = t * q * e;
  const float cdf = z >= 0.f ? 1.0f + tqe : -tqe;
  return fmaf(z * e, 0.39894228040143267794f, cdf);   // 1 / sqrt(2 pi)
}

// The same derivative with the library erf (fp32 layers).
__device__ __forceinline__ float gelu_grad_erf(float z) {
  return 0.5f * (1.0f + erff(z * 0.70710678118654752440f)) +
         z * expf(-0.5f * z * z) * 0.39894228040143267794f;
}

// Softmax over the N experts of one token row held by a wavefront (lane l
// holds experts l, l + 64, l + 128, l + 192; entries past N are ignored): the
// row max m (fp32), the exponentials ex[v] = exp(l[v] - m) (fp32, widened),
// and their sum (fp64; each lane adds its four in order, then a fixed
// butterfly).  The aux-loss, z-loss and routing kernels all use this one
// routine, so the probabilities and logsumexps they derive from a row are
// the same bits wherever they are computed.
__device__ __forceinline__ double row_softmax_terms(const float (&l)[4], int lane, int N,
                                                    double (&ex)[4], float& m) {
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

template <typename T> struct Elem;
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p, int64_t i) { return p[i]; }
  static __device__ __forceinline__ void store(float* p, int64_t i, float v) { p[i] = v; }
};
template <> struct Elem<uint16_t> {
  static __device__ __forceinline__ float load(const uint16_t* p, int64_t i) { return bf16_to_f32(p[i]); }
  static __device__ __forceinline__ void store(uint16_t* p, int64_t i, float v) { p[i] = f32_to_bf16(v); }
};

// ---------------------------------------------------------------- launchers
// Each returns the hipError_t of its launch(es).

// Router logits (fp64 MFMA split over the model dimension, or the certified
// bf16-MFMA path) + Top-K + softmax over the K chosen.  `ws` holds
// route_ws_bytes(T, d, N, certified) bytes, 256-byte aligned.
int route_splits(int T, int d, int N);
size_t route_ws_bytes(int T, int d, int N, bool certified);
struct RoutePartials;
hipError_t launch_route(int dtype, bool certified, const void* x, const void* w_router,
                        const float* b_router, const float* logit_offset, const float* sel_bias,
                        float* logits, int32_t* topk_idx, float* topk_w, void* ws, int T, int d,
                        int N, int K, const RoutePartials* parts, hipStream_t s);

// Dispatch: histogram, scan, stable rank and row copy.
constexpr int kDispatchTokensPerBlock = 256;
inline int dispatch_blocks(int T) { return (T + kDispatchTokensPerBlock - 1) / kDispatchTokensPerBlock; }
hipError_t launch_dispatch(const int32_t* topk_idx, const void* x, size_t row_bytes, int T, int K,
                           int N, int capacity, int32_t* counts, int32_t* offsets,
                           int32_t* slot_row, int32_t* row_token, void* x_perm,
                           int32_t* n_dropped, int32_t* blkcnt, int32_t* blkoff, hipStream_t s);

// Tile list of a grouped GEMM with BM x BN tiles over Nd output columns: one
// int4 {expert (-1: shared problem), first row, end row, first column} per
// workgroup tile, shared-problem tiles first, then expert by expert; count[0]
// receives the number of tiles.  A block's last remainder of at most `merge`
// rows (when the block has a full tile) is folded into its last full tile,
// which then spans up to BM + merge rows.
// max_tiles bounds the list (it sizes the launch: one workgroup per 2048 tiles).
// wide_rows > 0: an expert block of at most wide_rows rows gets one row of
// tiles 2 BN columns wide, marked by kWideTile in the expert field (never
// more tiles than with BN, so max_tiles still bounds the list).
constexpr int kWideTile = 1 << 16;
hipError_t launch_tile_list(const int32_t* offsets, int N, int BM, int BN, int Nd, int Ts,
                            int merge, int64_t max_tiles, int4* list, int32_t* count,
                            hipStream_t s, int wide_rows = 0);
inline int max_m_tiles(int64_t M_max, int N, int BM) {
  return static_cast<int>((M_max + BM - 1) / BM) + N;
}
inline int64_t max_tiles(int64_t M_max, int N, int Ts, int BM, int BN, int Nd) {
  return ((int64_t)max_m_tiles(M_max, N, BM) + (Ts + BM - 1) / BM) * ((Nd + BN - 1) / BN);
}

// Arguments of one grouped GEMM C = A . W_e^T (+ bias_e) (GELU) over the
// ragged expert row blocks, plus an optional dense "shared" problem.
struct GemmArgs {
  const void* A;        // [rows, Kd] routed activations
  const void* W;        // [E, Nd, Kd] stacked weights
  const void* bias;     // [E, Nd] or null
  void* C;              // [rows, Nd]
  const int32_t* offsets;   // [E+1] (skinny and fp32 kernels)
  const int4* tile_list;    // tiled kernels: tiles in execution order
  const int32_t* tile_count;
  const float* wscale;  // INT8 / INT4 weights: [E, Nd] fp32 row scales (W holds the codes);
                        // null: W is bf16
  bool w4;              // with wscale: INT4 codes, two per byte ([E, Nd, Kd / 2] bytes)
  const void* As;       // shared problem: [Ts, Kd] (null if none)
  const void* Ws;       // [Nd, Kd]
  void* Cs;             // [Ts, Nd]
  int Ts;
  int Kd, Nd;
  int E;
  int64_t grid_tiles;   // upper bound on the tile count (grid size)
  // Weight-gradient (k-segment) mode, tiled and fp32 kernels: when kseg is
  // set, expert e's tiles contract over columns [kseg[e], kseg[e+1]) of
  // A [wg_rows, Kd] and W [Nd, Kd] (both shared by all experts, row stride
  // Kd), writing C rows e * wg_rows + i; kseg entries are multiples of 32.
  const int32_t* kseg;
  int wg_rows;
  // k-major weights (tiled and fp32 kernels): W_e is stored [Kd, Nd], Nd
  // contiguous, instead of [Nd, Kd] (the backward's input gradients).
  bool wkmaj;
  // tiled kernel: eight-wavefront workgroups (launches bound by the weight
  // stream: few rows per expert, or short weight-gradient k-segments)
  bool waves8;
  // tiled kernel: the tile list was built with this wide_rows (routed blocks
  // of at most wide_rows rows have tiles 2 BN wide); 0 = none
  int wide_rows;
  // tiled kernel, weight-gradient mode: tiles of 256 x gemm_bf16_wg_narrow_bn()
  // columns, two workgroups per CU (tile list without folded remainders)
  bool wg_narrow;
  // tiled kernel: load the weights non-temporally (each weight panel is read
  // once, so it need not displace the activations from L2 and the MALL)
  bool w_stream;
};

// Prefill-shaped grouped GEMM (bf16 MFMA): tiles of gemm_bf16_bm() x
// gemm_bf16_bn() rows x columns; an expert block's last remainder of up to
// gemm_bf16_merge_rows() rows is folded into its last full tile.
int gemm_bf16_bm();
int gemm_bf16_bn();
int gemm_bf16_wide_rows();   // the largest block that takes wide tiles
int gemm_bf16_wg_narrow_bn();   // tile width of the narrow weight-gradient tiles
int gemm_bf16_merge_rows();
hipError_t launch_gemm_bf16(const GemmArgs& a, bool gelu, hipStream_t s);
// fp32 grouped GEMM (VALU), BM rows per tile.
int gemm_f32_bm();
int gemm_f32_bn();
hipError_t launch_gemm_f32(const GemmArgs& a, bool gelu, hipStream_t s);
// Decode-shaped grouped GEMM (bf16): streams each touched expert's weights once.
hipError_t launch_gemm_skinny_bf16(const GemmArgs& a, bool gelu, int max_rows_per_expert,
                                   hipStream_t s);
// Decode-shaped GEMM with k-major weights (W_e stored [Kd, Nd]; bf16, no
// bias or activation): the backward's input gradients.
hipError_t launch_gemm_skinny_kmaj_bf16(const GemmArgs& a, hipStream_t s);

// Bytes of per-slot rows (T*K rows of d elements) above which the combine,
// combine-backward and unpermute kernels load them non-temporally: half of
// the 256 MB MALL.  MOE_NONTEMPORAL_ROWS_BYTES (a decimal byte count) in the
// environment replaces it, read on every launch; tests set it to 0 to run the
// non-temporal variants on small layers.
int64_t nontemporal_rows_bytes();

// Combine.
hipError_t launch_combine(int dtype, const void* y_perm, const int32_t* slot_row,
                          const float* topk_w, const void* y_shared, void* out, int T, int d,
                          int K, hipStream_t s);

// Routing partials: per block of kAuxTokensPerBlock tokens, the sums over
// its tokens (in token order) of softmax_N(logits_t) (ppart [nblk, N]), of
// lse_t^2 (zpart [nblk]), and, per expert, the count and the routing-weight
// sum of the (token, slot) pairs routed to it (spcnt, spw [nblk, N], pairs in
// token-major order).  The select kernel writes them when asked, and the aux
// loss, z-loss and statistics kernels write the same bits from the logits /
// routing alone.
struct RoutePartials {
  double* ppart;
  double* zpart;
  double* spw;
  int32_t* spcnt;
};
// Routing partials from the logits (ppart, zpart) and from the routing
// (spcnt, spw); the final reductions of the aux loss (term: N doubles), the
// z-loss and the statistics.
constexpr int kAuxTokensPerBlock = 4;
inline int aux_blocks(int T) { return (T + kAuxTokensPerBlock - 1) / kAuxTokensPerBlock; }
hipError_t launch_logit_partials(const float* logits, int T, int N, const RoutePartials& rp,
                                 hipStream_t s);
hipError_t launch_routing_partials(const int32_t* topk_idx, const float* topk_w, int T, int K,
                                   int N, const RoutePartials& rp, hipStream_t s);
hipError_t launch_aux_final(const RoutePartials& rp, const int32_t* counts, int T, int N,
                            float alpha, double* term, float* loss_out, hipStream_t s);
hipError_t launch_zloss_final(const RoutePartials& rp, int T, float beta, float* loss_out,
                              hipStream_t s);
hipError_t launch_stats_final(const RoutePartials& rp, int T, int N, int32_t* counts, float* wmean,
                              hipStream_t s);
// Per-row symmetric INT8 quantisation (dtype 0 fp32, 1 bf16 input).
hipError_t launch_quantize_int8(const void* w, int dtype, int64_t rows, int cols, int8_t* q,
                                float* scale, hipStream_t s);
// int8 -> bf16 of 8 codes (exact: |q| <= 127), two per 32-bit word.
__device__ __forceinline__ uint4 int8x8_to_bf16x8(uint2 v) {
  uint32_t o[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t wd = j < 2 ? v.x : v.y;
    const int sh = (j & 1) * 16;
    const float f0 = (float)(int32_t)(int8_t)(wd >> sh);
    const float f1 = (float)(int32_t)(int8_t)(wd >> (sh + 8));
    // small integers are exact in fp32 with the low 16 bits zero: the bf16 is
    // the high half; v_perm_b32 packs the two high halves in one instruction
    o[j] = __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}
// int4 -> bf16 of the 8 codes of a 32-bit word (element i in bits 4i .. 4i+3,
// 4-bit two's complement; exact: |q| <= 8), two per output word.
__device__ __forceinline__ uint4 int4x8_to_bf16x8(uint32_t v) {
  uint32_t o[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    // arithmetic shifts sign-extend nibbles 2j and 2j + 1 (v_bfe_i32)
    const float f0 = (float)(static_cast<int32_t>(v << (28 - 8 * j)) >> 28);
    const float f1 = (float)(static_cast<int32_t>(v << (24 - 8 * j)) >> 28);
    o[j] = __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}
// The same 8 codes widened with an offset: bf16(136 + q) = 0x4300 | (n ^ 8)
// for the nibble n of q (exact: 128 + (q + 8) with q + 8 in [0, 15] is the
// mantissa of a bf16 in [128, 256)).  Two logic operations split the word's
// nibbles into bytes, one byte permutation and one OR per output word --
// about 1.5 operations per code against 2.5 for the conversions above; the
// caller removes 136 * sum(activations).
__device__ __forceinline__ uint4 int4x8_to_bf16x8_o136(uint32_t v) {
  const uint32_t u = v ^ 0x88888888u;
  const uint32_t lo = u & 0x0F0F0F0Fu;            // nibbles 0, 2, 4, 6 as bytes
  const uint32_t hi = (u >> 4) & 0x0F0F0F0Fu;     // nibbles 1, 3, 5, 7
  uint32_t o[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)   // bytes: lo[j], 0, hi[j], 0
    o[j] = __builtin_amdgcn_perm(hi, lo, 0x0C000C00u | ((4u + j) << 16) | (uint32_t)j) |
           0x43004300u;
  return make_uint4(o[0], o[1], o[2], o[3]);
}
hipError_t launch_quantize_int4(const void* w, int dtype, int64_t rows, int cols, uint8_t* q,
                                float* scale, hipStream_t s);
// ---------------------------------------------------------------- backward
// h = GELU(z) and d_z = d_h * GELU'(z) over rows [0, *nrows) (or rows_max
// when nrows is null) of [*, width] matrices.
hipError_t launch_gelu_fwd(int dtype, const void* z, void* h, const int32_t* nrows, int rows_max,
                           int width, hipStream_t s);
hipError_t launch_gelu_bwd(int dtype, const void* z, void* dh, const int32_t* nrows, int rows_max,
                           int width, hipStream_t s);
// d_y_perm rows of the kept slots and d_topk_w (0 for dropped slots).
hipError_t launch_combine_bwd(int dtype, const void* d_out, const void* y_perm,
                              const int32_t* slot_row, const float* topk_w, void* d_y_perm,
                              float* d_topk_w, int T, int d, int K, hipStream_t s);
// d_x[t] = sum of the kept d_x_perm rows + d_x_shared[t] + d_x_router[t].
hipError_t launch_unpermute(int dtype, const void* d_x_perm, const int32_t* slot_row,
                            const void* d_x_shared, const float* d_x_router, void* d_x, int T,
                            int d, int K, hipStream_t s);
// Rows of segment e of in [*, C] -> columns [kseg[e], kseg[e+1]) of out
// [C, ldo], zero padded; colsum [nseg, C] (or null) = per-segment column sums.
// max_rows: an upper bound of a single segment's rows (splits its rows over
// workgroups), 0 if unknown.
hipError_t launch_transpose_segments(int dtype, const void* in, const int32_t* off,
                                     const int32_t* kseg, int nseg, int C, int ldo, void* out,
                                     void* colsum, hipStream_t s, int max_rows = 0);
// kseg = scan of the segment lengths rounded up to 32; wa[e] = e * ra,
// wb[e] = e * rb (the output-row offsets of two weight-gradient GEMMs).
hipError_t launch_seg_offsets(const int32_t* off, int N, int ra, int rb, int32_t* kseg,
                              int32_t* wa, int32_t* wb, hipStream_t s);
// One segment of T rows (off = {0, T}).
hipError_t launch_dense_offsets(int T, int ra, int rb, int32_t* off, int32_t* kseg, int32_t* wa,
                                int32_t* wb, hipStream_t s);
// Router backward: d_logits, then d_w_router (part holds
// router_dw_slices(T, N, d) * N * d floats), d_b_router (or null) and
// d_x_router [T, d] fp32 (or null).
int router_dw_slices(int T, int N, int d);
hipError_t launch_route_bwd(int dtype, const void* x, const void* w_router, const float* logits,
                            const int32_t* topk_idx, const float* topk_w, const float* d_topk_w,
                            const int32_t* counts, float aux_coef, float z_coef, float* dl,
                            float* part, float* d_w_router, float* d_b_router, float* d_x_router,
                            int T, int d, int N, int K, hipStream_t s);

}  // namespace moe
