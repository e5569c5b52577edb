// Prefill-shaped grouped GEMM on the bf16 matrix cores of gfx950.
//
// What it computes (yunthe.com "MoE混合专家模型实战", reference forward and
// the note after it: each expert is Linear -> GELU -> Linear, and production
// code batches the tokens of one expert into a grouped GEMM):
//   C[r, n] = epi( sum_k A[r, k] * W_e[n, k] + bias_e[n] ) for every row r of
//   expert e's block, epi = exact GELU for the first Linear, identity for the
//   second.  bf16 operands, fp32 accumulation, bf16 result.
//
// Design for CDNA4:
//   - workgroup tile BM x BN = 128 x 128, BK = 64; 4 wavefronts in 2 x 2,
//     each owning a 64 x 64 sub-tile as 2 x 2 v_mfma_f32_32x32x16_bf16 tiles;
//   - A and W are both K-contiguous, so every operand fragment is one 16-byte
//     LDS read per lane; LDS rows are 128 bytes, their 16-byte chunks XOR-
//     swizzled by (row mod 8) so a fragment read touches every bank once;
//   - global -> LDS through registers, double-buffered: the loads of k-step
//     i+1 are in flight while the MFMAs of step i run; one barrier per step;
//   - rows past an expert's end read a clamped valid row and are not stored,
//     so a tile never touches memory outside its operands.
#include "gemm_common.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int NTHR = 256;
constexpr int CHUNKS = BK / 8;               // 16-byte chunks per LDS row
constexpr int A_LOADS = BM * CHUNKS / NTHR;  // 16-byte global loads per thread
constexpr int B_LOADS = BN * CHUNKS / NTHR;

__device__ __forceinline__ int swz(int row, int chunk) { return chunk ^ (row & 7); }

template <bool GELU>
__global__ __launch_bounds__(NTHR, 2) void gemm_bf16_kernel(GemmArgs a) {
  const TileRef tr = map_tile<BM, BN>(a);
  if (!tr.valid) return;

  __shared__ uint4 As[2][BM][CHUNKS];
  __shared__ uint4 Bs[2][BN][CHUNKS];

  const int Kd = a.Kd, Nd = a.Nd;
  const uint16_t* A;
  const uint16_t* W;
  const uint16_t* bias = nullptr;
  uint16_t* C;
  if (tr.shared) {
    A = static_cast<const uint16_t*>(a.As);
    W = static_cast<const uint16_t*>(a.Ws);
    C = static_cast<uint16_t*>(a.Cs);
  } else {
    A = static_cast<const uint16_t*>(a.A);
    W = static_cast<const uint16_t*>(a.W) + (int64_t)tr.e * Nd * Kd;
    if (a.bias) bias = static_cast<const uint16_t*>(a.bias) + (int64_t)tr.e * Nd;
    C = static_cast<uint16_t*>(a.C);
  }
  const int rows = tr.row_end - tr.row0;

  const int tid = threadIdx.x;
  // per-thread global sources (row clamped into the valid range)
  const uint4* a_src[A_LOADS];
  const uint4* b_src[B_LOADS];
  int a_row[A_LOADS], a_chk[A_LOADS], b_row[B_LOADS], b_chk[B_LOADS];
#pragma unroll
  for (int j = 0; j < A_LOADS; ++j) {
    const int q = tid + j * NTHR;
    a_row[j] = q / CHUNKS;
    a_chk[j] = q % CHUNKS;
    const int r = tr.row0 + min(a_row[j], rows - 1);
    a_src[j] = reinterpret_cast<const uint4*>(A + (int64_t)r * Kd) + a_chk[j];
  }
#pragma unroll
  for (int j = 0; j < B_LOADS; ++j) {
    const int q = tid + j * NTHR;
    b_row[j] = q / CHUNKS;
    b_chk[j] = q % CHUNKS;
    const int n = min(tr.n0 + b_row[j], Nd - 1);
    b_src[j] = reinterpret_cast<const uint4*>(W + (int64_t)n * Kd) + b_chk[j];
  }

  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  uint4 ra[A_LOADS], rb[B_LOADS];
  const int KT = Kd / BK;
  // prologue: k-step 0 into buffer 0
#pragma unroll
  for (int j = 0; j < A_LOADS; ++j) ra[j] = a_src[j][0];
#pragma unroll
  for (int j = 0; j < B_LOADS; ++j) rb[j] = b_src[j][0];
#pragma unroll
  for (int j = 0; j < A_LOADS; ++j) As[0][a_row[j]][swz(a_row[j], a_chk[j])] = ra[j];
#pragma unroll
  for (int j = 0; j < B_LOADS; ++j) Bs[0][b_row[j]][swz(b_row[j], b_chk[j])] = rb[j];
  __syncthreads();

  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) {
      const int koff = (kt + 1) * CHUNKS;
#pragma unroll
      for (int j = 0; j < A_LOADS; ++j) ra[j] = a_src[j][koff];
#pragma unroll
      for (int j = 0; j < B_LOADS; ++j) rb[j] = b_src[j][koff];
    }
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const int chunk = kk * 2 + (lane >> 5);
      bf16x8 fa[2], fb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = wm * 64 + i * 32 + (lane & 31);
        fa[i] = __builtin_bit_cast(bf16x8, As[buf][r][swz(r, chunk)]);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int r = wn * 64 + j * 32 + (lane & 31);
        fb[j] = __builtin_bit_cast(bf16x8, Bs[buf][r][swz(r, chunk)]);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < KT) {
      const int nb = buf ^ 1;
#pragma unroll
      for (int j = 0; j < A_LOADS; ++j) As[nb][a_row[j]][swz(a_row[j], a_chk[j])] = ra[j];
#pragma unroll
      for (int j = 0; j < B_LOADS; ++j) Bs[nb][b_row[j]][swz(b_row[j], b_chk[j])] = rb[j];
    }
    __syncthreads();
  }

  // epilogue: 32x32 accumulator layout -- element v of lane l holds
  // row (v/4)*8 + (l/32)*4 + v%4, column l%32.
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int col = tr.n0 + wn * 64 + j * 32 + (lane & 31);
    if (col >= Nd) continue;
    const float bv = bias ? bf16_to_f32(bias[col]) : 0.f;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int rl = wm * 64 + i * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
        if (rl < rows) {
          float z = acc[i][j][v] + bv;
          if (GELU) z = gelu_erf(z);
          C[(int64_t)(tr.row0 + rl) * Nd + col] = f32_to_bf16(z);
        }
      }
    }
  }
}

}  // namespace

int gemm_bf16_bm() { return BM; }

hipError_t launch_gemm_bf16(const GemmArgs& a, bool gelu, hipStream_t s) {
  const int grid = gemm_grid(a, BM, BN);
  if (grid == 0) return hipSuccess;
  if (gelu)
    hipLaunchKernelGGL(gemm_bf16_kernel<true>, dim3(grid), dim3(NTHR), 0, s, a);
  else
    hipLaunchKernelGGL(gemm_bf16_kernel<false>, dim3(grid), dim3(NTHR), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
