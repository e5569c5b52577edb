// fp32 grouped GEMM on the vector ALUs (the fp32 layer precision).
//
// Same contraction and epilogues as the bf16 kernel (Linear -> GELU -> Linear
// per expert, yunthe.com "MoE混合专家模型实战" reference forward), in fp32
// throughout.  64 x 64 workgroup tiles, BK = 16 staged in LDS k-major, each
// of the 256 threads owning a 4 x 4 block of outputs.  Used for fp32 layers,
// which are small; the products accumulate in k order with fma.  With
// GemmArgs::kseg set it runs the weight-gradient (k-segment) form; with
// GemmArgs::wkmaj it reads k-major weights.
#include "gemm_common.h"

namespace moe {
namespace {

constexpr int BM = 64, BN = 64, BK = 16, NTHR = 256;

template <bool GELU>
__global__ __launch_bounds__(NTHR) void gemm_f32_kernel(GemmArgs a) {
  const TileRef tr = map_tile(a);
  if (!tr.valid) return;
  __shared__ float As[BK][BM + 4];
  __shared__ float Bs[BK][BN + 4];

  const int Kd = a.Kd, Nd = a.Nd;
  const float* A;
  const float* W;
  const float* bias = nullptr;
  float* C;
  int arow0 = tr.row0, kbeg = 0, kend = Kd;
  if (a.kseg) {   // weight-gradient (k-segment) mode
    A = static_cast<const float*>(a.A);
    W = static_cast<const float*>(a.W);
    C = static_cast<float*>(a.C);
    kbeg = a.kseg[tr.e];
    kend = a.kseg[tr.e + 1];
    arow0 = tr.row0 - tr.e * a.wg_rows;
  } else if (tr.shared) {
    A = static_cast<const float*>(a.As);
    W = static_cast<const float*>(a.Ws);
    C = static_cast<float*>(a.Cs);
  } else {
    A = static_cast<const float*>(a.A);
    W = static_cast<const float*>(a.W) + (int64_t)tr.e * Nd * Kd;
    if (a.bias) bias = static_cast<const float*>(a.bias) + (int64_t)tr.e * Nd;
    C = static_cast<float*>(a.C);
  }
  const int rows = tr.row_end - tr.row0;
  const int tid = threadIdx.x;
  const int tx = tid % 16, ty = tid / 16;

  float acc[4][4] = {};
  for (int k0 = kbeg; k0 < kend; k0 += BK) {
    for (int i = tid; i < BM * BK; i += NTHR) {
      const int r = i / BK, k = i % BK;
      As[k][r] = (r < rows) ? A[(int64_t)(arow0 + r) * Kd + k0 + k] : 0.f;
      const int n = tr.n0 + r;
      Bs[k][r] = (n >= Nd) ? 0.f
                 : a.wkmaj ? W[(int64_t)(k0 + k) * Nd + n] : W[(int64_t)n * Kd + k0 + k];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < BK; ++k) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = As[k][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) bv[j] = Bs[k][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = ty * 4 + i;
    if (r >= rows) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = tr.n0 + tx * 4 + j;
      if (n >= Nd) continue;
      float z = acc[i][j] + (bias ? bias[n] : 0.f);
      if (GELU) z = gelu_erf(z);
      C[(int64_t)(tr.row0 + r) * Nd + n] = z;
    }
  }
}

}  // namespace

int gemm_f32_bm() { return BM; }
int gemm_f32_bn() { return BN; }

hipError_t launch_gemm_f32(const GemmArgs& a, bool gelu, hipStream_t s) {
  const int grid = gemm_grid(a);
  if (grid == 0) return hipSuccess;
  if (gelu)
    hipLaunchKernelGGL(gemm_f32_kernel<true>, dim3(grid), dim3(NTHR), 0, s, a);
  else
    hipLaunchKernelGGL(gemm_f32_kernel<false>, dim3(grid), dim3(NTHR), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
