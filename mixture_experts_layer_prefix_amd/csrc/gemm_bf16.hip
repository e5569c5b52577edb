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
//   - workgroup tile BM x BN = 256 x 256, BK = 32; 4 wavefronts in 2 x 2,
//     each owning 128 x 128 outputs as 4 x 4 tiles of
//     v_mfma_f32_32x32x16_bf16 (256 fp32 accumulators per lane, one
//     workgroup per CU), so each LDS byte read feeds 64 MFMA flops;
//   - operands move global -> LDS with 16-byte direct-to-LDS loads (no
//     VGPR staging); one wave instruction fills 16 LDS rows of 64 bytes.
//     The 16-byte chunks of a row are XOR-swizzled (swz below): the lane that
//     fills physical chunk p of row r loads logical chunk p ^ swz(r), so the
//     fragment reads (16 bytes per lane, 32 rows per half-wave) hit every
//     bank exactly once per 16 lanes;
//   - four LDS stages (4 x 32 KiB): the loads of k-step i+3 are issued while
//     the MFMAs of step i run, so each load has three k-steps to land; one
//     barrier per k-step; fragment registers are double-buffered so the LDS
//     reads of the second k-substep overlap the MFMAs of the first;
//   - the MFMA takes the weight fragment as its first operand, so each lane
//     ends up with 4 consecutive output columns of one row and the epilogue
//     writes 8-byte runs;
//   - rows past an expert's end read a clamped valid row and are not stored;
//   - the GELU epilogue uses the Abramowitz-Stegun 7.1.26 erf (gelu_as).
#include "gemm_common.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = 256, BN = 256, BK = 32, NST = 4;
constexpr int NTHR = 256;
constexpr int CH = BK / 8;                 // 16-byte chunks per LDS row (64-byte rows)
constexpr int RPI = 64 / CH;               // LDS rows filled by one wave instruction
constexpr int A_INS = BM / RPI / 4;        // direct loads per lane per stage (A)
constexpr int B_INS = BN / RPI / 4;        // (B)
constexpr int LOADS = A_INS + B_INS;       // vector-memory ops per lane per stage
constexpr int STAGE = (BM + BN) * BK;      // bf16 elements per LDS stage

// Chunk swizzle of LDS row r (rows of 64 bytes, 4 chunks).  A ds_read_b128
// serves 16 lanes per cycle over 64 four-byte banks (256 bytes); the 16 lanes
// of a fragment read hit 16 consecutive rows, i.e. 4 groups of 4 rows that
// each span the 256 bytes once, so the chunk is XORed with the group index.
__device__ __forceinline__ int swz(int r) { return (r >> 2) & 3; }

__device__ __forceinline__ void lds_load16(const uint16_t* g, uint16_t* l) {
  __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(g), reinterpret_cast<void*>(l),
                                   16, 0, 0);
}

// Wait until at most `ahead` stages of this lane's loads are still in flight.
__device__ __forceinline__ void wait_stages(int ahead) {
  if (ahead >= 2)
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * LOADS) : "memory");
  else if (ahead == 1)
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LOADS) : "memory");
  else
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

template <bool GELU>
__global__ __launch_bounds__(NTHR, 1) void gemm_bf16_kernel(GemmArgs a) {
  static_assert(NST == 4, "wait_stages assumes up to 2 younger stages in flight");
  const TileRef tr = map_tile(a);
  if (!tr.valid) return;

  __shared__ __attribute__((aligned(1024))) uint16_t lds[NST * STAGE];

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
  const int lane = tid & 63, wave = tid >> 6;

  // Direct-load sources: lane -> (row r_in of a RPI-row group, physical chunk
  // pc), loading logical chunk pc ^ swz(row) of that row.
  const int r_in = lane / CH;
  uint32_t a_off[A_INS], b_off[B_INS];
#pragma unroll
  for (int j = 0; j < A_INS; ++j) {
    const int row = (j * 4 + wave) * RPI + r_in;
    const int lchunk = (lane % CH) ^ swz(row);
    a_off[j] = (uint32_t)(tr.row0 + min(row, rows - 1)) * (uint32_t)Kd + lchunk * 8;
  }
#pragma unroll
  for (int j = 0; j < B_INS; ++j) {
    const int row = (j * 4 + wave) * RPI + r_in;
    const int lchunk = (lane % CH) ^ swz(row);
    const int n = min(tr.n0 + row, Nd - 1);
    b_off[j] = (uint32_t)n * (uint32_t)Kd + lchunk * 8;
  }

  auto issue = [&](int stage, int k0) {
    uint16_t* base = lds + stage * STAGE;
#pragma unroll
    for (int j = 0; j < A_INS; ++j)
      lds_load16(A + a_off[j] + k0, base + (j * 4 + wave) * RPI * BK);
#pragma unroll
    for (int j = 0; j < B_INS; ++j)
      lds_load16(W + b_off[j] + k0, base + BM * BK + (j * 4 + wave) * RPI * BK);
  };

  const int wm = wave >> 1, wn = wave & 1;
  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int KT = Kd / BK;
  const int sw = swz(lane & 31);   // the same for every fragment row this lane reads
  bf16x8 fa[2][4], fb[2][4];
  auto read_frags = [&](const uint16_t* As, int kk, int buf) {
    const int pc = ((kk * 2 + (lane >> 5)) ^ sw) * 8;
    const uint16_t* Bs = As + BM * BK;
#pragma unroll
    for (int mi = 0; mi < 4; ++mi)
      fa[buf][mi] = *reinterpret_cast<const bf16x8*>(As + (wm * 128 + mi * 32 + (lane & 31)) * BK + pc);
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
      fb[buf][ni] = *reinterpret_cast<const bf16x8*>(Bs + (wn * 128 + ni * 32 + (lane & 31)) * BK + pc);
  };
  auto mfmas = [&](int buf) {
#pragma unroll
    for (int ni = 0; ni < 4; ++ni)
#pragma unroll
      for (int mi = 0; mi < 4; ++mi)
        acc[ni][mi] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[buf][ni], fa[buf][mi], acc[ni][mi], 0, 0, 0);
  };

  // Prologue: the first NST-1 stages in flight.
#pragma unroll
  for (int st = 0; st < NST - 1; ++st)
    if (st < KT) issue(st, st * BK);

  for (int kt = 0; kt < KT; ++kt) {
    // Stage kt has landed for every lane once each waited for its own loads
    // and all passed the barrier.  The barrier also ends every wavefront's
    // use of the stage consumed in iteration kt-1 (its fragments all fed
    // MFMAs before the barrier), which is refilled next.  A bare s_barrier:
    // __syncthreads() would add a fence that drains every load in flight.
    wait_stages(min(NST - 2, KT - 1 - kt));
    __builtin_amdgcn_s_barrier();
    const uint16_t* As = lds + (kt % NST) * STAGE;
    read_frags(As, 0, 0);
    if (kt + NST - 1 < KT) issue((kt + NST - 1) % NST, (kt + NST - 1) * BK);
    read_frags(As, 1, 1);
    mfmas(0);
    mfmas(1);
    // interleave the fragment reads of k-substep 1 and the next stage's loads
    // with the MFMAs of k-substep 0
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 24, 0);
  }

  // Epilogue.  The 32x32 accumulator of (ni, mi) holds C^T: element v of lane l
  // is output row mi*32 + l%32, column ni*32 + (v/4)*8 + (l/32)*4 + v%4.
#pragma unroll
  for (int mi = 0; mi < 4; ++mi) {
    const int ml = wm * 128 + mi * 32 + (lane & 31);
    if (ml >= rows) continue;
    uint16_t* crow = C + (int64_t)(tr.row0 + ml) * Nd;
#pragma unroll
    for (int ni = 0; ni < 4; ++ni) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = tr.n0 + wn * 128 + ni * 32 + g * 8 + (lane >> 5) * 4;
        if (n >= Nd) continue;
        float z[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          z[q] = acc[ni][mi][g * 4 + q];
          if (bias) z[q] += bf16_to_f32(bias[n + q]);
          if (GELU) z[q] = gelu_as(z[q]);
        }
        uint2 pk;
        pk.x = (uint32_t)f32_to_bf16(z[0]) | ((uint32_t)f32_to_bf16(z[1]) << 16);
        pk.y = (uint32_t)f32_to_bf16(z[2]) | ((uint32_t)f32_to_bf16(z[3]) << 16);
        *reinterpret_cast<uint2*>(crow + n) = pk;
      }
    }
  }
}

}  // namespace

int gemm_bf16_bm() { return BM; }
int gemm_bf16_bn() { return BN; }

hipError_t launch_gemm_bf16(const GemmArgs& a, bool gelu, hipStream_t s) {
  const int grid = gemm_grid(a);
  if (grid == 0) return hipSuccess;
  if (gelu)
    hipLaunchKernelGGL(gemm_bf16_kernel<true>, dim3(grid), dim3(NTHR), 0, s, a);
  else
    hipLaunchKernelGGL(gemm_bf16_kernel<false>, dim3(grid), dim3(NTHR), 0, s, a);
  return hipGetLastError();
}

}  // namespace moe
