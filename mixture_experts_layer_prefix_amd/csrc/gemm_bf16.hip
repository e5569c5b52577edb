// Prefill-shaped grouped GEMM on the bf16 matrix cores of gfx950.
//
// What it computes (yunthe.com "MoE混合专家模型实战", reference forward and
// the note after it: each expert is Linear -> GELU -> Linear, and production
// code batches the tokens of one expert into a grouped GEMM):
//   C[r, n] = epi( sum_k A[r, k] * W_e[n, k] + bias_e[n] ) for every row r of
//   expert e's block, epi = GELU for the first Linear, identity for the
//   second.  bf16 operands, fp32 accumulation, bf16 result.
//
// Design for CDNA4:
//   - workgroup tile BM x BN = 256 x 256, BK = 32, 8 wavefronts = two groups
//     of four; the hardware places wavefront w on SIMD w mod 4, so every SIMD
//     holds one wavefront of each group.  Group g owns output rows
//     [g*BM/2, (g+1)*BM/2); wavefront j of a group owns columns [64j, 64j+64)
//     as (BM/64) x 2 tiles of v_mfma_f32_32x32x16_bf16;
//   - ping-pong: in each k-step, while one group issues its 16 MFMAs from
//     fragments already in registers (at raised wave priority), the other
//     group reads its fragments for the next MFMA burst from LDS and issues
//     its share of the global loads; one barrier per k-step swaps the roles,
//     so each SIMD's MFMA pipe runs the two groups' bursts back to back while
//     memory work hides in their shadow;
//   - operands move global -> LDS with 16-byte direct-to-LDS loads (no VGPR
//     staging); a wave instruction fills 16 LDS rows of 64 bytes; group 0
//     loads the A half of a stage, group 1 the W half.  The 16-byte chunks of
//     a row are XOR-swizzled (swz below) so fragment reads hit every bank
//     once per 16 lanes;
//   - four LDS stages (4 x 32 KiB); loads run two to three k-steps ahead;
//     after the last k-step every lane drains its loads before the epilogue;
//   - the MFMA takes the weight fragment as its first operand, so each lane
//     ends up with 4 consecutive output columns of one row and the epilogue
//     writes 8-byte runs; the GELU epilogue uses the Abramowitz-Stegun 7.1.26
//     erf (gelu_as);
//   - rows past an expert's end read a clamped valid row and are not stored.
#include "gemm_common.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BN = 256, BK = 32;
constexpr int NTHR = 512;
constexpr int CH = BK / 8;                 // 16-byte chunks per LDS row (64-byte rows)
constexpr int RPI = 64 / CH;               // LDS rows filled by one wave instruction (16)
constexpr int LB = BN / RPI / 4;           // direct loads per group-1 wavefront per stage (W half)

// Chunk swizzle of LDS row r (rows of 64 bytes, 4 chunks).  A ds_read_b128
// serves 16 lanes per cycle over 64 four-byte banks (256 bytes); the 16 lanes
// of a fragment read hit 16 consecutive rows, i.e. 4 groups of 4 rows that
// each span the 256 bytes once, so the chunk is XORed with the group index.
__device__ __forceinline__ int swz(int r) { return (r >> 2) & 3; }

__device__ __forceinline__ void lds_load16(const uint16_t* g, uint16_t* l) {
  __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(g), reinterpret_cast<void*>(l),
                                   16, 0, 0);
}

// s_barrier with a compiler memory fence: no LDS access moves across it.
__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

// BM = 256 or 128 rows per tile; each group owns BM/2 rows (MI tiles of 32).
template <int BM, bool GELU>
__global__ __launch_bounds__(NTHR, 1) void gemm_bf16_kernel(GemmArgs a) {
  constexpr int MI = BM / 64;                 // 32-row MFMA tiles per wavefront
  constexpr int LA = BM / RPI / 4;            // direct loads per group-0 wavefront (A half)
  constexpr int STAGE = (BM + BN) * BK;       // bf16 elements per LDS stage
  // LDS stages: 4 x 32 KiB for 256-row tiles; 6 x 24 KiB for 128-row tiles,
  // which stream weights from HBM and need more bytes in flight.
  constexpr int NST = BM == 256 ? 4 : 6;
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
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int grp = wave >> 2, wj = wave & 3;

  // Direct loads of this wavefront: group 0 fills the A half of a stage (LA
  // instructions), group 1 the W half (LB); instruction i covers LDS rows
  // (wj*L + i)*RPI .. +RPI of its half.  Lane -> (row r_in, physical chunk),
  // loading logical chunk pc ^ swz(row).
  const int r_in = lane / CH;
  const uint16_t* src = grp == 0 ? A : W;
  constexpr int LMAX = LA > LB ? LA : LB;
  const int nload = grp == 0 ? LA : LB;
  uint32_t off[LMAX];
#pragma unroll
  for (int i = 0; i < LMAX; ++i) {
    const int row = (wj * nload + i) * RPI + r_in;
    const int lchunk = (lane % CH) ^ swz(row);
    const int g_row = grp == 0 ? tr.row0 + min(row, rows - 1) : min(tr.n0 + row, Nd - 1);
    off[i] = (uint32_t)g_row * (uint32_t)Kd + lchunk * 8;
  }
  const int half = grp == 0 ? 0 : BM * BK;
  auto issue = [&](int stage, int k0) {
    uint16_t* base = lds + stage * STAGE + half;
#pragma unroll
    for (int i = 0; i < LMAX; ++i)
      if (i < nload) lds_load16(src + off[i] + k0, base + (wj * nload + i) * RPI * BK);
  };

  f32x16 acc[2][MI];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < MI; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int sw = swz(lane & 31);   // the same for every fragment row this lane reads
  bf16x8 fa[MI][2], fb[2][2];
  auto read_frags = [&](int stage) {
    const uint16_t* As = lds + stage * STAGE;
    const uint16_t* Bs = As + BM * BK;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int pc = ((kk * 2 + (lane >> 5)) ^ sw) * 8;
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
        fa[mi][kk] = *reinterpret_cast<const bf16x8*>(
            As + (grp * (BM / 2) + mi * 32 + (lane & 31)) * BK + pc);
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
        fb[ni][kk] = *reinterpret_cast<const bf16x8*>(
            Bs + (wj * 64 + ni * 32 + (lane & 31)) * BK + pc);
    }
  };
  auto mfmas = [&]() {
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
          acc[ni][mi] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[ni][kk], fa[mi][kk],
                                                                acc[ni][mi], 0, 0, 0);
    __builtin_amdgcn_s_setprio(0);
  };

  const int KT = Kd / BK;
  // Prologue: stages 0 .. NST-2 in flight (chunks past the end re-read the
  // last chunk into stages nobody reads, so every k-step issues the same
  // number of loads and the wait counts below are constants).
#pragma unroll
  for (int st = 0; st < NST - 1; ++st) issue(st, min(st, KT - 1) * BK);
  if (grp == 0)
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LA * (NST - 2)) : "memory");
  else
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LB * (NST - 2)) : "memory");
  barrier();
  if (grp == 0) read_frags(0);

  for (int kt = 0; kt < KT; ++kt) {
    const int nxt = min(kt + NST - 1, KT - 1) * BK;
    // Phase A: group 0 runs its MFMAs on stage kt; group 1 reads its stage-kt
    // fragments and loads its half of stage kt+NST-1 into the buffer freed
    // by the previous k-step's last barrier.
    if (grp == 0) {
      mfmas();
    } else {
      read_frags(kt % NST);
      issue((kt + NST - 1) % NST, nxt);
    }
    // Each lane's own loads of stage kt+1 have landed (group 1 has NST-2
    // younger stages in flight, group 0 NST-3), and group 1's reads of stage
    // kt are complete; after the barrier every half of stage kt+1 is in LDS
    // and nobody reads stage kt any more.
    if (grp == 0)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LA * (NST - 3)) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(LB * (NST - 2)) : "memory");
    barrier();
    // Phase B: group 1 runs its MFMAs on stage kt; group 0 reads its stage
    // kt+1 fragments and loads its half of stage kt+NST-1.  No second
    // barrier: group 0's stage-kt+1 reads feed its next MFMA burst, which
    // precedes the next barrier, so they are complete before that buffer is
    // refilled two k-steps later.
    if (grp == 1) {
      mfmas();
    } else {
      if (kt + 1 < KT) read_frags((kt + 1) % NST);
      issue((kt + NST - 1) % NST, nxt);
    }
  }
  // no direct-to-LDS load may still be in flight when the workgroup ends
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // Epilogue.  The 32x32 accumulator of (ni, mi) holds C^T: element v of lane l
  // is output row mi*32 + l%32, column ni*32 + (v/4)*8 + (l/32)*4 + v%4.
#pragma unroll
  for (int mi = 0; mi < MI; ++mi) {
    const int ml = grp * (BM / 2) + mi * 32 + (lane & 31);
    if (ml >= rows) continue;
    uint16_t* crow = C + (int64_t)(tr.row0 + ml) * Nd;
#pragma unroll
    for (int ni = 0; ni < 2; ++ni) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = tr.n0 + wj * 64 + ni * 32 + g * 8 + (lane >> 5) * 4;
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

int gemm_bf16_bn() { return BN; }

hipError_t launch_gemm_bf16(const GemmArgs& a, int bm, bool gelu, hipStream_t s) {
  const int grid = gemm_grid(a);
  if (grid == 0) return hipSuccess;
  if (bm == 128) {
    if (gelu)
      hipLaunchKernelGGL((gemm_bf16_kernel<128, true>), dim3(grid), dim3(NTHR), 0, s, a);
    else
      hipLaunchKernelGGL((gemm_bf16_kernel<128, false>), dim3(grid), dim3(NTHR), 0, s, a);
  } else {
    if (gelu)
      hipLaunchKernelGGL((gemm_bf16_kernel<256, true>), dim3(grid), dim3(NTHR), 0, s, a);
    else
      hipLaunchKernelGGL((gemm_bf16_kernel<256, false>), dim3(grid), dim3(NTHR), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace moe
