// Prefill-shaped grouped GEMM on the bf16 matrix cores of gfx950.
//
// What it computes (yunthe.com "MoE混合专家模型实战", reference forward and
// the note after it: each expert is Linear -> GELU -> Linear, and production
// code batches the tokens of one expert into a grouped GEMM):
//   C[r, n] = epi( sum_k A[r, k] * W_e[n, k] + bias_e[n] ) for every row r of
//   expert e's block, epi = GELU for the first Linear, identity for the
//   second.  bf16 operands, fp32 accumulation, bf16 result.
//
// Design for CDNA4 (details at the kernel):
//   - tiles of 256 rows x 256 columns, four wavefronts (one per SIMD); the
//     wave arrangement is picked per tile from its row count, and a short
//     remainder of an expert's rows rides in its last full tile;
//   - operands move global -> LDS with 16-byte direct-to-LDS loads (no VGPR
//     staging), 32-wide k-steps.  Forward tiles load k-pairs: one wave
//     instruction fills 8 LDS rows of 128 bytes (two k-steps of an
//     activation or bf16 weight row) or 16 rows of 64 bytes (two k-steps of
//     INT8 codes, four of INT4 codes) into two pair buffers; weight-gradient
//     and k-major tiles fill 16 rows of 64 bytes per instruction into four
//     stages.  The 16-byte chunks of each LDS row are XOR-swizzled (swz,
//     swz8) so fragment reads hit every bank once per 16 lanes;
//   - the MFMA takes the weight fragment as its first operand, so each lane
//     ends up with 4 consecutive output columns of one row; the output tile
//     is staged through LDS and written as whole rows;
//   - rows past an expert's end read a clamped valid row and are not stored;
//     the GELU epilogue uses the Abramowitz-Stegun 7.1.26 erf (gelu_as);
//   - variants: INT8 and INT4 weights (codes widened in registers), weight gradients
//     over per-expert k-segments (and a two-workgroups-per-CU kernel of 256 x
//     128 tiles for short segments), k-major weights for input gradients.
// MOE_KPAIRS=0 builds the four-stage loop for the forward tiles too.
#include <type_traits>

#include "gemm_common.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int BN = 256, BK = 32;
constexpr int W4_NS = 4;                   // LDS stages
constexpr int CH = BK / 8;                 // 16-byte chunks per LDS row (64-byte rows)
constexpr int RPI = 64 / CH;               // LDS rows filled by one wave instruction (16)

// Chunk swizzle of LDS row r (rows of 64 bytes, 4 chunks).  A ds_read_b128
// serves 16 lanes per cycle over 64 four-byte banks (256 bytes); the 16 lanes
// of a fragment read hit 16 consecutive rows, i.e. 4 groups of 4 rows that
// each span the 256 bytes once, so the chunk is XORed with the group index.
__device__ __forceinline__ int swz(int r) { return (r >> 2) & 3; }

// k-pairs (bf16 forward tiles): LDS rows of 128 bytes hold two 32-wide
// k-steps (8 chunks of 16 bytes); chunk c of row r sits at c ^ swz8(r).  A
// ds_read_b128 serves 16 lanes = 16 consecutive rows: rows of equal parity
// share a 32-bank half, and the XOR spreads each half's 8 rows over its 8
// chunks, so the 16 reads cover the 64 banks once.
__device__ __forceinline__ int swz8(int r) { return (r >> 1) & 7; }
#ifndef MOE_KPAIRS
#define MOE_KPAIRS 1
#endif

// AUX = 2: non-temporal (nt), for bf16 weights streamed once
// (GemmArgs::w_stream; the kernels' NTW instantiations)
template <int AUX = 0>
__device__ __forceinline__ void lds_load16(const void* g, void* l) {
  __builtin_amdgcn_global_load_lds(g, l, 16, 0, AUX);
}

// INT8 weights: the weight region of an even stage (16 KiB, sized for bf16)
// takes the codes of two k-steps, 256 rows of 64 bytes laid out and swizzled
// like the bf16 rows, and the odd stage after it reads the second half of
// every row.  The direct loads thus move 64 contiguous bytes per row, which
// streams ~20% faster than 32-byte rows.  A lane reads one 16-byte chunk (16
// codes) per k-step with a ds_read_b128 and feeds its first 8 codes to the
// first half's MFMAs and the other 8 to the second half's; the A fragments
// follow the same order of k (see read_half).

// k-major weights (KM): a stage holds 32 k-rows of 256 bf16 (512 bytes, 32
// chunks of 16 bytes); chunk c of k-row r sits at chunk c ^ (4 (r mod 4)).  A
// fragment is two ds_read_b64_tr_b16: in each group of 16 lanes, result lane
// m receives element m mod 4 of the 8 bytes addressed by source lanes m/4,
// m/4 + 4, m/4 + 8, m/4 + 12 -- i.e. 4 consecutive k of one n column when
// source lane 4q + u points at k-row q, columns 4u .. 4u + 3.  The 16 lanes
// of a half-group read 4 k-rows x 8 chunks that the swizzle spreads over all
// 64 banks.
__device__ __forceinline__ int kswz(int r) { return 4 * (r & 3); }

typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4_lds;

__device__ __forceinline__ bf16x4 lds_read_tr(const char* p) {
  return __builtin_bit_cast(
      bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                  (__attribute__((address_space(3))) bf16x4_lds*)(p)));
}

// s_barrier with a compiler memory fence: no LDS access moves across it.
__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }

// 256-row tiles: four wavefronts, one per SIMD.  The wave arrangement is
// chosen per tile from its valid row count R:
//   256 < R <= 320: 2 x 2 wavefronts of 128 x 128 plus, per wavefront, 32
//                   more rows x 128 columns held in ordinary VGPRs: the tile
//                   list folds a remainder of up to 64 rows into an expert's
//                   last full tile, which streams the weight rows anyway,
//   192 < R <= 256: 2 x 2 wavefronts of 128 x 128 (4 x 4 MFMA tiles of 32 x 32),
//   128 < R <= 192: 2 x 2 wavefronts of  96 x 128,
//   96 < R <= 128:  1 x 4 wavefronts of 128 x 64,
//   64 < R <= 96:   1 x 4 wavefronts of  96 x 64 (128 A rows loaded),
//   R <= 64:        1 x 4 wavefronts of  64 x 64;
// A rows past the arrangement's height are neither loaded nor multiplied, so
// a tile multiplies fewer than 32 rows past its end (fewer than 64 below 64).
// The loads of this kernel run at the L2's pace (an expert's weight panel
// is streamed once per m-tile), so a separate tile for a short remainder
// would cost nearly as much as a full one.
// The 2 x 2 arrangement keeps 256 fp32 accumulators per lane in the
// accumulation registers and reads 512 bytes of fragments from LDS per MFMA
// (a 128 x 64 wavefront tile needs 768); one wavefront draws at most about
// 32 bytes per clock from LDS on this chip.
//
// Each k-step has two halves (k 0-15 and 16-31 of the step).  While one
// half's MFMAs run on one register set of fragments, the other set is filled
// from LDS for the next half, and the wavefront issues its share of the
// direct-to-LDS loads of the stage NS-1 steps ahead (A rows in the first
// half, W rows in the second).  One barrier per k-step, between the halves:
// before it every lane has its own loads of the next stage landed and its
// reads of the current stage done, so after it the next stage is whole and
// the current one may be refilled.
//
// Eight-wavefront workgroups (layouts 4, 5, 7; two wavefronts per SIMD, 128
// accumulators each) serve the backward's routed GEMMs when experts have few
// rows: one workgroup of four wavefronts per CU streams direct-to-LDS loads
// at about 4.9 TB/s over the chip whatever the pipeline depth, eight
// wavefronts at about 5.7 TB/s (a plain streaming probe), and a second
// wavefront per SIMD overlaps the many short tiles of the weight gradients.
//   256 < R <= 320: 2 x 4 wavefronts of 128 x 64 plus 32 folded rows each,
//   128 < R <= 256: 2 x 4 wavefronts of 128 x 64,
//   R <= 128:       2 x 4 wavefronts of  64 x 64.
constexpr int cmax(int a, int b) { return a > b ? a : b; }
constexpr int W4_TM = 256;
constexpr int W4_MERGE = 64;                  // remainder rows folded into the previous tile
constexpr int W4_AR = W4_TM + W4_MERGE;       // A rows held per LDS stage
constexpr int W4_STAGE = (W4_AR + BN) * BK;   // bf16 elements per LDS stage (36 KiB)
constexpr int W4_CST = BN + 8;                // staged output row stride in bf16 (528 bytes)
constexpr int W8_AR = 384;                    // eight wavefronts, folded tiles: 3 loads per wave
constexpr int W8_STAGE = (W8_AR + BN) * BK;   // 40 KiB: four stages fill the 160 KiB of LDS

// Wide tiles (tile lists built with wide_rows = 128): an expert block of at
// most 128 rows takes 512 columns per tile, 1 x 4 wavefronts of 128 x 128.
// Per k-step the tile loads 8 KiB of A rows and 32 KiB of weight rows for
// twice the MFMAs of a 128 x 256 tile (which loads 8 + 16 KiB), and each
// wavefront reads 16 KiB of fragments from LDS per 32 MFMAs instead of 12
// KiB per 16: the short tiles of the fine-grained shapes are bound by these
// two rates.
constexpr int WIDE_BN = 2 * BN, WIDE_AR = 128;
constexpr int WIDE_STAGE = (WIDE_AR + WIDE_BN) * BK;   // 40 KiB
constexpr int WIDE_CST = WIDE_BN + 8;

// Per layout: BNL columns per tile, CST = staged output row stride (bf16).
struct W4Cols {
  static constexpr int BNL = BN, CST = W4_CST;
};
template <int L>
struct W4Layout;
template <>
struct W4Layout<0> : W4Cols {   // 128 < R <= 256
  static constexpr int NW = 4, WN = 2, MI = 4, NI = 4, AROWS = 256, AR = W4_AR;
  static constexpr bool EXTRA = false;
};
template <>
struct W4Layout<1> : W4Cols {   // 64 < R <= 128
  static constexpr int NW = 4, WN = 4, MI = 4, NI = 2, AROWS = 128, AR = W4_AR;
  static constexpr bool EXTRA = false;
};
template <>
struct W4Layout<2> : W4Cols {   // R <= 64
  static constexpr int NW = 4, WN = 4, MI = 2, NI = 2, AROWS = 64, AR = W4_AR;
  static constexpr bool EXTRA = false;
};
template <>
struct W4Layout<3> : W4Cols {   // 256 < R <= 320
  static constexpr int NW = 4, WN = 2, MI = 4, NI = 4, AROWS = 320, AR = W4_AR;
  static constexpr bool EXTRA = true;
};
template <>
struct W4Layout<14> : W4Cols {   // 128 < R <= 160: one row of four 160 x 64 wavefront tiles
  static constexpr int NW = 4, WN = 4, MI = 5, NI = 2, AROWS = 192, AR = W4_AR;
  static constexpr bool EXTRA = false;
};
template <>
struct W4Layout<8> : W4Cols {   // 160 < R <= 192
  static constexpr int NW = 4, WN = 2, MI = 3, NI = 4, AROWS = 192, AR = W4_AR;
  static constexpr bool EXTRA = false;
};
template <>
struct W4Layout<9> : W4Cols {   // 64 < R <= 96 (the load split needs a multiple of 64 A rows)
  static constexpr int NW = 4, WN = 4, MI = 3, NI = 2, AROWS = 128, AR = W4_AR;
  static constexpr bool EXTRA = false;
};
template <>
struct W4Layout<10> {   // wide tiles: 96 < R <= 128, 512 columns
  static constexpr int NW = 4, WN = 4, MI = 4, NI = 4, AROWS = WIDE_AR, AR = WIDE_AR;
  static constexpr int BNL = WIDE_BN, CST = WIDE_CST;
  static constexpr bool EXTRA = false;
};
// Wide tiles of fewer rows multiply fewer padding rows (the fine-grained
// shape's experts hold 20-300 rows; 121 of its 256 have at most 96): the
// same LDS layout, 64 or 128 A rows loaded (the load split needs a multiple
// of 64), 64 or 96 rows multiplied.
template <>
struct W4Layout<12> {   // wide tiles: R <= 64
  static constexpr int NW = 4, WN = 4, MI = 2, NI = 4, AROWS = 64, AR = WIDE_AR;
  static constexpr int BNL = WIDE_BN, CST = WIDE_CST;
  static constexpr bool EXTRA = false;
};
template <>
struct W4Layout<13> {   // wide tiles: 64 < R <= 96
  static constexpr int NW = 4, WN = 4, MI = 3, NI = 4, AROWS = WIDE_AR, AR = WIDE_AR;
  static constexpr int BNL = WIDE_BN, CST = WIDE_CST;
  static constexpr bool EXTRA = false;
};
// Weight gradients of launches bound by the weight stream (few rows per
// expert, so k-segments of a few k-steps): tiles of 256 x 128, 2 x 2
// wavefronts of 128 x 64 (128 accumulators each), three 24 KiB stages.  Two
// workgroups fit on a CU (at most 256 registers per lane and 72 KiB of LDS
// each), so one's epilogue stores and prologue loads overlap the other's
// MFMAs; a 256 x 256 tile holds half of a CU's registers and all its LDS.
constexpr int WG2_BN = BN / 2, WG2_NS = 3;
constexpr int WG2_STAGE = (W4_TM + WG2_BN) * BK;   // 24 KiB
constexpr int WG2_CST = WG2_BN + 8;
template <>
struct W4Layout<11> {   // weight gradients, 256 x 128 tiles, no folded rows
  static constexpr int NW = 4, WN = 2, MI = 4, NI = 2, AROWS = W4_TM, AR = W4_TM;
  static constexpr int BNL = WG2_BN, CST = WG2_CST;
  static constexpr bool EXTRA = false;
};
template <>
struct W4Layout<4> : W4Cols {   // eight wavefronts, 128 < R <= 256
  static constexpr int NW = 8, WN = 4, MI = 4, NI = 2, AROWS = 256, AR = W4_AR;
  static constexpr bool EXTRA = false;
};
template <>
struct W4Layout<5> : W4Cols {   // eight wavefronts, R <= 128
  static constexpr int NW = 8, WN = 4, MI = 2, NI = 2, AROWS = 128, AR = W4_AR;
  static constexpr bool EXTRA = false;
};
template <>
struct W4Layout<7> : W4Cols {   // eight wavefronts, 256 < R <= 320 (384 A rows loaded, the last clamped)
  static constexpr int NW = 8, WN = 4, MI = 4, NI = 2, AROWS = W8_AR, AR = W8_AR;
  static constexpr bool EXTRA = true;
};


// 16 output bytes staged in LDS to memory, as non-temporal stores (NT) for
// the weight gradients and the first GEMM's GELU output.  Nothing later in
// the pass reads the gradients, and with ~128-row k-segments their kernels
// are bound by these stores (the expert backward of the Switch- and
// DeepSeek-shaped layers ran 8% and 4% faster with them).  The GELU output
// is read once more, by the second GEMM; the forward expert stage still ran
// 0.6-0.8% faster on the three prefill shapes (the second GEMM's output,
// which the combine reads right away, measured better without).
// Accumulator (ni, mi) of a wavefront tile: acc[ni][mi] for up to 4 x 4
// blocks; layouts with more than four row blocks (and at most 16 blocks in
// all) number the blocks ni * MI + mi across the same 16 registers tiles.
constexpr int acc_r(int MI, int ni, int mi) { return MI <= 4 ? ni : (ni * MI + mi) >> 2; }
constexpr int acc_c(int MI, int ni, int mi) { return MI <= 4 ? mi : (ni * MI + mi) & 3; }

template <bool NT>
__device__ __forceinline__ void store_out(uint16_t* dst, const uint16_t* src) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = *reinterpret_cast<const u32x4*>(src);
  if constexpr (NT)
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(dst));
  else
    *reinterpret_cast<u32x4*>(dst) = v;
}

// QW: the routed weights are INT8 codes with one fp32 scale per output row
// (a.wscale); the shared problem's tiles keep bf16 weights and take the
// kernel's bf16 path.  The codes travel to LDS as bytes (half the bytes of
// bf16), each fragment is widened to bf16 in registers (exact: |q| <= 127)
// just before its MFMAs, and the epilogue multiplies by the row scale before
// the bias.
// WG: weight-gradient (k-segment) mode -- expert e's tile contracts over
// columns [kseg[e], kseg[e+1]) of A [wg_rows, Kd] and W [Nd, Kd], both shared
// by all experts; an empty segment leaves the accumulators at zero.
// KM: k-major weights, W_e stored [Kd, Nd] (the input gradients of the
// backward read the forward's weights as they are).
// NTW: the weights' direct loads are non-temporal (lds_load16<2>).
template <bool GELU, bool QW, int NS, int LAY, bool WG, bool KM, bool NTW = false,
          bool Q4 = false>
__device__ __forceinline__ void w4_tile(const GemmArgs& a, const TileRef& tr, uint16_t* lds,
                                        f32x16 (&acc)[4][4]) {
  using Lay = W4Layout<LAY>;
  constexpr int MI = Lay::MI, NI = Lay::NI, WN = Lay::WN;
  constexpr bool EX = Lay::EXTRA;
  constexpr int NW = Lay::NW;
  constexpr int NLA = Lay::AROWS / RPI / NW;   // direct loads per wavefront per stage, A rows
  // W rows: 16 rows of 64 bytes per wave instruction (bf16 rows of one
  // k-step, INT8 rows of two)
  constexpr int NLB = Lay::BNL / RPI / NW;
  static_assert(!KM || Lay::BNL == BN, "k-major weight stages hold 256 columns");
  static_assert(!QW || NS == 4, "the INT8 / INT4 wait counts below assume four stages");
  static_assert(!Q4 || QW, "INT4 codes are a form of quantised weights");
  static_assert(NLA * RPI * NW == Lay::AROWS && NLB > 0, "loads split evenly over the waves");
  constexpr int NLS = NLA + NLB;
  const int Kd = a.Kd, Nd = a.Nd;
  const uint16_t* A;
  const char* W;                // bf16 or INT8 weights of this tile's expert
  const uint16_t* bias = nullptr;
  const float* wsc = nullptr;
  uint16_t* C;
  int arow0 = tr.row0;          // A row of the tile's first row
  int kbeg = 0, KT = Kd / BK;   // contraction columns [kbeg, kbeg + KT * BK)
  if constexpr (WG) {
    A = static_cast<const uint16_t*>(a.A);
    W = static_cast<const char*>(a.W);
    C = static_cast<uint16_t*>(a.C);
    kbeg = a.kseg[tr.e];
    KT = (a.kseg[tr.e + 1] - kbeg) / BK;
    arow0 = tr.row0 - tr.e * a.wg_rows;
  } else if (tr.shared) {
    A = static_cast<const uint16_t*>(a.As);
    W = static_cast<const char*>(a.Ws);
    C = static_cast<uint16_t*>(a.Cs);
  } else {
    A = static_cast<const uint16_t*>(a.A);
    W = static_cast<const char*>(a.W) + (Q4 ? (int64_t)tr.e * Nd * (Kd / 2)
                                            : (int64_t)tr.e * Nd * Kd * (QW ? 1 : 2));
    if (a.bias) bias = static_cast<const uint16_t*>(a.bias) + (int64_t)tr.e * Nd;
    if (QW) wsc = a.wscale + (int64_t)tr.e * Nd;
    C = static_cast<uint16_t*>(a.C);
  }
  const int rows = tr.row_end - tr.row0;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / WN, wn = wave % WN;
  constexpr int WROWS = MI * 32, WCOLS = NI * 32;   // wavefront tile

  // Wavefront w fills A rows [NLA*16*w, +NLA*16) and W rows [64w, 64w+64) of
  // a stage; instruction i covers 16 rows; lane -> (row r_in, physical
  // chunk), loading logical chunk pc ^ swz(row).
  const int r_in = lane / CH;
  uint32_t offA[NLA], offB[NLB];
#pragma unroll
  for (int i = 0; i < NLA; ++i) {
    const int row = (wave * NLA + i) * RPI + r_in;
    const int lchunk = (lane % CH) ^ swz(row);
    offA[i] = (uint32_t)(arow0 + min(row, rows - 1)) * (uint32_t)Kd + lchunk * 8 + kbeg;
  }
  // (byte offsets of the W rows)
#pragma unroll
  for (int i = 0; i < NLB; ++i) {
    if constexpr (QW) {
      const int row = (wave * NLB + i) * RPI + r_in;
      const int lchunk = (lane % CH) ^ swz(row);
      offB[i] = (uint32_t)min(tr.n0 + row, Nd - 1) * (uint32_t)(Q4 ? Kd / 2 : Kd) + lchunk * 16;
    } else if constexpr (KM) {
      // instruction i fills k-rows 2 (w NLB + i) and + 1, 32 lanes per row;
      // columns past Nd (partial tiles) read a valid chunk and are not stored
      const int row = (wave * NLB + i) * 2 + (lane >> 5);
      const int lchunk = (lane & 31) ^ kswz(row);
      offB[i] = ((uint32_t)row * (uint32_t)Nd + (uint32_t)min(tr.n0 + lchunk * 8, Nd - 8)) * 2;
    } else {
      const int row = (wave * NLB + i) * RPI + r_in;
      const int lchunk = (lane % CH) ^ swz(row);
      offB[i] = ((uint32_t)min(tr.n0 + row, Nd - 1) * (uint32_t)Kd + lchunk * 8 + kbeg) * 2;
    }
  }
  constexpr int STG = (Lay::AR + Lay::BNL) * BK;   // bf16 elements per LDS stage
  auto issue_a = [&](int buf, int k0) {
    uint16_t* base = lds + buf * STG + wave * NLA * RPI * BK;
#pragma unroll
    for (int i = 0; i < NLA; ++i) lds_load16(A + offA[i] + k0, base + i * RPI * BK);
  };
  auto issue_b = [&](int buf, int k0) {
    char* base = reinterpret_cast<char*>(lds + buf * STG + Lay::AR * BK) + wave * NLB * 1024;
    const uint32_t kb = KM ? (uint32_t)k0 * (uint32_t)Nd * 2 : (Q4 ? k0 / 2 : k0 * (QW ? 1 : 2));
    if constexpr (NTW) {
#pragma unroll
      for (int i = 0; i < NLB; ++i) lds_load16<2>(W + offB[i] + kb, base + i * 1024);
    } else {
#pragma unroll
      for (int i = 0; i < NLB; ++i) lds_load16(W + offB[i] + kb, base + i * 1024);
    }
  };

  // k-pairs: one direct load moves 8 rows x 128 bytes (two k-steps of a
  // row), into two pair buffers of (AR + BNL) rows x 128 bytes each.  INT8
  // codes: the weight region of a pair buffer holds the codes of its two
  // k-steps as 64-byte rows, 16 rows per direct load, laid out and swizzled
  // like the four-stage loop's even stages; the activation rows stay 128
  // bytes (they are most of an INT8 tile's load bytes).  INT4 codes: a
  // 64-byte row holds four k-steps (two pairs), so pairs 2g and 2g + 1 read
  // the codes that were loaded with pair 2g into the weight region of
  // buffer g mod 2, and only the odd pairs issue code loads (for the next
  // group, into the other region).
  constexpr bool P2 = MOE_KPAIRS && !WG && !KM;
  constexpr int NLA2 = Lay::AROWS / 8 / NW, NLB2 = Lay::BNL / 8 / NW;
  constexpr int NLBP = QW ? NLB : NLB2;   // weight loads per wavefront per pair
  static_assert(!P2 || (NLA2 * 8 * NW == Lay::AROWS && NLBP % 2 == 0), "pair loads split evenly");
  constexpr int PST = (Lay::AR + Lay::BNL) * 2 * BK;   // bf16 elements per pair buffer
  static_assert(!P2 || NS == 4, "the pair buffers take the four stages' LDS");
  uint32_t oA2[P2 ? NLA2 : 1], oB2[P2 ? NLB2 : 1];
  if constexpr (P2) {
#pragma unroll
    for (int i = 0; i < NLA2; ++i) {
      const int row = (wave * NLA2 + i) * 8 + (lane >> 3);
      oA2[i] = (uint32_t)(arow0 + min(row, rows - 1)) * (uint32_t)Kd + ((lane & 7) ^ swz8(row)) * 8;
    }
#pragma unroll
    for (int i = 0; i < NLB2; ++i) {
      const int row = (wave * NLB2 + i) * 8 + (lane >> 3);
      oB2[i] = ((uint32_t)min(tr.n0 + row, Nd - 1) * (uint32_t)Kd + ((lane & 7) ^ swz8(row)) * 8) * 2;
    }
  }
  auto issue_a2 = [&](int buf, int k0) {
    uint16_t* base = lds + buf * PST + wave * NLA2 * 8 * 2 * BK;
#pragma unroll
    for (int i = 0; i < NLA2; ++i) lds_load16(A + oA2[i] + k0, base + i * 8 * 2 * BK);
  };
  auto issue_b2 = [&](int buf, int k0, auto i0_tag, auto i1_tag) {
    char* base = reinterpret_cast<char*>(lds + buf * PST + Lay::AR * 2 * BK) + wave * NLBP * 1024;
    if constexpr (QW) {
#pragma unroll
      for (int i = decltype(i0_tag)::value; i < decltype(i1_tag)::value; ++i)
        lds_load16(W + offB[i] + (uint32_t)(Q4 ? k0 / 2 : k0), base + i * 1024);
    } else if constexpr (NTW) {
#pragma unroll
      for (int i = decltype(i0_tag)::value; i < decltype(i1_tag)::value; ++i)
        lds_load16<2>(W + oB2[i] + (uint32_t)k0 * 2, base + i * 1024);
    } else {
#pragma unroll
      for (int i = decltype(i0_tag)::value; i < decltype(i1_tag)::value; ++i)
        lds_load16(W + oB2[i] + (uint32_t)k0 * 2, base + i * 1024);
    }
  };

  const int sw = swz(lane & 31);   // the same for every fragment row this lane reads
  const int sw8 = swz8(lane & 31);   // (k-pairs; fragment rows start at multiples of 16)
  const int arow = (wm * WROWS + (lane & 31)) * BK, brow = (wn * WCOLS + (lane & 31)) * BK;
  // rows 256 + 32*wm .. +32 of a 320-row tile (EX only)
  const int xrow = (W4_TM + wm * 32 + (lane & 31)) * BK;
  constexpr int MX = MI + (EX ? 1 : 0);   // A fragments per half
  // W fragments: bf16x8, or 8 INT8 codes widened just before their MFMAs
  // (INT4: one 32-bit word of 8 codes)
  using BF = typename std::conditional<Q4, uint32_t,
                                       typename std::conditional<QW, uint2, bf16x8>::type>::type;
  // INT8: byte offset of this lane's row (n = lane mod 32) in a pair region
  const int browq = (wn * WCOLS + (lane & 31)) * 64;
  // KM: this lane's byte offset inside a stage's weight region (source role:
  // group g = lane / 16, q = (lane mod 16) / 4, u = lane mod 4), without the
  // half, the second read's 4 k-rows and the fragment's 32-column group
  const int kg = lane >> 4, kq = (lane & 15) >> 2, ku = lane & 3;
  const int kmb = (8 * (kg >> 1) + kq) * 512 + (2 * (kg & 1) + (ku >> 1)) * 16 + (ku & 1) * 8;
  bf16x8 fa0[MX], fa1[MX];
  BF fb0[NI], fb1[NI];
  BF fbq[QW ? NI : 1];   // INT8 / INT4: the second half's codes, read with the first's
  f32x16 accx[EX ? NI : 1];
  if constexpr (EX) {
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) accx[i][v] = 0.f;
  }
  // Fragments of half kk: lane half h = lane / 32 holds k = 16 kk + 8 h + 0..7
  // of the step (bf16 weights), or k = 16 h + 8 kk + 0..7 (INT8 weights, so
  // that one 16-byte chunk of codes serves both halves).
  // kabs: the k-step's index (INT4: which of the two code regions holds it)
  auto read_half = [&](bf16x8 (&fa)[MX], BF (&fb)[NI], int buf, int kk, int kabs) {
    const uint16_t* As = lds + buf * STG;
    const uint16_t* Bs = As + Lay::AR * BK;
    const int pc = ((QW ? (lane >> 5) * 2 + kk : kk * 2 + (lane >> 5)) ^ sw) * 8;
#pragma unroll
    for (int i = 0; i < MI; ++i)
      fa[i] = *reinterpret_cast<const bf16x8*>(As + arow + i * 32 * BK + pc);
    if constexpr (EX) fa[MI] = *reinterpret_cast<const bf16x8*>(As + xrow + pc);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      if constexpr (Q4) {
        if (kk == 0) {
          // INT4: chunk buf (= k-step mod 4) of the region of stage 0 or 2
          // holding this group of four k-steps; lane half h reads its 8 bytes
          const char* Bq = reinterpret_cast<const char*>(lds + ((kabs >> 2) & 1) * 2 * STG +
                                                         Lay::AR * BK);
          const uint2 q = *reinterpret_cast<const uint2*>(
              Bq + browq + i * 32 * 64 + ((buf ^ sw) * 16) + (lane >> 5) * 8);
          fb[i] = q.x;
          fbq[i] = q.y;
        } else {
          fb[i] = fbq[i];
        }
      } else if constexpr (QW) {
        if (kk == 0) {
          // chunk 2 (buf mod 2) + lane / 32 of the pair region of the even stage
          const char* Bq = reinterpret_cast<const char*>(lds + (buf & ~1) * STG + Lay::AR * BK);
          const uint4 q = *reinterpret_cast<const uint4*>(
              Bq + browq + i * 32 * 64 + (((2 * (buf & 1) + (lane >> 5)) ^ sw) * 16));
          fb[i] = make_uint2(q.x, q.y);
          fbq[i] = make_uint2(q.z, q.w);
        } else {
          fb[i] = fbq[i];
        }
      } else if constexpr (KM) {
        const char* p = reinterpret_cast<const char*>(Bs) + kk * 8192 + kmb +
                        ((((wn * WCOLS + i * 32) >> 3) ^ (4 * kq)) << 4);
        const bf16x4 lo = lds_read_tr(p), hi = lds_read_tr(p + 2048);
        fb[i] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      } else {
        fb[i] = *reinterpret_cast<const bf16x8*>(Bs + brow + i * 32 * BK + pc);
      }
    }
  };
  // k-pairs: fragments of half kk of k-step ks (0, 1) of the pair in buffer buf
  // (INT8 codes: the k order of read_half's INT8 fragments, k = 16 h + 8 kk
  // + 0..7 of the step; the half kk = 0 reads the 16 codes of both halves)
  // (pq: the pair's index, which places INT4 codes)
  auto read_q = [&](bf16x8 (&fa)[MX], BF (&fb)[NI], int buf, int ks, int kk, int pq) {
    const uint16_t* As = lds + buf * PST;
    const uint16_t* Bs = As + Lay::AR * 2 * BK;
    const int pc = ((ks * 4 + (QW ? (lane >> 5) * 2 + kk : kk * 2 + (lane >> 5))) ^ sw8) * 8;
    const int ar = (wm * WROWS + (lane & 31)) * 2 * BK, br = (wn * WCOLS + (lane & 31)) * 2 * BK;
#pragma unroll
    for (int i = 0; i < MI; ++i)
      fa[i] = *reinterpret_cast<const bf16x8*>(As + ar + i * 32 * 2 * BK + pc);
    if constexpr (EX)
      fa[MI] = *reinterpret_cast<const bf16x8*>(As + (W4_TM + wm * 32 + (lane & 31)) * 2 * BK + pc);
    if constexpr (Q4) {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        if (kk == 0) {
          // chunk 2 (pq mod 2) + ks (the k-step inside the group of four) of
          // the region of buffer (pq / 2) mod 2; lane half h reads its 8 bytes
          const char* Bq =
              reinterpret_cast<const char*>(lds + ((pq >> 1) & 1) * PST + Lay::AR * 2 * BK);
          const uint2 q = *reinterpret_cast<const uint2*>(
              Bq + browq + i * 32 * 64 + (((2 * (pq & 1) + ks) ^ sw) * 16) + (lane >> 5) * 8);
          fb[i] = q.x;
          fbq[i] = q.y;
        } else {
          fb[i] = fbq[i];
        }
      }
    } else if constexpr (QW) {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        if (kk == 0) {
          const uint4 q = *reinterpret_cast<const uint4*>(
              reinterpret_cast<const char*>(Bs) + browq + i * 32 * 64 +
              (((2 * ks + (lane >> 5)) ^ sw) * 16));
          fb[i] = make_uint2(q.x, q.y);
          fbq[i] = make_uint2(q.z, q.w);
        } else {
          fb[i] = fbq[i];
        }
      }
    } else if constexpr (!QW) {
#pragma unroll
      for (int i = 0; i < NI; ++i)
        fb[i] = *reinterpret_cast<const bf16x8*>(Bs + br + i * 32 * 2 * BK + pc);
    }
  };
  auto wfrag = [&](const BF& f) -> bf16x8 {
    if constexpr (Q4)
      return __builtin_bit_cast(bf16x8, int4x8_to_bf16x8(f));
    else if constexpr (QW)
      return __builtin_bit_cast(bf16x8, int8x8_to_bf16x8(f));
    else
      return f;
  };
  auto mfma_half = [&](const bf16x8 (&fa)[MX], const BF (&fbr)[NI]) {
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
      const bf16x8 fb = wfrag(fbr[ni]);
#pragma unroll
      for (int mi = 0; mi < MI; ++mi)
        acc[acc_r(MI, ni, mi)][acc_c(MI, ni, mi)] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            fb, fa[mi], acc[acc_r(MI, ni, mi)][acc_c(MI, ni, mi)], 0, 0, 0);
      // The folded rows' accumulators live in ordinary VGPRs (the 256
      // accumulation registers hold the main 256 x 256): the compiler keeps
      // all MFMA results in one register class, so these four are written
      // out with VGPR operands.  The compiler does not see an MFMA here and
      // inserts no wait states for it, and it may schedule the statement
      // right after the VALU instructions that write its operands (the INT8
      // weight fragment is widened by v_perm_b32 code; the compiler was seen
      // to place this MFMA one instruction after that write, which made the
      // folded rows' results depend on timing).  So the statement carries
      // its own pad: s_nop 4 gives 5 wait states, more than a VALU write
      // followed by an MFMA source read needs.  fa[MI] comes from an LDS
      // read covered by the wait counts; each accx[ni] is next read by the
      // same MFMA a whole half later, and the epilogue pads before reading it.
      if constexpr (EX)
        asm("s_nop 4\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
            : "+v"(accx[ni])
            : "v"(fb), "v"(fa[MI]));
    }
  };
  // one half: MI*NI MFMAs interleaved with the half's fragment reads (MX
  // for A plus NB for the weights) and NV direct loads; RPS reads follow
  // each MFMA
  auto interleave = [&](auto nv_tag, auto nb_tag) {
    constexpr int NV = decltype(nv_tag)::value;
    constexpr int NM = MX * NI, ND = MX + decltype(nb_tag)::value;
    constexpr int RPS = (ND + NM - 1) / NM, NSL = (ND + RPS - 1) / RPS;
    constexpr int VS = NSL >= NV ? NSL - NV : 0;    // first slot with a direct load
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i < NSL) __builtin_amdgcn_sched_group_barrier(0x100, RPS, 0);
      if (i >= VS && i < VS + NV) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    }
    static_assert(VS + NV <= NM, "every load sits between two MFMAs");
  };

  if constexpr (P2) {
  // k-pairs: pair p covers k-steps 2p, 2p+1 (KT is even: Kd is a multiple of
  // 64) in buffer p mod 2, four halves per pair.  The weight rows of pair
  // p+1 are issued in the first two halves of pair p into the other buffer
  // (its reads ended before the previous pair's barrier); one barrier after
  // the third half, once every lane has its own loads of pair p+1 landed and
  // its reads of pair p done; the fourth half reads pair p+1's first
  // fragments and issues the A rows of pair p+2 into the buffer just freed.
  const int NP = KT / 2;
  issue_a2(0, 0);
  issue_b2(0, 0, std::integral_constant<int, 0>{}, std::integral_constant<int, NLBP>{});
  issue_a2(1, min(1, NP - 1) * 2 * BK);
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NLA2) : "memory");
  barrier();
  read_q(fa0, fb0, 0, 0, 0, 0);
  // pair p; PH = p mod 2 (INT4 codes: the odd pairs load the next group's)
  auto pair_step = [&](int p, auto ph_tag) {
    constexpr bool LOADW = !Q4 || decltype(ph_tag)::value == 1;
    constexpr int NVW = LOADW ? NLBP / 2 : 0;
    const int buf = p & 1, nb = buf ^ 1;
    const int kn2 = min(p + 2, NP - 1) * 2 * BK;
    // weight rows of pair p + 1 into buffer nb; INT4: the codes of group
    // (p + 1) / 2 into region ((p + 1) / 2) mod 2 (past the end: the last
    // group's codes again, into the region no pair reads any more)
    const int wreg = Q4 ? ((p + 1) >> 1) & 1 : nb;
    const int kw = (Q4 ? min(p + 1, NP - 2) : min(p + 1, NP - 1)) * 2 * BK;
    __builtin_amdgcn_sched_barrier(0);
    read_q(fa1, fb1, buf, 0, 1, p);
    if constexpr (LOADW)
      issue_b2(wreg, kw, std::integral_constant<int, 0>{}, std::integral_constant<int, NLBP / 2>{});
    mfma_half(fa0, fb0);
    // (INT8 / INT4 codes: weight fragments are read in the halves kk = 0 only)
    interleave(std::integral_constant<int, NVW>{}, std::integral_constant<int, QW ? 0 : NI>{});
    __builtin_amdgcn_sched_barrier(0);
    read_q(fa0, fb0, buf, 1, 0, p);
    if constexpr (LOADW)
      issue_b2(wreg, kw, std::integral_constant<int, NLBP / 2>{}, std::integral_constant<int, NLBP>{});
    mfma_half(fa1, fb1);
    interleave(std::integral_constant<int, LOADW ? NLBP - NLBP / 2 : 0>{},
               std::integral_constant<int, NI>{});
    __builtin_amdgcn_sched_barrier(0);
    read_q(fa1, fb1, buf, 1, 1, p);
    mfma_half(fa0, fb0);
    interleave(std::integral_constant<int, 0>{}, std::integral_constant<int, QW ? 0 : NI>{});
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    barrier();
    __builtin_amdgcn_sched_barrier(0);
    read_q(fa0, fb0, nb, 0, 0, p + 1);
    issue_a2(buf, kn2);
    mfma_half(fa1, fb1);
    interleave(std::integral_constant<int, NLA2>{}, std::integral_constant<int, NI>{});
    __builtin_amdgcn_sched_barrier(0);
  };
  if constexpr (Q4) {
    // Kd is a multiple of 128 for INT4 codes: NP is even
    for (int p = 0; p < NP; p += 2) {
      pair_step(p, std::integral_constant<int, 0>{});
      pair_step(p + 1, std::integral_constant<int, 1>{});
    }
  } else {
    for (int p = 0; p < NP; ++p) pair_step(p, std::integral_constant<int, 0>{});
  }
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  } else if (!WG || KT > 0) {
  // Prologue: stages 0 .. NS-2 in flight (chunks past the end re-read the
  // last chunk into buffers nobody reads again, so every k-step issues the
  // same number of loads and the wait counts are constants).  INT8: the even
  // stages load the codes of their pair (Kd is a multiple of 64, so KT is
  // even), and a k-step waits for fewer younger loads when the stage it
  // waits for is even (no codes were issued with the stage after it).
  // INT4: stages 4g load the codes of k-steps 4g .. 4g+3 (64 bytes a row,
  // Kd a multiple of 128) into the weight region of stage 0 (g even) or 2 (g
  // odd); with codes issued at one step in four, the k-step of phase 2 is
  // the one that waits for fewer younger loads.
  constexpr int CPL = Q4 ? 4 : 2;   // quantised: k-steps per code load
#pragma unroll
  for (int st = 0; st < NS - 1; ++st) {
    issue_a(st, min(st, KT - 1) * BK);
    if (!QW)
      issue_b(st, min(st, KT - 1) * BK);
    else if (st % CPL == 0)
      issue_b(st, min(st, KT - CPL) * BK);
  }
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(Q4 ? 2 * NLA : QW ? 2 * NLA + NLB : NLS * (NS - 2))
               : "memory");
  barrier();
  read_half(fa0, fb0, 0, 0, 0);

  // one k-step; PH (quantised weights only): kt mod CPL.  The quantised loops
  // run CPL steps per iteration so that the phase is known at compile time.
  auto step = [&](int kt, auto ph_tag) {
    constexpr int PH = decltype(ph_tag)::value;
    // the step whose second half issues the codes of stage kt+NS-1, and the
    // step that then waits for one code load fewer (INT8: PH 1 and 0; INT4:
    // PH 1 and 2)
    constexpr bool CODES = QW && PH == 1;
    constexpr bool WAIT_B = QW && PH == (Q4 ? 2 : 0);
    const int buf = kt % NS, nbuf = (kt + NS - 1) % NS;
    const int nk = min(kt + NS - 1, KT - 1) * BK;
    // first half: MFMAs on set 0; set 1 <- second half of this stage; A rows
    // of stage kt+NS-1 into the buffer last read before the previous barrier
    __builtin_amdgcn_sched_barrier(0);
    read_half(fa1, fb1, buf, 1, kt);
    issue_a(nbuf, nk);
    mfma_half(fa0, fb0);
    interleave(std::integral_constant<int, NLA>{},
               std::integral_constant<int, QW ? 0 : (KM ? 2 : 1) * NI>{});
    __builtin_amdgcn_sched_barrier(0);
    // own loads of stage kt+1 landed (younger: NS-3 whole stages and this
    // step's A rows), own reads of stage kt done
    if constexpr (QW && !WAIT_B)
      asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(2 * NLA) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(QW ? 2 * NLA + NLB : NLS * (NS - 3) + NLA)
                   : "memory");
    barrier();
    // second half: MFMAs on set 1; set 0 <- first half of stage kt+1 (in the
    // last step this reads a stale buffer that nobody uses); W rows of stage
    // kt+NS-1 (quantised: only when that stage starts a code load, into the
    // region of its group)
    __builtin_amdgcn_sched_barrier(0);
    read_half(fa0, fb0, (kt + 1) % NS, 0, kt + 1);
    if constexpr (QW && !CODES) {
      mfma_half(fa1, fb1);
      interleave(std::integral_constant<int, 0>{}, std::integral_constant<int, NI>{});
    } else {
      if constexpr (Q4)
        issue_b((((kt + NS - 1) >> 2) & 1) * 2, min(kt + NS - 1, KT - CPL) * BK);
      else
        issue_b(nbuf, QW ? min(kt + NS - 1, KT - CPL) * BK : nk);
      mfma_half(fa1, fb1);
      interleave(std::integral_constant<int, NLB>{},
                 std::integral_constant<int, (KM ? 2 : 1) * NI>{});
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  if constexpr (Q4) {
    for (int kt = 0; kt < KT; kt += 4) {
      step(kt, std::integral_constant<int, 0>{});
      step(kt + 1, std::integral_constant<int, 1>{});
      step(kt + 2, std::integral_constant<int, 2>{});
      step(kt + 3, std::integral_constant<int, 3>{});
    }
  } else if constexpr (QW) {
    for (int kt = 0; kt < KT; kt += 2) {
      step(kt, std::integral_constant<int, 0>{});
      step(kt + 1, std::integral_constant<int, 1>{});
    }
  } else {
    for (int kt = 0; kt < KT; ++kt) step(kt, std::integral_constant<int, 0>{});
  }
  // no direct-to-LDS load may still be in flight past this point
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
  }

  // Epilogue.  The 32x32 accumulator of (ni, mi) holds C^T: element v of lane l
  // is output row mi*32 + l%32, column ni*32 + (v/4)*8 + (l/32)*4 + v%4.
  // Bias and GELU are applied in registers, the bf16 tile goes to LDS, and
  // the workgroup then writes whole 512-byte rows with 16-byte stores.
  barrier();
#pragma unroll
  for (int ni = 0; ni < NI; ++ni) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int nl = wn * WCOLS + ni * 32 + g * 8 + (lane >> 5) * 4;
      float bv[4] = {0.f, 0.f, 0.f, 0.f};
      if (bias) {
        // columns past Nd (partial tiles) read a valid chunk and are not stored
        const uint2 braw = *reinterpret_cast<const uint2*>(bias + min(tr.n0 + nl, Nd - 4));
        bv[0] = __uint_as_float(braw.x << 16);
        bv[1] = __uint_as_float(braw.x & 0xffff0000u);
        bv[2] = __uint_as_float(braw.y << 16);
        bv[3] = __uint_as_float(braw.y & 0xffff0000u);
      }
      float sv[4] = {1.f, 1.f, 1.f, 1.f};
      if constexpr (QW) {
        const float4 sr = *reinterpret_cast<const float4*>(wsc + min(tr.n0 + nl, Nd - 4));
        sv[0] = sr.x; sv[1] = sr.y; sv[2] = sr.z; sv[3] = sr.w;
      }
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        const int ml = wm * WROWS + mi * 32 + (lane & 31);
        float z[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float av = acc[acc_r(MI, ni, mi)][acc_c(MI, ni, mi)][g * 4 + q];
          z[q] = QW ? fmaf(av, sv[q], bv[q]) : av + bv[q];
          if (GELU) z[q] = gelu_as(z[q]);
        }
        // v_cvt_pk_bf16_f32: round to nearest even, two values per instruction
        const bf16x4 pk = __builtin_convertvector((f32x4){z[0], z[1], z[2], z[3]}, bf16x4);
        *reinterpret_cast<bf16x4*>(lds + ml * Lay::CST + nl) = pk;
      }
    }
  }
  __syncthreads();
  // TPR threads x 16 bytes per staged row; 64 NW / TPR rows per pass
  constexpr int TPR = Lay::BNL / 8;
  const int cc = (threadIdx.x % TPR) * 8;
  const int ncol = tr.n0 + cc;
  const int nrow = min(rows, W4_TM);
  for (int ml = threadIdx.x / TPR; ml < nrow; ml += 64 * NW / TPR)
    if (ncol < Nd)
      store_out<WG || GELU>(C + (int64_t)(tr.row0 + ml) * Nd + ncol, lds + ml * Lay::CST + cc);
  if constexpr (EX) {
    // the folded remainder: rows 256 .. R-1, staged as LDS rows 0 .. 63.
    // 24 wait states between the last MFMA writing accx and its first VALU
    // read (the tie to accx keeps the pad after those MFMAs)
    if constexpr (NI == 4)
      asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
                   : "+v"(accx[0]), "+v"(accx[1]), "+v"(accx[2]), "+v"(accx[3]));
    else
      asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(accx[0]), "+v"(accx[1]));
    __syncthreads();
#pragma unroll
    for (int ni = 0; ni < NI; ++ni) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int nl = wn * WCOLS + ni * 32 + g * 8 + (lane >> 5) * 4;
        float bv[4] = {0.f, 0.f, 0.f, 0.f};
        if (bias) {
          const uint2 braw = *reinterpret_cast<const uint2*>(bias + min(tr.n0 + nl, Nd - 4));
          bv[0] = __uint_as_float(braw.x << 16);
          bv[1] = __uint_as_float(braw.x & 0xffff0000u);
          bv[2] = __uint_as_float(braw.y << 16);
          bv[3] = __uint_as_float(braw.y & 0xffff0000u);
        }
        float sv[4] = {1.f, 1.f, 1.f, 1.f};
        if constexpr (QW) {
          const float4 sr = *reinterpret_cast<const float4*>(wsc + min(tr.n0 + nl, Nd - 4));
          sv[0] = sr.x; sv[1] = sr.y; sv[2] = sr.z; sv[3] = sr.w;
        }
        float z[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          z[q] = QW ? fmaf(accx[ni][g * 4 + q], sv[q], bv[q]) : accx[ni][g * 4 + q] + bv[q];
          if (GELU) z[q] = gelu_as(z[q]);
        }
        const bf16x4 pk = __builtin_convertvector((f32x4){z[0], z[1], z[2], z[3]}, bf16x4);
        *reinterpret_cast<bf16x4*>(lds + (wm * 32 + (lane & 31)) * Lay::CST + nl) = pk;
      }
    }
    __syncthreads();
    for (int ml = threadIdx.x / TPR; ml < rows - W4_TM; ml += 64 * NW / TPR)
      if (ncol < Nd)
        store_out<WG || GELU>(C + (int64_t)(tr.row0 + W4_TM + ml) * Nd + ncol, lds + ml * Lay::CST + cc);
  }
}

// Four-wavefront tile: the wave arrangement from the tile's row count.
template <bool GELU, bool QW, int NS, bool WG, bool KM, bool NTW = false, bool Q4 = false>
__device__ __forceinline__ void w4_rows(const GemmArgs& a, const TileRef& tr, uint16_t* lds,
                                        f32x16 (&acc)[4][4]) {
  const int rows = tr.row_end - tr.row0;
  if (rows > W4_TM)
    w4_tile<GELU, QW, NS, 3, WG, KM, NTW, Q4>(a, tr, lds, acc);
  else if (rows > 192)
    w4_tile<GELU, QW, NS, 0, WG, KM, NTW, Q4>(a, tr, lds, acc);
  else if (rows > 160)
    w4_tile<GELU, QW, NS, 8, WG, KM, NTW, Q4>(a, tr, lds, acc);
  else if (rows > 128)
    w4_tile<GELU, QW, NS, 14, WG, KM, NTW, Q4>(a, tr, lds, acc);
  else if (rows > 96)
    w4_tile<GELU, QW, NS, 1, WG, KM, NTW, Q4>(a, tr, lds, acc);
  else if (rows > 64)
    w4_tile<GELU, QW, NS, 9, WG, KM, NTW, Q4>(a, tr, lds, acc);
  else
    w4_tile<GELU, QW, NS, 2, WG, KM, NTW, Q4>(a, tr, lds, acc);
}

template <bool GELU, bool QW, int NS, bool WG, bool KM, bool NTW = false, bool Q4 = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void
gemm_bf16_w4_kernel(GemmArgs a) {
  // the output tile is staged through the same LDS after the main loop
  // (wide tiles: four 40 KiB stages, the whole 160 KiB)
  constexpr int LDS_ELEMS = cmax(cmax(NS * W4_STAGE, W4_TM * W4_CST),
                                 KM || WG ? 0 : cmax(NS * WIDE_STAGE, WIDE_AR * WIDE_CST));
  __shared__ __attribute__((aligned(1024))) uint16_t lds[LDS_ELEMS];
  const TileRef tr = map_tile(a);
  if (!tr.valid) return;
  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  if constexpr (!KM && !WG) {
    if (tr.wide) {   // routed tiles only
      const int rows = tr.row_end - tr.row0;
      if (rows > 96)
        w4_tile<GELU, QW, NS, 10, WG, KM, false, Q4>(a, tr, lds, acc);
      else if (rows > 64)
        w4_tile<GELU, QW, NS, 13, WG, KM, false, Q4>(a, tr, lds, acc);
      else
        w4_tile<GELU, QW, NS, 12, WG, KM, false, Q4>(a, tr, lds, acc);
      return;
    }
  }
  if (QW && tr.shared)
    w4_rows<GELU, false, NS, WG, KM>(a, tr, lds, acc);
  else
    w4_rows<GELU, QW, NS, WG, KM, NTW, Q4>(a, tr, lds, acc);
}

// The same tiles with eight wavefronts (two per SIMD, at most 256 registers
// each; only acc[0..1][0..3] are live).
template <bool GELU, bool QW, int NS, bool WG, bool KM>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void
gemm_bf16_w8_kernel(GemmArgs a) {
  constexpr int LDS_ELEMS = NS * W8_STAGE > W4_TM * W4_CST ? NS * W8_STAGE : W4_TM * W4_CST;
  __shared__ __attribute__((aligned(1024))) uint16_t lds[LDS_ELEMS];
  const TileRef tr = map_tile(a);
  if (!tr.valid) return;
  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  const int rows = tr.row_end - tr.row0;
  if (rows > W4_TM)
    w4_tile<GELU, QW, NS, 7, WG, KM>(a, tr, lds, acc);
  else if (rows > 128)
    w4_tile<GELU, QW, NS, 4, WG, KM>(a, tr, lds, acc);
  else
    w4_tile<GELU, QW, NS, 5, WG, KM>(a, tr, lds, acc);
}

template <int NS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void
gemm_bf16_wg2_kernel(GemmArgs a) {
  constexpr int LDS_ELEMS = cmax(NS * WG2_STAGE, W4_TM * WG2_CST);
  __shared__ __attribute__((aligned(1024))) uint16_t lds[LDS_ELEMS];
  const TileRef tr = map_tile(a);
  if (!tr.valid) return;
  f32x16 acc[4][4];   // acc[0..1][0..3] live
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;
  w4_tile<false, false, NS, 11, true, false>(a, tr, lds, acc);
}

// Eight wavefronts serve the backward's GEMMs, which never have INT8 weights
// or wide tiles.
template <bool GELU, bool QW, bool WG, bool KM, bool NTW = false, bool Q4 = false>
void launch_w(const GemmArgs& a, int grid, hipStream_t s) {
  if constexpr (!QW) {
    if (a.waves8 && a.wide_rows == 0) {
      hipLaunchKernelGGL((gemm_bf16_w8_kernel<GELU, false, W4_NS, WG, KM>), dim3(grid), dim3(512),
                         0, s, a);
      return;
    }
  }
  hipLaunchKernelGGL((gemm_bf16_w4_kernel<GELU, QW, W4_NS, WG, KM, NTW, Q4>), dim3(grid),
                     dim3(256), 0, s, a);
}

}  // namespace

int gemm_bf16_bm() { return W4_TM; }
int gemm_bf16_bn() { return BN; }
int gemm_bf16_wide_rows() { return WIDE_AR; }
int gemm_bf16_wg_narrow_bn() { return WG2_BN; }
int gemm_bf16_merge_rows() { return W4_MERGE; }

hipError_t launch_gemm_bf16(const GemmArgs& a, bool gelu, hipStream_t s) {
  const int grid = gemm_grid(a);
  if (grid == 0) return hipSuccess;
  if (a.kseg && a.wg_narrow)
    hipLaunchKernelGGL((gemm_bf16_wg2_kernel<WG2_NS>), dim3(grid), dim3(256), 0, s, a);
  else if (a.kseg)
    launch_w<false, false, true, false>(a, grid, s);
  else if (a.wkmaj)
    launch_w<false, false, false, true>(a, grid, s);
  else if (a.wscale && a.w4)
    gelu ? launch_w<true, true, false, false, false, true>(a, grid, s)
         : launch_w<false, true, false, false, false, true>(a, grid, s);
  else if (a.wscale)
    gelu ? launch_w<true, true, false, false>(a, grid, s)
         : launch_w<false, true, false, false>(a, grid, s);
  else
    a.w_stream ? (gelu ? launch_w<true, false, false, false, true>(a, grid, s)
                       : launch_w<false, false, false, false, true>(a, grid, s))
               : (gelu ? launch_w<true, false, false, false>(a, grid, s)
                       : launch_w<false, false, false, false>(a, grid, s));
  return hipGetLastError();
}

}  // namespace moe
