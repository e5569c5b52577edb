// Dispatch: permute (token, slot) pairs from token order into contiguous
// per-expert row blocks, with an optional per-expert capacity.
//
// What it computes (lmnt.cn MoE walkthrough §3.1: reorder the input from
// "by token" to "by expert" so each expert gets one contiguous block; §3.3
// capacity equation: over-capacity tokens skip the expert):
//   pairs p = t*K + k in token-major order; e = idx[p];
//   pos(p)  = #{p' < p : idx[p'] = e}            (stable, token order)
//   kept    = pos(p) < C;  counts[e] = #pairs of e; kept_e = min(counts[e], C)
//   off     = exclusive scan of kept_e;  row = off[e] + pos(p)
//   slot_row[p] = kept ? row : -1;  row_token[row] = t;  x_perm[row] = x[t].
//
// Four launches (two when the tokens form one chunk of 256: hist, scan and
// rank then run in one workgroup), all deterministic (no result depends on
// atomic order):
//   1. hist:    each workgroup counts its 256-token chunk per expert (LDS).
//   2. scan:    one workgroup turns the per-chunk counts into per-chunk
//               starting positions, counts, kept counts, offsets, n_dropped.
//   3. rank:    one wavefront per chunk walks its pairs in order, 64 at a
//               time; lanes with equal experts are matched with ballots, so
//               each pair's position is its chunk start + earlier matches.
//   4. permute: one wavefront per token reads x[t] once (16-byte loads, the
//               whole row in one batch for rows up to 16 KiB) and writes it to
//               each of its kept rows.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int DB = kDispatchTokensPerBlock;
constexpr int MAXN = 256;

__global__ __launch_bounds__(256) void hist_kernel(const int32_t* __restrict__ idx, int T, int K,
                                                   int N, int32_t* __restrict__ blkcnt) {
  __shared__ int hist[MAXN];
  for (int e = threadIdx.x; e < N; e += blockDim.x) hist[e] = 0;
  __syncthreads();
  const int64_t p0 = (int64_t)blockIdx.x * DB * K;
  const int64_t p1 = min((int64_t)(blockIdx.x + 1) * DB, (int64_t)T) * K;
  for (int64_t p = p0 + threadIdx.x; p < p1; p += blockDim.x) {
    const int e = idx[p];
    if (e >= 0 && e < N) atomicAdd(&hist[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < N; e += blockDim.x) blkcnt[(int64_t)blockIdx.x * N + e] = hist[e];
}

// Offsets from the per-expert pair counts: thread e (< N, of 256) holds expert
// e's count `run`; kept = min(run, cap), offsets = exclusive scan of kept,
// offsets[N] = the kept total, n_dropped = pairs - kept total.
__device__ __forceinline__ void expert_scan(int e, int run, int N, int cap, int64_t pairs,
                                            int32_t* __restrict__ offsets,
                                            int32_t* __restrict__ n_dropped, int* wsum) {
  const int kept = (e < N) ? min(run, cap) : 0;
  // exclusive scan of kept over e: wave-level inclusive scan, then wave sums
  const int lane = e & 63, wave = e >> 6;
  int v = kept;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(v, o, 64);
    if (lane >= o) v += u;
  }
  if (lane == 63) wsum[wave] = v;
  __syncthreads();
  int base = 0;
  for (int w = 0; w < wave; ++w) base += wsum[w];
  const int excl = base + v - kept;
  if (e < N) offsets[e] = excl;
  if (e == N - 1) {
    offsets[N] = excl + kept;
    n_dropped[0] = (int32_t)(pairs - (int64_t)(excl + kept));
  }
}

// One workgroup of 256 threads; thread e owns expert e (N <= 256).
__global__ __launch_bounds__(256) void scan_kernel(const int32_t* __restrict__ blkcnt, int nblk,
                                                   int N, int cap, int64_t pairs,
                                                   int32_t* __restrict__ blkoff,
                                                   int32_t* __restrict__ counts,
                                                   int32_t* __restrict__ offsets,
                                                   int32_t* __restrict__ n_dropped) {
  __shared__ int wsum[4];
  const int e = threadIdx.x;
  int run = 0;
  if (e < N) {
    // eight blocks' counts loaded together, then added in block order
    int b = 0;
    for (; b + 8 <= nblk; b += 8) {
      int c[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) c[u] = blkcnt[(int64_t)(b + u) * N + e];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        blkoff[(int64_t)(b + u) * N + e] = run;
        run += c[u];
      }
    }
    for (; b < nblk; ++b) {
      blkoff[(int64_t)b * N + e] = run;
      run += blkcnt[(int64_t)b * N + e];
    }
    counts[e] = run;
  }
  expert_scan(e, run, N, cap, pairs, offsets, n_dropped, wsum);
}

// Positions of the pairs [p0, p1), in order: run[e] holds the position the
// next pair of expert e takes and off_s[e] its block's first row.  Wavefront
// 0 (lanes `lane`) ranks 64 pairs per step; lanes with equal experts are
// matched with ballots.  Every wavefront of the workgroup calls this (the
// trip counts are uniform) and reaches its barriers; `active` is true in
// wavefront 0 only.
__device__ __forceinline__ void rank_walk(const int32_t* __restrict__ idx, int64_t p0, int64_t p1,
                                          int K, int N, int cap, int* run, const int* off_s,
                                          int32_t* __restrict__ slot_row,
                                          int32_t* __restrict__ row_token, int lane, bool active) {
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  // the expert indices of RB 64-slot steps are loaded together, then the
  // steps run in slot order
  constexpr int RB = 8;
  for (int64_t pc = p0; pc < p1; pc += 64 * RB) {
    int ev[RB];
#pragma unroll
    for (int u = 0; u < RB; ++u) {
      const int64_t p = pc + 64 * u + lane;
      ev[u] = (active && p < p1) ? idx[p] : -1;
    }
#pragma unroll
    for (int u = 0; u < RB; ++u) {
      const int64_t pb = pc + 64 * u;
      if (pb >= p1) break;   // uniform over the workgroup
      const int64_t p = pb + lane;
      const bool inb = active && p < p1;
      const int e = ev[u];
      const bool valid = inb && e >= 0 && e < N;
      // lanes holding the same valid expert: AND of per-bit ballots
      uint64_t match = __ballot(valid);
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        const bool bit = valid && ((e >> b) & 1);
        const uint64_t ones = __ballot(bit);
        match &= bit ? ones : ~ones;
      }
      if (!valid) match = 0;
      int pos = 0;
      if (valid) {
        const int rank = __popcll(match & below);
        const int start = run[e];
        pos = start + rank;
        const uint64_t above = (lane == 63) ? 0ull : (match >> (lane + 1));
        if (above == 0) run[e] = start + __popcll(match);   // last lane of its group
      }
      if (inb) {
        int r = -1;
        if (valid && pos < cap) {
          r = off_s[e] + pos;
          row_token[r] = (int32_t)(p / K);
        }
        slot_row[p] = r;
      }
      __syncthreads();
    }
  }
}

// One wavefront per chunk of DB tokens.
__global__ __launch_bounds__(64) void rank_kernel(const int32_t* __restrict__ idx, int T, int K,
                                                  int N, int cap,
                                                  const int32_t* __restrict__ blkoff,
                                                  const int32_t* __restrict__ offsets,
                                                  int32_t* __restrict__ slot_row,
                                                  int32_t* __restrict__ row_token) {
  __shared__ int run[MAXN];
  __shared__ int off_s[MAXN];
  const int lane = threadIdx.x;
  for (int e = lane; e < N; e += 64) {
    run[e] = blkoff[(int64_t)blockIdx.x * N + e];
    off_s[e] = offsets[e];
  }
  __syncthreads();
  const int64_t p0 = (int64_t)blockIdx.x * DB * K;
  const int64_t p1 = min((int64_t)(blockIdx.x + 1) * DB, (int64_t)T) * K;
  rank_walk(idx, p0, p1, K, N, cap, run, off_s, slot_row, row_token, lane, true);
}

// All of hist, scan and rank in one workgroup of 256 threads when the tokens
// form one chunk (T <= DB): the per-expert counts in LDS, thread e's scan,
// then wavefront 0's walk from position 0 of every expert.  The same results
// as the three launches (one chunk: every expert's chunk start is 0).
__global__ __launch_bounds__(256) void dispatch_small_kernel(
    const int32_t* __restrict__ idx, int T, int K, int N, int cap, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ n_dropped,
    int32_t* __restrict__ slot_row, int32_t* __restrict__ row_token) {
  __shared__ int hist[MAXN];
  __shared__ int off_s[MAXN];
  __shared__ int wsum[4];
  const int e = threadIdx.x;
  if (e < N) hist[e] = 0;
  __syncthreads();
  const int64_t pairs = (int64_t)T * K;
  for (int64_t p = threadIdx.x; p < pairs; p += blockDim.x) {
    const int x = idx[p];
    if (x >= 0 && x < N) atomicAdd(&hist[x], 1);
  }
  __syncthreads();
  const int run = e < N ? hist[e] : 0;
  if (e < N) counts[e] = run;
  expert_scan(e, run, N, cap, pairs, offsets, n_dropped, wsum);
  if (e < N) {
    off_s[e] = offsets[e];
    hist[e] = 0;              // the walk's running positions
  }
  __syncthreads();
  rank_walk(idx, 0, pairs, K, N, cap, hist, off_s, slot_row, row_token, threadIdx.x & 63,
            (threadIdx.x >> 6) == 0);
}

// One wavefront per token (its index made wave-uniform, so the slot rows are
// scalar loads); rows are copied as 16-byte units, up to U per lane loaded
// together before they are stored to each kept row.
template <int U>
__global__ __launch_bounds__(256) void permute_kernel(const uint4* __restrict__ x,
                                                      const int32_t* __restrict__ slot_row,
                                                      uint4* __restrict__ x_perm, int T, int K,
                                                      int row_vec) {
  const int t = __builtin_amdgcn_readfirstlane((int)(blockIdx.x * 4 + (threadIdx.x >> 6)));
  if (t >= T) return;
  const int lane = threadIdx.x & 63;
  const int32_t* sr = slot_row + (int64_t)t * K;
  bool any = false;
  for (int k = 0; k < K; ++k) any |= sr[k] >= 0;
  if (!any) return;
  const uint4* src = x + (int64_t)t * row_vec;
  // this lane's pieces are c = lane + 64 i, i < n
  const int n = (row_vec - lane + 63) / 64;
  for (int i0 = 0; i0 < n; i0 += U) {
    uint4 v[U];
    if (i0 + U <= n) {
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = src[lane + 64 * (i0 + u)];
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = (i0 + u < n) ? src[lane + 64 * (i0 + u)] : make_uint4(0, 0, 0, 0);
    }
    for (int k = 0; k < K; ++k) {
      const int r = sr[k];
      if (r < 0) continue;
      uint4* dst = x_perm + (int64_t)r * row_vec + lane;
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (i0 + u < n) dst[64 * (i0 + u)] = v[u];
    }
  }
}

// Tile list of a grouped GEMM (one workgroup; thread e owns expert e).
// Shared-problem tiles come first, then expert by expert.  Within an expert
// (or the shared problem) with mt m-tiles, tiles go in windows of about 32
// -- one XCD's worth of CUs: groups of gm = min(mt, 8) m-tiles by bands of
// max(1, 32 / gm) n-tiles, so the tiles of a window read each weight tile
// once and each activation panel once between them.
// Inside a band the tiles go m-tile by m-tile, and a last m-tile holding a
// folded remainder (more than BM rows, about 1.2 times a full tile's time)
// goes first.  An XCD hands each workgroup to the first CU that frees up,
// so a band's heavy tiles then land on the CUs that finished the previous
// band first; with the heavy tiles at the band's end they kept landing on
// the CUs that were already behind (a dispatch model of the Mixtral-shaped
// tile lists: 8.2 instead of 7.4 rounds of tiles for the first GEMM, 2.36
// instead of 2.18 for the second).  The order decides only when a tile
// runs, never what it computes.
__device__ __forceinline__ int4 band_tile(int j, int mt, int ntn, int BN, int e, int o0, int o1,
                                          int BM) {
  const int gm = min(mt, 8);
  const int g = j / (gm * ntn), r0 = j % (gm * ntn);       // m-group, index inside it
  const int gsz = min(gm, mt - g * gm);                      // m-tiles in this group
  const int band = max(1, 32 / gm);
  const int b = r0 / (band * gsz), r = r0 % (band * gsz);
  const int bw = min(band, ntn - b * band);                  // n-tiles in this band
  const int nt = b * band + r % bw;
  int mi = r / bw;                                           // m-tile inside the group
  const bool heavy_last = g * gm + gsz == mt && o1 - o0 - (mt - 1) * BM > BM;
  if (heavy_last) mi = mi == 0 ? gsz - 1 : mi - 1;
  const int i = g * gm + mi;
  // the last m-tile runs to the block's end (it may hold a folded remainder)
  return make_int4(e, o0 + i * BM, i == mt - 1 ? o1 : o0 + (i + 1) * BM, nt * BN);
}

// m-tiles of a block of `rows` rows; a last remainder of at most `merge` rows
// joins the previous full tile
__device__ __forceinline__ int m_tiles(int rows, int BM, int merge) {
  const int mt = (rows + BM - 1) / BM;
  return (mt >= 2 && rows - (mt - 1) * BM <= merge) ? mt - 1 : mt;
}

constexpr int TL_PER_WG = 2048;   // routed tiles written per workgroup

__global__ __launch_bounds__(256) void tile_list_kernel(const int32_t* __restrict__ offsets, int N,
                                                        int BM, int BN, int Nd, int Ts, int merge,
                                                        int wide_rows, int4* __restrict__ list,
                                                        int32_t* __restrict__ count) {
  __shared__ int wsum[4], s_nonuni;
  __shared__ int s_base[MAXN + 1], s_mt[MAXN], s_o0[MAXN], s_o1[MAXN], s_wide[MAXN];
  const int e = threadIdx.x;
  const int ntn = (Nd + BN - 1) / BN;
  if (e == 0) s_nonuni = 0;
  const int ms = m_tiles(Ts, BM, merge);
  const int shared_tiles = ms * ntn;
  int o0 = 0, o1 = 0, mt = 0, ntn_e = ntn;
  if (e < N) {
    o0 = offsets[e];
    o1 = offsets[e + 1];
    mt = m_tiles(o1 - o0, BM, merge);
    // a block of at most wide_rows rows: tiles of 2 BN columns
    const int wide = wide_rows > 0 && o1 - o0 <= wide_rows;
    if (wide) ntn_e = (Nd + 2 * BN - 1) / (2 * BN);
    s_mt[e] = mt;
    s_o0[e] = o0;
    s_o1[e] = o1;
    s_wide[e] = wide;
  }
  const int n = mt * ntn_e;
  const int lane = e & 63, wave = e >> 6;
  int v = n;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(v, o, 64);
    if (lane >= o) v += u;
  }
  if (lane == 63) wsum[wave] = v;
  __syncthreads();
  if (e < N && (s_mt[e] != s_mt[0] || s_wide[e] != s_wide[0])) s_nonuni = 1;
  int base = 0, total = 0;
  for (int w = 0; w < 4; ++w) {
    if (w < wave) base += wsum[w];
    total += wsum[w];
  }
  if (e < N) s_base[e] = base + v - n;
  if (e == 0) s_base[N] = total;
  __syncthreads();
  // every thread writes tiles: find the expert owning routed tile j (the last
  // expert whose first tile is <= j; experts without tiles share the next base).
  // Workgroup b writes tiles [b * TL_PER_WG, (b + 1) * TL_PER_WG); each
  // workgroup repeats the per-expert scan above (N <= 256 values).
  const int jend = min(total, (int)(blockIdx.x + 1) * TL_PER_WG);
  // Every expert with the same tile count (the same m-tiles and column
  // width): the list goes band by band across the experts (band 0 of every
  // expert, then band 1, ...) instead of expert by expert.  The list is cut
  // into one contiguous slice per XCD, so an XCD then runs bands of several
  // experts, and the bands holding a folded remainder (about 1.2 times a
  // full tile each) spread over the XCDs instead of filling the slices of
  // the experts that have one.  A band still runs on one XCD at once.
  const int mt0 = s_mt[0], wd0 = s_wide[0];
  const int ntn0 = wd0 ? (Nd + 2 * BN - 1) / (2 * BN) : ntn;
  const int gm0 = min(mt0, 8), band0 = max(1, 32 / max(gm0, 1));
  const bool uniform = N > 1 && !s_nonuni && mt0 > 0 &&
                       ((mt0 + gm0 - 1) / gm0) * ((ntn0 + band0 - 1) / band0) <= 512;
  for (int j = blockIdx.x * TL_PER_WG + threadIdx.x; j < jend; j += blockDim.x) {
    if (uniform) {
      // band k of expert x starts at N * (first local tile of band k) +
      // x * (size of band k)
      int rem = j, lb = 0, ex = 0, loc = 0;
      bool found = false;
      for (int g0 = 0; g0 < mt0 && !found; g0 += gm0) {
        const int gsz = min(gm0, mt0 - g0);
        for (int b0 = 0; b0 < ntn0 && !found; b0 += band0) {
          const int size = min(band0, ntn0 - b0) * gsz;
          if (rem < N * size) {
            ex = rem / size;
            loc = lb + rem % size;
            found = true;
          } else {
            rem -= N * size;
            lb += size;
          }
        }
      }
      list[shared_tiles + j] = band_tile(loc, mt0, ntn0, wd0 ? 2 * BN : BN,
                                         ex | (wd0 ? kWideTile : 0), s_o0[ex], s_o1[ex], BM);
      continue;
    }
    int lo = 0, hi = N - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_base[mid] <= j) lo = mid; else hi = mid - 1;
    }
    const int wd = s_wide[lo];
    list[shared_tiles + j] = band_tile(j - s_base[lo], s_mt[lo], ntn, wd ? 2 * BN : BN,
                                       lo | (wd ? kWideTile : 0), s_o0[lo], s_o1[lo], BM);
  }
  if (blockIdx.x == 0) {
    for (int j = threadIdx.x; j < shared_tiles; j += blockDim.x)
      list[j] = band_tile(j, ms, ntn, BN, -1, 0, Ts, BM);
    if (threadIdx.x == 0) count[0] = shared_tiles + total;
  }
}

}  // namespace

hipError_t launch_dispatch(const int32_t* topk_idx, const void* x, size_t row_bytes, int T, int K,
                           int N, int capacity, int32_t* counts, int32_t* offsets,
                           int32_t* slot_row, int32_t* row_token, void* x_perm,
                           int32_t* n_dropped, int32_t* blkcnt, int32_t* blkoff, hipStream_t s) {
  const int nblk = dispatch_blocks(T);
  const int cap = capacity > 0 ? capacity : 0x7fffffff;
  if (nblk == 1) {
    hipLaunchKernelGGL(dispatch_small_kernel, dim3(1), dim3(256), 0, s, topk_idx, T, K, N, cap,
                       counts, offsets, n_dropped, slot_row, row_token);
  } else {
    hipLaunchKernelGGL(hist_kernel, dim3(nblk), dim3(256), 0, s, topk_idx, T, K, N, blkcnt);
    hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(256), 0, s, blkcnt, nblk, N, cap,
                       (int64_t)T * K, blkoff, counts, offsets, n_dropped);
    hipLaunchKernelGGL(rank_kernel, dim3(nblk), dim3(64), 0, s, topk_idx, T, K, N, cap, blkoff,
                       offsets, slot_row, row_token);
  }
  // the pieces a lane copies per row, all in one batch when they fit in 16
  const int row_vec = (int)(row_bytes / 16), per_lane = (row_vec + 63) / 64;
  const uint4* xs = static_cast<const uint4*>(x);
  uint4* xd = static_cast<uint4*>(x_perm);
  const dim3 pg((T + 3) / 4), pb(256);
  if (per_lane <= 4)
    hipLaunchKernelGGL(permute_kernel<4>, pg, pb, 0, s, xs, slot_row, xd, T, K, row_vec);
  else if (per_lane <= 8)
    hipLaunchKernelGGL(permute_kernel<8>, pg, pb, 0, s, xs, slot_row, xd, T, K, row_vec);
  else
    hipLaunchKernelGGL(permute_kernel<16>, pg, pb, 0, s, xs, slot_row, xd, T, K, row_vec);
  return hipGetLastError();
}

hipError_t launch_tile_list(const int32_t* offsets, int N, int BM, int BN, int Nd, int Ts,
                            int merge, int64_t max_tiles, int4* list, int32_t* count,
                            hipStream_t s, int wide_rows) {
  const unsigned nwg = (unsigned)((max_tiles + TL_PER_WG - 1) / TL_PER_WG);
  hipLaunchKernelGGL(tile_list_kernel, dim3(nwg < 1 ? 1 : nwg), dim3(256), 0, s, offsets, N, BM,
                     BN, Nd, Ts, merge, wide_rows, list, count);
  return hipGetLastError();
}

}  // namespace moe
