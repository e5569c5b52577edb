// Tile scheduling shared by the tiled grouped-GEMM kernels.
//
// A grouped GEMM runs C = A . W_e^T over the ragged row blocks of the routed
// experts (their starts come from the device-side tile map, so no host
// synchronisation is needed) plus, optionally, one dense "shared" problem.
// The m-tiles are numbered shared first, then routed; each m-tile pairs with
// every n-tile.  The grid is sized for the worst case and surplus workgroups
// exit at once.
//
// Order: the hardware hands workgroup b to XCD (b mod 8), and each XCD has
// its own L2.  The active tiles are split into 8 contiguous ranges, one per
// XCD, so that the tiles an XCD runs at the same time are neighbours; inside
// a range, tiles go in groups of GM m-tiles by all n-tiles (m fastest), so
// concurrently running tiles share A rows and weight rows in that L2.
#pragma once

#include "moe_internal.h"

namespace moe {

struct TileRef {
  bool valid;
  bool shared;
  int e;        // expert (routed tiles)
  int row0;     // first row of the tile
  int row_end;  // one past the last valid row
  int n0;       // first output column
};

template <int BM, int BN, int GM = 8>
__device__ __forceinline__ TileRef map_tile(const GemmArgs& a) {
  TileRef r;
  r.valid = false;
  r.shared = false;
  r.e = 0;
  r.row0 = r.row_end = r.n0 = 0;
  const int ntn = (a.Nd + BN - 1) / BN;
  const int Ms = a.As ? (a.Ts + BM - 1) / BM : 0;
  const int Mr = a.tile_map ? a.tile_count[0] : 0;
  const int Mt = Ms + Mr;
  const int total = Mt * ntn;
  const int xcd = blockIdx.x & 7;
  const int slot = blockIdx.x >> 3;
  const int per = total >> 3, extra = total & 7;
  if (slot >= per + (xcd < extra ? 1 : 0)) return r;
  const int L = xcd * per + min(xcd, extra) + slot;
  const int g = L / (GM * ntn);
  const int first_m = g * GM;
  const int gsz = min(GM, Mt - first_m);
  const int Lin = L - g * GM * ntn;
  const int mt = first_m + Lin % gsz;
  const int nt = Lin / gsz;
  r.valid = true;
  r.n0 = nt * BN;
  if (mt < Ms) {
    r.shared = true;
    r.row0 = mt * BM;
    r.row_end = min(r.row0 + BM, a.Ts);
  } else {
    const int2 tm = a.tile_map[mt - Ms];
    r.e = tm.x;
    r.row0 = tm.y;
    r.row_end = min(r.row0 + BM, a.offsets[tm.x + 1]);
  }
  return r;
}

// Workgroups to launch for a grouped GEMM with BM x BN tiles.
inline int gemm_grid(const GemmArgs& a, int BM, int BN) {
  const int ntn = (a.Nd + BN - 1) / BN;
  const int Ms = a.As ? (a.Ts + BM - 1) / BM : 0;
  const int Mr = a.tile_map ? a.max_tiles : 0;
  const long total = (long)(Ms + Mr) * ntn;
  return (int)(((total + 7) / 8) * 8);
}

}  // namespace moe
