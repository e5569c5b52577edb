// Tile scheduling shared by the tiled grouped-GEMM kernels.
//
// A grouped GEMM runs C = A . W_e^T over the ragged row blocks of the routed
// experts plus, optionally, one dense "shared" problem.  The tiles come from
// a device-side tile list (built after dispatch, so no host synchronisation
// is needed); the grid is sized for the worst case and surplus workgroups
// exit at once.
//
// Order: the hardware hands workgroup b to XCD (b mod 8), and each XCD has
// its own L2.  The list is cut into 8 contiguous slices, one per XCD, so the
// tiles an XCD runs at the same time are neighbours in the list; the list
// runs expert by expert, each expert in bands of n-tiles whose tiles
// together fill about one XCD (see the tile-list kernel), so tiles running
// together share the expert's activation rows and weight rows in that L2.
#pragma once

#include "moe_internal.h"

namespace moe {

struct TileRef {
  bool valid;
  bool shared;
  bool wide;    // 2 BN columns (tile lists built with wide_rows)
  int e;        // expert (routed tiles)
  int row0;     // first row of the tile
  int row_end;  // one past the last valid row
  int n0;       // first output column
};

__device__ __forceinline__ TileRef map_tile(const GemmArgs& a) {
  TileRef r;
  r.valid = false;
  r.shared = false;
  r.wide = false;
  r.e = 0;
  r.row0 = r.row_end = r.n0 = 0;
  const int total = a.tile_count[0];
  const int xcd = blockIdx.x & 7;
  const int slot = blockIdx.x >> 3;
  const int per = total >> 3, extra = total & 7;
  if (slot >= per + (xcd < extra ? 1 : 0)) return r;
  const int L = xcd * per + min(xcd, extra) + slot;
  const int4 t = a.tile_list[L];
  r.valid = true;
  r.shared = t.x < 0;
  r.wide = t.x >= 0 && (t.x & kWideTile);
  r.e = t.x < 0 ? 0 : (t.x & (kWideTile - 1));
  r.row0 = t.y;
  r.row_end = t.z;
  r.n0 = t.w;
  return r;
}

// Workgroups to launch: the tile bound rounded up to a multiple of 8.
inline int gemm_grid(const GemmArgs& a) { return (int)(((a.grid_tiles + 7) / 8) * 8); }

}  // namespace moe
