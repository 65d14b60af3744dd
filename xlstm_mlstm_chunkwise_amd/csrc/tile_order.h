// Placement of a workgroup's tile on the chip (gfx950: eight XCDs, each
// with its own L2).
#pragma once
#include <hip/hip_runtime.h>

namespace mlstm {

// Tile index (x, y) of this workgroup over a 2-D grid, placed so that
// neighbouring tiles (consecutive x, and the y slices of one x, y fastest)
// run on one XCD at about the same time: tiles of one chunk stage the same
// keys, values, states or partner tiles, which that XCD's L2 then serves.
// The hardware deals workgroups to the eight XCDs round-robin in launch
// order, so consecutive launch indices would land on different XCDs.
struct TileIdx {
  int x, y;
};
__device__ __forceinline__ TileIdx xcd_tile() {
  const unsigned long long gy = gridDim.y, n = (unsigned long long)gridDim.x * gy;
  unsigned long long lin = blockIdx.x + blockIdx.y * (unsigned long long)gridDim.x;
  if ((n & 7) == 0) lin = (lin & 7) * (n >> 3) + (lin >> 3);
  return {(int)(lin / gy), (int)(lin % gy)};
}

}  // namespace mlstm
