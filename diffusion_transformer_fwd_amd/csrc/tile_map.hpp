// Workgroup -> (problem, tile) map of a grouped GEMM launch, shared by the
// kernel and host-side checks (plain C++, no HIP dependency).
//
// The hardware hands the workgroups of a launch to the 8 XCDs round-robin by
// launch index: XCD x receives blocks x, x + 8, x + 16, ... in that order.
// Each XCD has its own L2, so the tiles an XCD runs together should share A
// and W panels, and every XCD should get the same mix of tile sizes. The map
// therefore deals every problem out separately: problem p's n_p tiles are
// cut into 8 contiguous ranges, one per XCD, of n_p / 8 tiles plus one more
// for the XCDs of a cyclic window of n_p % 8 XCDs that starts where the
// previous problems' windows ended. XCD x runs its range of problem 0, then
// its range of problem 1, ... . The windows of all problems together cover
// every XCD floor(sum / 8) times plus the first sum % 8 XCDs once more, which
// is exactly the count round-robin dealing gives each XCD, so the map is a
// bijection from launch indices onto tiles.
#pragma once

#ifndef DIT_HD
#if defined(__HIPCC__)
#define DIT_HD __host__ __device__
#else
#define DIT_HD
#endif
#endif

namespace dit {

// tiles_of(i): tile count of problem i < count (count <= MAXP). On return
// *problem and *tile name the tile of launch index `block`; returns false if
// `block` maps to no tile (only for block >= the sum of the counts).
template <int MAXP, class TilesOf>
DIT_HD inline bool tile_of_block(const TilesOf& tiles_of, int count, int block, int* problem,
                                 int* tile) {
  const int x = block & 7;
  int k = block >> 3;
  int start = 0;  // first XCD of the current problem's window
#if defined(__HIPCC__)
#pragma unroll
#endif
  for (int i = 0; i < MAXP; ++i) {
    if (i >= count) break;
    const int n = tiles_of(i), q = n >> 3, r = n & 7;
    const int share = q + ((((x - start) & 7) < r) ? 1 : 0);
    if (k < share) {
      // XCDs y < x inside the window [start, start + r) (mod 8)
      const int e = start + r;
      int before = x - start < 0 ? 0 : (x - start < r ? x - start : r);
      if (e > 8) before += x < e - 8 ? x : e - 8;
      *problem = i;
      *tile = x * q + before + k;
      return true;
    }
    k -= share;
    start = (start + r) & 7;
  }
  return false;
}

}  // namespace dit
