// tile_map.h -- workgroup id -> output tile, aware of the MI355X's 8 XCDs.
#pragma once

#include <hip/hip_runtime.h>

namespace miconv {

// The dispatcher hands workgroup ids to the 8 XCDs round-robin (id % 8).
// This bijection on [0, tiles) gives each XCD one contiguous run of logical
// tile ids, so the tiles that share input rows (same m tile, every n tile)
// land on the same XCD and its L2.
//
// rev != 0 runs the tiles in the opposite order (tile t -> tiles - 1 - t):
// every tile is still computed exactly once, by another workgroup and at
// another time, so a result that changes under it exposes a dependence
// between workgroups or a race on shared memory.  Only tests set it.
__host__ __device__ __forceinline__ int xcd_logical_tile(int bid, int tiles, int rev = 0)
{
    const int xcd = bid & 7;
    const int loc = bid >> 3;
    const int per = tiles >> 3;
    const int extra = tiles & 7;          // the first `extra` XCDs get one more tile
    const int t = xcd < extra ? xcd * (per + 1) + loc
                              : extra * (per + 1) + (xcd - extra) * per + loc;
    return rev ? tiles - 1 - t : t;
}

}  // namespace miconv
