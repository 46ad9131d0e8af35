// tile_map.h -- workgroup id -> output tile, aware of the MI355X's 8 XCDs.
#pragma once

#include <stdint.h>
#include <stdlib.h>

#include <hip/hip_runtime.h>

#include "conv_params.h"

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

// Logical tile t -> (m tile, n tile).  With ng <= 0 or ng >= n_tiles the n
// tiles of one m tile are consecutive (m tile outer).  Otherwise the n tiles
// go in groups of ng: the logical order runs over every m tile for the first
// group's ng n tiles, then for the next group, and so on.  Consecutive
// logical tiles run at the same time on one XCD and share its L2, so a
// narrow group makes the tiles in flight together share few filter columns
// (which stream through the L2 once per round) and many input rows.
struct TileRC {
    int mt, nt;
};

__host__ __device__ __forceinline__ TileRC grouped_tile(int t, int m_tiles, int n_tiles, int ng)
{
    TileRC rc;
    if (ng <= 0 || ng >= n_tiles) {
        rc.mt = t / n_tiles;
        rc.nt = t - rc.mt * n_tiles;
        return rc;
    }
    const int gsz = m_tiles * ng;                  // tiles of one full group
    const int g = t / gsz;
    const int r = t - g * gsz;
    const int wdt = n_tiles - g * ng < ng ? n_tiles - g * ng : ng;   // the last group may be narrower
    rc.mt = r / wdt;
    rc.nt = g * ng + (r - rc.mt * wdt);
    return rc;
}

// Group width for grouped_tile (host).  Model of the bytes an XCD's 4 MB L2
// misses: each XCD runs z = 32 CUs x wg_per_cu tiles at a time, a round of z
// consecutive tiles being z/ng m tiles x ng n tiles; a round reads its ng
// slices of the filter and its z/ng slices of the input once, so over the
// m_tiles * n_tiles / z rounds
//   traffic(ng) = m_tiles * ng * w_bytes / z + n_tiles * x_bytes / ng.
// Filters that fit in half an L2 stay there after the first round: then one
// group (ng = n_tiles, the input read once).  MIC_N_GROUP=<ng> (environment)
// overrides the choice (tuning runs; every choice computes the same result).
inline int choose_n_group(const ConvParams& p, int64_t x_bytes, int64_t w_bytes, int wg_per_cu)
{
    if (const char* e = getenv("MIC_N_GROUP")) {
        const int v = atoi(e);
        if (v > 0) return v;
    }
    if (p.n_tiles <= 1 || w_bytes <= (int64_t)2 << 20) return 0;
    const double z = 32.0 * (wg_per_cu > 0 ? wg_per_cu : 1);
    int best = 0;
    double best_t = 0;
    for (int ng = 1; ng <= p.n_tiles; ++ng) {
        const double t = (double)p.m_tiles * ng * (double)w_bytes / z + (double)p.n_tiles * (double)x_bytes / ng;
        if (best == 0 || t < best_t) {
            best = ng;
            best_t = t;
        }
    }
    return best >= p.n_tiles ? 0 : best;
}

}  // namespace miconv
