// fa_schedule.hpp -- which workgroup does which tiles.
//
// Every kernel runs a 1-D grid of units; these functions map a workgroup
// index to its (batch*head, unit) and a unit to its query or key tiles, and
// size the forward grid.  They are __host__ __device__ so that a host program
// can enumerate a whole grid and check that every tile is issued exactly once.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// Unit schedule of a 1-D grid of `total` = heads * per_head workgroups.
// Workgroup i runs on XCD i % 8.  XCD x takes heads x, x + 8, x + 16, ... in
// order, all units of a head together, so one head's K/V re-reads stay in
// one XCD's L2, and heads of unequal work (the sequences of a packed batch
// are consecutive heads) spread evenly over the eight XCDs.
__host__ __device__ __forceinline__ void unit_of(int i, int total, int per_head, int& head,
                                                 int& idx) {
    const int heads = total / per_head;
    if ((heads & 7) == 0) {
        const int s = i >> 3, k = s / per_head;
        head = (i & 7) + 8 * k;
        idx = s - k * per_head;
    } else {
        head = i / per_head;
        idx = i - head * per_head;
    }
}

// Causal schedule with a split tail.  Units of equal work (pairs of a light
// and a heavy tile) finish at scattered times, so the last round of a plain
// pair schedule ends raggedly.  Here XCD x still takes heads x, x + 8, ... in
// order, all units of a head together (heads % 8 == 0), but its last `tail`
// heads come as single tiles ordered from the heaviest down, which fills the
// end of the launch with ever smaller units.  Returns the head and either the
// pair index (rank < 0) or the single tile's rank from the heaviest
// (rank >= 0).
__host__ __device__ __forceinline__ void tail_unit(int i, int heads, int per_head, int tail,
                                                   int& head, int& uidx, int& rank) {
    const int x = i & 7, s = i >> 3;
    const int hx = heads >> 3;                      // heads per XCD
    const int lead = (hx - tail) * per_head;        // pair units before the tail
    if (s < lead) {
        const int k = s / per_head;
        head = x + 8 * k;
        uidx = s - k * per_head;
        rank = -1;
    } else {
        const int s2 = s - lead;
        head = x + 8 * (hx - tail + s2 % tail);
        uidx = 0;
        rank = s2 / tail;
    }
}

// Tiles of unit `uidx` of a sequence of n_tiles tiles.  Without pairing the
// unit is tile uidx.  With pairing (causal masking) it is the light tile
// uidx and the heavy tile n_tiles - 1 - uidx, so every unit carries about
// the same work; t0 is the heavy one if heavy_first, else the light one, and
// t1 = -1 when both are the same middle tile.  Returns false when the unit
// has no tile (past the end, or past the middle of the pairs).
__host__ __device__ __forceinline__ bool unit_tiles(bool pairs, bool heavy_first, int uidx,
                                                    int n_tiles, int& t0, int& t1) {
    if (!pairs) {
        t0 = uidx;
        t1 = -1;
        return uidx < n_tiles;
    }
    const int light = uidx, heavy = n_tiles - 1 - uidx;
    if (light > heavy) return false;
    t0 = heavy_first ? heavy : light;
    t1 = light == heavy ? -1 : (heavy_first ? light : heavy);
    return true;
}

// Query tiles of a forward unit: a single tile of the split tail (rank >= 0,
// counted from the heaviest), else the unit's pair or tile (heavy first; the
// forward kernel walks the keys of a pair's second, light tile downwards).
__host__ __device__ __forceinline__ bool fwd_tiles(bool pairs, int rank, int uidx, int n_tiles,
                                                   int& t0, int& t1) {
    if (rank >= 0) {
        t0 = n_tiles - 1 - rank;
        t1 = -1;
        return t0 >= 0;
    }
    return unit_tiles(pairs, true, uidx, n_tiles, t0, t1);
}

// Grid of the dense causal forward for `heads` = B*H heads of n_qt query
// tiles (per_head = ceil(n_qt / 2) pair units each).  With heads % 8 == 0,
// about one round of an XCD's 64 workgroup slots comes as single tiles: the
// last `tail` heads of each XCD.  Otherwise tail = 0 and the grid is the
// plain heads * per_head pairs.
struct FwdGrid {
    int tail;
    int64_t units;
};

inline FwdGrid fwd_causal_grid(int heads, int n_qt) {
    const int per_head = (n_qt + 1) / 2;
    if ((heads & 7) != 0) return {0, (int64_t)heads * per_head};
    const int hx = heads >> 3;
    const int tail = hx < (64 + per_head - 1) / per_head ? hx : (64 + per_head - 1) / per_head;
    return {tail, 8 * ((int64_t)(hx - tail) * per_head + (int64_t)tail * n_qt)};
}

}  // namespace fa
