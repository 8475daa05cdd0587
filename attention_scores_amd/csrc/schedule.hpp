// schedule.hpp -- workgroup -> output-tile map (the operand-reuse scheduler).
//
// Output tiles of one grid row consume the same A row-panel and those of one
// grid column the same B column-panel; the pages fan such a shared tile out
// to all its consumers from a single fetch (lesson 07 "Clusters, distributed
// shared memory & cluster launch control", section "TMA multicast -- one
// load, many CTAs": the tile scheduler groups tiles that share operands).
// gfx950 has no multicast, so the reuse must come from the caches: consumers
// of one panel are made to run at the same time on the same XCD, whose
// private L2 then serves every consumer after the first.
//
// Two facts of the MI355X dispatcher are used (both measured with a probe
// kernel reading HW_REG_XCC_ID): the 8 XCDs receive workgroups round-robin,
// so hardware workgroup id h runs on XCD h mod 8; and workgroups start in id
// order, so the (h div 8)-th workgroup of an XCD runs in its (h div 8)-th slot.
//
// Map, for a grid of `tiles` workgroups:
//   1. XCD split: XCD x owns the contiguous logical range
//      [x*q + min(x, r), ...) of q or q+1 tiles (q = tiles div 8,
//      r = tiles mod 8); slot s of XCD x takes logical tile x*q + min(x,r) + s.
//   2. Grouped order inside a batch: logical tiles walk a band of group_m
//      tile rows column by column, so the ~32 tiles an XCD runs at once span
//      group_m A row-panels and 32/group_m B column-panels.
// With grouping off (the ablation) the map is the identity in row-major
// tile order.  The map is a bijection on [0, tiles).
#pragma once

#include <hip/hip_runtime.h>

namespace asl {

constexpr int kXcds = 8;

template <typename I>
__host__ __device__ inline void remap_tile(I h, I tiles, I tiles_m, I tiles_n, I group_m, bool grouped,
                                           I& b, I& tm, I& tn) {
    I L = h;
    if (grouped) {
        I xcd = h % kXcds, slot = h / kXcds, q = tiles / kXcds, r = tiles % kXcds;
        L = xcd * q + (xcd < r ? xcd : r) + slot;
    }
    I per_b = tiles_m * tiles_n;
    b = L / per_b;
    I t = L - b * per_b;
    if (grouped) {
        I width = group_m * tiles_n;
        I gid = t / width;
        I first = gid * group_m;
        I gsz = (tiles_m - first) < group_m ? (tiles_m - first) : group_m;
        I in = t - gid * width;
        tm = first + in % gsz;
        tn = in / gsz;
    } else {
        tm = t / tiles_n;
        tn = t - tm * tiles_n;
    }
}

}  // namespace asl
