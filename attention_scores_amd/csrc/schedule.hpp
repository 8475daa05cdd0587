// schedule.hpp -- which output tiles a workgroup computes, in which order
// (the operand-reuse scheduler).
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
// order.
//
// The grid may be persistent (fewer workgroups than tiles, each walking
// several tiles -- the static persistent schedule of the same lesson,
// section "The second wall: the static schedule's tail").  With P
// workgroups:
//   1. XCD split: XCD x owns the contiguous logical range
//      [x*q + min(x, r), ...) of q or q+1 tiles (q = tiles div 8,
//      r = tiles mod 8).  Its workgroups (ids h = x mod 8, the s-th one being
//      h = 8s + x) take the range's tiles s, s + n, s + 2n, ... where n is
//      the number of workgroups on XCD x; so at any moment an XCD runs a run
//      of consecutive logical tiles.
//   2. Grouped order inside a batch: logical tiles walk a band of group_m
//      tile rows column by column, so the ~32 tiles an XCD runs at once span
//      group_m A row-panels and 32/group_m B column-panels.
// Two ablations: with grouping off, workgroup h takes tiles h, h + P, ... in
// row-major tile order; without the XCD split (step 1 skipped), workgroup h
// takes logical tiles h, h + P, ... of the grouped order of step 2, so
// consecutive tiles of a band run on different XCDs (the band order of a
// GPU whose workgroups all share one L2).  Every tile is visited exactly
// once.
#pragma once

#include <hip/hip_runtime.h>

namespace asl {

constexpr int kXcds = 8;

// Logical tile range owned by XCD x.
template <typename I>
__host__ __device__ inline void xcd_range(I x, I tiles, I& start, I& count) {
    const I q = tiles / kXcds, r = tiles % kXcds;
    start = x * q + (x < r ? x : r);
    count = q + (x < r ? 1 : 0);
}

// Logical tile L -> (batch, tile row, tile column).
template <typename I>
__host__ __device__ inline void logical_tile(I L, I tiles_m, I tiles_n, I group_m, bool grouped, I& b, I& tm,
                                             I& tn) {
    const I per_b = tiles_m * tiles_n;
    b = L / per_b;
    const I t = L - b * per_b;
    if (grouped) {
        const I width = group_m * tiles_n;
        const I gid = t / width;
        const I first = gid * group_m;
        const I gsz = (tiles_m - first) < group_m ? (tiles_m - first) : group_m;
        const I in = t - gid * width;
        tm = first + in % gsz;
        tn = in / gsz;
    } else {
        tm = t / tiles_n;
        tn = t - tm * tiles_n;
    }
}

// Logical tiles workgroup h of a P-workgroup grid visits: first, first +
// stride, ... while < end.  xcd_split: each XCD walks its own range (step 1).
template <typename I>
__host__ __device__ inline void tile_walk(I h, I P, I tiles, bool xcd_split, I& first, I& stride, I& end) {
    if (!xcd_split) {
        first = h;
        stride = P;
        end = tiles;
        return;
    }
    const I x = h % kXcds, s = h / kXcds;
    I start, count;
    xcd_range<I>(x, tiles, start, count);
    first = start + s;
    stride = P / kXcds + (x < P % kXcds ? 1 : 0);
    end = start + count;
}

// Tile computed in execution slot i = j*P + h (round j of workgroup h), for
// i < tiles; returns false if that slot is empty.  Slot i runs on XCD i mod 8
// when P is a multiple of 8 or P == tiles.
template <typename I>
__host__ __device__ inline bool tile_of_slot(I i, I P, I tiles, I tiles_m, I tiles_n, I group_m, bool grouped,
                                             bool xcd_split, I& b, I& tm, I& tn) {
    const I h = i % P, j = i / P;
    I first, stride, end;
    tile_walk<I>(h, P, tiles, xcd_split, first, stride, end);
    const I L = first + j * stride;
    if (L >= end) return false;
    logical_tile<I>(L, tiles_m, tiles_n, group_m, grouped, b, tm, tn);
    return true;
}

}  // namespace asl
