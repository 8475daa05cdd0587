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

#include <cstdint>

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

// Unsigned division by a divisor fixed for a whole launch, for dividends
// below 2^31.  With l = ceil(log2 d) and m = floor(2^32 (2^l - d) / d) + 1,
// n div d = (n + mulhi(m, n)) >> l (Granlund and Montgomery, "Division by
// invariant integers using multiplication", PLDI 1994, section 4, the
// unsigned case); mulhi(m, n) < n, so the sum stays below 2^32.  On the
// device a division by a run-time value is a loop of about forty scalar
// instructions; this is three.
struct DivU31 {
    uint32_t m, l;
    // 1 <= d < 2^31 (host).
    static DivU31 of(uint32_t d) {
        uint32_t l = 0;
        while ((uint64_t(1) << l) < d) ++l;
        return DivU31{(uint32_t)(((uint64_t(1) << 32) * ((uint64_t(1) << l) - d)) / d + 1), l};
    }
    __host__ __device__ uint32_t div(uint32_t n) const {
        return ((uint32_t)(((uint64_t)n * m) >> 32) + n) >> l;
    }
};

// logical_tile of one launch with its divisors prepared on the host: the
// form the kernels evaluate at every tile they visit (and gemm_plan_tile_of
// on the host).  Needs tiles_m * tiles_n * batch < 2^31 and
// group_m <= tiles_m, which the planner guarantees.
struct TileMap {
    int32_t tiles_m, tiles_n, group_m, grouped;
    DivU31 per_b, width, group, group_tail, cols;   // divisors tiles_m*tiles_n, group_m*tiles_n, group_m,
                                                    // tiles_m mod group_m (the last band, if partial), tiles_n
    static TileMap of(int64_t tiles_m, int64_t tiles_n, int64_t group_m, bool grouped) {
        TileMap t;
        t.tiles_m = (int32_t)tiles_m;
        t.tiles_n = (int32_t)tiles_n;
        t.group_m = (int32_t)group_m;
        t.grouped = grouped ? 1 : 0;
        t.per_b = DivU31::of((uint32_t)(tiles_m * tiles_n));
        t.width = DivU31::of((uint32_t)(group_m * tiles_n));
        t.group = DivU31::of((uint32_t)group_m);
        t.group_tail = DivU31::of(tiles_m % group_m ? (uint32_t)(tiles_m % group_m) : 1u);
        t.cols = DivU31::of((uint32_t)tiles_n);
        return t;
    }
    __host__ __device__ void coords(uint32_t L, int& b, int& tm, int& tn) const {
        const uint32_t bq = per_b.div(L);
        const uint32_t t = L - bq * (uint32_t)(tiles_m * tiles_n);
        b = (int)bq;
        if (grouped) {
            const uint32_t gid = width.div(t);
            const uint32_t first = gid * (uint32_t)group_m;
            const uint32_t in = t - gid * (uint32_t)(group_m * tiles_n);
            const bool tail = (uint32_t)tiles_m - first < (uint32_t)group_m;
            const uint32_t gsz = tail ? (uint32_t)tiles_m - first : (uint32_t)group_m;
            const uint32_t q = (tail ? group_tail : group).div(in);
            tm = (int)(first + (in - q * gsz));
            tn = (int)q;
        } else {
            const uint32_t q = cols.div(t);
            tm = (int)q;
            tn = (int)(t - q * (uint32_t)tiles_n);
        }
    }
};

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

}  // namespace asl
