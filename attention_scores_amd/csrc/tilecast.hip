// tilecast.hip -- tile fan-out microbenchmark for gfx950.
//
// The "Hopper TMA Multicast" deep-dive (sections "Microbenchmark source" and
// "run results") measures how often one 128x64 16-bit tile is fetched when
// several thread blocks consume it: unicast has every consumer issue its own
// load, multicast has one load fanned out by the cluster fabric.  Here every
// consumer always issues its own 128-bit loads (gfx950 has no fabric that
// writes one fetch into several CUs' LDS); what changes is WHERE the
// consumers of one tile run:
//   grouped   the `group` consumers of a tile share one XCD, so the first
//             fetch fills that XCD's L2 and the others hit in it -- HBM/EA
//             traffic per consumer falls towards tile/group;
//   ungrouped consumers of a tile are consecutive workgroup ids, which the
//             dispatcher spreads over different XCDs, so each XCD's L2
//             misses on its own and fetches the tile again.
// The L2 -> CU leg is one transfer per consumer in both arms: that part of
// the multicast saving has no gfx950 counterpart.
//
// Per iteration each workgroup loads its tile with global_load_dwordx4 into
// registers, adds every 32-bit word into a running checksum, writes the tile
// to LDS and waits at a workgroup barrier (the deep-dive's kernels wait on
// their barrier every iteration).  At the end it stores the running checksum
// and the sum of the tile left in LDS.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "internal.hpp"

namespace asl {
namespace kern {

constexpr int kTcThreads = 256;
constexpr int kTcMaxBytes = 65536;

struct TcArgs {
    const uint4* buf;
    int64_t cols_chunks;       // row length in 16-byte chunks
    int32_t tiles_x, tiles_y;  // tile grid
    int32_t tile_m, tile_chunks_x;
    int32_t consumers, group, grouped;
    int64_t iters, stride;
    uint32_t* out;
};

__device__ __forceinline__ uint32_t words(uint4 v) { return v.x + v.y + v.z + v.w; }

__global__ void __launch_bounds__(kTcThreads) tilecast_kernel(TcArgs a) {
    __shared__ uint4 tile[kTcMaxBytes / 16];
    __shared__ uint32_t red[kTcThreads];
    const int tid = threadIdx.x;
    const int w = blockIdx.x;
    int g;
    if (a.grouped) {
        const int per_xcd = a.consumers / 8;
        g = (w % 8) * (per_xcd / a.group) + (w / 8) / a.group;
    } else {
        g = w / a.group;
    }
    const int nchunks = a.tile_m * a.tile_chunks_x;
    uint32_t sum = 0;
    for (int64_t it = 0; it < a.iters; ++it) {
        const int64_t t = it * a.stride + g;
        const int64_t c0 = (t % a.tiles_x) * a.tile_chunks_x;
        const int64_t r0 = ((t / a.tiles_x) % a.tiles_y) * a.tile_m;
        const uint4* src = a.buf + r0 * a.cols_chunks + c0;
        for (int q = tid; q < nchunks; q += kTcThreads) {
            const int r = q / a.tile_chunks_x, c = q - r * a.tile_chunks_x;
            uint4 v = src[(int64_t)r * a.cols_chunks + c];
            sum += words(v);
            tile[q] = v;
        }
        __syncthreads();
    }
    uint32_t last = 0;
    for (int q = tid; q < nchunks; q += kTcThreads) last += words(tile[q]);
    red[tid] = sum;
    __syncthreads();
    if (tid == 0) {
        uint32_t s = 0;
        for (int i = 0; i < kTcThreads; ++i) s += red[i];
        a.out[2 * w] = s;
    }
    __syncthreads();
    red[tid] = last;
    __syncthreads();
    if (tid == 0) {
        uint32_t s = 0;
        for (int i = 0; i < kTcThreads; ++i) s += red[i];
        a.out[2 * w + 1] = s;
    }
}

}  // namespace kern

using namespace kern;

int launch_tilecast(const TilecastDesc& d, void* stream) {
    TcArgs a;
    a.buf = (const uint4*)d.buf;
    a.cols_chunks = d.cols / 8;
    a.tiles_x = (int32_t)(d.cols / d.tile_n);
    a.tiles_y = (int32_t)(d.rows / d.tile_m);
    a.tile_m = d.tile_m;
    a.tile_chunks_x = d.tile_n / 8;
    a.consumers = d.consumers;
    a.group = d.group;
    a.grouped = d.grouped;
    a.iters = d.iters;
    a.stride = d.stride;
    a.out = d.out;
    hipLaunchKernelGGL(tilecast_kernel, dim3((unsigned)d.consumers), dim3(kTcThreads), 0, (hipStream_t)stream, a);
    return (int)hipGetLastError();
}

}  // namespace asl
