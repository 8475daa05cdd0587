// splitk.hip -- the reduction step of a GEMM split over K (gfx950): the
// product kernel writes one fp32 partial product per K chunk into a
// workspace, and this kernel adds them, in chunk order, into C.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <mutex>

#include "internal.hpp"
#include "schedule.hpp"
#include "tile.hpp"

namespace asl {
namespace kern {

// Split-K reduction: C[i][j] = ws[0][i][j] + ws[1][i][j] + ... in chunk
// order, rounded to C's type.  Thread t takes the 4 consecutive columns of
// group t mod `groups` of row t div `groups` (one 16-byte load per chunk: ws
// rows are a multiple of 4 floats; the division by the launch constant is
// a multiply-high, DivU31), with two chunks' loads in flight at a time; the
// last group of a row stores only its columns below N.  Memory-bound: 4
// bytes read per chunk and element, 2 or 4 written.
template <bool OUT_BF16>
__global__ void __launch_bounds__(256) splitk_reduce_kernel(const float* __restrict__ ws, void* __restrict__ C,
                                                            int32_t N, DivU31 rows, int32_t groups, int32_t total,
                                                            int64_t ws_ld, int64_t ws_bs, int64_t c_ld, int32_t splits) {
    const int32_t t = blockIdx.x * 256 + threadIdx.x;
    if (t >= total) return;
    const int32_t i = (int32_t)rows.div((uint32_t)t), j = (t - i * groups) * 4;
    const float* p = ws + (int64_t)i * ws_ld + j;
    f32x4 acc = __builtin_nontemporal_load((const f32x4*)p);
    int32_t c = 1;
    for (; c + 2 < splits + 1; c += 2) {
        const f32x4 v0 = __builtin_nontemporal_load((const f32x4*)(p + c * ws_bs));
        const f32x4 v1 = __builtin_nontemporal_load((const f32x4*)(p + (c + 1) * ws_bs));
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = (acc[e] + v0[e]) + v1[e];
    }
    if (c < splits) {
        const f32x4 v = __builtin_nontemporal_load((const f32x4*)(p + c * ws_bs));
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] += v[e];
    }
    const int64_t o = (int64_t)i * c_ld + j;
    if (j + 4 <= N) {
        if constexpr (OUT_BF16) {
            typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
            bf16x4 y;
#pragma unroll
            for (int e = 0; e < 4; ++e) y[e] = (__bf16)acc[e];
            *((bf16x4*)((__bf16*)C + o)) = y;
        } else {
            *((f32x4*)((float*)C + o)) = acc;
        }
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (j + e < N) {
                if constexpr (OUT_BF16) ((__bf16*)C)[o + e] = (__bf16)acc[e];
                else ((float*)C)[o + e] = acc[e];
            }
    }
}

// Split-K workspace for callers that cannot allocate device memory
// (gemm_run_no_alloc): one array per GPU, which the GPU holds from the
// loading of the code object until the process ends.  Host code must never
// pass the name itself to a kernel (on the host it is only a stand-in, not
// the device address): scratch_address() looks up each device's address.
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

}  // namespace kern

int scratch_address(void** out) {
    // Device addresses of the array, looked up once per device with that
    // device current (each GPU has its own copy at its own address).
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return (int)e;
    if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        // Not a stream operation: allowed while a stream of this thread records.
        hipStreamCaptureMode mode = hipStreamCaptureModeRelaxed;
        (void)hipThreadExchangeStreamCaptureMode(&mode);
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(kern::scratch));
        (void)hipThreadExchangeStreamCaptureMode(&mode);
        if (e != hipSuccess) return (int)e;
        addr[dev] = p;
    }
    *out = addr[dev];
    return 0;
}

int launch_splitk_reduce(const GemmDesc& d, const void* ws, void* C, void* stream) {
    const int64_t groups = d.ws_ld / 4, total = d.M * groups;   // < 2^31: split plans are small grids
    const unsigned blocks = (unsigned)((total + 255) / 256);
    const DivU31 rows = DivU31::of((uint32_t)groups);
    hipStream_t s = (hipStream_t)stream;
    const float* w = (const float*)ws;
    if (d.c_bf16)
        kern::splitk_reduce_kernel<true><<<blocks, 256, 0, s>>>(w, C, (int32_t)d.N, rows, (int32_t)groups,
                                                                (int32_t)total, d.ws_ld, d.M * d.ws_ld, d.c_row,
                                                                d.splits);
    else
        kern::splitk_reduce_kernel<false><<<blocks, 256, 0, s>>>(w, C, (int32_t)d.N, rows, (int32_t)groups,
                                                                 (int32_t)total, d.ws_ld, d.M * d.ws_ld, d.c_row,
                                                                 d.splits);
    return (int)hipGetLastError();
}

}  // namespace asl
