// gemm.hip -- bf16 GEMM / attention-score kernels for gfx950 (MI355X).
//
// C[b] = A[b].B[b] with fp32 accumulation, one square output tile (256x256 or
// 128x128) per workgroup of 4 waves laid out 2x2; each wave owns a
// (TILE/2)x(TILE/2) block of 32x32 MFMA tiles.  The pages compute the same
// contraction with shared operand tiles fanned out to several consumers
// (lesson 07 "Clusters, distributed shared memory & cluster launch control",
// sections "Two CTAs, one MMA" and "TMA multicast"; "Hopper TMA Multicast"
// deep-dive, Attention/GEMM reuse use-case, S_i = Q_i K^T).  On gfx950 the
// reuse comes from the workgroup->tile map in schedule.hpp (consumers of a
// panel co-run on one XCD and share its L2) and, inside a workgroup, from
// the large output tile: every A element staged in LDS feeds TILE/32 MFMA
// columns and every B element TILE/32 MFMA rows.
//
// Data path of one K step (BK = 64):
//   global -> LDS   buffer_load_dwordx4 ... lds (no registers in between),
//                   double-buffered; the next step's tile is requested while
//                   the current one is multiplied.  LDS keeps each operand in
//                   its global orientation, 16-byte chunks XOR-swizzled so
//                   that the fragment reads below are bank-conflict free.
//   LDS -> VGPR     K-contiguous operands: ds_read_b128 (8 k values of one
//                   row per lane); MN-contiguous operands: two
//                   ds_read_b64_tr_b16, which transpose 4x16 blocks on the way
//                   out of LDS so each lane still receives 8 consecutive k.
//   MFMA            v_mfma_f32_32x32x16_bf16, fp32 accumulators.
//   epilogue        fp32 stores, or round-to-nearest-even to bf16.
//
// Lane maps (measured on gfx950 with a probe kernel):
//   MFMA 32x32x16 bf16: A operand lane l = row l%32, k (l/32)*8+e (e<8);
//     B operand lane l = column l%32, k (l/32)*8+e; result element e of lane
//     l = row 8*(e/4) + 4*(l/32) + e%4, column l%32.
//   ds_read_b64_tr_b16: within each 16-lane group, result lane i element j is
//     element i%4 of the 8 bytes addressed by lane 4j + i/4 of the group.
//   buffer/global_load ... lds dwordx4: lane l's 16 bytes land at
//     LDS base + 16*l.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "internal.hpp"
#include "schedule.hpp"

namespace asl {
namespace kern {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4_t;
typedef __attribute__((address_space(3))) i16x8 lds_i16x8_t;

constexpr int kBK = 64;        // K per pipeline step
constexpr int kWaves = 4;      // 2 x 2
constexpr int kThreads = 64 * kWaves;

// Word 3 of a raw buffer resource on gfx9-family parts: 32-bit data format,
// no swizzle, offsets checked against num_records.
constexpr int kRsrcWord3 = 0x00020000;

struct KArgs {
    const uint16_t* A;
    const uint16_t* B;
    void* C;
    int64_t a_ld, a_bs;   // A: stride of the non-contiguous index, batch stride
    int64_t b_ld, b_bs;
    int64_t c_ld, c_bs;
    int32_t ktiles;       // K / 64
    int32_t tiles, tiles_m, tiles_n, group_m, grouped;
};

// Swizzle of a K-contiguous tile (rows of 64 k = 8 chunks of 16 B): chunk c
// of row r is stored in slot c ^ swz_k(r).  Any 8 aligned consecutive rows
// read at one chunk index hit 8 distinct slots, and any 16 hit 16 distinct
// 16-byte bank groups of a 256-byte bank line.
__device__ __forceinline__ int swz_k(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// Swizzle of an MN-contiguous tile (rows are k, CH chunks of 16 B per row):
// chunk c of row k is stored in slot c ^ swz_mn(k).  The transposing reads
// touch 4 consecutive chunks of 4 consecutive rows; the XOR spreads them over
// 16 distinct bank groups.
template <int CH>
__device__ __forceinline__ int swz_mn(int k) { return ((k & 3) << 2) & (CH - 1); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, 0x7fffffff, kRsrcWord3);
}

// One operand tile of R (M or N extent) x 64 (K) bf16 per pipeline stage.
template <int R, bool KMAJ>
struct OperandTile {
    static constexpr int kBytes = R * kBK * 2;
    static constexpr int kLoadsPerWave = kBytes / 1024 / kWaves;   // 1 KiB per wave-wide load
    static constexpr int kCH = R / 8;                                // chunks per row (MN-major)

    // Byte offset, relative to the tile origin in global memory, of the 16
    // bytes that lane `lane` of wave `w` fetches in its i-th load; the data
    // lands at LDS byte (w*kLoadsPerWave + i)*1024 + lane*16.
    __device__ static uint32_t src_offset(int w, int i, int lane, int64_t ld) {
        int p = (w * kLoadsPerWave + i) * 64 + lane;      // destination chunk index
        if constexpr (KMAJ) {
            int r = p >> 3, s = p & 7;
            int c = s ^ swz_k(r);
            return (uint32_t)(((int64_t)r * ld + c * 8) * 2);
        } else {
            int k = p / kCH, s = p % kCH;
            int c = s ^ swz_mn<kCH>(k);
            return (uint32_t)(((int64_t)k * ld + c * 8) * 2);
        }
    }

    // Fragment for MFMA operand rows/columns [mn0, mn0+32) and k16 step j:
    // lane l receives 8 consecutive k of row/column mn0 + l%32.
    __device__ static bf16x8 frag(const char* lds, int mn0, int j, int lane) {
        if constexpr (KMAJ) {
            int r = mn0 + (lane & 31);
            int c = 2 * j + (lane >> 5);
            const lds_i16x8_t* p = (const lds_i16x8_t*)(lds + r * 128 + ((c ^ swz_k(r)) << 4));
            i16x8 v = *p;
            return __builtin_bit_cast(bf16x8, v);
        } else {
            int g = lane >> 4, s = lane & 15;
            int col = mn0 + (g & 1) * 16 + 4 * (s & 3);
            int cc = col >> 3, sub = (col & 7) * 2;
            int k0 = 16 * j + (g >> 1) * 8 + (s >> 2);
            int k1 = k0 + 4;
            const char* p0 = lds + k0 * (R * 2) + ((cc ^ swz_mn<kCH>(k0)) << 4) + sub;
            const char* p1 = lds + k1 * (R * 2) + ((cc ^ swz_mn<kCH>(k1)) << 4) + sub;
            i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)p0);
            i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)p1);
            i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            return __builtin_bit_cast(bf16x8, v);
        }
    }
};

// Request the K step `kt` tiles of A and B into LDS stage `stage`: wave w
// fills its own 1 KiB rows of the stage, one buffer_load ... lds per KiB.
template <class OpA, class OpB>
__device__ __forceinline__ void issue_loads(char* smem, int stage_bytes, int stage, int w,
                                            const uint16_t* a_src, const uint16_t* b_src,
                                            const uint32_t* aoff, const uint32_t* boff) {
    __amdgpu_buffer_rsrc_t ra = make_rsrc(a_src);
    __amdgpu_buffer_rsrc_t rb = make_rsrc(b_src);
    char* sa = smem + stage * stage_bytes + w * OpA::kLoadsPerWave * 1024;
    char* sb = smem + stage * stage_bytes + OpA::kBytes + w * OpB::kLoadsPerWave * 1024;
#pragma unroll
    for (int i = 0; i < OpA::kLoadsPerWave; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void_t*)(sa + i * 1024), 16, aoff[i], 0, 0, 0);
#pragma unroll
    for (int i = 0; i < OpB::kLoadsPerWave; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void_t*)(sb + i * 1024), 16, boff[i], 0, 0, 0);
}

template <int TILE, bool A_K, bool B_K, bool OUT_BF16>
__global__ void __launch_bounds__(kThreads, 1) gemm_kernel(KArgs a) {
    constexpr int WT = TILE / 2;         // wave tile
    constexpr int TM = WT / 32;          // MFMA tiles per wave along M
    constexpr int TN = WT / 32;          // ... along N
    using OpA = OperandTile<TILE, A_K>;
    using OpB = OperandTile<TILE, B_K>;
    constexpr int kStage = OpA::kBytes + OpB::kBytes;
    __shared__ __attribute__((aligned(1024))) char smem[2 * kStage];

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int wm = w >> 1, wn = w & 1;

    int bb, tm, tn;
    remap_tile<int>(blockIdx.x, a.tiles, a.tiles_m, a.tiles_n, a.group_m, a.grouped != 0, bb, tm, tn);

    // Tile origins and per-step advance (elements).
    const uint16_t* a0 = a.A + bb * a.a_bs + (A_K ? (int64_t)tm * TILE * a.a_ld : (int64_t)tm * TILE);
    const uint16_t* b0 = a.B + bb * a.b_bs + (B_K ? (int64_t)tn * TILE * a.b_ld : (int64_t)tn * TILE);
    const int64_t a_step = A_K ? kBK : (int64_t)kBK * a.a_ld;
    const int64_t b_step = B_K ? kBK : (int64_t)kBK * a.b_ld;

    uint32_t aoff[OpA::kLoadsPerWave], boff[OpB::kLoadsPerWave];
#pragma unroll
    for (int i = 0; i < OpA::kLoadsPerWave; ++i) aoff[i] = OpA::src_offset(w, i, lane, a.a_ld);
#pragma unroll
    for (int i = 0; i < OpB::kLoadsPerWave; ++i) boff[i] = OpB::src_offset(w, i, lane, a.b_ld);


    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = f32x16{};

    issue_loads<OpA, OpB>(smem, kStage, 0, w, a0, b0, aoff, boff);

    for (int kt = 0; kt < a.ktiles; ++kt) {
        const int stage = kt & 1;
        __builtin_amdgcn_s_waitcnt(0);     // this wave's loads of step kt have landed
        __syncthreads();                   // ... and every other wave's

        const char* sa = smem + stage * kStage;
        const char* sb = sa + OpA::kBytes;
        bf16x8 af[TM][4], bfr[TN][4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
            for (int i = 0; i < TM; ++i) af[i][j] = OpA::frag(sa, wm * WT + 32 * i, j, lane);
#pragma unroll
            for (int i = 0; i < TN; ++i) bfr[i][j] = OpB::frag(sb, wn * WT + 32 * i, j, lane);
        }
        // All fragment reads of this stage are issued before the next stage's
        // loads, so no read waits on them.
        __builtin_amdgcn_sched_barrier(0);
        if (kt + 1 < a.ktiles)
            issue_loads<OpA, OpB>(smem, kStage, stage ^ 1, w, a0 + (int64_t)(kt + 1) * a_step,
                                  b0 + (int64_t)(kt + 1) * b_step, aoff, boff);
        __builtin_amdgcn_sched_barrier(0);

#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int mi = 0; mi < TM; ++mi)
#pragma unroll
                for (int ni = 0; ni < TN; ++ni)
                    acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi][j], bfr[ni][j], acc[mi][ni], 0, 0, 0);
    }

    // Epilogue: element e of lane l of MFMA tile (mi, ni) is
    // C[row0 + 32*mi + 8*(e/4) + 4*(l/32) + e%4][col0 + 32*ni + l%32].
    const int64_t row0 = (int64_t)tm * TILE + wm * WT + 4 * (lane >> 5);
    const int64_t col0 = (int64_t)tn * TILE + wn * WT + (lane & 31);
    if constexpr (OUT_BF16) {
        __bf16* c = (__bf16*)a.C + bb * a.c_bs;
#pragma unroll
        for (int mi = 0; mi < TM; ++mi)
#pragma unroll
            for (int ni = 0; ni < TN; ++ni)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    int64_t r = row0 + 32 * mi + 8 * (e >> 2) + (e & 3);
                    c[r * a.c_ld + col0 + 32 * ni] = (__bf16)acc[mi][ni][e];
                }
    } else {
        float* c = (float*)a.C + bb * a.c_bs;
#pragma unroll
        for (int mi = 0; mi < TM; ++mi)
#pragma unroll
            for (int ni = 0; ni < TN; ++ni)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    int64_t r = row0 + 32 * mi + 8 * (e >> 2) + (e & 3);
                    c[r * a.c_ld + col0 + 32 * ni] = acc[mi][ni][e];
                }
    }
}

template <int TILE, bool A_K, bool B_K, bool OUT_BF16>
int launch_t(const GemmDesc& d, const KArgs& k, hipStream_t s) {
    gemm_kernel<TILE, A_K, B_K, OUT_BF16><<<dim3((unsigned)d.tiles), dim3(kThreads), 0, s>>>(k);
    return (int)hipGetLastError();
}

template <int TILE>
int launch_tile(const GemmDesc& d, const KArgs& k, hipStream_t s) {
    const int sel = (d.a_kmajor ? 4 : 0) | (d.b_kmajor ? 2 : 0) | (d.c_bf16 ? 1 : 0);
    switch (sel) {
        case 0: return launch_t<TILE, false, false, false>(d, k, s);
        case 1: return launch_t<TILE, false, false, true>(d, k, s);
        case 2: return launch_t<TILE, false, true, false>(d, k, s);
        case 3: return launch_t<TILE, false, true, true>(d, k, s);
        case 4: return launch_t<TILE, true, false, false>(d, k, s);
        case 5: return launch_t<TILE, true, false, true>(d, k, s);
        case 6: return launch_t<TILE, true, true, false>(d, k, s);
        default: return launch_t<TILE, true, true, true>(d, k, s);
    }
}

}  // namespace kern

void tile_of_workgroup(const GemmDesc& d, int64_t h, int64_t* b, int64_t* tm, int64_t* tn) {
    int64_t bb, m, n;
    remap_tile<int64_t>(h, d.tiles, d.tiles_m, d.tiles_n, d.group_m, d.grouped, bb, m, n);
    *b = bb;
    *tm = m;
    *tn = n;
}

using namespace kern;

int launch_gemm(const GemmDesc& d, const void* A, const void* B, void* C, void* stream) {
    KArgs k;
    k.A = (const uint16_t*)A;
    k.B = (const uint16_t*)B;
    k.C = C;
    k.a_ld = d.a_kmajor ? d.a_row : d.a_col;
    k.a_bs = d.a_batch;
    k.b_ld = d.b_kmajor ? d.b_col : d.b_row;
    k.b_bs = d.b_batch;
    k.c_ld = d.c_row;
    k.c_bs = d.c_batch;
    k.ktiles = (int32_t)(d.K / kBK);
    k.tiles = (int32_t)d.tiles;
    k.tiles_m = (int32_t)d.tiles_m;
    k.tiles_n = (int32_t)d.tiles_n;
    k.group_m = d.group_m;
    k.grouped = d.grouped ? 1 : 0;
    hipStream_t s = (hipStream_t)stream;
    if (d.tile == 256) return launch_tile<256>(d, k, s);
    return launch_tile<128>(d, k, s);
}

}  // namespace asl
