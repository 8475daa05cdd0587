// gemm.hip -- bf16 GEMM / attention-score kernels for gfx950 (MI355X).
//
// C[b] = A[b].B[b] with fp32 accumulation, one square output tile per
// workgroup: 256x256 with 8 waves laid out 2x4 (each wave a 128x64 block of
// 16x16 MFMA tiles, two waves per SIMD), 128x128 with 4 waves laid out 2x2
// (64x64 blocks of 32x32 MFMA tiles), or 64x64 with 4 waves of 32x32 for
// small grids; WaveGrid below.  The pages compute the same
// contraction with shared operand tiles fanned out to several consumers
// (lesson 07 "Clusters, distributed shared memory & cluster launch control",
// sections "Two CTAs, one MMA" and "TMA multicast"; "Hopper TMA Multicast"
// deep-dive, Attention/GEMM reuse use-case, S_i = Q_i K^T).  On gfx950 the
// reuse comes from the workgroup->tile map in schedule.hpp (consumers of a
// panel co-run on one XCD and share its L2) and, inside a workgroup, from
// the large output tile: every A element staged in LDS feeds the MFMA
// columns of a whole wave tile and every B element its MFMA rows.
//
// Data path of one K step (BK = 64):
//   global -> LDS   buffer_load_dwordx4 ... lds (no registers in between),
//                   double-buffered (A triple-buffered when it streams and
//                   every workgroup has one tile); the next step's tile is
//                   requested while the current one is multiplied.  LDS
//                   keeps each operand in its global orientation, 16-byte
//                   chunks XOR-swizzled so that the fragment reads below are
//                   bank-conflict free (one swizzle per MFMA shape, tile.hpp).
//   LDS -> VGPR     K-contiguous operands: ds_read_b128 (8 k values of one
//                   row per lane); MN-contiguous operands: two
//                   ds_read_b64_tr_b16, which transpose 4x16 blocks on the way
//                   out of LDS so each lane still receives 8 consecutive k.
//   MFMA            v_mfma_f32_16x16x32_bf16 (256 tile) or
//                   v_mfma_f32_32x32x16_bf16 (128 tile), fp32 accumulators.
//   epilogue        fp32 stores, or round-to-nearest-even to bf16.
//
// Lane maps and the operand tile's LDS layout: tile.hpp.
//
// Edges.  M and N need not be multiples of the tile, nor K of BK (K must be
// a multiple of 8, one 16-byte chunk).  Every stage's buffer resource covers
// exactly the operand bytes from the stage origin to the operand's last
// element, so rows past M or N and k rows past K (MN-contiguous operands)
// read as zero and never fault; in the last, partial K stage the chunks of a
// K-contiguous operand at k >= K (which would otherwise read the next row)
// are given out-of-range offsets and also read as zero.  Every product term
// with k >= K is therefore 0 * 0, and outputs outside M x N are not stored.
//
#include <hip/hip_runtime.h>

#include <cstdint>

#include "internal.hpp"
#include "schedule.hpp"
#include "tile.hpp"

namespace asl {
namespace kern {

struct KArgs {
    const uint16_t* A;
    const uint16_t* B;
    void* C;
    int64_t a_ld, a_bs;   // A: stride of the non-contiguous index, batch stride
    int64_t b_ld, b_bs;
    int64_t c_ld, c_bs;
    int64_t M, N, K;      // problem sizes (edge tiles are partial)
    int32_t ktiles;       // ceil(K / BK) stages per tile
    int32_t krem;         // K mod BK: valid k of the last stage (0: the last stage is full)
    int32_t tiles, xcd_split;
    int32_t rotate;       // tile row tm starts its K loop at stage tm mod ktiles
    TileMap map;          // logical tile -> (batch, tile row, tile column)
    DivU31 kdiv;          // division by ktiles
    int32_t c_keep;       // C is read again right away (a split product's partial sums): the
                          // general kernel stores it with ordinary stores, so its lines stay in
                          // L2 and the MALL; otherwise (and in the short-product kernel)
                          // non-temporal stores
};

// A compile-time flag passed as a value (to generic lambdas).
template <bool B>
struct Flag {
    static constexpr bool value = B;
};

// Per-lane source offsets of a wave's stage loads.  For the last, partial K
// stage of a K-contiguous operand, a chunk at k >= K would read the next
// row, so its offset is moved out of range there.  A load of such an operand
// covers 8 rows of 8 chunks and the chunk order depends only on the lane and
// on one bit of the load's row-group index (OperandTile::kGroupBit, from
// the swizzle in swz_k<8>); kc[p] is the lane's k offset in loads where that
// bit is p.  An MN-contiguous operand needs
// no mask: its k rows past K lie past the resource's range.
template <class OpA, class OpB>
struct LaneOffsets {
    uint32_t a[OpA::kLoadsPerWave], b[OpB::kLoadsPerWave];
    uint32_t akc[2], bkc[2];
};

// The per-stage global -> LDS loads of one wave: kLoadsPerWave for A then
// for B, each filling one 1 KiB row of the wave's part of the stage.  The
// resources cover the operands' valid bytes from the stage origin; for a
// dead stage (past the workgroup's last tile) they cover nothing: the loads
// fetch nothing and only keep the per-stage load count uniform.  `klim` is
// the stage's valid k (BK except in a partial last stage).
template <class OpA, class OpB, bool RAGGED, bool NT_A>
struct StageLoads {
    static constexpr int kCount = OpA::kLoadsPerWave + OpB::kLoadsPerWave;
    static_assert(OpA::kLoadsPerWave % (2 << OpA::kGroupBit) == 0 && OpB::kLoadsPerWave % (2 << OpB::kGroupBit) == 0,
                  "a wave's loads must start on a row group whose swizzle bit is 0");
    static_assert(OpA::kCHR == 8 && OpB::kCHR == 8, "the two-parity chunk order holds for 8-chunk rows");
    __amdgpu_buffer_rsrc_t ra, rb;
    uint32_t sa, sb;   // LDS byte addresses of this wave's first A / B row in the stage
    uint32_t klim;
    bool live;         // the stage exists (false past the workgroup's last tile: nothing is requested)

    __device__ void setup(const char* dst_a, const char* dst_b, int w, const uint16_t* a_src, const uint16_t* b_src,
                          int a_bytes, int b_bytes, int klim_, bool live_) {
        ra = make_rsrc(a_src, a_bytes);
        rb = make_rsrc(b_src, b_bytes);
        sa = lds_u32(dst_a + w * OpA::kLoadsPerWave * 1024);
        sb = lds_u32(dst_b + w * OpB::kLoadsPerWave * 1024);
        if constexpr (RAGGED) klim = (uint32_t)__builtin_amdgcn_readfirstlane(klim_);
        live = live_;
    }
    // Load i of a stage that lies a_add / b_add bytes past the resources'
    // origins and lds_add bytes past this wave's first LDS row (resources
    // set up once for a whole tile).
    __device__ void issue_at(int i, const LaneOffsets<OpA, OpB>& o, uint32_t a_add, uint32_t b_add,
                             uint32_t lds_add) const {
        if (i < OpA::kLoadsPerWave) {
            uint32_t v = o.a[i] + a_add;
            if constexpr (RAGGED && OpA::kKMaj) v = o.akc[(i >> OpA::kGroupBit) & 1] < klim ? v : kOob;
            if constexpr (NT_A) lds_dma16_nt(ra, v, sa + lds_add + i * 1024);
            else lds_dma16(ra, v, sa + lds_add + i * 1024);
        } else {
            const int j = i - OpA::kLoadsPerWave;
            uint32_t v = o.b[j] + b_add;
            if constexpr (RAGGED && OpB::kKMaj) v = o.bkc[(j >> OpB::kGroupBit) & 1] < klim ? v : kOob;
            lds_dma16(rb, v, sb + lds_add + j * 1024);
        }
    }
    __device__ void issue(int i, const LaneOffsets<OpA, OpB>& o) const {
        if (!live) return;
        if (i < OpA::kLoadsPerWave) {
            uint32_t v = o.a[i];
            if constexpr (RAGGED && OpA::kKMaj) v = o.akc[(i >> OpA::kGroupBit) & 1] < klim ? v : kOob;
            if constexpr (NT_A) lds_dma16_nt(ra, v, sa + i * 1024);
            else lds_dma16(ra, v, sa + i * 1024);
        } else {
            const int j = i - OpA::kLoadsPerWave;
            uint32_t v = o.b[j];
            if constexpr (RAGGED && OpB::kKMaj) v = o.bkc[(j >> OpB::kGroupBit) & 1] < klim ? v : kOob;
            lds_dma16(rb, v, sb + j * 1024);
        }
    }
};

template <int TM, int TN>
struct Frags {
    bf16x8 a[TM];
    bf16x8 b[TN];
};

// The MFMA of an MI x MI output block: 32x32x16 (16 fp32 results per lane)
// or 16x16x32 (4 per lane), both bf16 in, fp32 accumulate.
template <int MI>
struct Mfma;
template <>
struct Mfma<32> {
    using Acc = f32x16;
    static constexpr int kK = 16;        // k per instruction
    static __device__ __forceinline__ Acc run(bf16x8 a, bf16x8 b, Acc c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
};
template <>
struct Mfma<16> {
    using Acc = f32x4;
    static constexpr int kK = 32;
    static __device__ __forceinline__ Acc run(bf16x8 a, bf16x8 b, Acc c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};

// Fragment unit u of a 32x32x16 substep: u < TM is A tile u, else B tile
// u - TM.
template <class OpA, class OpB, int TM, int TN>
__device__ __forceinline__ void read_unit(Frags<TM, TN>& f, int u, const char* stage, int j, int m0, int n0,
                                          int lane) {
    if (u < TM) f.a[u] = OpA::frag(stage, m0 + 32 * u, j, lane);
    else f.b[u - TM] = OpB::frag(stage + OpA::kBytes, n0 + 32 * (u - TM), j, lane);
}

// One k16 substep of the 32x32x16 path: TM*TN MFMAs on fragments `f`; woven
// between them, one fragment unit of the next set `g` (stage `rd`, substep
// `j`) per MFMA and, when `LOADS` is set, one of this wave's global -> LDS
// loads of a future stage per MFMA.  Scheduling barriers keep that order, so every MFMA has
// independent work issued next to it and the LDS sees a steady stream of
// requests rather than bursts.
template <class OpA, class OpB, int MI, int TM, int TN, bool LOADS, bool RAGGED, bool NT_A>
__device__ __forceinline__ void substep(typename Mfma<MI>::Acc (&acc)[TM][TN], const Frags<TM, TN>& f, Frags<TM, TN>& g,
                                        const char* rd, int j, int m0, int n0, int lane,
                                        const StageLoads<OpA, OpB, RAGGED, NT_A>& ld, const LaneOffsets<OpA, OpB>& off) {
    constexpr int kMfma = TM * TN;
    constexpr int kUnits = TM + TN;
    constexpr int kLoads = StageLoads<OpA, OpB, RAGGED, NT_A>::kCount;
#pragma unroll
    for (int t = 0; t < kMfma; ++t) {
        const int mi = t / TN, ni = t % TN;
        acc[mi][ni] = Mfma<MI>::run(f.a[mi], f.b[ni], acc[mi][ni]);
        if constexpr (LOADS) {
            if (t < kLoads) ld.issue(t, off);
        }
        if (t < kUnits) read_unit<OpA, OpB>(g, t, rd, j, m0, n0, lane);
        __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (LOADS) {
#pragma unroll
        for (int t = kMfma; t < kLoads; ++t) ld.issue(t, off);
    }
#pragma unroll
    for (int t = kMfma; t < kUnits; ++t) read_unit<OpA, OpB>(g, t, rd, j, m0, n0, lane);
}

// Fragments of the 16x16x32 path.  A row block's fragment is replaced by
// the next substep's right after the row's MFMAs have issued (one set of A
// fragments); B has two sets, the one in use and the next.  With 16 units
// per substep in a 128x128 wave tile, two full sets of both would not fit
// next to the 256 accumulators.
template <int TM, int TN>
struct Frags16 {
    bf16x8 a[TM];
    bf16x8 b[2][TN];
};

// One k32 substep of the 16x16x32 path: TM*TN MFMAs row block by row block
// on B set P; woven between them, the next substep's B unit u at the first
// MFMA of row u (into set 1-P), the next A fragment of row mi at the third
// MFMA of row mi+1, and, when `LOADS` is set, this wave's global -> LDS
// loads of a future stage, evenly spread.  Two MFMAs between a row's B and
// A reads measured best: A at the second MFMA of the row was 3.6 % slower
// at 8192^3, and other placements of the two reads 2-5 % slower.  The last row has no next row: its
// next fragment goes into a spare register at the end of the row before it
// and is moved into place after the loop.  Read after the loop instead, it
// would still be in flight at the stage barrier's LDS wait that follows the
// first substep (measured 1-1.7 % slower on the large shapes).  The loads
// go out at the last MFMA of every group of kEvery: all in the first MFMAs
// (5 % slower at 8192^3: the burst competes with the fragment reads) or at
// the first of each group (0.3 % slower) measured worse.
template <class OpA, class OpB, int TM, int TN, int P, bool LOADS, bool RAGGED, bool NT_A, bool B_FIRST = false>
__device__ __forceinline__ void substep16(f32x4 (&acc)[TM][TN], Frags16<TM, TN>& f, const char* rd, const char* rdb,
                                          int j, int m0, int n0, int lane,
                                          const StageLoads<OpA, OpB, RAGGED, NT_A>& ld,
                                          const LaneOffsets<OpA, OpB>& off) {
    constexpr int kMfma = TM * TN;
    constexpr int kLoads = StageLoads<OpA, OpB, RAGGED, NT_A>::kCount;
    constexpr int kLA = OpA::kLoadsPerWave, kLB = OpB::kLoadsPerWave;
    static_assert(TN <= TM && TN >= 3, "B units ride on the first MFMA of a row, A on the third");
    static_assert(kLoads <= kMfma, "at most one load per MFMA");
    constexpr int kEvery = kMfma / kLoads;
    bf16x8 last;                       // the last row's next fragment, read early into a spare
#pragma unroll
    for (int t = 0; t < kMfma; ++t) {
        const int mi = t / TN, ni = t % TN;
        acc[mi][ni] = Mfma<16>::run(f.a[mi], f.b[P][ni], acc[mi][ni]);
        if constexpr (LOADS) {
            if (t % kEvery == kEvery - 1) {
                const int q = t / kEvery;   // B_FIRST: the B loads, then the A loads
                ld.issue(B_FIRST ? (q < kLB ? kLA + q : q - kLB) : q, off);
            }
        }
        if (ni == 0 && mi < TN) f.b[1 - P][mi] = OpB::frag16(rdb, n0 + 16 * mi, j, lane);
        if (ni == 2 && mi > 0) f.a[mi - 1] = OpA::frag16(rd, m0 + 16 * (mi - 1), j, lane);
        if (mi == TM - 2 && ni == TN - 1) last = OpA::frag16(rd, m0 + 16 * (TM - 1), j, lane);
        __builtin_amdgcn_sched_barrier(0);
    }
    f.a[TM - 1] = last;
}

// Epilogue staging region of one wave: ROWS rows of the wave's block as
// fp32, WTN*4 bytes per row and 64 more bytes after every 4 rows.  LDS
// serves 4-byte stores 32 lanes at a time over a 128-byte bank window, and
// 16-byte loads in passes of 16 lanes (see swz_k in tile.hpp).  The 64-byte
// step puts the two 16-lane halves of a 16x16 staging write (rows r and r+4)
// in different halves of the bank window, and the read-back below picks, per
// lane, which row piece it reads (ReadBack), so that every pass of it hits
// 16 distinct 16-byte groups: no bank conflicts on either side.  A tile
// followed by another tile of the same workgroup stages 8 rows at a time in
// a region past the LDS ring, so the next tile's stages can stream in
// meanwhile; a workgroup's last tile stages 32 rows at a time in the then
// idle ring (fewer LDS round trips per tile).
template <int WTN, int ROWS>
struct EpiRegion {
    static constexpr int kStride = WTN * 4;
    static constexpr int kBytes = ROWS * kStride + 64 * (ROWS / 4);
    // Byte offset of the fp32 element in row `row`, column `col`.
    __device__ static int offset(int row, int col) { return row * kStride + 64 * (row >> 2) + 4 * col; }
    // Row R + e of a lane whose own rows start at lr (R and lr multiples of
    // 4, e < 4): offset(lr, c) plus this constant.
    static constexpr int step(int R, int e) { return (R + e) * kStride + 16 * R; }
};

// Read-back order: lane l reads piece cp of row rl of each group of rows one
// read-back instruction covers (16-byte pieces for fp32, 32-byte pieces for
// bf16, read as two 16-byte halves, the upper one first where s = 1).  The
// maps were found by exhaustive search over the lane-bit assignments against
// the bank model: with them no pass of a read-back instruction meets a
// bank twice.
__device__ __forceinline__ int lane_bit(int l, int b) { return (l >> b) & 1; }
template <int WTN, bool OUT_BF16>
__device__ __forceinline__ void read_back_map(int l, int& rl, int& cp, int& s) {
    if constexpr (!OUT_BF16) {
        rl = l / (WTN / 4);
        cp = l % (WTN / 4);
        s = 0;
    } else if constexpr (WTN == 64) {
        rl = lane_bit(l, 0) | lane_bit(l, 2) << 1 | lane_bit(l, 1) << 2;
        cp = lane_bit(l, 3) | lane_bit(l, 5) << 1 | lane_bit(l, 4) << 2;
        s = lane_bit(l, 0);
    } else if constexpr (WTN == 128) {
        rl = lane_bit(l, 0) | lane_bit(l, 2) << 1;
        cp = lane_bit(l, 1) | lane_bit(l, 3) << 1 | lane_bit(l, 4) << 2 | lane_bit(l, 5) << 3;
        s = lane_bit(l, 0);
    } else {
        static_assert(WTN == 32, "read-back maps exist for 32-, 64- and 128-column wave blocks");
        rl = l & 15;
        cp = l >> 4;
        s = lane_bit(l, 1);
    }
}

// Write a wave's (WTM x WTN) accumulator block to C (row r0.., column c0..)
// through its LDS region, ROWS rows at a time.  With 32x32 MFMAs element e
// of lane l of MFMA tile (mi, ni) is row 32*mi + 8*(e/4) + 4*(l/32) + e%4,
// column 32*ni + l%32 of the block; with 16x16 MFMAs it is row
// 16*mi + 4*(l/16) + e, column 16*ni + l%16.  Either way a lane holds 4
// consecutive rows of one column, so direct stores would write only 32 or 16
// contiguous elements per row.  Staged, every row goes out as contiguous
// 16-byte pieces: WTN*4-byte (fp32) or WTN*2-byte (bf16, rounded to nearest
// even right before its store) runs, whole 128-byte lines for WTN >= 64.
// The stores are non-temporal: C is written once and not re-read, so it
// should not push A and B out of L2.  KEEP (fp32 only): C is a split
// product's partial sums, which the reduction reads next; ordinary stores
// leave them in L2 and the MALL for it.  (A run-time choice between the two
// store forms does not work: the compiler merges the two stores into one
// and drops the non-temporal hint.)
//
// EDGE (a tile that extends past C): only rows < m_lim and columns < n_lim
// of the block (counted from r0, c0) are stored; a 16-byte piece that
// straddles column n_lim goes out element by element.
template <int MI, int WTM, int WTN, int ROWS>
__device__ __forceinline__ void epilogue_stage(const typename Mfma<MI>::Acc (&acc)[WTM / MI][WTN / MI], int qc,
                                               char* region, int lane) {
    constexpr int TN = WTN / MI;
    using Region = EpiRegion<WTN, ROWS>;
    // Element at row R + lr + e, column C + lc of the chunk: the lane's base
    // plus a constant.
    auto put = [&](int base, int R, int e, int C, float x) {
        *(__attribute__((address_space(3))) float*)(lds_void_t*)(region + base + Region::step(R, e) + 4 * C) = x;
    };
    if constexpr (MI == 32) {
        constexpr int H = 32 / ROWS;                 // chunks per MFMA row block
        const int mi = qc / H, h = qc % H;           // rows ROWS*h .. +ROWS-1 of row block mi
        const int lr = 4 * (lane >> 5), lc = lane & 31;
        const int base = Region::offset(lr, lc);
#pragma unroll
        for (int ni = 0; ni < TN; ++ni)
#pragma unroll
            for (int e = (ROWS / 8) * 4 * h; e < (ROWS / 8) * 4 * (h + 1); ++e)
                put(base, 8 * (e >> 2) - ROWS * h, e & 3, 32 * ni, acc[mi][ni][e]);
    } else if constexpr (ROWS >= 16) {
        const int lr = 4 * (lane >> 4), lc = lane & 15;   // whole 16-row blocks per chunk
        const int base = Region::offset(lr, lc);
#pragma unroll
        for (int b = 0; b < ROWS / 16; ++b)
#pragma unroll
            for (int ni = 0; ni < TN; ++ni)
#pragma unroll
                for (int e = 0; e < 4; ++e) put(base, 16 * b, e, 16 * ni, acc[qc * (ROWS / 16) + b][ni][e]);
    } else {
        // 8-row chunks: half h of row block mi is held by lanes 32h .. 32h+31
        const int mi = qc / 2, h = qc % 2;
        const int lr = 4 * ((lane >> 4) & 1), lc = lane & 15;
        const int base = Region::offset(lr, lc);
        if ((lane >> 5) == h) {
#pragma unroll
            for (int ni = 0; ni < TN; ++ni)
#pragma unroll
                for (int e = 0; e < 4; ++e) put(base, 0, e, 16 * ni, acc[mi][ni][e]);
        }
    }
}

template <int MI, int WTM, int WTN, int ROWS, bool OUT_BF16, bool EDGE = false, bool KEEP = false>
__device__ __forceinline__ void epilogue(const typename Mfma<MI>::Acc (&acc)[WTM / MI][WTN / MI], char* region,
                                         void* Cv, int64_t c_off, int64_t r0, int64_t c0, int64_t ldc, int lane,
                                         int64_t m_lim = 0, int64_t n_lim = 0) {
    using Region = EpiRegion<WTN, ROWS>;
    constexpr int ELEMS = OUT_BF16 ? 8 : 4;          // elements per lane per store (16 bytes out)
    constexpr int PPR = WTN / ELEMS;                 // pieces per row
    constexpr int PIECES = ROWS * PPR;
    static_assert(ROWS == 8 || ROWS == 16 || ROWS == 32, "chunks are whole 8-row groups of a row block");
    static_assert(MI == 16 || ROWS <= 32, "a 32x32 row block splits into whole chunks");
    static_assert(PIECES % 64 == 0, "epilogue pieces must fill whole wave stores");
    // Read-back q covers rows RQ*q .. RQ*q + RQ-1; the lane's addresses are
    // its q = 0 ones plus a constant (RQ*q moves whole groups of 4 rows, or,
    // for RQ = 2, keeps the lane's row inside its group of 4).
    constexpr int RQ = 64 / PPR;
    static_assert(RQ % 4 == 0 || RQ == 2, "read-back steps keep the lane's offset within its 4-row group");
    int rl, cp, sw;
    read_back_map<WTN, OUT_BF16>(lane, rl, cp, sw);
    const int rd_a = Region::offset(rl, cp * ELEMS + 4 * sw);        // read first
    const int rd_b = Region::offset(rl, cp * ELEMS + 4 * (1 - sw));  // bf16: read second
#pragma unroll
    for (int qc = 0; qc < WTM / ROWS; ++qc) {        // rows ROWS*qc .. ROWS*qc+ROWS-1 of the block
        epilogue_stage<MI, WTM, WTN, ROWS>(acc, qc, region, lane);
        wave_lds_order();                            // other lanes' staged values are read below
#pragma unroll
        for (int q = 0; q < PIECES / 64; ++q) {
            const int row = RQ * q + rl;
            const int qoff = RQ * q * Region::kStride + 64 * ((RQ * q) >> 2);
            const int64_t gi = c_off + (r0 + ROWS * qc + row) * ldc + c0 + cp * ELEMS;
            if constexpr (EDGE) {
                const int rg = ROWS * qc + row, cl = cp * ELEMS;
                if (rg >= m_lim || cl >= n_lim) continue;
                if (cl + ELEMS > n_lim) {
#pragma unroll
                    for (int e = 0; e < ELEMS; ++e) {
                        if (cl + e < n_lim) {
                            const float x = *(const __attribute__((address_space(3))) float*)(lds_void_t*)(
                                region + Region::offset(row, cl + e));
                            if constexpr (OUT_BF16) ((__bf16*)Cv)[gi + e] = (__bf16)x;
                            else ((float*)Cv)[gi + e] = x;
                        }
                    }
                    continue;
                }
            }
            if constexpr (OUT_BF16) {
                const f32x4 fa = *(const lds_f32x4_t*)(lds_void_t*)(region + rd_a + qoff);
                const f32x4 fb = *(const lds_f32x4_t*)(lds_void_t*)(region + rd_b + qoff);
                bf16x8 o;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    o[k] = (__bf16)(sw ? fb[k] : fa[k]);
                    o[k + 4] = (__bf16)(sw ? fa[k] : fb[k]);
                }
                __builtin_nontemporal_store(__builtin_bit_cast(i16x8, o), (i16x8*)((__bf16*)Cv + gi));
            } else {
                const f32x4 v = *(const lds_f32x4_t*)(lds_void_t*)(region + rd_a + qoff);
                if constexpr (KEEP) *(f32x4*)((float*)Cv + gi) = v;
                else __builtin_nontemporal_store(v, (f32x4*)((float*)Cv + gi));
            }
        }
        wave_lds_order();                            // the next chunk overwrites what was just read
    }
}

// Global stores one wave issues in epilogue<MI, WTM, WTN, ROWS, OUT_BF16>.
template <int WTM, int WTN, int ROWS, bool OUT_BF16>
constexpr int epilogue_stores() {
    return (WTM / ROWS) * (ROWS * WTN / (OUT_BF16 ? 8 : 4)) / 64;
}

// Cursor over the stream of stages a workgroup loads: tile t (logical),
// stage k of it, and the global origins of that stage's A and B tiles.
template <int TILE, int BK, bool A_K, bool B_K, bool RAGGED>
struct StageCursor {
    const KArgs& a;
    int t, k, ks, stride, end;   // tile, stages of it so far, the stage's K index
    int tm, tn;
    int64_t a_step, b_step;
    const uint16_t *pa, *pb;

    __device__ StageCursor(const KArgs& args, int first, int stride_, int end_)
        : a(args), t(first), k(0), stride(stride_), end(end_) {
        a_step = A_K ? BK : (int64_t)BK * a.a_ld;
        b_step = B_K ? BK : (int64_t)BK * a.b_ld;
        origins();
    }
    __device__ bool live() const { return t < end; }
    __device__ void origins() {
        int bb;
        a.map.coords((uint32_t)t, bb, tm, tn);
        ks = a.rotate ? tm - (int)a.kdiv.div((uint32_t)tm) * a.ktiles : 0;
        pa = a.A + bb * a.a_bs + (A_K ? (int64_t)tm * TILE * a.a_ld : (int64_t)tm * TILE) + ks * a_step;
        pb = a.B + bb * a.b_bs + (B_K ? (int64_t)tn * TILE * a.b_ld : (int64_t)tn * TILE) + ks * b_step;
    }
    // Stages of a tile run ks, ks+1, ..., ktiles-1, 0, ..., ks-1 (rotated
    // start; without rotation ks starts at 0 and never wraps).
    __device__ void advance() {
        if (++k == a.ktiles) {
            k = 0;
            t += stride;
            if (t < end) origins();
        } else if (++ks == a.ktiles) {
            ks = 0;
            pa -= (int64_t)(a.ktiles - 1) * a_step;
            pb -= (int64_t)(a.ktiles - 1) * b_step;
        } else {
            pa += a_step;
            pb += b_step;
        }
    }
    // Bytes from a stage origin to the end of the 16-byte chunk holding the
    // operand's last element: `outer` rows of stride ld remain, the last with
    // `inner` contiguous elements.  A chunk is never split by the range, so a
    // 16-byte load is either wholly in range or wholly zero; the few bytes
    // past the last element that a final partial chunk covers share its
    // 16-byte-aligned block (never a new page) and feed only outputs past M or
    // N, which are not stored.
    static __device__ int extent(int64_t outer, int64_t inner, int64_t ld) {
        const int64_t e = ((outer - 1) * ld + ((inner + 7) & ~int64_t(7))) * 2;
        return e > 0x7fffffff ? 0x7fffffff : (int)e;
    }
    __device__ int a_bytes() const {
        if (!live()) return 0;
        if constexpr (!RAGGED) return 0x7fffffff;
        const int64_t mr = a.M - (int64_t)tm * TILE, kr = a.K - (int64_t)ks * BK;
        return A_K ? extent(mr, kr, a.a_ld) : extent(kr, mr, a.a_ld);
    }
    __device__ int b_bytes() const {
        if (!live()) return 0;
        if constexpr (!RAGGED) return 0x7fffffff;
        const int64_t nr = a.N - (int64_t)tn * TILE, kr = a.K - (int64_t)ks * BK;
        return B_K ? extent(nr, kr, a.b_ld) : extent(kr, nr, a.b_ld);
    }
    // Valid k of the stage: BK, or K mod BK in a partial last stage.
    __device__ int klim() const { return (a.krem != 0 && ks == a.ktiles - 1) ? a.krem : BK; }
    // The current tile's operand origins (K stage 0) and the bytes from
    // there to the end of each operand's last valid chunk.
    __device__ const uint16_t* tile_a() const { return pa - ks * a_step; }
    __device__ const uint16_t* tile_b() const { return pb - ks * b_step; }
    __device__ int tile_a_bytes() const {
        if constexpr (!RAGGED) return 0x7fffffff;
        const int64_t mr = a.M - (int64_t)tm * TILE;
        return A_K ? extent(mr, a.K, a.a_ld) : extent(a.K, mr, a.a_ld);
    }
    __device__ int tile_b_bytes() const {
        if constexpr (!RAGGED) return 0x7fffffff;
        const int64_t nr = a.N - (int64_t)tn * TILE;
        return B_K ? extent(nr, a.K, a.b_ld) : extent(a.K, nr, a.b_ld);
    }
};

// Pipeline (S LDS buffers; a stage is BK deep in K, NS = BK / (the MFMA's
// k) substeps: 4 of k16 for 32x32x16, 2 of k32 for 16x16x32).  The stages of
// all the tiles a workgroup visits form one stream; stream stage g lives in
// buffer g mod S.
//   prologue  request stages 0..S-1; wait for stage 0; barrier; read the
//             substep-0 fragments of stage 0.
//   step g    substeps 0..NS-2: MFMAs on the current fragments while the
//                        next substep's fragments of stage g are read
//                        (16x16x32: into the B set not in use and, row by
//                        row, in place of the A fragments just consumed);
//             sync:      this wave's loads of stage g+1 have landed
//                        (vmcnt <= the loads of stages g+2..g+S-1), its
//                        LDS reads are done, then a workgroup barrier: every
//                        wave's part of stage g+1 is in LDS and nobody
//                        reads buffer g mod S any more;
//             substep NS-1: request stage g+S into buffer g mod S, read the
//                        substep-0 fragments of stage g+1, MFMAs on the
//                        last fragments of stage g.
// After a tile's last step its accumulators go out through the wave's own
// epilogue region while the next tile's first stages are already landing.
// A stage is requested S-1 steps before it is consumed.  While stages
// remain, every step issues the same number of loads, so the wait count is a
// constant.  With a ring deeper than two stages, nothing is requested past
// the workgroup's last stage (each wave-wide load holds the issuing wave for
// tens of cycles even when it fetches nothing), and from the first skipped
// stage on the waits are for everything outstanding.
//
// NT_A (an A that streams from HBM, e.g. one tile column): A's loads carry
// the non-temporal hint, so its lines leave L2 first and B stays resident.
//
// SA = 3 (split ring; streaming A, one tile-aligned 256x256 tile per
// workgroup): A and B get rings of their own, A three stages deep and B two,
// which fill the 160 KiB of LDS (no room for a between-tiles epilogue
// region, and none is needed).  Step g requests B(g+2), then A(g+3), so the
// sync's wait for stage g+1 (its B was requested before A(g+2)) leaves A's
// next stage in flight: while the MFMAs of a step run, two stages of A are
// on their way from HBM instead of one, and B, which comes from L2, keeps
// its one-step lead.  The MFMA order is that of the two-stage ring, so C is
// bitwise the same.
//
// RAGGED: M or N is not a multiple of TILE or K not of BK.  The stage
// resources then cover exactly the valid bytes, the last partial K stage
// masks its K-contiguous chunks, and edge tiles use the predicated epilogue;
// otherwise none of that code is compiled in.
template <int TILE, int BK, int S, int WGM, int WGN, int MI, bool A_K, bool B_K, bool OUT_BF16, bool RAGGED,
          bool NT_A, int SA = 0>
__global__ void __launch_bounds__(64 * WGM * WGN, 1) gemm_kernel(KArgs a) {
    constexpr int NW = WGM * WGN;        // waves, WGM along M by WGN along N
    constexpr int WTM = TILE / WGM;      // wave tile rows
    constexpr int WTN = TILE / WGN;      // wave tile columns
    constexpr int TM = WTM / MI;         // MFMA tiles per wave along M
    constexpr int TN = WTN / MI;         // ... along N
    constexpr int NS = BK / Mfma<MI>::kK;   // MFMA substeps per stage
    static_assert(NS % 2 == 0, "fragment sets alternate; NS must be even");
    static_assert(MI == 32 || NS == 2, "the 16x16x32 path runs two k32 substeps per stage");
    using OpA = OperandTile<TILE, A_K, BK, NW, MI == 16>;
    using OpB = OperandTile<TILE, B_K, BK, NW, MI == 16>;
    constexpr int kStage = OpA::kBytes + OpB::kBytes;
    constexpr int L = OpA::kLoadsPerWave + OpB::kLoadsPerWave;   // loads per wave per stage
    constexpr int LA = OpA::kLoadsPerWave;
    static_assert(L * (S - 1) < 64, "vmcnt holds at most 63");
    // SA > S: A has a ring of its own, SA deep, B one of S (split ring).
    constexpr int kSA = SA ? SA : S;
    constexpr bool kSplit = kSA != S;
    static_assert(!kSplit || (S == 2 && kSA == 3 && MI == 16 && !RAGGED && NT_A),
                  "the split ring is built for streaming A on tile-aligned 16x16x32 products");
    constexpr int kRing = kSplit ? kSA * OpA::kBytes + S * OpB::kBytes : S * kStage;
    // loads issued after the awaited stage's (split ring: B goes first, so
    // only the next A stage is still on its way)
    constexpr int kWaitStage = kSplit ? LA : L * (S - 2);
    // Rows per chunk of a tile followed by another: 8, or 16 where 8 rows
    // of a narrow bf16 block are fewer than one 16-byte piece per lane.
    constexpr int ER = 8 * WTN / (OUT_BF16 ? 8 : 4) >= 64 ? 8 : 16;
    constexpr int kEpiStores = epilogue_stores<WTM, WTN, ER, OUT_BF16>();
    constexpr int kWaitAfterEpi = kWaitStage + kEpiStores < 63 ? kWaitStage + kEpiStores : 63;
    using Epi8 = EpiRegion<WTN, ER>;
    using Epi32 = EpiRegion<WTN, 32>;
    static_assert(NW * Epi32::kBytes <= kRing, "last-tile epilogue must fit in the ring");
    // The split ring leaves no room for the between-tiles region: it runs
    // one tile per workgroup, so every tile is a last tile.
    __shared__ __attribute__((aligned(1024))) char smem[kSplit ? kRing : S * kStage + NW * Epi8::kBytes];
    auto abuf = [&](int i) __attribute__((always_inline)) {
        return kSplit ? smem + i * OpA::kBytes : smem + i * kStage;
    };
    auto bbuf = [&](int i) __attribute__((always_inline)) {
        return kSplit ? smem + kSA * OpA::kBytes + i * OpB::kBytes : smem + i * kStage + OpA::kBytes;
    };

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int wm = w / WGN, wn = w % WGN;
    const int m0 = wm * WTM, n0 = wn * WTN;
    char* const epi = kSplit ? smem : smem + S * kStage + w * Epi8::kBytes;

    // The logical tiles this workgroup visits: first, first + stride, ... < end.
    int first, stride, end;
    tile_walk<int>(blockIdx.x, gridDim.x, a.tiles, a.xcd_split != 0, first, stride, end);
    if (first >= end) return;

    StageCursor<TILE, BK, A_K, B_K, RAGGED> cur_ld(a, first, stride, end);   // split ring: A's stages
    StageCursor<TILE, BK, A_K, B_K, RAGGED> cur_b(a, first, stride, end);    // split ring: B's stages
    LaneOffsets<OpA, OpB> off;
#pragma unroll
    for (int i = 0; i < OpA::kLoadsPerWave; ++i) off.a[i] = OpA::src_offset(w, i, lane, a.a_ld);
#pragma unroll
    for (int i = 0; i < OpB::kLoadsPerWave; ++i) off.b[i] = OpB::src_offset(w, i, lane, a.b_ld);
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        off.akc[p] = (uint32_t)OpA::inner_of(w, p << OpA::kGroupBit, lane);
        off.bkc[p] = (uint32_t)OpB::inner_of(w, p << OpB::kGroupBit, lane);
    }

    const int KT = a.ktiles;
    StageLoads<OpA, OpB, RAGGED, NT_A> ld;
    // Stages past the end are skipped only with a ring deeper than two (the
    // 64 tile, whose short products end with S-1 such steps); the two-stage
    // kernels keep one constant wait and a branch-free main loop.
    bool tail = false;                            // a stage past the last one was skipped
    if constexpr (kSplit) {
        // B(s) then A(s) for s < S, then A(s) for S <= s < SA: the order of
        // the main loop, where waiting for a stage's B leaves only the next
        // A stage in flight.  Stage 0 has landed once the loads after A(0)
        // are all that is left.
#pragma unroll
        for (int s = 0; s < kSA; ++s) {
            ld.setup(abuf(s), bbuf(s < S ? s : 0), w, cur_ld.pa, cur_b.pb, cur_ld.a_bytes(), cur_b.b_bytes(), BK,
                     true);
            if (s < S) {
#pragma unroll
                for (int i = LA; i < L; ++i) ld.issue(i, off);
                cur_b.advance();
            }
#pragma unroll
            for (int i = 0; i < LA; ++i) ld.issue(i, off);
            cur_ld.advance();
        }
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(L * (S - 1) + LA * (kSA - S), 0));
    } else {
#pragma unroll
        for (int s = 0; s < S; ++s) {
            const bool lv = S == 2 || cur_ld.live();
            tail |= !lv;
            ld.setup(abuf(s), bbuf(s), w, cur_ld.pa, cur_ld.pb, cur_ld.a_bytes(), cur_ld.b_bytes(), cur_ld.klim(),
                     lv);
#pragma unroll
            for (int i = 0; i < L; ++i) ld.issue(i, off);
            cur_ld.advance();
        }
        if (tail) __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
        else __builtin_amdgcn_s_waitcnt(waitcnt_imm(L * (S - 1), 0));
    }
    asm volatile("s_barrier" ::: "memory");

    Frags<TM, TN> f[2];
    Frags16<TM, TN> f16;
    if constexpr (MI == 32) {
#pragma unroll
        for (int u = 0; u < TM + TN; ++u) read_unit<OpA, OpB>(f[0], u, smem, 0, m0, n0, lane);
    } else {
#pragma unroll
        for (int u = 0; u < TM; ++u) f16.a[u] = OpA::frag16(smem, m0 + 16 * u, 0, lane);
#pragma unroll
        for (int u = 0; u < TN; ++u) f16.b[0][u] = OpB::frag16(bbuf(0), n0 + 16 * u, 0, lane);
    }

    int cur = 0;                                  // buffer of the current stage (split ring: its B)
    int cura = 0;                                 // split ring: A buffer of the current stage
    bool prev_full = true;                        // the previous tile stored every piece
    for (int t = first; t < end; t += stride) {
        typename Mfma<MI>::Acc acc[TM][TN];
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j) acc[i][j] = typename Mfma<MI>::Acc{};

        for (int kt = 0; kt < KT; ++kt) {
            char* st = smem + cur * kStage;
            const int nxt = (cur + 1 == S) ? 0 : cur + 1;
            const int nxta = (cura + 1 == kSA) ? 0 : cura + 1;   // split ring only
            char* const sta = kSplit ? abuf(cura) : st;
            char* const stb = kSplit ? bbuf(cur) : st + OpA::kBytes;
            if constexpr (MI == 32) {
#pragma unroll
                for (int j = 0; j + 1 < NS; ++j)
                    substep<OpA, OpB, MI, TM, TN, false, RAGGED, NT_A>(acc, f[j & 1], f[(j + 1) & 1], st, j + 1, m0, n0,
                                                                     lane, ld, off);
            } else {
                substep16<OpA, OpB, TM, TN, 0, false, RAGGED, NT_A>(acc, f16, sta, stb, 1, m0, n0, lane, ld, off);
            }
            // the next stage landed everywhere; nobody reads buffer `cur` any more
            __builtin_amdgcn_sched_barrier(0);
            if (tail) {
                __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
            } else if (kt == 0 && t != first && (!RAGGED || prev_full)) {
                // The previous tile's epilogue stores (all kEpiStores of
                // them: it was not an edge tile) were issued after the
                // awaited loads; vector memory operations retire in issue
                // order, so they may stay in flight.
                __builtin_amdgcn_s_waitcnt(waitcnt_imm(kWaitAfterEpi, 0));
            } else {
                __builtin_amdgcn_s_waitcnt(waitcnt_imm(kWaitStage, 0));
            }
            asm volatile("s_barrier" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
            const bool lv = S == 2 || cur_ld.live();
            tail |= !lv;
            if constexpr (kSplit)
                ld.setup(sta, stb, w, cur_ld.pa, cur_b.pb, cur_ld.a_bytes(), cur_b.b_bytes(), BK, true);
            else
                ld.setup(sta, stb, w, cur_ld.pa, cur_ld.pb, cur_ld.a_bytes(), cur_ld.b_bytes(), cur_ld.klim(), lv);
            if constexpr (MI == 32)
                substep<OpA, OpB, MI, TM, TN, true, RAGGED, NT_A>(acc, f[(NS - 1) & 1], f[0], smem + nxt * kStage, 0, m0,
                                                                n0, lane, ld, off);
            else if constexpr (kSplit)
                substep16<OpA, OpB, TM, TN, 1, true, RAGGED, NT_A, true>(acc, f16, abuf(nxta), bbuf(nxt), 0, m0, n0,
                                                                         lane, ld, off);
            else
                substep16<OpA, OpB, TM, TN, 1, true, RAGGED, NT_A>(acc, f16, smem + nxt * kStage,
                                                                 smem + nxt * kStage + OpA::kBytes, 0, m0, n0, lane,
                                                                 ld, off);
            __builtin_amdgcn_sched_barrier(0);
            cur_ld.advance();
            cur = nxt;
            if constexpr (kSplit) {
                cur_b.advance();
                cura = nxta;
            }
        }

        int bb, tm, tn;
        a.map.coords((uint32_t)t, bb, tm, tn);
        const int64_t r0 = (int64_t)tm * TILE + m0, c0 = (int64_t)tn * TILE + n0;
        const bool full = !RAGGED || (((int64_t)tm + 1) * TILE <= a.M && ((int64_t)tn + 1) * TILE <= a.N);
        const int64_t m_lim = a.M - r0, n_lim = a.N - c0;   // rows / columns of the wave's block inside C
        const bool last = kSplit || t + stride >= end;
        if (last) {
            // Last tile: only loads past the end (two-stage ring: they fetch
            // nothing but still complete into LDS) can be outstanding.  Once
            // they have landed and every wave is done reading the last stage,
            // the ring is free for 32-row staging.
            __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
            asm volatile("s_barrier" ::: "memory");
        }
        // The epilogues' per-lane index arithmetic depends only on the lane;
        // an opaque copy keeps the compiler from hoisting all of it out of
        // the tile loop, where it would stay live in registers throughout.
        int el = lane;
        if constexpr (RAGGED) asm volatile("" : "+v"(el));
        auto store = [&](auto keep) {
            constexpr bool K = decltype(keep)::value;
            if (RAGGED && !full)
                epilogue<MI, WTM, WTN, ER, OUT_BF16, RAGGED, K>(acc, epi, a.C, bb * a.c_bs, r0, c0, a.c_ld, el, m_lim,
                                                                n_lim);
            else if (last)
                epilogue<MI, WTM, WTN, 32, OUT_BF16, false, K>(acc, smem + w * Epi32::kBytes, a.C, bb * a.c_bs, r0, c0,
                                                               a.c_ld, el);
            else
                epilogue<MI, WTM, WTN, ER, OUT_BF16, false, K>(acc, epi, a.C, bb * a.c_bs, r0, c0, a.c_ld, el);
        };
        if constexpr (OUT_BF16) store(Flag<false>{});
        else if (a.c_keep) store(Flag<true>{});
        else store(Flag<false>{});
        prev_full = full;
    }
}

// Stage depth and ring length: 2 x 64 KiB of LDS for the 256 tile.  A
// 64-deep stage reads whole 128-byte lines of K-contiguous operands.  The
// 64 tile is for grids too small to fill the CUs, whose time is the latency
// of the dependent stage loads rather than bandwidth: its 16 KiB stages sit
// in a ring of 8, so a K of up to 512 is requested at once and deeper K
// keeps 7 stages in flight.
constexpr int kBK = 64;
template <int TILE>
constexpr int stages_of() { return TILE == 64 ? 8 : 2; }

// k16 substeps U0 .. U1-1 of a tile whose stages sit in the ring (substep u:
// stage u / NS, k16 step u % NS), fragments read three substeps ahead; the
// fixed order keeps every wait to the reads it needs.
template <class OpA, class OpB, int MI, int TM, int TN, int NS, int U0, int U1, int kStage>
__device__ __forceinline__ void ring_substeps(typename Mfma<MI>::Acc (&acc)[TM][TN], const char* smem, int m0, int n0,
                                              int lane) {
    constexpr int kAhead = 4;
    Frags<TM, TN> f[kAhead];
#pragma unroll
    for (int u = U0; u < U0 + kAhead - 1; ++u) {
        if (u < U1) {
#pragma unroll
            for (int q = 0; q < TM + TN; ++q)
                read_unit<OpA, OpB>(f[u % kAhead], q, smem + (u / NS) * kStage, u % NS, m0, n0, lane);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = U0; u < U1; ++u) {
        const int v = u + kAhead - 1;
        if (v < U1) {
#pragma unroll
            for (int q = 0; q < TM + TN; ++q)
                read_unit<OpA, OpB>(f[v % kAhead], q, smem + (v / NS) * kStage, v % NS, m0, n0, lane);
        }
#pragma unroll
        for (int t = 0; t < TM * TN; ++t)
            acc[t / TN][t % TN] = Mfma<MI>::run(f[u % kAhead].a[t / TN], f[u % kAhead].b[t % TN], acc[t / TN][t % TN]);
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Short products on the 64 tile: every workgroup has one tile, and all of
// the tile's K stages (KT <= 8) fit the 8-stage ring.  The general loop
// spends most of such a product's time on each wave's own stage loads (a
// wave-wide LDS-DMA load holds the wave that issues it for tens of cycles,
// and 512^3 asks 32 of each of 4 waves; the per-stage resources add
// dependent scalar work) and on a barrier and a fragment read latency per
// stage of only 4 MFMAs.  Here the roles are split: waves 4..7 request the
// first half of the stages, release it with a barrier once it has landed,
// then do the same for the second half; waves 0..3 (2 x 2 of 32 x 32, as in
// the general kernel) run the MFMAs of the first half while the second is
// still loading, reading fragments three k16 steps ahead across stage
// boundaries.  The loads use one buffer resource per operand at the tile
// origin and add each stage's offset to the lane offsets (the caller checks
// that those stay below 2^31).  Stage s of the ring holds K stage
// (ks + s) mod KT, and each output element accumulates the same MFMA chain
// as in the general kernel, so the results are bitwise the same.  512^3:
// 6.6 us per launch in the general loop, 4.3 us here.
template <int KT, bool A_K, bool B_K, bool OUT_BF16, bool RAGGED, bool NT_A>
__device__ __forceinline__ void short64_tile(const KArgs& a, char* smem, int w, int lane, int first) {
    constexpr int TILE = 64, BK = kBK, MI = 32, NW = 4;
    constexpr int WTM = 32, WTN = 32, TM = 1, TN = 1;
    constexpr int NS = BK / Mfma<MI>::kK;
    using OpA = OperandTile<TILE, A_K, BK, NW>;
    using OpB = OperandTile<TILE, B_K, BK, NW>;
    constexpr int kStage = OpA::kBytes + OpB::kBytes;
    constexpr int L = OpA::kLoadsPerWave + OpB::kLoadsPerWave;
    constexpr int KH = (KT + 1) / 2;                 // stages of the first release
    constexpr int ER = 8 * WTN / (OUT_BF16 ? 8 : 4) >= 64 ? 8 : 16;
    using Epi8 = EpiRegion<WTN, ER>;
    using Epi32 = EpiRegion<WTN, 32>;
    StageCursor<TILE, BK, A_K, B_K, RAGGED> cur(a, first, 1, first + 1);

    if (w >= NW) {
        // Loader: the pieces compute wave w - 4 loads in the general kernel.
        const int lw = w - NW;
        LaneOffsets<OpA, OpB> off;
#pragma unroll
        for (int i = 0; i < OpA::kLoadsPerWave; ++i) off.a[i] = OpA::src_offset(lw, i, lane, a.a_ld);
#pragma unroll
        for (int i = 0; i < OpB::kLoadsPerWave; ++i) off.b[i] = OpB::src_offset(lw, i, lane, a.b_ld);
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            off.akc[p] = (uint32_t)OpA::inner_of(lw, p << OpA::kGroupBit, lane);
            off.bkc[p] = (uint32_t)OpB::inner_of(lw, p << OpB::kGroupBit, lane);
        }
        StageLoads<OpA, OpB, RAGGED, NT_A> ld;
        ld.setup(smem, smem + OpA::kBytes, lw, cur.tile_a(), cur.tile_b(), cur.tile_a_bytes(), cur.tile_b_bytes(), BK,
                 true);
        const uint32_t astep = (uint32_t)(cur.a_step * 2), bstep = (uint32_t)(cur.b_step * 2);
        const int ks0 = cur.ks;
        auto issue_stage = [&](int s) __attribute__((always_inline)) {
            const int kk = ks0 + s < KT ? ks0 + s : ks0 + s - KT;
            if constexpr (RAGGED) ld.klim = (a.krem != 0 && kk == KT - 1) ? a.krem : BK;
#pragma unroll
            for (int i = 0; i < L; ++i) ld.issue_at(i, off, kk * astep, kk * bstep, s * kStage);
        };
#pragma unroll
        for (int s = 0; s < KH; ++s) issue_stage(s);
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
        asm volatile("s_barrier" ::: "memory");     // release the first half
#pragma unroll
        for (int s = KH; s < KT; ++s) issue_stage(s);
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
        asm volatile("s_barrier" ::: "memory");     // release the second half
        asm volatile("s_barrier" ::: "memory");     // the compute waves' last reads of the ring
        return;
    }

    const int wm = w / 2, wn = w % 2;
    const int m0 = wm * WTM, n0 = wn * WTN;
    typename Mfma<MI>::Acc acc[TM][TN];
    acc[0][0] = typename Mfma<MI>::Acc{};
    asm volatile("s_barrier" ::: "memory");         // stages 0 .. KH-1 are in the ring
    ring_substeps<OpA, OpB, MI, TM, TN, NS, 0, KH * NS, kStage>(acc, smem, m0, n0, lane);
    asm volatile("s_barrier" ::: "memory");         // stages KH .. KT-1 too
    ring_substeps<OpA, OpB, MI, TM, TN, NS, KH * NS, KT * NS, kStage>(acc, smem, m0, n0, lane);
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
    asm volatile("s_barrier" ::: "memory");         // every wave is done reading the ring

    int bb, tm, tn;
    a.map.coords((uint32_t)first, bb, tm, tn);
    const int64_t r0 = (int64_t)tm * TILE + m0, c0 = (int64_t)tn * TILE + n0;
    const bool full = !RAGGED || (((int64_t)tm + 1) * TILE <= a.M && ((int64_t)tn + 1) * TILE <= a.N);
    int el = lane;
    if constexpr (RAGGED) asm volatile("" : "+v"(el));
    if (RAGGED && !full)
        epilogue<MI, WTM, WTN, ER, OUT_BF16, RAGGED>(acc, smem + KT * kStage + w * Epi8::kBytes, a.C, bb * a.c_bs, r0,
                                                     c0, a.c_ld, el, a.M - r0, a.N - c0);
    else if constexpr (KT * kStage >= NW * Epi32::kBytes)
        epilogue<MI, WTM, WTN, 32, OUT_BF16>(acc, smem + w * Epi32::kBytes, a.C, bb * a.c_bs, r0, c0, a.c_ld, el);
    else
        epilogue<MI, WTM, WTN, ER, OUT_BF16>(acc, smem + KT * kStage + w * Epi8::kBytes, a.C, bb * a.c_bs, r0, c0,
                                             a.c_ld, el);
}

template <bool A_K, bool B_K, bool OUT_BF16, bool RAGGED, bool NT_A>
__global__ void __launch_bounds__(512, 1) gemm_short64_kernel(KArgs a) {
    constexpr int kStage = 2 * 64 * kBK * 2;
    constexpr int ER = 8 * 32 / (OUT_BF16 ? 8 : 4) >= 64 ? 8 : 16;
    __shared__ __attribute__((aligned(1024))) char smem[8 * kStage + 4 * EpiRegion<32, ER>::kBytes];
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int first, stride, end;
    tile_walk<int>(blockIdx.x, gridDim.x, a.tiles, a.xcd_split != 0, first, stride, end);
    if (first >= end) return;
    switch (a.ktiles) {
        case 1: short64_tile<1, A_K, B_K, OUT_BF16, RAGGED, NT_A>(a, smem, w, lane, first); break;
        case 2: short64_tile<2, A_K, B_K, OUT_BF16, RAGGED, NT_A>(a, smem, w, lane, first); break;
        case 3: short64_tile<3, A_K, B_K, OUT_BF16, RAGGED, NT_A>(a, smem, w, lane, first); break;
        case 4: short64_tile<4, A_K, B_K, OUT_BF16, RAGGED, NT_A>(a, smem, w, lane, first); break;
        case 5: short64_tile<5, A_K, B_K, OUT_BF16, RAGGED, NT_A>(a, smem, w, lane, first); break;
        case 6: short64_tile<6, A_K, B_K, OUT_BF16, RAGGED, NT_A>(a, smem, w, lane, first); break;
        case 7: short64_tile<7, A_K, B_K, OUT_BF16, RAGGED, NT_A>(a, smem, w, lane, first); break;
        default: short64_tile<8, A_K, B_K, OUT_BF16, RAGGED, NT_A>(a, smem, w, lane, first); break;
    }
}

// Wave grid and MFMA of a workgroup.
//   256 tile: 16x16x32 MFMAs; 2 x 4 waves of 128 x 64, two waves per SIMD,
//     so that while one waits on its fragment reads or the stage barrier
//     the other's MFMAs keep the matrix unit busy.  Edge-tile (RAGGED)
//     kernels with fp32 output need a few more registers than two waves
//     per SIMD leave and run 2 x 2 waves of 128 x 128 instead; every output
//     element accumulates the same MFMA chain either way, so the bits agree.
//   128 tile: 32x32x16 MFMAs; 2 x 2 waves of 64 x 64 (8 waves would leave
//     2 MFMAs per substep).
//   64 tile: 32x32x16 MFMAs; 2 x 2 waves of 32 x 32.
// Against 32x32x16, the 16x16x32 MFMA reads and writes half the accumulator
// bytes per multiply-add; on this power-limited part the clock it keeps
// makes 8192^3 7 % faster (measured, interleaved: 0.800 -> 0.744 ms).
template <int TILE, bool RAGGED, bool OUT_BF16>
struct WaveGrid {
    static constexpr int M = 2;
    static constexpr int N = TILE == 256 && !(RAGGED && !OUT_BF16) ? 4 : 2;
    static constexpr int MI = TILE == 256 ? 16 : 32;
};

// A 64-tile product whose workgroups each get one tile with all K stages in
// the ring, and whose stage offsets fit the 32-bit lane offsets, runs
// gemm_short64_kernel.
inline bool short64_fits(const GemmDesc& d, const KArgs& k) {
    if (k.ktiles > 8 || d.grid < d.tiles) return false;
    const int64_t a_step = d.a_kmajor ? kBK : (int64_t)kBK * k.a_ld;
    const int64_t b_step = d.b_kmajor ? kBK : (int64_t)kBK * k.b_ld;
    const int64_t a_span = (int64_t)(k.ktiles - 1) * a_step * 2 + (int64_t)(d.a_kmajor ? 64 : kBK) * k.a_ld * 2;
    const int64_t b_span = (int64_t)(k.ktiles - 1) * b_step * 2 + (int64_t)(d.b_kmajor ? 64 : kBK) * k.b_ld * 2;
    return a_span < 0x7fffffff && b_span < 0x7fffffff;
}

template <int TILE, bool A_K, bool B_K, bool OUT_BF16, bool NT_A>
void launch_nt(const GemmDesc& d, const KArgs& k, hipStream_t s) {
    using WR = WaveGrid<TILE, true, OUT_BF16>;
    using WF = WaveGrid<TILE, false, OUT_BF16>;
    const bool ragged = d.M % TILE || d.N % TILE || d.K % kBK;
    const dim3 grid((unsigned)d.grid);
    constexpr int S = stages_of<TILE>();
    if constexpr (TILE == 64) {
        if (short64_fits(d, k)) {
            if (ragged) gemm_short64_kernel<A_K, B_K, OUT_BF16, true, NT_A><<<grid, dim3(512), 0, s>>>(k);
            else gemm_short64_kernel<A_K, B_K, OUT_BF16, false, NT_A><<<grid, dim3(512), 0, s>>>(k);
            return;
        }
    }
    // Streaming A with one tile-aligned 256x256 tile per workgroup: the split
    // ring (A three stages deep).
    if constexpr (TILE == 256 && NT_A) {
        if (!ragged && d.grid >= d.tiles) {
            gemm_kernel<TILE, kBK, S, WF::M, WF::N, WF::MI, A_K, B_K, OUT_BF16, false, NT_A, 3>
                <<<grid, dim3(64 * WF::M * WF::N), 0, s>>>(k);
            return;
        }
    }
    if (ragged)
        gemm_kernel<TILE, kBK, S, WR::M, WR::N, WR::MI, A_K, B_K, OUT_BF16, true, NT_A>
            <<<grid, dim3(64 * WR::M * WR::N), 0, s>>>(k);
    else
        gemm_kernel<TILE, kBK, S, WF::M, WF::N, WF::MI, A_K, B_K, OUT_BF16, false, NT_A>
            <<<grid, dim3(64 * WF::M * WF::N), 0, s>>>(k);
}

template <int TILE, bool A_K, bool B_K, bool OUT_BF16>
int launch_t(const GemmDesc& d, KArgs k, hipStream_t s) {
    k.ktiles = (int32_t)((d.K + kBK - 1) / kBK);
    k.krem = (int32_t)(d.K % kBK);
    if (d.nt_a) launch_nt<TILE, A_K, B_K, OUT_BF16, true>(d, k, s);
    else launch_nt<TILE, A_K, B_K, OUT_BF16, false>(d, k, s);
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

// Slot i is round i div P of hardware workgroup i mod P (P = d.grid); the
// tile comes from the kernels' own walk and map.
bool tile_of_slot(const GemmDesc& d, int64_t i, int64_t* b, int64_t* tm, int64_t* tn) {
    const int64_t h = i % d.grid, j = i / d.grid;
    int64_t first, stride, end;
    tile_walk<int64_t>(h, d.grid, d.tiles, d.xcd_split, first, stride, end);
    const int64_t L = first + j * stride;
    if (L >= end) return false;
    int bb, m, n;
    TileMap::of(d.tiles_m, d.tiles_n, d.group_m, d.grouped).coords((uint32_t)L, bb, m, n);
    *b = bb;
    *tm = m;
    *tn = n;
    return true;
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
    k.M = d.M;
    k.N = d.N;
    k.K = d.K;
    k.tiles = (int32_t)d.tiles;
    k.xcd_split = d.xcd_split ? 1 : 0;
    k.rotate = d.rotate_k ? 1 : 0;
    k.map = TileMap::of(d.tiles_m, d.tiles_n, d.group_m, d.grouped);
    k.kdiv = DivU31::of((uint32_t)((d.K + kBK - 1) / kBK));
    k.c_keep = d.c_keep ? 1 : 0;
    hipStream_t s = (hipStream_t)stream;
    if (d.tile == 256) return launch_tile<256>(d, k, s);
    if (d.tile == 64) return launch_tile<64>(d, k, s);
    return launch_tile<128>(d, k, s);
}

}  // namespace asl
