// tile.hpp -- gfx950 building blocks shared by the contraction kernels
// (gemm.hip, attn.hip): vector types, LDS swizzles, buffer resources, the
// global -> LDS DMA load, wait-count immediates and the bf16 operand tile
// (its global -> LDS load offsets and its MFMA fragment reads).
//
// Lane maps (measured on gfx950 with a probe kernel):
//   MFMA 32x32x16 bf16: A operand lane l = row l%32, k (l/32)*8+e (e<8);
//     B operand lane l = column l%32, k (l/32)*8+e; result element e of lane
//     l = row 8*(e/4) + 4*(l/32) + e%4, column l%32.
//   MFMA 16x16x32 bf16: A operand lane l = row l%16, k (l/16)*8+e (e<8);
//     B operand lane l = column l%16, k (l/16)*8+e; result element e (e<4)
//     of lane l = row 4*(l/16) + e, column l%16.
//   ds_read_b64_tr_b16: within each 16-lane group, result lane i element j is
//     element i%4 of the 8 bytes addressed by lane 4j + i/4 of the group.
//   buffer/global_load ... lds dwordx4: lane l's 16 bytes land at
//     LDS base + 16*l.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace asl {
namespace kern {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4_t;
typedef __attribute__((address_space(3))) i16x8 lds_i16x8_t;
typedef __attribute__((address_space(3))) f32x4 lds_f32x4_t;

// Word 3 of a raw buffer resource on gfx9-family parts: 32-bit data format,
// no swizzle, offsets checked against num_records.
constexpr int kRsrcWord3 = 0x00020000;

// A lane offset past any buffer resource's range (ranges are < 2^31 bytes):
// the load returns zeros.
constexpr uint32_t kOob = 0x80000000u;

// LDS banks (measured on gfx950 with SQ_LDS_BANK_CONFLICT and lane-pair
// probes): 64 banks of 4 bytes, i.e. 16 groups of 16 bytes per 256-byte
// line.  A 16-byte-per-lane read (ds_read_b128) is served in four passes of
// 16 lanes: in each 32-lane half, the lanes whose quad index (lane / 4 mod
// 8) has even bit parity form one pass and the odd ones the other (lane 0
// shares its pass with lanes 1-3, 12-15, 20-23 and 24-27).  An 8-byte read
// (ds_read_b64, ds_read_b64_tr_b16) is served in two passes of 32
// consecutive lanes.  Lanes of one pass that read different addresses in
// one bank serialize.
//
// Two layouts, one per fragment shape (L16 selects the second):
//   32x32x16 reads: lane l reads row l%32 (K-contiguous) or rows k, k+4 of
//     4 column chunks (MN-contiguous, see frag);
//   16x16x32 reads: lane l reads row l%16 at chunk 4j + l/16 (K-contiguous)
//     or k rows 8*(l/16) + (l%16)/4 (+4) of 2 column chunks (MN-contiguous).
//
// Swizzle of a K-contiguous tile (rows of BK k = CHR chunks of 16 B): chunk
// c of row r is stored in slot c ^ swz_k<CHR, L16>(r).
//   CHR = 4 (64-byte rows): rows with equal r mod 4 get distinct slots;
//   CHR = 8 (128-byte rows), 32x32 reads: any 8 consecutive rows fall in 8
//     distinct groups of a 128-byte half line, any 16 in 16 groups;
//   CHR = 8, 16x16 reads: rows r and r ^ 8 share a group (their lanes,
//     l and l ^ 8, are never in one pass), and rows 0..7 of a 16-row block
//     times the two chunks that lanes l and l + 16 read cover all 16
//     groups.  Bit 4 of r only flips the slot order of the next 16 rows.
template <int CHR, bool L16 = false>
__device__ __forceinline__ int swz_k(int r) {
    static_assert(!L16 || CHR == 8, "the 16x16 layout is for 128-byte rows");
    if constexpr (L16) return (r & 6) | ((r >> 4) & 1);
    else if constexpr (CHR == 4) return ((r >> 2) ^ (r >> 1)) & 3;
    else return (r & 7) ^ ((r >> 3) & 1);
}

// Swizzle of an MN-contiguous tile (rows are k, CH chunks of 16 B per row):
// chunk c of row k is stored in slot c ^ swz_mn<CH, L16>(k).  The
// transposing reads of one pass touch 2 (16x16) or 4 (32x32) consecutive
// chunks of 4 consecutive rows, plus, for 16x16, the same chunks of the 4
// rows 8 further on; the XOR spreads them over 16 distinct groups (bit 3
// of k moves the second set of rows to the other chunk pairs).  With
// 128-byte rows (CH = 8) two rows share a 256-byte line, so rows k and
// k + 2 must take the other half of the line's chunks: bit 1 of k.
template <int CH, bool L16 = false>
__device__ __forceinline__ int swz_mn(int k) {
    static_assert(CH >= 8, "rows of at least 128 bytes");
    if constexpr (L16) return (((k & 3) << 2) ^ (((k >> 3) & 1) << 1)) & (CH - 1);
    else if constexpr (CH == 8) return ((k >> 1) & 1) << 2;
    else return (k & 3) << 2;
}

// Buffer resource over `bytes` bytes at `base`.  The operands are wave
// uniform by construction; readfirstlane makes that visible to the compiler
// so the descriptor lives in SGPRs (the loads take it as a scalar operand).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
    const uint64_t p = (uint64_t)(uintptr_t)base;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
    void* q = (void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(q, (short)0, __builtin_amdgcn_readfirstlane(bytes), kRsrcWord3);
}

// s_waitcnt immediate for the gfx9 family: vmcnt <= vm (6 bits, split
// [3:0] and [15:14]), lgkmcnt <= lgkm (4 bits [11:8]), expcnt unconstrained.
constexpr int waitcnt_imm(int vm, int lgkm) {
    return (vm & 0xF) | ((vm >> 4) << 14) | (0x7 << 4) | ((lgkm & 0xF) << 8);
}

// One operand tile of R (M or N extent) x BK (K) bf16 per pipeline stage,
// loaded by the NW waves of a workgroup, in the LDS layout of the 16x16x32
// fragment reads (L16) or of the 32x32x16 ones.
template <int R, bool KMAJ, int BK, int NW, bool L16 = false>
struct OperandTile {
    static constexpr int kBytes = R * BK * 2;
    static constexpr int kCHR = BK / 8;                              // chunks per row (K-major)
    static constexpr int kLoadsPerWave = kBytes / 1024 / NW;       // 1 KiB per wave-wide load
    static_assert(kLoadsPerWave >= 1 && kLoadsPerWave * NW * 1024 == kBytes, "tile must split into whole loads");
    static constexpr int kCH = R / 8;                                // chunks per row (MN-major)
    static constexpr bool kKMaj = KMAJ;
    // K-contiguous, 8-chunk rows: a 1 KiB load covers 8 rows, whose chunk
    // order depends on the lane and on one bit of the load's row-group index
    // (bit 0 for the 32x32 layout, bit 1 for the 16x16 one).
    static constexpr int kGroupBit = L16 ? 1 : 0;

    // Byte offset, relative to the tile origin in global memory, of the 16
    // bytes that lane `lane` of wave `w` fetches in its i-th load; the data
    // lands at LDS byte (w*kLoadsPerWave + i)*1024 + lane*16.
    __device__ static uint32_t src_offset(int w, int i, int lane, int64_t ld) {
        int p = (w * kLoadsPerWave + i) * 64 + lane;      // destination chunk index
        if constexpr (KMAJ) {
            int r = p / kCHR, s = p % kCHR;
            int c = s ^ swz_k<kCHR, L16>(r);
            return (uint32_t)(((int64_t)r * ld + c * 8) * 2);
        } else {
            int k = p / kCH, s = p % kCH;
            int c = s ^ swz_mn<kCH, L16>(k);
            return (uint32_t)(((int64_t)k * ld + c * 8) * 2);
        }
    }

    // Element offset, along the contiguous dimension, of the chunk that lane
    // `lane` of wave `w` fetches in its i-th load (k within the stage for a
    // K-contiguous operand).
    __device__ static int inner_of(int w, int i, int lane) {
        int p = (w * kLoadsPerWave + i) * 64 + lane;
        if constexpr (KMAJ) {
            int r = p / kCHR, s = p % kCHR;
            return (s ^ swz_k<kCHR, L16>(r)) * 8;
        } else {
            int k = p / kCH, s = p % kCH;
            return (s ^ swz_mn<kCH, L16>(k)) * 8;
        }
    }

    // K-contiguous operand only: lane l receives k 16*j + 8*(l/32) .. +7 of
    // tile row r (any row the caller picks for the lane).
    __device__ static bf16x8 frag_row(const char* lds, int r, int j, int lane) {
        static_assert(KMAJ, "row-addressed fragments are for K-contiguous tiles");
        int c = 2 * j + (lane >> 5);
        const lds_i16x8_t* p = (const lds_i16x8_t*)(lds + r * (BK * 2) + ((c ^ swz_k<kCHR, L16>(r)) << 4));
        i16x8 v = *p;
        return __builtin_bit_cast(bf16x8, v);
    }

    // Fragment of the 16x16x32 MFMA for operand rows/columns [mn0, mn0+16)
    // and k32 substep j (< BK/32): lane l receives k 32*j + 8*(l/16) .. +7
    // of row/column mn0 + l%16.
    __device__ static bf16x8 frag16(const char* lds, int mn0, int j, int lane) {
        if constexpr (KMAJ) {
            const int r = mn0 + (lane & 15), c = 4 * j + (lane >> 4);
            const lds_i16x8_t* p = (const lds_i16x8_t*)(lds + r * (BK * 2) + ((c ^ swz_k<kCHR, L16>(r)) << 4));
            i16x8 v = *p;
            return __builtin_bit_cast(bf16x8, v);
        } else {
            // Each 16-lane group reads 4 rows of 16 columns, transposed: lane
            // i of the group receives column mn0 + i of the group's 4 rows.
            int g = lane >> 4, s = lane & 15;
            int col = mn0 + 4 * (s & 3);
            int cc = col >> 3, sub = (col & 7) * 2;
            int k0 = 32 * j + g * 8 + (s >> 2);
            int k1 = k0 + 4;
            const char* p0 = lds + k0 * (R * 2) + ((cc ^ swz_mn<kCH, L16>(k0)) << 4) + sub;
            const char* p1 = lds + k1 * (R * 2) + ((cc ^ swz_mn<kCH, L16>(k1)) << 4) + sub;
            i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)p0);
            i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)p1);
            i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            return __builtin_bit_cast(bf16x8, v);
        }
    }

    // Fragment for MFMA operand rows/columns [mn0, mn0+32) and k16 substep j
    // (< BK/16): lane l receives 8 consecutive k of row/column mn0 + l%32.
    __device__ static bf16x8 frag(const char* lds, int mn0, int j, int lane) {
        if constexpr (KMAJ) {
            return frag_row(lds, mn0 + (lane & 31), j, lane);
        } else {
            int g = lane >> 4, s = lane & 15;
            int col = mn0 + (g & 1) * 16 + 4 * (s & 3);
            int cc = col >> 3, sub = (col & 7) * 2;
            int k0 = 16 * j + (g >> 1) * 8 + (s >> 2);
            int k1 = k0 + 4;
            const char* p0 = lds + k0 * (R * 2) + ((cc ^ swz_mn<kCH, L16>(k0)) << 4) + sub;
            const char* p1 = lds + k1 * (R * 2) + ((cc ^ swz_mn<kCH, L16>(k1)) << 4) + sub;
            i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)p0);
            i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)p1);
            i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            return __builtin_bit_cast(bf16x8, v);
        }
    }
};

// One 16-byte-per-lane global -> LDS load: lane l's bytes at rsrc base +
// voff land at LDS address m0 + 16*l.  Issued as inline assembly so that the
// compiler does not insert its own (conservative) vmcnt waits before later
// LDS reads; the kernel orders these loads explicitly (s_waitcnt vmcnt + s_barrier).
// The compiler's hazard checks do not look inside inline assembly, and it
// may build the resource with v_readfirstlane (or reload spilled SGPRs with
// v_readlane) right before the load: an SGPR written by a VALU instruction
// needs 5 wait states before a VMEM instruction reads it (and M0 one before
// an LDS-DMA load), or the load may use the old value -- a wrong range
// check or LDS address.  The s_nop 4 in front supplies them whatever the
// compiler schedules there.
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t lds_addr) {
    asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" : : "v"(voff), "s"(rsrc), "{m0}"(lds_addr)
                 : "memory");
}

// The same load with the non-temporal hint: lines of an operand that is
// read once (streamed) are the first that L2 evicts, so they do not push out
// operands that other workgroups re-read.
__device__ __forceinline__ void lds_dma16_nt(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t lds_addr) {
    asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen nt lds" : : "v"(voff), "s"(rsrc), "{m0}"(lds_addr)
                 : "memory");
}

// Lanes of one wave that exchange values through LDS (one lane writes, another
// reads) share no address per lane, so nothing stops the compiler from moving
// one lane's read ahead of another's write, or a later write ahead of an
// earlier read of the same bytes.  This compiler barrier keeps the LDS
// accesses on each side of it in program order.  No wait is needed: LDS
// executes one wave's instructions in order.
__device__ __forceinline__ void wave_lds_order() { asm volatile("" ::: "memory"); }

__device__ __forceinline__ uint32_t lds_u32(const void* p) {
    return (uint32_t)(uintptr_t)(const lds_void_t*)p;
}

}  // namespace kern
}  // namespace asl
