// internal.hpp -- host-side interface between the C ABI (api.cpp) and the
// kernel launchers (gemm.hip, tilecast.hip).  Not installed, not part of the ABI.
#pragma once

#include <cstdint>

namespace asl {

// K extent of one pipeline stage (the last stage of a tile may be partial).
constexpr int kTileK = 64;

// Everything a GEMM launch needs, fixed at plan time.  Strides are elements.
struct GemmDesc {
    int64_t M, N, K, batch;
    int64_t a_row, a_col, a_batch;   // A[b,i,k]
    int64_t b_row, b_col, b_batch;   // B[b,k,j]
    int64_t c_row, c_batch;          // C[b,i,j], column stride 1
    bool a_kmajor;                   // A[i, k..k+7] contiguous
    bool b_kmajor;                   // B[k..k+7, j] contiguous
    bool c_bf16;                     // output rounded to bf16 (else fp32)
    bool c_keep;                     // output read again right away (split-K partial sums): cached stores
    int tile;                        // 256 or 128 (square output tile)
    int group_m;                     // rows of tiles per group in the grouped order
    bool grouped;                    // band order of group_m tile rows (false: row-major, the identity)
    bool xcd_split;                  // each XCD walks a contiguous range of that order
    bool nt_a;                       // A's loads carry the non-temporal hint (A streams)
    bool rotate_k;                   // tile row tm starts its K loop at stage tm mod (K stages)
    int64_t tiles_m, tiles_n, tiles; // output tiles
    int64_t grid;                    // workgroups launched (tiles, or fewer: persistent)
    // Split K (batch 1 only): the product runs as `splits` products over
    // consecutive K chunks of kc, each writing fp32 partial sums to its own
    // slice of a workspace (row stride ws_ld, ws_bytes in all); a second
    // kernel adds the slices in chunk order into C.  splits == 1: no split.
    int32_t splits;
    int64_t kc, ws_ld, ws_bytes;
};

// Launch the planned product.  Returns 0 or a hipError_t value.
int launch_gemm(const GemmDesc& d, const void* A, const void* B, void* C, void* stream);

// C = sum over chunks s = 0 .. splits-1 (in that order) of workspace slice s,
// rounded to C's type.  Returns 0 or a hipError_t value.
int launch_splitk_reduce(const GemmDesc& d, const void* ws, void* C, void* stream);

// Bytes of the static split-K scratch array (per GPU) that gemm_run_no_alloc
// uses instead of a plan's own workspace.  It holds every workspace the
// planner makes: K is split only when tiles x chunks fit the 256-workgroup
// resident grid (256 x 256 x 256 x 4 bytes) or the 512-workgroup one of
// 128 x 128 tiles (half that).
constexpr int64_t kScratchBytes = INT64_C(64) << 20;

// Device address of the scratch array on the current device (looked up once
// per device).  Returns 0 or a hipError_t value.
int scratch_address(void** out);

// Tile computed in execution slot i (round i div grid of workgroup i mod
// grid; the device schedule, shared with the kernels).  False if empty.
bool tile_of_slot(const GemmDesc& d, int64_t i, int64_t* b, int64_t* tm, int64_t* tn);

// Attention forward O = softmax(scale Q K^T) V, d == dv in {64, 128}.
// Strides are elements; every operand's last dimension is contiguous.
// key_split 1: 256 queries per workgroup; 2: 128 queries, the keys of each
// stage split over the two waves of a SIMD.
constexpr int attn_queries_per_workgroup(int key_split) { return key_split == 2 ? 128 : 256; }
struct AttnDesc {
    int64_t batch, Lq, Lk, d;
    int64_t q_row, q_batch, k_row, k_batch, v_row, v_batch, o_row, o_batch;
    bool o_bf16;
    bool causal;                     // query i sees keys j <= i + (Lk - Lq)
    float c;                         // scale * log2(e)
    int key_split;                   // 1 or 2
    int64_t kv_group;                // query slice b reads K and V slice b / kv_group
    int sched;                       // 0: one workgroup per item; 1: persistent, static; 2: persistent, queue
    int64_t qtiles, tiles;           // query tiles per slice, work items (batch * qtiles)
    int64_t grid;                    // workgroups launched
};

int launch_attn(const AttnDesc& d, const void* Q, const void* K, const void* V, void* O, void* stream);

struct TilecastDesc {
    const void* buf;
    int64_t rows, cols;
    int32_t tile_m, tile_n;
    int32_t consumers, group, grouped;
    int64_t iters, stride;
    uint32_t* out;
};

int launch_tilecast(const TilecastDesc& d, void* stream);

}  // namespace asl
