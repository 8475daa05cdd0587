// attn.hip -- fused attention forward for gfx950 (MI355X):
//   O[b] = softmax(scale * Q[b] K[b]^T) V[b]
// in one pass over the keys, the scores never leaving registers.
//
// The score product S = Q K^T is the inner step of the FlashAttention-class
// operators in which neighbouring query tiles consume the same key and value
// tiles ("Hopper TMA Multicast" deep-dive, Attention/GEMM reuse use-case,
// S_0 = Q_0 K^T, S_1 = Q_1 K^T, and the comparison table's "Attention K/V"
// row).  Here the query tiles of one slice run on one XCD (the same
// XCD-contiguous ranges as the GEMM schedule), so each K/V tile comes from
// HBM once per XCD and from its L2 for the other query tiles.
//
// Workgroup: 8 waves, 256 queries (32 per wave, two waves per SIMD), key
// stages of 64 keys double-buffered in LDS by buffer_load ... lds.  Everything is computed
// transposed, so that a lane owns one query:
//   S^T = K Q^T   MFMA A = K fragment (LDS, rows = keys), B = Q fragment
//                 (registers for the whole kernel).  Result lane l holds query
//                 l%32 and 16 of the 32 keys of the tile; lane l^32 holds the
//                 other 16.  The K rows are read with bits 2 and 3 of the row
//                 index exchanged, which makes lane half h hold keys
//                 16*s + 8*h + e (e < 8) in elements 8*s + e: exactly the B
//                 operand of a k16 step over those keys.
//   softmax       online (running max m and sum l per query, base 2 with
//                 scale*log2(e) folded into one fma per score): max and sum
//                 over a lane's keys in registers, one exchange with lane l^32
//                 for the max; the max is refreshed lazily (O is rescaled
//                 only when a query's scores outgrow it by 2^8).
//   O^T += V^T P^T  MFMA A = V fragment (LDS, transposing reads), B = P
//                 (the probabilities, rounded to bf16).  Result lane l holds
//                 query l%32: the running rescale by 2^(m_old - m_new) is a
//                 per-lane multiply.
// Ragged shapes: K and V stage resources cover exactly the valid rows, so
// rows past Lk read as zero; their scores are set to -inf before the max.
// Query rows past Lq read as zero and are not stored.  Causal mask (query i
// sees keys j <= i + Lk - Lq): a workgroup visits only the key tiles its
// last query sees, and tiles crossing a wave's diagonal get the same -inf
// treatment per key.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "internal.hpp"
#include "schedule.hpp"
#include "tile.hpp"

namespace asl {
namespace kern {

struct AttnArgs {
    const uint16_t *Q, *K, *V;
    void* O;
    int64_t q_ld, q_bs, k_ld, k_bs, v_ld, v_bs, o_ld, o_bs;
    int32_t Lq, Lk, qtiles, tiles, ktiles;
    int32_t causal;       // query i sees keys j <= i + (Lk - Lq) only
    float c;   // scale * log2(e)
};

constexpr int kBN = 64;               // keys per stage
constexpr int kBQ = kAttnQueriesPerWorkgroup;   // queries per workgroup (256)
// 32-query MFMA tiles per wave.  One (8 waves of 32 queries, two waves per
// SIMD) measured 67.8 us against 77.8 us for two (4 waves of 64 queries,
// one per SIMD) on 32 slices of 2048 x 2048 x 128: the second wave on a SIMD
// covers LDS latency and softmax arithmetic, and the smaller register set
// needs no accumulator copies.
constexpr int kAttnJQ = 1;

// Row of an MFMA A-operand tile that lane row r reads: bits 2 and 3 exchanged.
__device__ __forceinline__ int swap23(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

// Bytes from a stage origin to the end of the last valid row: `rows` rows of
// stride ld remain, each with `len` valid elements (0 rows: nothing).
__device__ __forceinline__ int rows_extent(int64_t rows, int64_t len, int64_t ld) {
    if (rows <= 0) return 0;
    const int64_t e = ((rows - 1) * ld + len) * 2;
    return e > 0x7fffffff ? 0x7fffffff : (int)e;
}

// Issue key/value stage j of one slice (kb, vb: the slice's K and V) into
// the LDS stage at dst: K as DH [64 keys][64 d] halves, then V [64 keys][D].
template <int D, class OpK, class OpV>
__device__ __forceinline__ void issue_kv_stage(const AttnArgs& a, const uint16_t* kb, const uint16_t* vb, int j,
                                               char* dst, int w, const uint32_t* koff, const uint32_t* voff) {
    constexpr int DH = D / 64;
    const int64_t rows = (int64_t)a.Lk - (int64_t)j * kBN;
#pragma unroll
    for (int hh = 0; hh < DH; ++hh) {
        const __amdgpu_buffer_rsrc_t r =
            make_rsrc(kb + (int64_t)j * kBN * a.k_ld + 64 * hh, rows_extent(rows, D - 64 * hh, a.k_ld));
        const uint32_t base = lds_u32(dst + hh * OpK::kBytes + w * OpK::kLoadsPerWave * 1024);
#pragma unroll
        for (int i = 0; i < OpK::kLoadsPerWave; ++i) lds_dma16(r, koff[i], base + i * 1024);
    }
    const __amdgpu_buffer_rsrc_t r = make_rsrc(vb + (int64_t)j * kBN * a.v_ld, rows_extent(rows, D, a.v_ld));
    const uint32_t base = lds_u32(dst + DH * OpK::kBytes + w * OpV::kLoadsPerWave * 1024);
#pragma unroll
    for (int i = 0; i < OpV::kLoadsPerWave; ++i) lds_dma16(r, voff[i], base + i * 1024);
}

// CPOS: the scale is positive (c > 0; a zero scale arrives as the smallest
// positive normal float, which leaves every 2^(c*s - m) at 1 to fp32
// precision); otherwise negative.
//
// JQ: 32-query MFMA tiles per wave (2: 4 waves of 64 queries; 1: 8 waves of
// 32 queries, two per SIMD, which hide each other's latencies but read every
// K and V fragment twice as often per MFMA).
template <int D, bool OUT_BF16, bool CPOS, int JQ>
__global__ void __launch_bounds__(64 * kBQ / (32 * JQ), 1) attn_fwd_kernel(AttnArgs a) {
    constexpr int QW = 32 * JQ;                   // queries per wave
    constexpr int NW = kBQ / QW;                  // waves per workgroup
    constexpr int DH = D / 64;                    // 64-deep halves of a key row
    constexpr int DS = D / 16;                    // k16 steps of K Q^T
    constexpr int VT = D / 32;                    // 32-wide value-column tiles
    using OpK = OperandTile<kBN, true, 64, NW>;   // [64 keys][64 d], d contiguous
    using OpV = OperandTile<D, false, kBN, NW>;   // [64 keys][D], value columns contiguous
    constexpr int kKBytes = DH * OpK::kBytes;
    constexpr int kStage = kKBytes + OpV::kBytes;
    __shared__ __attribute__((aligned(1024))) char smem[2 * kStage];

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int h = lane >> 5, col = lane & 31;

    // (slice, query tile) of this workgroup; an XCD runs a contiguous range.
    int first, stride, end;
    tile_walk<int>(blockIdx.x, gridDim.x, a.tiles, true, first, stride, end);
    if (first >= end) return;
    const int bb = first / a.qtiles;
    const int qt0 = (first - bb * a.qtiles) * kBQ;             // the workgroup's first query
    const int q0 = qt0 + w * QW;                               // this wave's first query
    // Key tiles the workgroup visits: all of them, or with the causal mask
    // those up to the last key its last query sees.
    const int off = a.Lk - a.Lq;
    int nkt = a.ktiles;
    if (a.causal) {
        const int qlast = (qt0 + kBQ < a.Lq ? qt0 + kBQ : a.Lq) - 1;
        const int kend = qlast + off + 1;                      // keys 0 .. kend-1
        nkt = (kend + kBN - 1) / kBN;
    }

    // Stage loads: K halves then V, each lane's 16-byte pieces.
    uint32_t koff[OpK::kLoadsPerWave], voff[OpV::kLoadsPerWave];
#pragma unroll
    for (int i = 0; i < OpK::kLoadsPerWave; ++i) koff[i] = OpK::src_offset(w, i, lane, a.k_ld);
#pragma unroll
    for (int i = 0; i < OpV::kLoadsPerWave; ++i) voff[i] = OpV::src_offset(w, i, lane, a.v_ld);
    const uint16_t* kb = a.K + bb * a.k_bs;
    const uint16_t* vb = a.V + bb * a.v_bs;

    // Q fragments (B operand of K Q^T): query q0 + 32*jq + col, d 16*s + 8*h ..+7.
    bf16x8 qf[JQ][DS];
    const uint16_t* qb = a.Q + bb * a.q_bs;
#pragma unroll
    for (int jq = 0; jq < JQ; ++jq) {
        const int q = q0 + 32 * jq + col;
#pragma unroll
        for (int s = 0; s < DS; ++s) {
            if (q < a.Lq) qf[jq][s] = *(const bf16x8*)(qb + (int64_t)q * a.q_ld + 16 * s + 8 * h);
            else qf[jq][s] = bf16x8{};
        }
    }

    issue_kv_stage<D, OpK, OpV>(a, kb, vb, 0, smem, w, koff, voff);
    if (nkt > 1) issue_kv_stage<D, OpK, OpV>(a, kb, vb, 1, smem + kStage, w, koff, voff);
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));   // Q and the first stages
    asm volatile("s_barrier" ::: "memory");

    f32x16 o[VT][JQ];
#pragma unroll
    for (int vt = 0; vt < VT; ++vt)
#pragma unroll
        for (int jq = 0; jq < JQ; ++jq) o[vt][jq] = f32x16{};
    // Running max m (base-2 units) and lane-partial sum l per query tile.
    // The max is refreshed lazily: while no lane's new scores exceed its m by
    // more than kLazy, m stays (probabilities then reach at most 2^kLazy) and
    // O and l need no rescale; when one lane's max grows further, every lane
    // of the wave moves to its exact running max.
    constexpr float kLazy = 8.0f;
    float m[JQ], l[JQ];
#pragma unroll
    for (int jq = 0; jq < JQ; ++jq) {
        m[jq] = -INFINITY;
        l[jq] = 0.f;
    }

    for (int j = 0; j < nkt; ++j) {
        const char* st = smem + (j & 1) * kStage;
        const char* sv = st + kKBytes;

        // S^T = K Q^T for 2 key tiles x 2 query tiles.
        f32x16 s[2][JQ];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int jq = 0; jq < JQ; ++jq) s[kt][jq] = f32x16{};
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) {
            bf16x8 kf[2];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
                kf[kt] = OpK::frag_row(st + (ds / 4) * OpK::kBytes, 32 * kt + swap23(col), ds % 4, lane);
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int jq = 0; jq < JQ; ++jq)
                    s[kt][jq] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kt], qf[jq][ds], s[kt][jq], 0, 0, 0);
        }

        // Keys past Lk (last tile only) get the neutral score of the max,
        // so their probability comes out as exactly 0.  Element e of
        // s[kt][.] is key 32*kt + 16*(e/8) + 8*h + e%8 of the tile.
        // With the causal mask, query q sees tile keys k < q + off - j*kBN + 1;
        // only tiles crossing this wave's diagonal need the per-key test.
        const int valid = a.Lk - j * kBN;
        const bool diag = a.causal && j * kBN + kBN - 1 > q0 + off;
        if (valid < kBN || diag) {
#pragma unroll
            for (int jq = 0; jq < JQ; ++jq) {
                const int lim_c = a.causal ? q0 + 32 * jq + col + off - j * kBN + 1 : kBN;
                const int lim = lim_c < valid ? lim_c : valid;     // keys < lim are visible
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int e = 0; e < 16; ++e)
                        if (32 * kt + 16 * (e / 8) + 8 * h + e % 8 >= lim) s[kt][jq][e] = CPOS ? -INFINITY : INFINITY;
            }
        }

        // Largest scaled score per query (scale > 0: the max of S, scale < 0:
        // the min), one exchange with lane l^32, which holds the query's
        // other 32 keys.
        float mn[JQ];
        bool grow = false;
#pragma unroll
        for (int jq = 0; jq < JQ; ++jq) {
            float x = CPOS ? -INFINITY : INFINITY;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int e = 0; e < 16; ++e) x = CPOS ? fmaxf(x, s[kt][jq][e]) : fminf(x, s[kt][jq][e]);
            float mt = x * a.c;
            mt = fmaxf(mt, __shfl_xor(mt, 32));
            mn[jq] = fmaxf(m[jq], mt);
            grow |= mn[jq] > m[jq] + kLazy;
        }
        if (__any(grow)) {
#pragma unroll
            for (int jq = 0; jq < JQ; ++jq) {
                const float alpha = __builtin_amdgcn_exp2f(m[jq] - mn[jq]);
                m[jq] = mn[jq];
                l[jq] *= alpha;
#pragma unroll
                for (int vt = 0; vt < VT; ++vt) o[vt][jq] *= alpha;
            }
        }

        // p = 2^(c*s - m), rounded to bf16 as the B operand of V^T P^T.
        bf16x8 pf[JQ][4];
#pragma unroll
        for (int jq = 0; jq < JQ; ++jq) {
            float sum = 0.f;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kt][jq][e], a.c, -m[jq]));
                    s[kt][jq][e] = p;
                    sum += p;
                }
            l[jq] += sum;
#pragma unroll
            for (int js = 0; js < 4; ++js)
#pragma unroll
                for (int e = 0; e < 8; ++e) pf[jq][js][e] = (__bf16)s[js / 2][jq][8 * (js % 2) + e];
        }

        // O^T += V^T P^T over the tile's 4 k16 key steps.
#pragma unroll
        for (int js = 0; js < 4; ++js) {
#pragma unroll
            for (int vt = 0; vt < VT; ++vt) {
                const bf16x8 vf = OpV::frag(sv, 32 * vt, js, lane);
#pragma unroll
                for (int jq = 0; jq < JQ; ++jq)
                    o[vt][jq] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[jq][js], o[vt][jq], 0, 0, 0);
            }
        }

        // Stage j+1 has landed and every wave is done with buffer j&1: refill
        // it with stage j+2.
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
        asm volatile("s_barrier" ::: "memory");
        if (j + 2 < nkt) issue_kv_stage<D, OpK, OpV>(a, kb, vb, j + 2, smem + (j & 1) * kStage, w, koff, voff);
    }

    // O = O^T / l: lane holds query q0 + 32*jq + col, value columns
    // 32*vt + 8*g + 4*h + (0..3) in elements 4*g .. 4*g+3.
#pragma unroll
    for (int jq = 0; jq < JQ; ++jq) {
        const float lt = l[jq] + __shfl_xor(l[jq], 32);
        const float inv = 1.0f / lt;
        const int q = q0 + 32 * jq + col;
        if (q >= a.Lq) continue;
        char* orow = (char*)a.O + ((int64_t)bb * a.o_bs + (int64_t)q * a.o_ld) * (OUT_BF16 ? 2 : 4);
#pragma unroll
        for (int vt = 0; vt < VT; ++vt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int c0 = 32 * vt + 8 * g + 4 * h;
                f32x4 x;
#pragma unroll
                for (int i = 0; i < 4; ++i) x[i] = o[vt][jq][4 * g + i] * inv;
                if constexpr (OUT_BF16) {
                    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
                    bf16x4 y;
#pragma unroll
                    for (int i = 0; i < 4; ++i) y[i] = (__bf16)x[i];
                    *(bf16x4*)(orow + c0 * 2) = y;
                } else {
                    *(f32x4*)(orow + c0 * 4) = x;
                }
            }
    }
}

template <int D, bool OUT_BF16>
int launch_attn_t(const AttnDesc& d, const AttnArgs& k, hipStream_t s) {
    constexpr int JQ = kAttnJQ;
    constexpr unsigned threads = 64 * kBQ / (32 * JQ);
    if (k.c > 0.f) attn_fwd_kernel<D, OUT_BF16, true, JQ><<<dim3((unsigned)d.tiles), dim3(threads), 0, s>>>(k);
    else attn_fwd_kernel<D, OUT_BF16, false, JQ><<<dim3((unsigned)d.tiles), dim3(threads), 0, s>>>(k);
    return (int)hipGetLastError();
}

}  // namespace kern

using namespace kern;

int launch_attn(const AttnDesc& d, const void* Q, const void* K, const void* V, void* O, void* stream) {
    AttnArgs k;
    k.Q = (const uint16_t*)Q;
    k.K = (const uint16_t*)K;
    k.V = (const uint16_t*)V;
    k.O = O;
    k.q_ld = d.q_row;
    k.q_bs = d.q_batch;
    k.k_ld = d.k_row;
    k.k_bs = d.k_batch;
    k.v_ld = d.v_row;
    k.v_bs = d.v_batch;
    k.o_ld = d.o_row;
    k.o_bs = d.o_batch;
    k.Lq = (int32_t)d.Lq;
    k.Lk = (int32_t)d.Lk;
    k.qtiles = (int32_t)d.qtiles;
    k.tiles = (int32_t)d.tiles;
    k.ktiles = (int32_t)((d.Lk + kBN - 1) / kBN);
    k.causal = d.causal ? 1 : 0;
    // A zero scale makes every probability 1: the smallest positive normal
    // c keeps c*s - m at 0 to fp32 precision and masked keys at -inf.
    k.c = d.c == 0.f ? 1.17549435e-38f : d.c;
    hipStream_t s = (hipStream_t)stream;
    if (d.d == 128) return d.o_bf16 ? launch_attn_t<128, true>(d, k, s) : launch_attn_t<128, false>(d, k, s);
    return d.o_bf16 ? launch_attn_t<64, true>(d, k, s) : launch_attn_t<64, false>(d, k, s);
}

}  // namespace asl
