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
// Workgroup: 8 waves of 32 queries (two waves per SIMD), key stages
// double-buffered in LDS by buffer_load ... lds, in one of two shapes:
//   KS = 1  256 queries, 64-key stages; every wave sweeps all keys.
//   KS = 2  128 queries, 128-key stages; the two waves of a SIMD take the
//           same 32 queries and one 64-key half of every stage each, with
//           their own running max, sum and O, merged through LDS at the end.
//           A work item (128 queries x their keys) is then half as long,
//           which is what lets unequal causal items and small grids balance
//           over the CUs.
// Everything is computed transposed, so that a lane owns one query:
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
// sees keys j <= i + Lk - Lq): a workgroup visits only the key stages its
// last query sees, a wave skips the 64-key tiles none of its queries sees,
// and tiles crossing a wave's diagonal get the same -inf treatment per key.
// Causal items cost different amounts (lesson 07 "Clusters, distributed
// shared memory & cluster launch control", section "The second wall: the
// static schedule's tail"), so they are launched heaviest first: the
// dispatcher starts workgroups in id order as CUs free up, which is the
// longest-first greedy assignment.
#include <hip/hip_runtime.h>

#include <atomic>
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
    int32_t batch, Lq, Lk, qtiles, tiles;
    int32_t causal;       // query i sees keys j <= i + (Lk - Lq) only
    int32_t heavy_first;  // items in heaviest-first order (below)
    int32_t kv_group;     // query slice b reads K and V slice b / kv_group
    int32_t sched;        // 0: one workgroup per item; 1: persistent, static stride; 2: persistent, queue
    int32_t qslot;        // queue counters used by this launch (sched 2)
    float c;   // scale * log2(e)
};

// Work-queue counters for the persistent schedule: per launch slot and
// queue (XCD), a claim counter and a done counter, each in its own 128-byte
// line.  Zero at load; the last workgroup of a queue to finish sets both back
// to zero, so a launch leaves its slot as it found it.
constexpr int kQueueSlots = 64;
__device__ __attribute__((aligned(128))) uint32_t g_attn_queue[kQueueSlots][kXcds][2][32];

constexpr int kBN = 64;               // keys per wave per stage
constexpr int kNW = 8;                // waves per workgroup
// 32 queries per wave.  8 waves of 32 queries (two waves per SIMD) measured
// 67.8 us against 77.8 us for 4 waves of 64 queries (one per SIMD) on 32
// slices of 2048 x 2048 x 128: the second wave on a SIMD covers LDS latency
// and softmax arithmetic, and the smaller register set needs no accumulator
// copies.

// Row of an MFMA A-operand tile that lane row r reads: bits 2 and 3 exchanged.
__device__ __forceinline__ int swap23(int r) { return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1); }

// Bytes from a stage origin to the end of the last valid row: `rows` rows of
// stride ld remain, each with `len` valid elements (0 rows: nothing).
__device__ __forceinline__ int rows_extent(int64_t rows, int64_t len, int64_t ld) {
    if (rows <= 0) return 0;
    const int64_t e = ((rows - 1) * ld + len) * 2;
    return e > 0x7fffffff ? 0x7fffffff : (int)e;
}

// Issue key/value stage j (BN keys) of one slice (kb, vb: the slice's K and
// V) into the LDS stage at dst: K as DH [BN keys][64 d] halves, then V
// [BN keys][D].
template <int D, int BN, class OpK, class OpV>
__device__ __forceinline__ void issue_kv_stage(const AttnArgs& a, const uint16_t* kb, const uint16_t* vb, int j,
                                               char* dst, int w, const uint32_t* koff, const uint32_t* voff) {
    constexpr int DH = D / 64;
    const int64_t rows = (int64_t)a.Lk - (int64_t)j * BN;
#pragma unroll
    for (int hh = 0; hh < DH; ++hh) {
        const __amdgpu_buffer_rsrc_t r =
            make_rsrc(kb + (int64_t)j * BN * a.k_ld + 64 * hh, rows_extent(rows, D - 64 * hh, a.k_ld));
        const uint32_t base = lds_u32(dst + hh * OpK::kBytes + w * OpK::kLoadsPerWave * 1024);
#pragma unroll
        for (int i = 0; i < OpK::kLoadsPerWave; ++i) lds_dma16(r, koff[i], base + i * 1024);
    }
    const __amdgpu_buffer_rsrc_t r = make_rsrc(vb + (int64_t)j * BN * a.v_ld, rows_extent(rows, D, a.v_ld));
    const uint32_t base = lds_u32(dst + DH * OpK::kBytes + w * OpV::kLoadsPerWave * 1024);
#pragma unroll
    for (int i = 0; i < OpV::kLoadsPerWave; ++i) lds_dma16(r, voff[i], base + i * 1024);
}

// CPOS: the scale is positive (c > 0; a zero scale arrives as the smallest
// positive normal float, which leaves every 2^(c*s - m) at 1 to fp32
// precision); otherwise negative.  KS: key groups per workgroup (above).
// PERSIST: the grid is persistent and each workgroup walks several items
// (compiled separately, so that one workgroup per item keeps the simpler
// straight-line code and its lower scalar-register pressure).
template <int D, bool OUT_BF16, bool CPOS, int KS, bool PERSIST>
__global__ void __launch_bounds__(64 * kNW, 1) attn_fwd_kernel(AttnArgs a) {
    constexpr int QB = kNW / KS;                  // 32-query blocks per workgroup
    constexpr int BQ = 32 * QB;                   // queries per workgroup
    constexpr int BN = kBN * KS;                  // keys per stage
    constexpr int DH = D / 64;                    // 64-deep halves of a key row
    constexpr int DS = D / 16;                    // k16 steps of K Q^T
    constexpr int VT = D / 32;                    // 32-wide value-column tiles
    using OpK = OperandTile<BN, true, 64, kNW>;   // [BN keys][64 d], d contiguous
    using OpV = OperandTile<D, false, BN, kNW>;   // [BN keys][D], value columns contiguous
    constexpr int kKBytes = DH * OpK::kBytes;
    constexpr int kStage = kKBytes + OpV::kBytes;
    // KS = 2 merge: per wave, VT/2 value tiles of O (f32x4 pieces, lane
    // contiguous) in the idle ring, and m, l of its 32 queries past it.
    constexpr int kMergeO = (VT / 2) * 4 * 64 * 16;
    constexpr int kML = KS == 2 ? kNW * 2 * 32 * 4 : 0;
    static_assert(KS == 1 || kNW * kMergeO <= 2 * kStage, "merge buffer must fit in the ring");
    __shared__ __attribute__((aligned(1024))) char smem[2 * kStage + kML + 16];

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int h = lane >> 5, col = lane & 31;
    const int qb = w % QB, kg = w / QB;           // query block, key group (waves w, w+4 share a SIMD)

    // Stage loads: K halves then V, each lane's 16-byte pieces.
    uint32_t koff[OpK::kLoadsPerWave], voff[OpV::kLoadsPerWave];
#pragma unroll
    for (int i = 0; i < OpK::kLoadsPerWave; ++i) koff[i] = OpK::src_offset(w, i, lane, a.k_ld);
#pragma unroll
    for (int i = 0; i < OpV::kLoadsPerWave; ++i) voff[i] = OpV::src_offset(w, i, lane, a.v_ld);

    // Work items.  Queue x = blockIdx mod 8 (the workgroup's XCD) lists its
    // items in order k = 0, 1, ...: with heavy_first the items g = x + 8k of
    // the heaviest-first list (item g is query tile qtiles-1 - g/batch of
    // slice g mod batch), otherwise the XCD's contiguous range of the
    // (slice, query tile) list, so a slice's K and V stay in one L2.  The
    // nx workgroups of a queue start at k = their index on it; with one
    // workgroup per item that is their only item.  A persistent workgroup
    // then moves on by the static formula k += nx, or (sched 2) asks the
    // queue for its next k two key stages before the current item ends: late
    // enough that the workgroups which run dry first ask first (so the
    // heaviest remaining items go to the earliest free CUs), early enough
    // that the answer arrives while the last stages compute (lesson 07,
    // "The work-stealing loop -- ask first, then compute").
    const int x = blockIdx.x % kXcds, sidx = blockIdx.x / kXcds;
    const int nx = (int)gridDim.x / kXcds + (x < (int)gridDim.x % kXcds ? 1 : 0);
    int qstart = 0, cnt;
    if (a.heavy_first) cnt = x < a.tiles ? (a.tiles - x + kXcds - 1) / kXcds : 0;
    else xcd_range<int>(x, a.tiles, qstart, cnt);
    uint32_t* const claim_ctr = &g_attn_queue[a.qslot][x][0][0];
    uint32_t* const done_ctr = &g_attn_queue[a.qslot][x][1][0];
    __attribute__((address_space(3))) int* const next_k =
        (__attribute__((address_space(3))) int*)(smem + 2 * kStage + kML);

    for (int k = sidx; k < cnt;) {
    uint32_t claim = 0;
    int bb, u;                                     // slice, query tile
    if (a.heavy_first) {
        const int g = x + kXcds * k;
        const int r = g % a.batch;
        // With batch a multiple of 8, item g runs on XCD g mod 8 = r mod 8:
        // give that XCD the contiguous slices x*(batch/8) .. so that query
        // slices sharing K and V (a key/value group) share its L2.
        bb = a.batch % kXcds == 0 ? (r % kXcds) * (a.batch / kXcds) + r / kXcds : r;
        u = a.qtiles - 1 - g / a.batch;
    } else {
        const int L = qstart + k;
        bb = L / a.qtiles;
        u = L - bb * a.qtiles;
    }
    const int qt0 = u * BQ;                        // the workgroup's first query
    const int q0 = qt0 + 32 * qb;                  // this wave's first query
    // Key stages the workgroup visits: all of them, or with the causal mask
    // those up to the last key its last query sees.
    const int off = a.Lk - a.Lq;
    int kend = a.Lk;
    if (a.causal) kend = (qt0 + BQ < a.Lq ? qt0 + BQ : a.Lq) + off;   // keys 0 .. kend-1
    const int nst = (kend + BN - 1) / BN;

    const int bkv = bb / a.kv_group;               // key/value slice
    const uint16_t* kb = a.K + bkv * a.k_bs;
    const uint16_t* vb = a.V + bkv * a.v_bs;

    // Q fragments (B operand of K Q^T): query q0 + col, d 16*s + 8*h ..+7.
    bf16x8 qf[DS];
    const uint16_t* qp = a.Q + bb * a.q_bs;
    {
        const int q = q0 + col;
#pragma unroll
        for (int s = 0; s < DS; ++s) {
            if (q < a.Lq) qf[s] = *(const bf16x8*)(qp + (int64_t)q * a.q_ld + 16 * s + 8 * h);
            else qf[s] = bf16x8{};
        }
    }

    issue_kv_stage<D, BN, OpK, OpV>(a, kb, vb, 0, smem, w, koff, voff);
    if (nst > 1) issue_kv_stage<D, BN, OpK, OpV>(a, kb, vb, 1, smem + kStage, w, koff, voff);
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));   // Q and the first stages
    asm volatile("s_barrier" ::: "memory");

    f32x16 o[VT];
#pragma unroll
    for (int vt = 0; vt < VT; ++vt) o[vt] = f32x16{};
    // Running max m (base-2 units) and lane-partial sum l of the lane's
    // query.  The max is refreshed lazily: while no lane's new scores exceed
    // its m by more than kLazy, m stays (probabilities then reach at most
    // 2^kLazy) and O and l need no rescale; when one lane's max grows
    // further, every lane of the wave moves to its exact running max.  m
    // starts at the lowest finite float rather than -inf, so that a lane
    // whose first keys are all masked gets 2^(-inf) = 0 instead of
    // 2^(-inf + inf); its first visible key then rescales O and l (both 0)
    // by 2^(-huge) = 0.
    constexpr float kLazy = 8.0f;
    float m = -3.40282347e38f, l = 0.f;

    // The last query of this wave that exists decides which of its key
    // tiles can hold a visible key (queries past Lq are never stored).
    const int qlast = (q0 + 31 < a.Lq ? q0 + 31 : a.Lq - 1);

    const int claim_at = nst > 2 ? nst - 2 : 0;
    for (int j = 0; j < nst; ++j) {
        const char* st = smem + (j & 1) * kStage;
        const char* sv = st + kKBytes;
        if (PERSIST && a.sched == 2 && j == claim_at && w == 0 && lane == 0)
            claim = __hip_atomic_fetch_add(claim_ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        const int kb0 = j * BN + kBN * kg;         // first key of this wave's 64
        const bool act = kb0 < a.Lk && (!a.causal || kb0 <= qlast + off);

        if (act) {
            // S^T = K Q^T for the wave's 2 key tiles of 32.
            f32x16 s[2];
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) s[kt] = f32x16{};
#pragma unroll
            for (int ds = 0; ds < DS; ++ds) {
                bf16x8 kf[2];
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
                    kf[kt] = OpK::frag_row(st + (ds / 4) * OpK::kBytes, kBN * kg + 32 * kt + swap23(col), ds % 4, lane);
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
                    s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kt], qf[ds], s[kt], 0, 0, 0);
            }

            // Keys past Lk get the neutral score of the max, so their
            // probability comes out as exactly 0.  Element e of s[kt] is key
            // kb0 + 32*kt + 16*(e/8) + 8*h + e%8.  With the causal mask,
            // query q sees keys k < q + off - kb0 + 1 of the wave's 64; only
            // tiles crossing this wave's diagonal need the per-key test.
            const int valid = a.Lk - kb0;
            const bool diag = a.causal && kb0 + kBN - 1 > q0 + off;
            if (valid < kBN || diag) {
                const int lim_c = a.causal ? q0 + col + off - kb0 + 1 : kBN;
                const int lim = lim_c < valid ? lim_c : valid;     // keys < lim are visible
#pragma unroll
                for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                    for (int e = 0; e < 16; ++e)
                        if (32 * kt + 16 * (e / 8) + 8 * h + e % 8 >= lim) s[kt][e] = CPOS ? -INFINITY : INFINITY;
            }

            // Largest scaled score per query (scale > 0: the max of S, scale
            // < 0: the min), one exchange with lane l^32, which holds the
            // query's other 32 keys.
            float x = CPOS ? -INFINITY : INFINITY;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int e = 0; e < 16; ++e) x = CPOS ? fmaxf(x, s[kt][e]) : fminf(x, s[kt][e]);
            float mt = x * a.c;
            mt = fmaxf(mt, __shfl_xor(mt, 32));
            const float mn = fmaxf(m, mt);
            if (__any(mn > m + kLazy)) {
                const float alpha = __builtin_amdgcn_exp2f(m - mn);
                m = mn;
                l *= alpha;
#pragma unroll
                for (int vt = 0; vt < VT; ++vt) o[vt] *= alpha;
            }

            // p = 2^(c*s - m), rounded to bf16 as the B operand of V^T P^T.
            bf16x8 pf[4];
            float sum = 0.f;
#pragma unroll
            for (int kt = 0; kt < 2; ++kt)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kt][e], a.c, -m));
                    s[kt][e] = p;
                    sum += p;
                }
            l += sum;
#pragma unroll
            for (int js = 0; js < 4; ++js)
#pragma unroll
                for (int e = 0; e < 8; ++e) pf[js][e] = (__bf16)s[js / 2][8 * (js % 2) + e];

            // O^T += V^T P^T over the wave's 4 k16 key steps.
#pragma unroll
            for (int js = 0; js < 4; ++js) {
#pragma unroll
                for (int vt = 0; vt < VT; ++vt) {
                    const bf16x8 vf = OpV::frag(sv, 32 * vt, 4 * kg + js, lane);
                    o[vt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[js], o[vt], 0, 0, 0);
                }
            }
        }

        // Stage j+1 has landed and every wave is done with buffer j&1: refill
        // it with stage j+2.
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
        asm volatile("s_barrier" ::: "memory");
        if (j + 2 < nst) issue_kv_stage<D, BN, OpK, OpV>(a, kb, vb, j + 2, smem + (j & 1) * kStage, w, koff, voff);
    }

    // Lane holds query q0 + col, value columns 32*vt + 8*g + 4*h + (0..3) in
    // elements 4*g .. 4*g+3 of o[vt].
    float lt = l + __shfl_xor(l, 32);
    int vt0 = 0, vt1 = VT;                         // value tiles this wave stores
    if constexpr (KS == 2) {
        // Merge the two key halves of each query: wave (qb, kg) finishes value
        // tiles [kg*VT/2, (kg+1)*VT/2) and hands the other half of its O, with
        // its m and l, to its partner (qb, 1-kg).  The ring is idle: the last
        // stage wait and barrier above saw every load land and every read end.
        char* mine = smem + w * kMergeO;
        const int pw = (1 - kg) * QB + qb;         // partner wave
        const char* theirs = smem + pw * kMergeO;
        float* ml = (float*)(smem + 2 * kStage);
        // (Value tiles are picked by a wave-uniform test on constant indices,
        // so o[] stays in registers.)
#pragma unroll
        for (int vt = 0; vt < VT; ++vt) {
            if (vt / (VT / 2) == kg) continue;      // a tile this wave finishes itself
            const int t = vt % (VT / 2);
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                f32x4 x;
#pragma unroll
                for (int i = 0; i < 4; ++i) x[i] = o[vt][4 * g + i];
                *(lds_f32x4_t*)(mine + ((t * 4 + g) * 64 + lane) * 16) = x;
            }
        }
        if (h == 0) {
            ml[(w * 2 + 0) * 32 + col] = m;
            ml[(w * 2 + 1) * 32 + col] = lt;
        }
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
        asm volatile("s_barrier" ::: "memory");
        const float pm = ml[(pw * 2 + 0) * 32 + col], pl = ml[(pw * 2 + 1) * 32 + col];
        const float mm = fmaxf(m, pm);
        const float sa = __builtin_amdgcn_exp2f(m - mm), sb = __builtin_amdgcn_exp2f(pm - mm);
        lt = lt * sa + pl * sb;
        vt0 = kg * (VT / 2);
        vt1 = vt0 + VT / 2;
#pragma unroll
        for (int vt = 0; vt < VT; ++vt) {
            if (vt / (VT / 2) != kg) continue;
            const int t = vt % (VT / 2);
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const f32x4 y = *(const lds_f32x4_t*)(theirs + ((t * 4 + g) * 64 + lane) * 16);
#pragma unroll
                for (int i = 0; i < 4; ++i) o[vt][4 * g + i] = o[vt][4 * g + i] * sa + y[i] * sb;
            }
        }
    }

    // O = O^T / l for the lane's query.
    const float inv = 1.0f / lt;
    const int q = q0 + col;
    if (q < a.Lq) {
        char* orow = (char*)a.O + ((int64_t)bb * a.o_bs + (int64_t)q * a.o_ld) * (OUT_BF16 ? 2 : 4);
#pragma unroll
        for (int vt = 0; vt < VT; ++vt) {
            if (vt < vt0 || vt >= vt1) continue;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int c0 = 32 * vt + 8 * g + 4 * h;
                f32x4 y;
#pragma unroll
                for (int i = 0; i < 4; ++i) y[i] = o[vt][4 * g + i] * inv;
                if constexpr (OUT_BF16) {
                    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
                    bf16x4 z;
#pragma unroll
                    for (int i = 0; i < 4; ++i) z[i] = (__bf16)y[i];
                    *(bf16x4*)(orow + c0 * 2) = z;
                } else {
                    *(f32x4*)(orow + c0 * 4) = y;
                }
            }
        }
    }

    if constexpr (!PERSIST) break;
    // Next item.  The barrier also keeps the next item's stage loads out of
    // the ring until every wave has finished reading the merge data.
    if (a.sched == 2 && w == 0 && lane == 0) *next_k = nx + (int)claim;
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
    asm volatile("s_barrier" ::: "memory");
    k = a.sched == 2 ? __builtin_amdgcn_readfirstlane(*next_k) : k + nx;
    }

    // Queue bookkeeping: every workgroup reports once after its last
    // (failed) claim; the last one of the queue resets both counters.
    if (PERSIST && a.sched == 2 && w == 0 && lane == 0) {
        const uint32_t done = __hip_atomic_fetch_add(done_ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        if (done == (uint32_t)nx - 1) {
            __hip_atomic_store(claim_ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
            __hip_atomic_store(done_ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        }
    }
}

template <int D, bool OUT_BF16, int KS>
int launch_attn_t(const AttnDesc& d, const AttnArgs& k, hipStream_t s) {
    constexpr unsigned threads = 64 * kNW;
    const dim3 grid((unsigned)(k.sched == 0 ? d.tiles : d.grid)), block(threads);
    if (k.sched == 0) {
        if (k.c > 0.f) attn_fwd_kernel<D, OUT_BF16, true, KS, false><<<grid, block, 0, s>>>(k);
        else attn_fwd_kernel<D, OUT_BF16, false, KS, false><<<grid, block, 0, s>>>(k);
    } else {
        if (k.c > 0.f) attn_fwd_kernel<D, OUT_BF16, true, KS, true><<<grid, block, 0, s>>>(k);
        else attn_fwd_kernel<D, OUT_BF16, false, KS, true><<<grid, block, 0, s>>>(k);
    }
    return (int)hipGetLastError();
}

template <int D, bool OUT_BF16>
int launch_attn_ks(const AttnDesc& d, const AttnArgs& k, hipStream_t s) {
    return d.key_split == 2 ? launch_attn_t<D, OUT_BF16, 2>(d, k, s) : launch_attn_t<D, OUT_BF16, 1>(d, k, s);
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
    k.batch = (int32_t)d.batch;
    k.Lq = (int32_t)d.Lq;
    k.Lk = (int32_t)d.Lk;
    k.qtiles = (int32_t)d.qtiles;
    k.tiles = (int32_t)d.tiles;
    k.causal = d.causal ? 1 : 0;
    k.heavy_first = d.causal ? 1 : 0;
    k.kv_group = (int32_t)d.kv_group;
    k.sched = d.sched;
    static std::atomic<uint32_t> launches{0};
    k.qslot = (int32_t)(launches.fetch_add(1, std::memory_order_relaxed) % kQueueSlots);
    // A zero scale makes every probability 1: the smallest positive normal
    // c keeps c*s - m at 0 to fp32 precision and masked keys at -inf.
    k.c = d.c == 0.f ? 1.17549435e-38f : d.c;
    hipStream_t s = (hipStream_t)stream;
    if (d.d == 128) return d.o_bf16 ? launch_attn_ks<128, true>(d, k, s) : launch_attn_ks<128, false>(d, k, s);
    return d.o_bf16 ? launch_attn_ks<64, true>(d, k, s) : launch_attn_ks<64, false>(d, k, s);
}

}  // namespace asl
