// api.cpp -- the C ABI (include/attn_scores.h): argument checks, planning,
// plan registry, error reporting.  Every check runs before any HIP call.
#include "attn_scores.h"

#include <cinttypes>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>
#include <algorithm>
#include <utility>
#include <string>
#include <memory>
#include <unordered_map>

#include <hip/hip_runtime_api.h>

#include "internal.hpp"
#include "schedule.hpp"

struct as_gemm_plan {
    asl::GemmDesc d;
    // Split-K workspace (device memory of d.ws_bytes), allocated by the first
    // run on a device and kept until the plan is released.
    std::mutex ws_mu;
    void* ws = nullptr;
    int ws_dev = -1;
    ~as_gemm_plan() {
        if (!ws) return;
        int cur = 0;
        (void)hipGetDevice(&cur);
        (void)hipSetDevice(ws_dev);
        (void)hipFree(ws);
        (void)hipSetDevice(cur);
    }
};

namespace {

thread_local std::string g_last_error;

// Live plans.  A run holds its own reference for as long as it reads the
// plan, so a gemm_destroy racing with it on another thread only drops the
// registry's reference; the plan (and its workspace) goes when the last
// reference does.
std::mutex g_plans_mu;
std::unordered_map<const as_gemm_plan*, std::shared_ptr<as_gemm_plan>>& plans() {
    static std::unordered_map<const as_gemm_plan*, std::shared_ptr<as_gemm_plan>> s;
    return s;
}

as_status fail(as_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
as_status fail(as_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

as_status ok() {
    g_last_error.clear();
    return AS_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

constexpr uint32_t kKnownFlags = AS_FLAG_NO_GROUPING | AS_FLAG_TILE_128 | AS_FLAG_TILE_256 | AS_FLAG_TILE_64 |
                                 AS_FLAG_ONE_TILE_PER_WORKGROUP | AS_FLAG_NO_SPLIT_K | AS_FLAG_NT_A |
                                 AS_FLAG_NO_NT_A | AS_FLAG_ROTATE_K | AS_FLAG_NO_ROTATE_K | AS_FLAG_NO_XCD_SPLIT;
constexpr int64_t kBK = asl::kTileK;
constexpr int64_t kCus = 256;   // MI355X compute units
constexpr int64_t kMinSplitK = 1024;   // shallowest K chunk of a split product

// Workgroups that stay resident at once: one per CU for the 256 tile's
// 146 KiB and the 64 tile's 133 KiB of LDS (its 8-stage ring), two for the
// 128 tile's 73 KiB.
int64_t resident_of(int tile) { return (tile == 128 ? 2 : 1) * kCus; }

// K chunks of a split product (1: no split).  K is split when the output
// tiles leave CUs idle (fewer tiles than CUs): into 2, 4, 8 or 16 chunks,
// each a multiple of the K stage and at least kMinSplitK deep, as many as
// keep tiles x chunks within the resident grid.  The fp32 partial sums then
// cost 8 bytes per output element and chunk (written, then read back by the
// reduction), against 2*kc flop per element and chunk.  (With a tile per CU
// already, a second workgroup per CU gained nothing: 2048^2 x 4096 ran
// 43.3 us unsplit, 44.4 us in two chunks.)
int64_t split_count(int64_t tiles, int tile, int64_t K, int64_t batch, uint32_t flags) {
    int64_t s = 1;
    if (!(flags & AS_FLAG_NO_SPLIT_K) && batch == 1 && tiles < kCus)
        while (s < 16 && tiles * s * 2 <= resident_of(tile) && K % (kBK * s * 2) == 0 && K / (s * 2) >= kMinSplitK)
            s *= 2;
    return s;
}

// Rows of tiles per group.  The cost of a candidate is the operand-panel
// traffic one XCD's L2 would take from memory, estimated on XCD 0's share
// of the grid: its tiles run 32 at a time (one workgroup per CU); a wave of
// 32 fetches every A row-panel and B column-panel it touches, unless the
// whole share's panels fit in the 4 MiB L2 together, in which case each is
// fetched once.  Ties go to the smaller group.  Panels are counted with
// stamp arrays (the logical order is batch-major, so a panel (b, row) is new
// to the share when its row was last stamped with an earlier batch), which
// keeps the simulation linear in the share.
int choose_group_m(int64_t tiles, int64_t tiles_m, int64_t tiles_n, int64_t tile, int64_t K) {
    constexpr int64_t kCusPerXcd = 32;
    constexpr int64_t kL2Bytes = INT64_C(4) << 20;
    const int64_t panel_bytes = tile * K * 2;
    const int64_t q = tiles / asl::kXcds, r = tiles % asl::kXcds;
    const int64_t share = q + (r > 0 ? 1 : 0);           // XCD 0's tiles: logical [0, share)
    std::vector<int64_t> all_a(tiles_m), all_b(tiles_n), wave_a(tiles_m), wave_b(tiles_n);
    int best = 1;
    int64_t best_cost = INT64_MAX;
    for (int64_t gm = 1; gm <= tiles_m && gm <= 64; gm *= 2) {
        std::fill(all_a.begin(), all_a.end(), -1);
        std::fill(all_b.begin(), all_b.end(), -1);
        std::fill(wave_a.begin(), wave_a.end(), -1);
        std::fill(wave_b.begin(), wave_b.end(), -1);
        int64_t whole = 0, per_wave = 0;
        for (int64_t L = 0; L < share; ++L) {
            int64_t bb, tm, tn;
            asl::logical_tile<int64_t>(L, tiles_m, tiles_n, gm, true, bb, tm, tn);
            // (wave, batch) stamp; a wave spans at most a few batches and L
            // only grows, so equal stamps mean the same panel of this wave.
            const int64_t ws = (L / kCusPerXcd) * (share + 1) + bb;
            if (all_a[tm] != bb) { all_a[tm] = bb; ++whole; }
            if (all_b[tn] != bb) { all_b[tn] = bb; ++whole; }
            if (wave_a[tm] != ws) { wave_a[tm] = ws; ++per_wave; }
            if (wave_b[tn] != ws) { wave_b[tn] = ws; ++per_wave; }
        }
        const int64_t cost = (whole * panel_bytes <= kL2Bytes) ? whole : per_wave;
        if (cost < best_cost) {
            best = (int)gm;
            best_cost = cost;
        }
    }
    return best;
}

as_status plan_desc(asl::GemmDesc* out, int64_t M, int64_t N, int64_t K, int64_t batch,
                    as_strides a, as_strides b, as_strides c,
                    as_dtype a_t, as_dtype b_t, as_dtype c_t, uint32_t flags) {
    if (M <= 0 || N <= 0 || K <= 0 || batch <= 0)
        return fail(AS_ERR_INVALID, "sizes must be positive (M=%" PRId64 " N=%" PRId64 " K=%" PRId64
                    " batch=%" PRId64 ")", M, N, K, batch);
    if (flags & ~kKnownFlags) return fail(AS_ERR_INVALID, "unknown flag bits 0x%x", flags & ~kKnownFlags);
    if (__builtin_popcount(flags & (AS_FLAG_TILE_64 | AS_FLAG_TILE_128 | AS_FLAG_TILE_256)) > 1)
        return fail(AS_ERR_INVALID, "AS_FLAG_TILE_64, AS_FLAG_TILE_128 and AS_FLAG_TILE_256 are exclusive");
    if ((flags & AS_FLAG_NT_A) && (flags & AS_FLAG_NO_NT_A))
        return fail(AS_ERR_INVALID, "AS_FLAG_NT_A and AS_FLAG_NO_NT_A are exclusive");
    if ((flags & AS_FLAG_ROTATE_K) && (flags & AS_FLAG_NO_ROTATE_K))
        return fail(AS_ERR_INVALID, "AS_FLAG_ROTATE_K and AS_FLAG_NO_ROTATE_K are exclusive");
    for (as_dtype t : {a_t, b_t, c_t})
        if (t != AS_BF16 && t != AS_F32) return fail(AS_ERR_INVALID, "unknown dtype %d", (int)t);
    if (a_t != AS_BF16 || b_t != AS_BF16)
        return fail(AS_ERR_UNSUPPORTED, "A and B must be bf16");
    const int64_t sv[9] = {a.row, a.col, a.batch, b.row, b.col, b.batch, c.row, c.col, c.batch};
    for (int64_t v : sv)
        if (v < 0) return fail(AS_ERR_INVALID, "negative stride %" PRId64, v);

    asl::GemmDesc d{};
    d.M = M; d.N = N; d.K = K; d.batch = batch;
    d.a_row = a.row; d.a_col = a.col; d.a_batch = a.batch;
    d.b_row = b.row; d.b_col = b.col; d.b_batch = b.batch;
    d.c_row = c.row; d.c_batch = c.batch;
    d.c_bf16 = (c_t == AS_BF16);

    // Operand orientation.
    if (a.col == 1) d.a_kmajor = true;
    else if (a.row == 1) d.a_kmajor = false;
    else return fail(AS_ERR_UNSUPPORTED, "A needs a unit row or column stride");
    if (b.row == 1 && b.col != 1) d.b_kmajor = true;
    else if (b.col == 1) d.b_kmajor = false;
    else return fail(AS_ERR_UNSUPPORTED, "B needs a unit row or column stride");
    if (c.col != 1) return fail(AS_ERR_UNSUPPORTED, "C must have column stride 1");

    const int64_t a_ld = d.a_kmajor ? a.row : a.col;
    const int64_t b_ld = d.b_kmajor ? b.col : b.row;
    if (a_ld % 8 || b_ld % 8)
        return fail(AS_ERR_UNSUPPORTED, "leading strides must be multiples of 8 elements (A %" PRId64
                    ", B %" PRId64 ")", a_ld, b_ld);
    const int64_t c_align = d.c_bf16 ? 8 : 4;
    if (c.row % c_align)
        return fail(AS_ERR_UNSUPPORTED, "C row stride must be a multiple of %" PRId64 " elements", c_align);
    // Every batch origin must start a 16-byte chunk like row origins do:
    // the kernels move operands and C in 16-byte pieces from there.
    if (batch > 1 && (a.batch % 8 || b.batch % 8 || c.batch % c_align))
        return fail(AS_ERR_UNSUPPORTED, "batch strides must be multiples of 8 elements (fp32 C: 4); got A %" PRId64
                    ", B %" PRId64 ", C %" PRId64, a.batch, b.batch, c.batch);
    if (M > 1 && c.row < N) return fail(AS_ERR_INVALID, "C rows overlap (row stride %" PRId64 " < N)", c.row);
    if (batch > 1 && c.batch < M * c.row)
        return fail(AS_ERR_INVALID, "C batches overlap (batch stride %" PRId64 ")", c.batch);

    if (K % 8)
        return fail(AS_ERR_UNSUPPORTED, "K must be a multiple of 8 (K=%" PRId64 ")", K);

    // Tile choice.  256x256 tiles when K is deep enough to amortise the
    // epilogue, the grid still fills most CUs and edge tiles waste little;
    // otherwise 128x128 tiles, whose 73 KiB of LDS lets two workgroups share
    // a CU so one's stores overlap the other's loads (store-bound shapes such
    // as attention scores with a short K).
    auto cdiv = [](int64_t x, int64_t y) { return (x + y - 1) / y; };
    // A grid of 128 tiles that would fill at most a quarter of the CUs and
    // cannot split K (too shallow, or batched) is latency-bound: its few
    // workgroups wait on one stage load after another.  64 tiles give it 4x
    // the workgroups, each with every stage of a K up to 512 in flight.
    int tile;
    if (flags & AS_FLAG_TILE_256) tile = 256;
    else if (flags & AS_FLAG_TILE_128) tile = 128;
    else if (flags & AS_FLAG_TILE_64) tile = 64;
    else {
        const int64_t area256 = cdiv(M, 256) * cdiv(N, 256) * 4, area128 = cdiv(M, 128) * cdiv(N, 128);
        const bool deep = K >= 512, many = batch * cdiv(M, 256) * cdiv(N, 256) >= 128;
        tile = (deep && many && area256 * 100 <= area128 * 106) ? 256 : 128;
        if (tile == 128 && batch * cdiv(M, 64) * cdiv(N, 64) <= kCus &&
            split_count(batch * area128, 128, K, batch, flags) == 1)
            tile = 64;
    }
    // Per-lane 32-bit byte offsets inside one staged tile.
    const int64_t a_span = (d.a_kmajor ? tile : kBK) * a_ld * 2;
    const int64_t b_span = (d.b_kmajor ? tile : kBK) * b_ld * 2;
    if (a_span >= (INT64_C(1) << 31) || b_span >= (INT64_C(1) << 31))
        return fail(AS_ERR_UNSUPPORTED, "leading strides too large for 32-bit tile offsets");
    if (cdiv(K, kBK) > INT32_MAX) return fail(AS_ERR_UNSUPPORTED, "K too large");

    d.tile = tile;
    d.tiles_m = cdiv(M, tile);
    d.tiles_n = cdiv(N, tile);
    if (d.tiles_m > INT32_MAX / d.tiles_n || d.tiles_m * d.tiles_n > INT32_MAX / batch)
        return fail(AS_ERR_UNSUPPORTED, "too many output tiles");
    d.tiles = batch * d.tiles_m * d.tiles_n;
    d.grouped = !(flags & AS_FLAG_NO_GROUPING);
    d.xcd_split = d.grouped && !(flags & AS_FLAG_NO_XCD_SPLIT);
    // With one tile column every A row panel has a single consumer: A
    // streams from HBM once while every tile re-reads all of B.  A's loads
    // then carry the non-temporal hint (its lines leave L2 before B's), and
    // the K loop is rotated: otherwise all running workgroups read the same
    // 128-byte column block of every A row at once (rows 2*K bytes apart),
    // an access pattern that HBM serves at about 4.4 TB/s against 6.1 TB/s
    // for rotated columns.
    const bool streams_a = d.tiles_n == 1;
    d.nt_a = (flags & AS_FLAG_NT_A) ? true : (flags & AS_FLAG_NO_NT_A) ? false : streams_a;
    d.rotate_k = (flags & AS_FLAG_ROTATE_K) ? true : (flags & AS_FLAG_NO_ROTATE_K) ? false : streams_a;
    d.splits = 1;
    d.kc = K;
    if (const int64_t sk = split_count(d.tiles, tile, K, batch, flags); sk > 1) {
        d.splits = (int32_t)sk;
        d.kc = K / sk;
        d.ws_ld = (N + 3) & ~INT64_C(3);
        d.ws_bytes = sk * M * d.ws_ld * 4;
    }
    // As many workgroups as stay resident, each walking its XCD's tiles
    // with the LDS ring streaming across tile boundaries, so one tile's
    // stores drain while the next tile computes; or, for the ablation, one
    // workgroup per tile.
    const int64_t resident = resident_of(tile);
    const int64_t launched = d.tiles * d.splits;   // split: every (chunk, tile) pair
    d.grid = !(flags & AS_FLAG_ONE_TILE_PER_WORKGROUP) && launched > resident ? resident : launched;
    d.group_m = choose_group_m(launched, d.tiles_m, d.tiles_n, tile, d.kc);
    *out = d;
    return AS_OK;
}

as_status check_attn_flags(uint32_t flags) {
    constexpr uint32_t kAttnFlags = AS_ATTN_CAUSAL | AS_ATTN_QUERIES_256 | AS_ATTN_QUERIES_128 |
                                    AS_ATTN_SCHED_STATIC | AS_ATTN_SCHED_QUEUE;
    if (flags & ~kAttnFlags) return fail(AS_ERR_INVALID, "unknown flag bits 0x%x", flags & ~kAttnFlags);
    if ((flags & AS_ATTN_QUERIES_256) && (flags & AS_ATTN_QUERIES_128))
        return fail(AS_ERR_INVALID, "AS_ATTN_QUERIES_256 and AS_ATTN_QUERIES_128 are exclusive");
    if ((flags & AS_ATTN_SCHED_STATIC) && (flags & AS_ATTN_SCHED_QUEUE))
        return fail(AS_ERR_INVALID, "AS_ATTN_SCHED_STATIC and AS_ATTN_SCHED_QUEUE are exclusive");
    return AS_OK;
}

// Attention schedule: one workgroup per item (the dispatcher starts them in
// id order as CUs free up), or a persistent grid of one workgroup per CU
// that walks items by a static stride or claims them from a queue.
int attn_sched(uint32_t flags) {
    if (flags & AS_ATTN_SCHED_STATIC) return 1;
    if (flags & AS_ATTN_SCHED_QUEUE) return 2;
    return 0;
}

// Attention work items: 256 queries, or 128 with each stage's keys split
// over the two waves of a SIMD (returns 1 or 2).  One workgroup runs per CU,
// so the grid runs in rounds of kCus items; a 128-query item takes 0.565 of
// a 256-query one (measured: 78.2 vs 69.1 us for the same 32 x 2048^2 x 128
// work in twice the items).  The shorter items win where they fill the
// rounds better, and always with the causal mask, whose items cost
// different amounts and balance only when each is short.
int attn_key_split(int64_t batch, int64_t Lq, uint32_t flags) {
    if (flags & AS_ATTN_QUERIES_256) return 1;
    if (flags & AS_ATTN_QUERIES_128) return 2;
    if (flags & AS_ATTN_CAUSAL) return 2;
    const int64_t n256 = batch * ((Lq + 255) / 256), n128 = batch * ((Lq + 127) / 128);
    const int64_t r256 = (n256 + kCus - 1) / kCus, r128 = (n128 + kCus - 1) / kCus;
    return 565 * r128 < 1000 * r256 ? 2 : 1;
}

// The product kernel launch of a split plan: `splits` products over the K
// chunks (chunk s of A and B starts s*kc along K), each into its own fp32
// slice of the workspace.
asl::GemmDesc split_launch_desc(const asl::GemmDesc& d) {
    asl::GemmDesc e = d;
    e.batch = d.splits;
    e.K = d.kc;
    e.a_batch = d.kc * d.a_col;        // A[i, k] at i*a_row + k*a_col
    e.b_batch = d.kc * d.b_row;        // B[k, j] at k*b_row + j*b_col
    e.c_row = d.ws_ld;
    e.c_batch = d.M * d.ws_ld;
    e.c_bf16 = false;
    e.c_keep = true;   // the reduction reads the partial sums next
    e.tiles = d.tiles * d.splits;
    e.splits = 1;
    return e;
}

std::shared_ptr<as_gemm_plan> acquire(const as_gemm_plan* p) {
    std::lock_guard<std::mutex> lk(g_plans_mu);
    auto it = p ? plans().find(p) : plans().end();
    return it == plans().end() ? nullptr : it->second;
}

as_status run_desc(const asl::GemmDesc& d, const void* A, const void* B, void* C, void* stream) {
    if (!A || !B || !C) return fail(AS_ERR_INVALID, "null device pointer");
    if (!aligned16(A) || !aligned16(B) || !aligned16(C))
        return fail(AS_ERR_UNSUPPORTED, "device pointers must be 16-byte aligned");
    int e = asl::launch_gemm(d, A, B, C, stream);
    if (e != 0) return fail(AS_ERR_HIP, "kernel launch failed: HIP error %d", e);
    return ok();
}

}  // namespace

extern "C" {

as_status gemm_create(as_gemm_t* out, int64_t M, int64_t N, int64_t K, int64_t batch,
                      as_strides a, as_strides b, as_strides c,
                      as_dtype a_t, as_dtype b_t, as_dtype c_t, uint32_t flags) {
    if (!out) return fail(AS_ERR_INVALID, "null plan output pointer");
    *out = nullptr;
    asl::GemmDesc d;
    as_status s = plan_desc(&d, M, N, K, batch, a, b, c, a_t, b_t, c_t, flags);
    if (s != AS_OK) return s;
    std::shared_ptr<as_gemm_plan> p;
    try {
        p = std::make_shared<as_gemm_plan>();
        p->d = d;
        std::lock_guard<std::mutex> lk(g_plans_mu);
        plans().emplace(p.get(), p);
    } catch (const std::bad_alloc&) {
        return fail(AS_ERR_NOMEM, "out of host memory");
    }
    *out = p.get();
    return ok();
}

as_status gemm_run(as_gemm_t plan, const void* A, const void* B, void* C, void* hip_stream) {
    const std::shared_ptr<as_gemm_plan> p = acquire(plan);
    if (!p) return fail(AS_ERR_INVALID, "null or unknown plan");
    const asl::GemmDesc& d = p->d;
    if (d.splits == 1) return run_desc(d, A, B, C, hip_stream);
    if (!A || !B || !C) return fail(AS_ERR_INVALID, "null device pointer");
    if (!aligned16(A) || !aligned16(B) || !aligned16(C))
        return fail(AS_ERR_UNSUPPORTED, "device pointers must be 16-byte aligned");
    void* ws;
    {
        std::lock_guard<std::mutex> lk(p->ws_mu);
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess) return fail(AS_ERR_HIP, "hipGetDevice failed");
        if (!p->ws || p->ws_dev != dev) {
            if (p->ws) {
                // A run on another device: its workspace moves here.  Freeing
                // waits for the device, which a capture cannot record.
                hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
                if (hipStreamIsCapturing((hipStream_t)hip_stream, &cs) != hipSuccess) {
                    (void)hipGetLastError();
                    cs = hipStreamCaptureStatusNone;
                }
                if (cs != hipStreamCaptureStatusNone)
                    return fail(AS_ERR_UNSUPPORTED, "split-K workspace lives on device %d: run the plan once on "
                                "device %d outside graph capture first", p->ws_dev, dev);
                (void)hipSetDevice(p->ws_dev);
                (void)hipFree(p->ws);
                (void)hipSetDevice(dev);
                p->ws = nullptr;
            }
            // The allocation is not a stream operation: with the calling
            // thread's capture mode relaxed for it (as a caching allocator
            // does), it is allowed while a stream records a graph, and the
            // recorded launches use this workspace on every replay.
            hipStreamCaptureMode mode = hipStreamCaptureModeRelaxed;
            (void)hipThreadExchangeStreamCaptureMode(&mode);
            const hipError_t e = hipMalloc(&p->ws, (size_t)d.ws_bytes);
            (void)hipThreadExchangeStreamCaptureMode(&mode);
            if (e != hipSuccess) {
                p->ws = nullptr;
                (void)hipGetLastError();
                return fail(AS_ERR_NOMEM, "split-K workspace of %" PRId64 " bytes: %s", d.ws_bytes,
                            hipGetErrorString(e));
            }
            p->ws_dev = dev;
        }
        ws = p->ws;
    }
    int e = asl::launch_gemm(split_launch_desc(d), A, B, ws, hip_stream);
    if (e == 0) e = asl::launch_splitk_reduce(d, ws, C, hip_stream);
    if (e != 0) return fail(AS_ERR_HIP, "kernel launch failed: HIP error %d", e);
    return ok();
}

as_status gemm_run_no_alloc(as_gemm_t plan, const void* A, const void* B, void* C, void* hip_stream) {
    const std::shared_ptr<as_gemm_plan> p = acquire(plan);
    if (!p) return fail(AS_ERR_INVALID, "null or unknown plan");
    const asl::GemmDesc& d = p->d;
    if (d.splits == 1) return run_desc(d, A, B, C, hip_stream);   // no workspace: gemm_run itself
    if (!A || !B || !C) return fail(AS_ERR_INVALID, "null device pointer");
    if (!aligned16(A) || !aligned16(B) || !aligned16(C))
        return fail(AS_ERR_UNSUPPORTED, "device pointers must be 16-byte aligned");
    if (d.ws_bytes > asl::kScratchBytes)
        return fail(AS_ERR_UNSUPPORTED, "split-K workspace of %" PRId64 " bytes exceeds the %" PRId64
                    "-byte static scratch array", d.ws_bytes, asl::kScratchBytes);
    void* ws = nullptr;
    if (int e = asl::scratch_address(&ws); e != 0)
        return fail(AS_ERR_HIP, "scratch array address: HIP error %d", e);
    int e = asl::launch_gemm(split_launch_desc(d), A, B, ws, hip_stream);
    if (e == 0) e = asl::launch_splitk_reduce(d, ws, C, hip_stream);
    if (e != 0) return fail(AS_ERR_HIP, "kernel launch failed: HIP error %d", e);
    return ok();
}

as_status gemm_destroy(as_gemm_t plan) {
    std::shared_ptr<as_gemm_plan> p;
    {
        std::lock_guard<std::mutex> lk(g_plans_mu);
        auto it = plan ? plans().find(plan) : plans().end();
        if (it == plans().end()) return fail(AS_ERR_INVALID, "null or unknown plan");
        p = std::move(it->second);
        plans().erase(it);
    }
    p.reset();   // frees the plan here, or at the end of a run still holding it
    return ok();
}

as_status gemm_plan_info(as_gemm_t plan, int32_t* tile_m, int32_t* tile_n, int32_t* tile_k, int64_t* tiles,
                         int64_t* workgroups) {
    const std::shared_ptr<as_gemm_plan> p = acquire(plan);
    if (!p) return fail(AS_ERR_INVALID, "null or unknown plan");
    if (tile_m) *tile_m = p->d.tile;
    if (tile_n) *tile_n = p->d.tile;
    if (tile_k) *tile_k = (int32_t)kBK;
    if (tiles) *tiles = p->d.tiles;
    if (workgroups) *workgroups = p->d.grid;
    return ok();
}

as_status gemm_plan_tile_of(as_gemm_t plan, int64_t workgroup, int64_t* batch, int64_t* tile_row,
                            int64_t* tile_col) {
    const std::shared_ptr<as_gemm_plan> p = acquire(plan);
    if (!p) return fail(AS_ERR_INVALID, "null or unknown plan");
    const asl::GemmDesc L = p->d.splits > 1 ? split_launch_desc(p->d) : p->d;
    if (workgroup < 0 || workgroup >= L.tiles || !batch || !tile_row || !tile_col)
        return fail(AS_ERR_INVALID, "execution slot out of range or null output");
    if (!asl::tile_of_slot(L, workgroup, batch, tile_row, tile_col))
        return fail(AS_ERR_INVALID, "execution slot %" PRId64 " is empty", workgroup);
    return ok();
}

as_status gemm_plan_split_k(as_gemm_t plan, int32_t* splits, int64_t* workspace_bytes) {
    const std::shared_ptr<as_gemm_plan> p = acquire(plan);
    if (!p) return fail(AS_ERR_INVALID, "null or unknown plan");
    if (splits) *splits = p->d.splits;
    if (workspace_bytes) *workspace_bytes = p->d.splits > 1 ? p->d.ws_bytes : 0;
    return ok();
}

as_status sscore_run(const void* Q, const void* K, void* S,
                     int64_t batch, int64_t Lq, int64_t Lk, int64_t dim,
                     as_strides q, as_strides k, as_strides s,
                     as_dtype qk_t, as_dtype s_t, void* hip_stream) {
    if (q.col != 1 || k.col != 1 || s.col != 1) {
        if (q.col < 0 || k.col < 0 || s.col < 0) return fail(AS_ERR_INVALID, "negative stride");
        return fail(AS_ERR_UNSUPPORTED, "Q, K and S need column stride 1");
    }
    // S = Q . K^T: A = Q, B[d, j] = K[j, d] (row stride 1, column stride k.row).
    as_strides a = {q.row, 1, q.batch};
    as_strides b = {1, k.row, k.batch};
    // Plans depend only on the sizes, strides and types: a few recent ones
    // are kept per thread, so a loop of calls plans once.
    struct Cached {
        int64_t key[14];
        asl::GemmDesc d;
    };
    thread_local Cached cache[8];
    thread_local int cached = 0, next_slot = 0;
    const int64_t key[14] = {batch, Lq, Lk, dim, q.row, q.col, q.batch, k.row, k.col, k.batch,
                             s.row, s.batch, (int64_t)qk_t, (int64_t)s_t};
    for (int i = 0; i < cached; ++i)
        if (std::memcmp(cache[i].key, key, sizeof key) == 0) return run_desc(cache[i].d, Q, K, S, hip_stream);
    asl::GemmDesc d;
    as_status st = plan_desc(&d, Lq, Lk, dim, batch, a, b, s, qk_t, qk_t, s_t, AS_FLAG_NO_SPLIT_K);
    if (st != AS_OK) return st;
    Cached& slot = cache[next_slot];
    std::memcpy(slot.key, key, sizeof key);
    slot.d = d;
    next_slot = (next_slot + 1) % 8;
    if (cached < 8) ++cached;
    return run_desc(d, Q, K, S, hip_stream);
}

as_status attn_fwd_run(const void* Q, const void* K, const void* V, void* O, int64_t batch, int64_t Lq,
                       int64_t Lk, int64_t d, int64_t dv, as_strides q, as_strides k, as_strides v,
                       as_strides o, float scale, as_dtype qkv_t, as_dtype o_t, uint32_t flags,
                       void* hip_stream) {
    return attn_fwd_run_gqa(Q, K, V, O, batch, 1, Lq, Lk, d, dv, q, k, v, o, scale, qkv_t, o_t, flags, hip_stream);
}

as_status attn_fwd_run_gqa(const void* Q, const void* K, const void* V, void* O, int64_t batch, int64_t kv_group,
                           int64_t Lq, int64_t Lk, int64_t d, int64_t dv, as_strides q, as_strides k,
                           as_strides v, as_strides o, float scale, as_dtype qkv_t, as_dtype o_t, uint32_t flags,
                           void* hip_stream) {
    if (kv_group <= 0 || (batch > 0 && batch % kv_group))
        return fail(AS_ERR_INVALID, "kv_group must be positive and divide batch (batch=%" PRId64 " kv_group=%" PRId64
                    ")", batch, kv_group);
    if (batch <= 0 || Lq <= 0 || Lk <= 0 || d <= 0 || dv <= 0)
        return fail(AS_ERR_INVALID, "sizes must be positive (batch=%" PRId64 " Lq=%" PRId64 " Lk=%" PRId64
                    " d=%" PRId64 " dv=%" PRId64 ")", batch, Lq, Lk, d, dv);
    for (as_dtype t : {qkv_t, o_t})
        if (t != AS_BF16 && t != AS_F32) return fail(AS_ERR_INVALID, "unknown dtype %d", (int)t);
    if (!std::isfinite(scale)) return fail(AS_ERR_INVALID, "scale must be finite");
    if (as_status st = check_attn_flags(flags); st != AS_OK) return st;
    const bool causal = (flags & AS_ATTN_CAUSAL) != 0;
    if (causal && Lk < Lq)
        return fail(AS_ERR_INVALID, "causal attention needs Lk >= Lq (Lq=%" PRId64 " Lk=%" PRId64 ")", Lq, Lk);
    const int64_t sv[12] = {q.row, q.col, q.batch, k.row, k.col, k.batch, v.row, v.col, v.batch,
                            o.row, o.col, o.batch};
    for (int64_t x : sv)
        if (x < 0) return fail(AS_ERR_INVALID, "negative stride %" PRId64, x);
    if (o.row < dv && Lq > 1) return fail(AS_ERR_INVALID, "O rows overlap (row stride %" PRId64 " < dv)", o.row);
    if (batch > 1 && o.batch < Lq * o.row)
        return fail(AS_ERR_INVALID, "O batches overlap (batch stride %" PRId64 ")", o.batch);
    if (!Q || !K || !V || !O) return fail(AS_ERR_INVALID, "null device pointer");
    if (qkv_t != AS_BF16) return fail(AS_ERR_UNSUPPORTED, "Q, K and V must be bf16");
    if (d != dv || (d != 64 && d != 128))
        return fail(AS_ERR_UNSUPPORTED, "head dimensions d = dv in {64, 128} only (d=%" PRId64 " dv=%" PRId64 ")",
                    d, dv);
    if (q.col != 1 || k.col != 1 || v.col != 1 || o.col != 1)
        return fail(AS_ERR_UNSUPPORTED, "Q, K, V and O need a contiguous last dimension (column stride 1)");
    if (q.row % 8 || k.row % 8 || v.row % 8 || o.row % 4)
        return fail(AS_ERR_UNSUPPORTED, "row strides must be multiples of 8 elements (O: 4)");
    // Batch origins of the slices that are used start 16-byte chunks too
    // (Q is read 16 bytes at a time, K and V by 16-byte LDS-DMA loads).
    if ((batch > 1 && (q.batch % 8 || o.batch % 4)) || (batch / kv_group > 1 && (k.batch % 8 || v.batch % 8)))
        return fail(AS_ERR_UNSUPPORTED, "batch strides must be multiples of 8 elements (O: 4)");
    if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O))
        return fail(AS_ERR_UNSUPPORTED, "device pointers must be 16-byte aligned");
    if (Lq > INT32_MAX / 2 || Lk > INT32_MAX / 2) return fail(AS_ERR_UNSUPPORTED, "sequence too long");
    // 32-bit offsets inside one staged tile of up to 128 keys.
    if (128 * k.row * 2 >= (INT64_C(1) << 31) || 128 * v.row * 2 >= (INT64_C(1) << 31))
        return fail(AS_ERR_UNSUPPORTED, "K or V row stride too large for 32-bit tile offsets");
    asl::AttnDesc ad{};
    ad.batch = batch; ad.Lq = Lq; ad.Lk = Lk; ad.d = d;
    ad.q_row = q.row; ad.q_batch = q.batch;
    ad.k_row = k.row; ad.k_batch = k.batch;
    ad.v_row = v.row; ad.v_batch = v.batch;
    ad.o_row = o.row; ad.o_batch = o.batch;
    ad.o_bf16 = (o_t == AS_BF16);
    ad.causal = causal;
    ad.kv_group = kv_group;
    ad.c = (float)((double)scale * 1.4426950408889634);   // log2(e)
    ad.key_split = attn_key_split(batch, Lq, flags);
    const int64_t bq = asl::attn_queries_per_workgroup(ad.key_split);
    ad.qtiles = (Lq + bq - 1) / bq;
    if (ad.qtiles > INT32_MAX / batch) return fail(AS_ERR_UNSUPPORTED, "too many query tiles");
    ad.tiles = batch * ad.qtiles;
    ad.sched = attn_sched(flags);
    ad.grid = ad.sched == 0 ? ad.tiles : std::min<int64_t>(ad.tiles, kCus);
    if (ad.sched == 2) {
        // A queue launch takes its counters' slot when it is launched; a
        // graph would replay the recorded slot, which an eager launch or
        // another replay may hold at the same time.
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        if (hipStreamIsCapturing((hipStream_t)hip_stream, &cs) != hipSuccess) {
            (void)hipGetLastError();
            cs = hipStreamCaptureStatusNone;
        }
        if (cs != hipStreamCaptureStatusNone)
            return fail(AS_ERR_UNSUPPORTED, "AS_ATTN_SCHED_QUEUE cannot be recorded into a graph capture "
                        "(use the default or the static schedule there)");
    }
    int e = asl::launch_attn(ad, Q, K, V, O, hip_stream);
    if (e != 0) return fail(AS_ERR_HIP, "kernel launch failed: HIP error %d", e);
    return ok();
}

as_status attn_fwd_plan_info(int64_t batch, int64_t Lq, uint32_t flags, int32_t* queries_per_workgroup,
                             int32_t* keys_per_stage, int64_t* workgroups) {
    if (batch <= 0 || Lq <= 0) return fail(AS_ERR_INVALID, "sizes must be positive");
    if (as_status st = check_attn_flags(flags); st != AS_OK) return st;
    const int ks = attn_key_split(batch, Lq, flags);
    const int64_t bq = asl::attn_queries_per_workgroup(ks);
    const int64_t items = batch * ((Lq + bq - 1) / bq);
    if (queries_per_workgroup) *queries_per_workgroup = (int32_t)bq;
    if (keys_per_stage) *keys_per_stage = 64 * ks;
    if (workgroups) *workgroups = attn_sched(flags) == 0 ? items : std::min<int64_t>(items, kCus);
    return ok();
}

as_status tilecast_run(const void* buf, int64_t rows, int64_t cols, int32_t tile_m, int32_t tile_n,
                       int32_t consumers, int32_t group, int32_t grouped, int64_t iters,
                       int64_t warmup, int64_t stride, uint32_t* out_checksum, void* hip_stream) {
    if (!buf || !out_checksum) return fail(AS_ERR_INVALID, "null pointer");
    if (rows <= 0 || cols <= 0 || tile_m <= 0 || tile_n <= 0)
        return fail(AS_ERR_INVALID, "sizes must be positive");
    if (consumers <= 0 || consumers > 4096 || consumers % 8)
        return fail(AS_ERR_INVALID, "consumers must be a positive multiple of 8, at most 4096");
    if (group <= 0 || consumers % group) return fail(AS_ERR_INVALID, "group must divide consumers");
    if (grouped && (consumers / 8) % group)
        return fail(AS_ERR_INVALID, "grouped: group must divide consumers/8 (workgroups per XCD)");
    if (iters < 0 || warmup < 0 || stride < 0) return fail(AS_ERR_INVALID, "negative iteration count or stride");
    if (tile_n % 8) return fail(AS_ERR_UNSUPPORTED, "tile_n must be a multiple of 8");
    if ((int64_t)tile_m * tile_n * 2 > 65536) return fail(AS_ERR_UNSUPPORTED, "tile larger than 64 KiB");
    if (rows % tile_m || cols % tile_n) return fail(AS_ERR_UNSUPPORTED, "matrix not a multiple of the tile");
    if (rows / tile_m > INT32_MAX || cols / tile_n > INT32_MAX) return fail(AS_ERR_UNSUPPORTED, "too many tiles");
    if (!aligned16(buf)) return fail(AS_ERR_UNSUPPORTED, "buffer must be 16-byte aligned");
    if (stride > 0 && (iters + warmup) > INT64_MAX / stride) return fail(AS_ERR_INVALID, "tile index overflow");
    asl::TilecastDesc d{buf, rows, cols, tile_m, tile_n, consumers, group, grouped ? 1 : 0,
                        iters + warmup, stride, out_checksum};
    int e = asl::launch_tilecast(d, hip_stream);
    if (e != 0) return fail(AS_ERR_HIP, "kernel launch failed: HIP error %d", e);
    return ok();
}

const char* as_status_str(as_status s) {
    switch (s) {
        case AS_OK: return "AS_OK";
        case AS_ERR_INVALID: return "AS_ERR_INVALID";
        case AS_ERR_UNSUPPORTED: return "AS_ERR_UNSUPPORTED";
        case AS_ERR_HIP: return "AS_ERR_HIP";
        case AS_ERR_NOMEM: return "AS_ERR_NOMEM";
    }
    return "AS_UNKNOWN_STATUS";
}

const char* as_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
