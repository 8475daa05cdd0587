/*
 * attn_scores.h -- C ABI of the MI355X (gfx950) operand-reuse contraction library.
 *
 * Operations
 *   gemm_*      C[b,i,j] = sum_k A[b,i,k] * B[b,k,j]          (beta = 0, no alpha)
 *   sscore_run  S[b,i,j] = sum_d Q[b,i,d] * K[b,j,d]  = Q.K^T  (no scale, no softmax)
 *   attn_fwd_run  O = softmax(scale * Q.K^T) V, fused (the scores stay on chip)
 *   tilecast_run  tile fan-out microbenchmark
 *
 * Where the operations are defined:
 *   - The GEMM over a tile grid whose rows share an A row-panel and whose
 *     columns share a B column-panel: lesson 07 "Clusters, distributed shared
 *     memory & cluster launch control", section "TMA multicast -- one load,
 *     many CTAs".
 *   - The attention scores S_i = Q_i K^T, computed by neighbouring workgroups
 *     that consume the same key tile: "Hopper TMA Multicast" deep-dive,
 *     Attention/GEMM reuse use-case, equation S_0 = Q_0 K^T, S_1 = Q_1 K^T.
 *     The equation carries no scale and no softmax, and neither does sscore_run.
 *   - The fan-out microbenchmark: same deep-dive, sections "Microbenchmark
 *     source" (128x64 16-bit tiles, consumers loading tile
 *     iteration*stride + group each iteration) and "run results" (hot-tile
 *     and streaming scenarios).
 *
 * Numerics: A and B (Q and K) are bf16; products are accumulated in fp32 by
 * v_mfma_f32_16x16x32_bf16 (256x256 tiles) or v_mfma_f32_32x32x16_bf16
 * (128x128 tiles); C is written as fp32, or rounded to bf16 with
 * round-to-nearest-even.  Results are deterministic run to run: no atomics,
 * and a split-K plan adds its chunks in a fixed order.  The order of the fp32
 * sum depends on the plan (K split, rotated K loop), never on the run.
 *
 * Layout conventions.  All strides are ELEMENT strides (not bytes).  A matrix
 * X[b, r, c] lives at base + b*batch + r*row + c*col.  A batch stride of 0
 * broadcasts one matrix to every batch entry.  For A (M x K) exactly one of
 * row/col must be 1: col == 1 is "K-major" (row-major A), row == 1 is
 * "M-major" (column-major A).  For B (K x N): row == 1 is "K-major" (B given
 * as its transpose, like K in Q.K^T), col == 1 is "N-major" (row-major B).
 * C must have col == 1.  The leading (non-unit) stride of every operand must
 * be a multiple of 8 elements, every base pointer 16-byte aligned, and every
 * batch stride that is used (batch > 1) a multiple of 8 elements (fp32 C and
 * O: 4), so that each batch origin starts a 16-byte chunk.
 *
 * Ownership.  The caller owns every device buffer; the library never
 * allocates, frees or keeps user memory.  A plan (as_gemm_t) is host memory,
 * plus a device workspace when it splits K (gemm_create below).  A plan
 * without a split may be destroyed as soon as gemm_run returns, because
 * kernel arguments are captured by value at launch; a split plan's launches
 * use its workspace until they complete, so a split plan must outlive every
 * HIP graph that recorded one of its runs.  `hip_stream` is the caller's
 * hipStream_t (NULL = the null stream); every run call is asynchronous on it
 * and never synchronizes.  Calls are thread-safe: a run holds the plan for
 * as long as it reads it, so a gemm_destroy on another thread at the same
 * time releases the plan only when that run returns.  as_last_error() is
 * per-thread.
 *
 * Errors.  Every entry point returns an as_status.  All argument checks
 * happen before any HIP call, so invalid calls are rejected without a GPU:
 *   AS_ERR_INVALID      null/negative/zero sizes, null pointers, an output
 *                       whose rows or batches overlap, unknown flags or
 *                       dtypes, a null or unknown plan
 *   AS_ERR_UNSUPPORTED  a well-formed request the kernels do not cover
 *                       (operand dtypes other than bf16, a contiguous stride
 *                       other than 1, unaligned pointers, leading or batch
 *                       strides, K not a multiple of 8)
 *   AS_ERR_HIP          a HIP launch error (the text is in as_last_error())
 *   AS_ERR_NOMEM        host allocation of a plan failed
 * Nothing is ever computed silently wrong: an unsupported case is refused.
 */
#ifndef ATTN_SCORES_H
#define ATTN_SCORES_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__) || defined(__clang__)
#define AS_API __attribute__((visibility("default")))
#else
#define AS_API
#endif

typedef enum {
    AS_OK = 0,
    AS_ERR_INVALID = 1,
    AS_ERR_UNSUPPORTED = 2,
    AS_ERR_HIP = 3,
    AS_ERR_NOMEM = 4
} as_status;

typedef enum { AS_BF16 = 0, AS_F32 = 1 } as_dtype;

/* Element strides of X[b, r, c]. */
typedef struct {
    int64_t row;
    int64_t col;
    int64_t batch;
} as_strides;

/* gemm_create flags */
#define AS_FLAG_NO_GROUPING 0x1u  /* ablation: workgroup id -> tile is the identity (row-major tile order) */
#define AS_FLAG_TILE_128    0x2u  /* force 128x128 output tiles */
#define AS_FLAG_TILE_256    0x4u  /* force 256x256 output tiles */
#define AS_FLAG_TILE_64     0x400u /* force 64x64 output tiles (8 K stages in flight) */
#define AS_FLAG_ONE_TILE_PER_WORKGROUP 0x8u  /* ablation: one workgroup per output tile instead of a resident
                                               * (persistent) grid whose workgroups walk several tiles */
#define AS_FLAG_NO_SPLIT_K  0x10u /* never split K over workgroups (no workspace) */
#define AS_FLAG_NT_A        0x20u /* load A with the non-temporal hint (the default when every A row panel
                                   * feeds a single output tile) */
#define AS_FLAG_NO_NT_A     0x40u /* ablation: ordinary loads for A */
#define AS_FLAG_ROTATE_K    0x80u /* tile row tm starts its K loop at K stage tm mod (K / 64): concurrent tiles read
                                   * different K columns (the default when every A row panel feeds a single tile) */
#define AS_FLAG_NO_ROTATE_K 0x100u /* ablation: every tile walks K from 0 */
#define AS_FLAG_NO_XCD_SPLIT 0x200u /* ablation: the grouped band order of tiles, but workgroup h takes its tiles
                                     * h, h + grid, ... of that order instead of a range owned by its XCD, so
                                     * tiles that share panels run on different XCDs (no effect with
                                     * AS_FLAG_NO_GROUPING) */

typedef struct as_gemm_plan* as_gemm_t;

/*
 * Plan C = A.B for `batch` independent (M x K).(K x N) products.
 *   out          receives the plan handle (host memory)
 *   M, N, K      sizes, > 0; M and N arbitrary, K a multiple of 8.  Edge tiles
 *                are partial: operand reads past M, N or K return zero
 *                (range-checked buffer loads) and only C[0..M) x [0..N) is
 *                written.
 *   batch        number of products, > 0
 *   a, b, c      element strides of A[b,i,k], B[b,k,j], C[b,i,j]
 *   a_t, b_t     must be AS_BF16
 *   c_t          AS_F32, or AS_BF16 (round-to-nearest-even)
 *   flags        AS_FLAG_* bits
 * Chooses the output tile (256x256 with 8 waves, 128x128 with 4, or 64x64
 * with 4 for a grid of 128x128 tiles that would fill at most a quarter of
 * the CUs without splitting K), the workgroup grouping and the grid: by
 * default as many workgroups as stay resident (256 for the 256x256 and
 * 64x64 tiles, 512 for 128x128; fewer if there are fewer tiles), each
 * walking several tiles.  Makes no HIP call.
 * Split K: when batch == 1 and there are fewer output tiles than the 256
 * CUs, the plan splits K into 2, 4, 8 or 16 equal chunks
 * (each a multiple of 64 and at least 1024 deep), as many as keep tiles x
 * chunks within the resident grid.  Each chunk's product goes to an fp32
 * slice of a workspace and a second kernel adds the slices in chunk order
 * into C (deterministic; the sum is ordered differently from an unsplit
 * product, within the same rounding bound).  The workspace
 * (gemm_plan_split_k) is device memory that the plan allocates on its first
 * gemm_run on a device and frees in gemm_destroy; runs of one plan share it,
 * so they must not overlap (the same stream, or ordered streams).
 * AS_FLAG_NO_SPLIT_K turns splitting off.
 * Streaming A: when N fits one output tile, each A row panel is read by one
 * workgroup only and streams from HBM.  The plan then (1) loads A with the
 * non-temporal hint, so its lines leave L2 before B's, which every tile
 * re-reads, and (2) rotates the K loop: tile row tm accumulates its K
 * stages starting at stage tm mod (K / 64), so the workgroups running at
 * one time read different K columns of A instead of one column block of
 * every row.  Rotation changes only the order of the fp32 accumulation.
 * AS_FLAG_NT_A / AS_FLAG_NO_NT_A and AS_FLAG_ROTATE_K / AS_FLAG_NO_ROTATE_K
 * override the two choices; each pair is exclusive.
 */
AS_API as_status gemm_create(as_gemm_t* out, int64_t M, int64_t N, int64_t K, int64_t batch,
                      as_strides a, as_strides b, as_strides c,
                      as_dtype a_t, as_dtype b_t, as_dtype c_t, uint32_t flags);

/* Launch the planned product on `hip_stream`.  A, B: device bf16; C: device
 * fp32 or bf16 as planned.  Pointers must be 16-byte aligned.  A split plan
 * launches two kernels and, on its first run on a device, allocates its
 * workspace (hipMalloc; AS_ERR_NOMEM if that fails).
 * Graph capture: the launches clear and synchronize nothing, so a run may be
 * recorded into a HIP graph on a capturing stream and replayed.  A split
 * plan's first run on a device allocates its workspace even while a stream
 * records (with the calling thread's capture mode relaxed for the
 * allocation, which is not a stream operation); a replay reuses the pointers
 * and the workspace of the recorded run, so the plan must outlive the graph.
 * A plan whose workspace lives on another device moves it only outside
 * capture (inside, AS_ERR_UNSUPPORTED and nothing is recorded). */
AS_API as_status gemm_run(as_gemm_t plan, const void* A, const void* B, void* C, void* hip_stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): gemm_run
 * without any allocation.  A plan that does not split K runs exactly as in
 * gemm_run.  A split plan's partial sums go to the library's static scratch
 * array instead of the plan's own workspace: 64 MiB of device memory per
 * GPU, held from the loading of the library's kernels until the process
 * ends, which covers every workspace the planner makes (gemm_plan_split_k
 * reports the bytes; a larger one would be refused with
 * AS_ERR_UNSUPPORTED).  The first call on a device looks up that device's
 * array address (hipGetSymbolAddress; no allocation).  Every call on a GPU
 * shares its one array, which keeps the last call's contents (nothing in it
 * needs to start at zero): calls that overlap on one GPU -- on different
 * streams, or from threads whose calls are not otherwise ordered -- race and
 * give wrong results; calls on one stream are ordered and safe.  Results
 * are bitwise those of gemm_run.  Errors as for gemm_run. */
AS_API as_status gemm_run_no_alloc(as_gemm_t plan, const void* A, const void* B, void* C, void* hip_stream);

/* Whether a plan splits K: number of K chunks (1: no split) and the bytes
 * of device workspace its runs use (0 without a split).  Any output pointer
 * may be NULL.  AS_ERR_INVALID on a bad plan. */
AS_API as_status gemm_plan_split_k(as_gemm_t plan, int32_t* splits, int64_t* workspace_bytes);

/* Release a plan created by gemm_create (NULL or unknown -> AS_ERR_INVALID).
 * Frees a split plan's workspace (hipFree, which waits for the device), so
 * a graph that recorded a run of it must not be replayed afterwards, and a
 * split plan must not be destroyed while a stream records a graph.  A run
 * of the plan in progress on another thread keeps it until that run
 * returns.  The handle is dead afterwards; a later gemm_create may return
 * the same value. */
AS_API as_status gemm_destroy(as_gemm_t plan);

/* What a plan chose (for reporting): output tile shape and K stage depth,
 * the number of output tiles, and the number of workgroups launched (equal
 * to the tiles, or fewer when the grid is persistent and each workgroup walks
 * several tiles).  Any output pointer may be NULL.  AS_ERR_INVALID on a bad
 * plan. */
AS_API as_status gemm_plan_info(as_gemm_t plan, int32_t* tile_m, int32_t* tile_n, int32_t* tile_k,
                                int64_t* tiles, int64_t* workgroups);

/* Output tile computed in execution slot `slot` (0 <= slot < tiles): slot
 * i is round i div W of hardware workgroup i mod W (W = workgroups), which
 * runs on XCD i mod 8.  Writes batch index, tile row and tile column under
 * the plan's XCD-aware grouped order.  Host-only; for inspection and tests. */
AS_API as_status gemm_plan_tile_of(as_gemm_t plan, int64_t slot, int64_t* batch, int64_t* tile_row,
                                   int64_t* tile_col);

/*
 * Attention scores S[b,i,j] = sum_d Q[b,i,d] * K[b,j,d] for b < batch,
 * i < Lq, j < Lk, d < dim.  Q is [batch, Lq, dim], K is [batch, Lk, dim],
 * S is [batch, Lq, Lk], each addressed by its own (row, col, batch) element
 * strides with col == 1 for all three (the head dimension and the key index
 * contiguous).  qk_t must be AS_BF16; s_t AS_F32 or AS_BF16.  This is the
 * GEMM with A = Q and B = K^T, planned and launched in one call (same
 * kernels, same errors).  The plans of the last 8 distinct size/stride/type
 * combinations are kept per calling thread (host memory only), so a loop of
 * calls plans once.  Asynchronous on `hip_stream`.  It never splits K, so
 * every call may be recorded into a HIP graph (see gemm_run).
 */
AS_API as_status sscore_run(const void* Q, const void* K, void* S,
                     int64_t batch, int64_t Lq, int64_t Lk, int64_t dim,
                     as_strides q, as_strides k, as_strides s,
                     as_dtype qk_t, as_dtype s_t, void* hip_stream);

/*
 * Attention forward O[b] = softmax(scale * Q[b] K[b]^T) V[b]: for every
 * query i, O[b,i,:] = sum_j p_j V[b,j,:] / sum_j p_j with
 * p_j = exp(scale * S[b,i,j] - max_j scale * S[b,i,j]) and S the scores of
 * sscore_run.  With AS_ATTN_CAUSAL in `flags`, query i sees only keys
 * j <= i + (Lk - Lq) (the mask aligned to the last key: with Lq == Lk,
 * keys 0..i; Lk >= Lq required, AS_ERR_INVALID otherwise); lesson 07 names
 * causal attention as the case whose tiles cost different amounts ("The
 * second wall: the static schedule's tail").  The score product is the inner step of the
 * FlashAttention-class operators whose neighbouring query tiles consume the
 * same key and value tiles ("Hopper TMA Multicast" deep-dive, Attention/GEMM
 * reuse use-case and the comparison table's "Attention K/V" row); the
 * softmax is the textbook scaled dot-product attention, which the pages name
 * but do not write out.  One fused kernel: the scores stay in registers.
 *   Q [batch, Lq, d], K [batch, Lk, d], V [batch, Lk, dv], O [batch, Lq, dv],
 *   each addressed by (row, col, batch) element strides with col == 1;
 *   row strides multiples of 8 (O: 4), pointers 16-byte aligned, batch
 *   strides of the slices used multiples of 8 (O: 4).
 *   d == dv, 64 or 128.  Lq, Lk >= 1, any length.  qkv_t AS_BF16; o_t AS_BF16
 *   (round-to-nearest-even) or AS_F32.  scale finite.
 * Numerics: scores accumulate in fp32; probabilities are rounded to bf16
 * before the P.V product (fp32 accumulation); the result is divided by the
 * fp32 sum of the unrounded probabilities.  Errors as for the other entry
 * points (AS_ERR_UNSUPPORTED: other head sizes, dtypes, strides or
 * alignments).  Asynchronous on `hip_stream`.
 * Work items: one workgroup computes 256 queries of a slice over all the keys
 * they see, or 128 queries with the keys of each stage split over two waves
 * and merged at the end.  By default the 128-query items are used with the
 * causal mask (items then cost different amounts, and shorter ones balance
 * better; they are launched heaviest first) and when 256-query items would
 * number fewer than the 256 CUs; AS_ATTN_QUERIES_256 / AS_ATTN_QUERIES_128
 * force one shape (AS_ERR_INVALID if both).  The shapes sum in different
 * orders, so their results differ within the rounding bound; each is
 * deterministic run to run.
 * Schedule: by default one workgroup per item, which the dispatcher starts
 * in id order as CUs free up (with the causal mask the ids run heaviest
 * item first).  AS_ATTN_SCHED_STATIC / AS_ATTN_SCHED_QUEUE launch instead a
 * persistent grid of one workgroup per CU that walks the items by a static
 * stride, or claims each next item from a per-XCD queue two key stages
 * before its current item ends (lesson 07 "Clusters, distributed shared
 * memory & cluster launch control": "The second wall: the static
 * schedule's tail" and "The work-stealing loop").  Every schedule gives
 * bitwise the same O.  The queue counters live in the library (64 slots per
 * device, taken in turn by successive launches; each launch leaves its slot
 * at zero): at most 64 queue launches may run at once on one device.
 * Graph capture: a launch allocates and clears nothing, so the default and
 * the static schedules may be recorded into a HIP graph and replayed.  A
 * queue launch takes its counters' slot at launch time, and a replay would
 * reuse the recorded slot while an eager launch or another replay may hold
 * it: AS_ATTN_SCHED_QUEUE on a capturing stream returns AS_ERR_UNSUPPORTED
 * and records nothing.
 */
#define AS_ATTN_CAUSAL 0x1u   /* attn_fwd_run: query i sees keys j <= i + (Lk - Lq) only */
#define AS_ATTN_QUERIES_256 0x2u  /* force work items of 256 queries (each wave sweeps all keys) */
#define AS_ATTN_QUERIES_128 0x4u  /* force work items of 128 queries (two waves split each key stage) */
#define AS_ATTN_SCHED_STATIC 0x8u /* persistent grid (one workgroup per CU), items by a static stride */
#define AS_ATTN_SCHED_QUEUE 0x10u /* persistent grid, items claimed from a per-XCD work queue */

AS_API as_status attn_fwd_run(const void* Q, const void* K, const void* V, void* O,
                              int64_t batch, int64_t Lq, int64_t Lk, int64_t d, int64_t dv,
                              as_strides q, as_strides k, as_strides v, as_strides o,
                              float scale, as_dtype qkv_t, as_dtype o_t, uint32_t flags,
                              void* hip_stream);

/*
 * Attention forward with grouped key/value heads: as attn_fwd_run, but query
 * slice b (0 <= b < batch) attends to key/value slice b / kv_group, so K and
 * V hold batch / kv_group slices (their batch strides step over those).
 * kv_group must be positive and divide batch (AS_ERR_INVALID otherwise);
 * kv_group == 1 is attn_fwd_run.  Query slices sharing K and V are many
 * consumers of the same key/value tiles, the reuse the deep-dive's
 * Attention/GEMM use-case describes: with the causal mask and batch a
 * multiple of 8 each XCD runs a contiguous block of slices, so a group's
 * K and V come from HBM once per XCD.
 */
AS_API as_status attn_fwd_run_gqa(const void* Q, const void* K, const void* V, void* O,
                                  int64_t batch, int64_t kv_group, int64_t Lq, int64_t Lk, int64_t d, int64_t dv,
                                  as_strides q, as_strides k, as_strides v, as_strides o,
                                  float scale, as_dtype qkv_t, as_dtype o_t, uint32_t flags, void* hip_stream);

/* The work items attn_fwd_run chooses for `batch` slices of Lq queries under
 * `flags`: queries per workgroup (256 or 128), keys per LDS stage (64 or
 * 128) and workgroups launched.  Any output pointer may be NULL.  Host-only,
 * no HIP call; AS_ERR_INVALID on non-positive sizes or bad flags. */
AS_API as_status attn_fwd_plan_info(int64_t batch, int64_t Lq, uint32_t flags, int32_t* queries_per_workgroup,
                                    int32_t* keys_per_stage, int64_t* workgroups);

/*
 * Tile fan-out microbenchmark.  `consumers` workgroups (a multiple of 8, at
 * most 4096) each load, once per iteration, one tile_m x tile_n tile of the
 * bf16 row-major matrix `buf` (rows x cols, leading dimension cols) into
 * LDS with 128-bit loads.  In iteration `it` the workgroups of group g load
 * tile index it*stride + g, at tile row ((it*stride+g) div (cols/tile_n))
 * mod (rows/tile_m) and tile column (it*stride+g) mod (cols/tile_n).
 * Groups hold `group` workgroups:
 *   grouped != 0  members run on one XCD: workgroup w runs on XCD w mod 8
 *                 and is the (w div 8)-th there; `group` consecutive ones of
 *                 an XCD form a group (so `group` must divide consumers/8);
 *   grouped == 0  members are `group` consecutive workgroup ids.
 * The launch runs warmup + iters iterations (it = 0 .. warmup+iters-1; the
 * split only mirrors the deep-dive's kernel arguments).  out_checksum
 * (device, 2*consumers uint32) receives, per workgroup w: [2w] the sum
 * modulo 2^32 of every little-endian 32-bit word of every tile it loaded in
 * all iterations, and [2w+1] the same sum over the tile held in its LDS at
 * the end (the last one loaded).
 * tile_n must be a multiple of 8, tile_m*tile_n*2 at most 65536 bytes, rows
 * and cols multiples of tile_m and tile_n.  Asynchronous on `hip_stream`.
 */
AS_API as_status tilecast_run(const void* buf, int64_t rows, int64_t cols, int32_t tile_m, int32_t tile_n,
                       int32_t consumers, int32_t group, int32_t grouped, int64_t iters,
                       int64_t warmup, int64_t stride, uint32_t* out_checksum, void* hip_stream);

/* Static text for a status code. */
AS_API const char* as_status_str(as_status s);

/* Text of the last error reported on the calling thread ("" if none). */
AS_API const char* as_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_SCORES_H */
