/*
 * oracle.c -- plain CPU reference for the dense bf16 contractions.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  It shares no code,
 * header, table or helper with the GPU library and includes nothing from it.
 *
 * What is computed, and where the pages define it:
 *
 *  - The GEMM C = A.B over a tile grid in which the output tiles of one grid
 *    row consume the same A row-panel and those of one grid column the same B
 *    column-panel (lesson 07 "Clusters, distributed shared memory & cluster
 *    launch control", section "TMA multicast -- one load, many CTAs").
 *  - The attention-score product S_i = Q_i K^T, where the query tiles of
 *    neighbouring workgroups consume one and the same key tile ("Hopper TMA
 *    Multicast" deep-dive, section on the Attention/GEMM reuse use-case, the
 *    CTA0/CTA1 equation S_0 = Q_0 K^T, S_1 = Q_1 K^T).  No scale factor and no
 *    softmax are applied: the pages' equation has none.
 *  - Attention forward O = softmax(scale * Q K^T) V, the FlashAttention-class
 *    operator the score product belongs to (see oracle_attention).
 *  - The tile fan-out microbenchmark's accounting and data checksum (same
 *    deep-dive, sections "Microbenchmark source" and "run results": each
 *    iteration every consumer loads the tile with index
 *    iteration*stride + group, at tile coordinates
 *    (idx mod tiles_x, (idx div tiles_x) mod tiles_y); traffic is
 *    consumers x iterations x tile bytes).
 *
 * Arithmetic: every bf16 input is decoded exactly to double.  For each output
 * element the products a*b are formed in double (exact: two 8-bit
 * significands give at most 16 significant bits) and summed in ascending k
 * order, together with the magnitude sum T = sum_k |a*b| that the tolerance
 * |C_gpu - C| <= 1e-3*T + 1e-5 is stated against.  No blocking, fusion or
 * reordering of the k sum.  Threads split the output rows only.
 *
 * All strides are ELEMENT strides: X[b,r,c] lives at b*s_batch + r*s_row +
 * c*s_col.  A batch stride of 0 broadcasts one matrix to every batch.
 *
 * Built with plain gcc -O2 (no fast-math) as liboracle.so.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

/* ---------------------------------------------------------------- bf16 -- */

/* bf16 is the upper half of an IEEE binary32: decode is a 16-bit shift. */
double oracle_bf16_to_f64(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/*
 * Round a double to the nearest bf16, ties to even (diagnostics and the
 * bit-exact integer pin of bf16 outputs).  Written from the definition:
 * bf16 has 8 significant bits, the binary32 exponent range, subnormals with
 * quantum 2^-133, and overflow to infinity.
 */
uint16_t oracle_f64_to_bf16_rne(double x) {
    uint16_t sign = signbit(x) ? 0x8000u : 0u;
    double ax = fabs(x);
    if (isnan(x)) return (uint16_t)(sign | 0x7fc0u);
    if (isinf(x)) return (uint16_t)(sign | 0x7f80u);
    if (ax == 0.0) return sign;
    int e;
    (void)frexp(ax, &e);               /* ax = m * 2^e, 0.5 <= m < 1 */
    int q_exp = e - 8;                 /* quantum of an 8-bit significand */
    if (q_exp < -133) q_exp = -133;    /* subnormal range */
    double q = ldexp(ax, -q_exp);      /* exact: scaling by a power of two */
    double fl = floor(q);
    double frac = q - fl;
    if (frac > 0.5 || (frac == 0.5 && fmod(fl, 2.0) != 0.0)) fl += 1.0;
    double r = ldexp(fl, q_exp);
    if (r >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7f80u);
    float rf = (float)r;               /* exact: r has <= 8 significant bits */
    uint32_t u;
    memcpy(&u, &rf, sizeof u);
    return (uint16_t)(sign | (uint16_t)((u >> 16) & 0x7fffu));
}

/* ---------------------------------------------------------------- GEMM -- */

typedef struct {
    const uint16_t *A, *B;
    double *C, *T;
    int64_t batch, M, N, K;
    int64_t a_row, a_col, a_batch, b_row, b_col, b_batch;
    int64_t row_begin, row_end;      /* flattened (batch, i) rows */
} gemm_job;

/* One output row: C[b,i,j] = sum_k A[b,i,k] * B[b,k,j], k ascending. */
static void gemm_row(const gemm_job* g, int64_t bi, double* acc, double* mag) {
    int64_t b = bi / g->M, i = bi % g->M;
    const uint16_t* a = g->A + b * g->a_batch + i * g->a_row;
    const uint16_t* bm = g->B + b * g->b_batch;
    for (int64_t j = 0; j < g->N; ++j) { acc[j] = 0.0; mag[j] = 0.0; }
    for (int64_t k = 0; k < g->K; ++k) {
        double aik = oracle_bf16_to_f64(a[k * g->a_col]);
        const uint16_t* brow = bm + k * g->b_row;
        for (int64_t j = 0; j < g->N; ++j) {
            double p = aik * oracle_bf16_to_f64(brow[j * g->b_col]);
            acc[j] += p;
            mag[j] += fabs(p);
        }
    }
    double* c = g->C + bi * g->N;
    double* t = g->T ? g->T + bi * g->N : NULL;
    for (int64_t j = 0; j < g->N; ++j) {
        c[j] = acc[j];
        if (t) t[j] = mag[j];
    }
}

static void* gemm_worker(void* arg) {
    const gemm_job* g = (const gemm_job*)arg;
    double* acc = (double*)malloc(sizeof(double) * (size_t)g->N);
    double* mag = (double*)malloc(sizeof(double) * (size_t)g->N);
    if (!acc || !mag) { free(acc); free(mag); return (void*)1; }
    for (int64_t bi = g->row_begin; bi < g->row_end; ++bi) gemm_row(g, bi, acc, mag);
    free(acc);
    free(mag);
    return NULL;
}

static int resolve_threads(int nthreads) {
    if (nthreads > 0) return nthreads;
    long n = sysconf(_SC_NPROCESSORS_ONLN);
    return n > 0 ? (int)n : 1;
}

/*
 * Full product.  C and T (T may be NULL) are dense row-major
 * [batch][M][N] doubles.  Returns 0, or -1 on bad arguments / no memory.
 */
int oracle_gemm(const uint16_t* A, const uint16_t* B, double* C, double* T,
                int64_t batch, int64_t M, int64_t N, int64_t K,
                int64_t a_row, int64_t a_col, int64_t a_batch,
                int64_t b_row, int64_t b_col, int64_t b_batch, int nthreads) {
    if (!A || !B || !C || batch <= 0 || M <= 0 || N <= 0 || K <= 0) return -1;
    int nt = resolve_threads(nthreads);
    int64_t rows = batch * M;
    if (nt > rows) nt = (int)rows;
    pthread_t* th = (pthread_t*)calloc((size_t)nt, sizeof(pthread_t));
    gemm_job* jobs = (gemm_job*)calloc((size_t)nt, sizeof(gemm_job));
    if (!th || !jobs) { free(th); free(jobs); return -1; }
    int rc = 0;
    for (int t = 0; t < nt; ++t) {
        gemm_job g = {A, B, C, T, batch, M, N, K, a_row, a_col, a_batch,
                      b_row, b_col, b_batch, rows * t / nt, rows * (t + 1) / nt};
        jobs[t] = g;
        if (pthread_create(&th[t], NULL, gemm_worker, &jobs[t]) != 0) { jobs[t].row_end = -1; rc = -1; }
    }
    for (int t = 0; t < nt; ++t) {
        if (jobs[t].row_end < 0) continue;
        void* ret = NULL;
        pthread_join(th[t], &ret);
        if (ret) rc = -1;
    }
    free(th);
    free(jobs);
    return rc;
}

/*
 * Selected elements only: pts holds npts triples (b, i, j).  Same arithmetic
 * as oracle_gemm, element by element, for checks at sizes where the full
 * product is out of reach on the CPU.
 */
typedef struct {
    const uint16_t *A, *B;
    const int64_t* pts;
    double *C, *T;
    int64_t K, a_row, a_col, a_batch, b_row, b_col, b_batch;
    int64_t begin, end;
} points_job;

static void* points_worker(void* arg) {
    const points_job* g = (const points_job*)arg;
    for (int64_t p = g->begin; p < g->end; ++p) {
        int64_t b = g->pts[3 * p], i = g->pts[3 * p + 1], j = g->pts[3 * p + 2];
        const uint16_t* a = g->A + b * g->a_batch + i * g->a_row;
        const uint16_t* bb = g->B + b * g->b_batch + j * g->b_col;
        double acc = 0.0, mag = 0.0;
        for (int64_t k = 0; k < g->K; ++k) {
            double prod = oracle_bf16_to_f64(a[k * g->a_col]) * oracle_bf16_to_f64(bb[k * g->b_row]);
            acc += prod;
            mag += fabs(prod);
        }
        g->C[p] = acc;
        if (g->T) g->T[p] = mag;
    }
    return NULL;
}

int oracle_gemm_points(const uint16_t* A, const uint16_t* B, const int64_t* pts, int64_t npts,
                       double* C, double* T, int64_t K,
                       int64_t a_row, int64_t a_col, int64_t a_batch,
                       int64_t b_row, int64_t b_col, int64_t b_batch, int nthreads) {
    if (!A || !B || !pts || !C || npts < 0 || K <= 0) return -1;
    if (npts == 0) return 0;
    int nt = resolve_threads(nthreads);
    if (nt > npts) nt = (int)npts;
    pthread_t* th = (pthread_t*)calloc((size_t)nt, sizeof(pthread_t));
    points_job* jobs = (points_job*)calloc((size_t)nt, sizeof(points_job));
    if (!th || !jobs) { free(th); free(jobs); return -1; }
    int rc = 0;
    for (int t = 0; t < nt; ++t) {
        points_job g = {A, B, pts, C, T, K, a_row, a_col, a_batch, b_row, b_col, b_batch,
                        npts * t / nt, npts * (t + 1) / nt};
        jobs[t] = g;
        if (pthread_create(&th[t], NULL, points_worker, &jobs[t]) != 0) { jobs[t].end = -1; rc = -1; }
    }
    for (int t = 0; t < nt; ++t)
        if (jobs[t].end >= 0) pthread_join(th[t], NULL);
    free(th);
    free(jobs);
    return rc;
}

/*
 * Attention scores S[b,i,j] = sum_d Q[b,i,d] * K[b,j,d]: the product with
 * the transpose of K, i.e. the GEMM whose B operand is B[b,d,j] = K[b,j,d].
 * The transpose is taken by exchanging K's row and column strides.
 */
int oracle_sscore(const uint16_t* Q, const uint16_t* Kt, double* S, double* T,
                  int64_t batch, int64_t Lq, int64_t Lk, int64_t d,
                  int64_t q_row, int64_t q_col, int64_t q_batch,
                  int64_t k_row, int64_t k_col, int64_t k_batch, int nthreads) {
    return oracle_gemm(Q, Kt, S, T, batch, Lq, Lk, d, q_row, q_col, q_batch,
                       /* B row (index d) */ k_col, /* B column (index j) */ k_row, k_batch, nthreads);
}

int oracle_sscore_points(const uint16_t* Q, const uint16_t* Kt, const int64_t* pts, int64_t npts,
                         double* S, double* T, int64_t d,
                         int64_t q_row, int64_t q_col, int64_t q_batch,
                         int64_t k_row, int64_t k_col, int64_t k_batch, int nthreads) {
    return oracle_gemm_points(Q, Kt, pts, npts, S, T, d, q_row, q_col, q_batch,
                              k_col, k_row, k_batch, nthreads);
}

/* ---------------------------------------------------- attention forward -- */

/*
 * Attention forward over the same Q and K: O = softmax(scale * Q K^T) V.
 * The pages introduce the score product as the inner step of
 * FlashAttention-class operators whose neighbouring query tiles consume the
 * same key and value tiles ("Hopper TMA Multicast" deep-dive, Attention/GEMM
 * reuse use-case and the comparison table's "Attention K/V" row); they do
 * not spell out the softmax, so this is the textbook scaled-dot-product
 * attention, without a mask:
 *   S[b,i,j] = sum_d Q[b,i,d] K[b,j,d]               (d ascending, exact)
 *   t_j      = scale * S[b,i,j]
 *   p_j      = exp(t_j - max_j t_j)                  (the max only keeps
 *                                                      exp in range)
 *   O[b,i,c] = sum_j p_j V[b,j,c] / sum_j p_j        (j ascending)
 * and, for the tolerance of a result whose p_j pass through bf16,
 *   TO[b,i,c] = sum_j p_j |V[b,j,c]| / sum_j p_j.
 * Rows are the flattened (b, i) pairs listed in `rows` (npairs of them), or
 * every one of batch*Lq when rows is NULL; O and TO are [rows][dv].
 *
 * causal != 0: query i sees only keys j <= i + (Lk - Lq), the sums above
 * running over those keys alone (the last query sees every key; with
 * Lq == Lk, query i sees keys 0..i).  Lesson 07 ("The second wall: the static
 * schedule's tail") names causal attention as the case whose tiles cost
 * different amounts; the mask itself is the textbook one, aligned to the
 * last key so that a query block appended after a key cache sees the cache.
 * Requires Lk >= Lq, so that every query sees at least one key.
 *
 * kv_group: query slice b reads key/value slice b / kv_group (grouped
 * key/value heads; 1: each query slice has its own).  The grouping only
 * decides which K and V a slice reads; the arithmetic above is unchanged.
 */
typedef struct {
    const uint16_t *Q, *K, *V;
    const int64_t* rows;
    double *O, *TO;
    int64_t Lq, Lk, d, dv;
    int64_t q_row, q_col, q_batch, k_row, k_col, k_batch, v_row, v_col, v_batch;
    double scale;
    int causal;
    int64_t kv_group;
    int64_t begin, end;
} attn_job;

static void* attn_worker(void* arg) {
    const attn_job* g = (const attn_job*)arg;
    double* t = (double*)malloc(sizeof(double) * (size_t)g->Lk);
    if (!t) return (void*)1;
    for (int64_t r = g->begin; r < g->end; ++r) {
        int64_t b, i;
        if (g->rows) { b = g->rows[2 * r]; i = g->rows[2 * r + 1]; }
        else { b = r / g->Lq; i = r % g->Lq; }
        const uint16_t* q = g->Q + b * g->q_batch + i * g->q_row;
        const int64_t bk = b / g->kv_group;                                /* key/value slice */
        const int64_t nk = g->causal ? i + (g->Lk - g->Lq) + 1 : g->Lk;   /* keys 0 .. nk-1 */
        double m = -INFINITY;
        for (int64_t j = 0; j < nk; ++j) {
            const uint16_t* k = g->K + bk * g->k_batch + j * g->k_row;
            double s = 0.0;
            for (int64_t x = 0; x < g->d; ++x)
                s += oracle_bf16_to_f64(q[x * g->q_col]) * oracle_bf16_to_f64(k[x * g->k_col]);
            t[j] = g->scale * s;
            if (t[j] > m) m = t[j];
        }
        double l = 0.0;
        for (int64_t j = 0; j < nk; ++j) {
            t[j] = exp(t[j] - m);
            l += t[j];
        }
        double* o = g->O + r * g->dv;
        double* to = g->TO ? g->TO + r * g->dv : NULL;
        for (int64_t c = 0; c < g->dv; ++c) {
            double acc = 0.0, mag = 0.0;
            for (int64_t j = 0; j < nk; ++j) {
                double v = oracle_bf16_to_f64(g->V[bk * g->v_batch + j * g->v_row + c * g->v_col]);
                acc += t[j] * v;
                mag += t[j] * fabs(v);
            }
            o[c] = acc / l;
            if (to) to[c] = mag / l;
        }
    }
    free(t);
    return NULL;
}

int oracle_attention(const uint16_t* Q, const uint16_t* K, const uint16_t* V, const int64_t* rows,
                     int64_t npairs, double* O, double* TO, int64_t batch, int64_t Lq, int64_t Lk,
                     int64_t d, int64_t dv, int64_t q_row, int64_t q_col, int64_t q_batch,
                     int64_t k_row, int64_t k_col, int64_t k_batch,
                     int64_t v_row, int64_t v_col, int64_t v_batch, double scale, int causal, int64_t kv_group,
                     int nthreads) {
    if (!Q || !K || !V || !O || batch <= 0 || Lq <= 0 || Lk <= 0 || d <= 0 || dv <= 0) return -1;
    if (kv_group <= 0 || batch % kv_group) return -1;
    if (causal && Lk < Lq) return -1;
    int64_t n = rows ? npairs : batch * Lq;
    if (n < 0) return -1;
    if (n == 0) return 0;
    int nt = resolve_threads(nthreads);
    if (nt > n) nt = (int)n;
    pthread_t* th = (pthread_t*)calloc((size_t)nt, sizeof(pthread_t));
    attn_job* jobs = (attn_job*)calloc((size_t)nt, sizeof(attn_job));
    if (!th || !jobs) { free(th); free(jobs); return -1; }
    int rc = 0;
    for (int w = 0; w < nt; ++w) {
        attn_job g = {Q, K, V, rows, O, TO, Lq, Lk, d, dv, q_row, q_col, q_batch, k_row, k_col, k_batch,
                      v_row, v_col, v_batch, scale, causal ? 1 : 0, kv_group, n * w / nt, n * (w + 1) / nt};
        jobs[w] = g;
        if (pthread_create(&th[w], NULL, attn_worker, &jobs[w]) != 0) { jobs[w].end = -1; rc = -1; }
    }
    for (int w = 0; w < nt; ++w) {
        if (jobs[w].end < 0) continue;
        void* ret = NULL;
        pthread_join(th[w], &ret);
        if (ret) rc = -1;
    }
    free(th);
    free(jobs);
    return rc;
}

/* ------------------------------------------------- tile fan-out bench -- */

/*
 * Traffic the microbenchmark moves into on-chip memory: every consumer loads
 * one tile per iteration (the deep-dive's accounting: CTAs x iterations x
 * tile bytes, e.g. 132 x 5000 x 16384 B for its H100 run).
 */
double oracle_tilecast_bytes(int64_t consumers, int64_t iters, int64_t tile_bytes) {
    return (double)consumers * (double)iters * (double)tile_bytes;
}

/*
 * Group that consumer (workgroup) w belongs to, for `consumers` workgroups in
 * groups of `group` members.
 *   grouped:   members share an XCD.  Workgroup w runs on XCD w mod 8 and is
 *              the (w div 8)-th workgroup there; the group is formed by
 *              `group` consecutive workgroups of one XCD.
 *   ungrouped: members are `group` consecutive workgroup ids.
 * Returns -1 on an invalid combination.
 */
int64_t oracle_tilecast_group(int64_t w, int64_t consumers, int64_t group, int grouped) {
    if (group <= 0 || consumers <= 0 || consumers % group != 0 || w < 0 || w >= consumers) return -1;
    if (!grouped) return w / group;
    if (consumers % 8 != 0) return -1;
    int64_t per_xcd = consumers / 8;
    if (per_xcd % group != 0) return -1;
    int64_t xcd = w % 8, slot = w / 8;
    return xcd * (per_xcd / group) + slot / group;
}

/*
 * Checksum of everything consumer w loads over `iters` iterations: the sum,
 * modulo 2^32, of every 32-bit word (two consecutive bf16 of a tile row,
 * little-endian) of every tile it loads.  Tile t of a rows x cols matrix
 * (row-major, ld = cols) sits at row (t div tiles_x mod tiles_y)*tile_m and
 * column (t mod tiles_x)*tile_n.  Also returns, through last_sum, the same
 * sum over the last tile alone.
 */
uint32_t oracle_tilecast_checksum(const uint16_t* buf, int64_t rows, int64_t cols,
                                  int64_t tile_m, int64_t tile_n, int64_t w, int64_t consumers,
                                  int64_t group, int grouped, int64_t iters, int64_t stride,
                                  uint32_t* last_sum) {
    int64_t g = oracle_tilecast_group(w, consumers, group, grouped);
    int64_t tiles_x = cols / tile_n, tiles_y = rows / tile_m;
    uint32_t total = 0, last = 0;
    for (int64_t it = 0; it < iters; ++it) {
        int64_t t = it * stride + g;
        int64_t c0 = (t % tiles_x) * tile_n;
        int64_t r0 = ((t / tiles_x) % tiles_y) * tile_m;
        uint32_t s = 0;
        for (int64_t r = 0; r < tile_m; ++r)
            for (int64_t c = 0; c < tile_n; c += 2) {
                const uint16_t* p = buf + (r0 + r) * cols + c0 + c;
                s += (uint32_t)p[0] | ((uint32_t)p[1] << 16);
            }
        total += s;
        last = s;
    }
    if (last_sum) *last_sum = last;
    return total;
}

/* Element-wise oracle_f64_to_bf16_rne over an array (n values). */
void oracle_f64_to_bf16_rne_array(const double* x, uint16_t* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f64_to_bf16_rne(x[i]);
}
