/*
 * rmsn_ref.c -- CPU oracle for the row-wise RMSNorm (test infrastructure only;
 * see rmsn_ref.h for the definition it follows and who may call it).
 *
 * Plain C99, written step by step in the order of the definition so that it
 * can be checked by eye. Build flags keep IEEE binary32 semantics:
 * -O2 -ffp-contract=off, no -ffast-math; fmaf, sqrtf and '/' are the C
 * library's correctly rounded operations (C11 F.10, IEEE 754-2008 5.4).
 *
 * Sources: Lecture 04 "Launch Geometry: Grids, Occupancy, and 327 Norms per
 * Token", section 2.1 (the narrow sum of squares, the block sum, the inverse
 * from ss/(float)n + eps, then the wide elementwise apply); Lecture 08
 * "Graph-resident decode", section 8 (short sequential chains combined by a
 * balanced tree).
 */
#include "rmsn_ref.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

#define LANES 256      /* R256 step 1: number of lane chains          */
#define WAVE 64        /* R256 step 2: width of each halving tree     */
#define WAVES (LANES / WAVE)
#define MAX_LANES 256  /* the lane counts defined here: 256 and 128   */

float rmsn_ref_bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;   /* exact: bf16 is the top half of binary32 */
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

uint16_t rmsn_ref_f32_to_bf16(float v)
{
    uint32_t u;
    memcpy(&u, &v, sizeof u);
    if (isnan(v))
        return (uint16_t)(0x7FC0u | ((u >> 16) & 0x8000u));
    /* Round to nearest, ties to even, on the 16 dropped bits. A carry out of
     * the mantissa correctly moves to the next binade or to infinity. */
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (uint16_t)(u >> 16);
}

void rmsn_ref_f32_to_bf16_range(uint32_t first_bits, int64_t count, uint16_t* out)
{
    for (int64_t i = 0; i < count; ++i) {
        const uint32_t u = first_bits + (uint32_t)i;
        float v;
        memcpy(&v, &u, sizeof v);
        out[i] = rmsn_ref_f32_to_bf16(v);
    }
}

/* Steps 1-3 given the row as binary32 values produced by `get`. */
typedef float (*getter)(const void* row, int64_t d);

static float get_f32(const void* row, int64_t d) { return ((const float*)row)[d]; }
static float get_bf16(const void* row, int64_t d)
{
    return rmsn_ref_bf16_to_f32(((const uint16_t*)row)[d]);
}

static void lane_chains(const void* row, int64_t n, getter get, int lanes, float p[MAX_LANES])
{
    /* Step 1: lane l accumulates x[l], x[l+L], x[l+2L], ... in ascending
     * order (L = lanes: 256 for R256). */
    for (int l = 0; l < lanes; ++l) {
        float acc = 0.0f;
        for (int64_t d = l; d < n; d += lanes) {
            float xd = get(row, d);
            acc = fmaf(xd, xd, acc);
        }
        p[l] = acc;
    }
}

static void wave_trees(const float p[MAX_LANES], int lanes, float W[WAVES])
{
    /* Step 2: each of the four groups of L/4 lanes (64 for R256) is reduced
     * by descending halving. */
    const int group = lanes / WAVES;
    for (int w = 0; w < WAVES; ++w) {
        float q[MAX_LANES / WAVES];
        for (int j = 0; j < group; ++j) q[j] = p[group * w + j];
        for (int s = group / 2; s >= 1; s /= 2)
            for (int j = 0; j < s; ++j) q[j] = q[j] + q[j + s];
        W[w] = q[0];
    }
}

static float block_tree(const float W[WAVES])
{
    /* Step 3: the same halving applied to the four group totals. */
    float a = W[0] + W[2];
    float b = W[1] + W[3];
    return a + b;
}

static float sumsq(const void* row, int64_t n, getter get, int lanes)
{
    float p[MAX_LANES], W[WAVES];
    lane_chains(row, n, get, lanes, p);
    wave_trees(p, lanes, W);
    return block_tree(W);
}

float rmsn_ref_sumsq_f32(const float* x, int64_t n) { return sumsq(x, n, get_f32, LANES); }
float rmsn_ref_sumsq_bf16(const uint16_t* x, int64_t n) { return sumsq(x, n, get_bf16, LANES); }

void rmsn_ref_wave_totals_f32(const float* x, int64_t n, float out_w[4])
{
    float p[MAX_LANES];
    lane_chains(x, n, get_f32, LANES, p);
    wave_trees(p, LANES, out_w);
}

static int valid_lanes(int lanes) { return lanes == 128 || lanes == 256; }

float rmsn_ref_sumsq_lanes(int dtype, const void* x, int64_t n, int lanes)
{
    if (!valid_lanes(lanes)) return NAN;
    return sumsq(x, n, dtype == RMSN_REF_F32 ? get_f32 : get_bf16, lanes);
}

float rmsn_ref_inv(float ss, int64_t n, float eps)
{
    float m = ss / (float)n;   /* step 4: mean of squares, n exact in binary32 */
    float t = m + eps;         /* step 5                                        */
    float r = sqrtf(t);        /* step 6: correctly rounded square root         */
    float inv = 1.0f / r;      /* step 7: correctly rounded reciprocal          */
    return inv;
}

static void row_f32(const float* x, const float* w, float* y, int64_t n, float eps, int lanes)
{
    float inv = rmsn_ref_inv(sumsq(x, n, get_f32, lanes), n, eps);
    for (int64_t d = 0; d < n; ++d) {
        float a = x[d] * inv;  /* step 8, left to right */
        y[d] = a * w[d];
    }
}

static void row_bf16(const uint16_t* x, const uint16_t* w, uint16_t* y, int64_t n, float eps,
                     int lanes)
{
    float inv = rmsn_ref_inv(sumsq(x, n, get_bf16, lanes), n, eps);
    for (int64_t d = 0; d < n; ++d) {
        float a = rmsn_ref_bf16_to_f32(x[d]) * inv;
        float b = a * rmsn_ref_bf16_to_f32(w[d]);
        y[d] = rmsn_ref_f32_to_bf16(b);
    }
}

void rmsn_ref_row_f32(const float* x, const float* w, float* y, int64_t n, float eps)
{
    row_f32(x, w, y, n, eps, LANES);
}

void rmsn_ref_row_bf16(const uint16_t* x, const uint16_t* w, uint16_t* y, int64_t n, float eps)
{
    row_bf16(x, w, y, n, eps, LANES);
}

/* ---- many rows, optionally on several threads ---------------------------- */

typedef struct {
    int dtype;
    const void* x; int64_t xs;
    const void* w;
    void* y; int64_t ys;
    int64_t r0, r1, n;
    float eps;
    int lanes;
} rows_job;

static void run_rows(const rows_job* j)
{
    for (int64_t r = j->r0; r < j->r1; ++r) {
        if (j->dtype == RMSN_REF_F32)
            row_f32((const float*)j->x + r * j->xs, (const float*)j->w,
                    (float*)j->y + r * j->ys, j->n, j->eps, j->lanes);
        else
            row_bf16((const uint16_t*)j->x + r * j->xs, (const uint16_t*)j->w,
                     (uint16_t*)j->y + r * j->ys, j->n, j->eps, j->lanes);
    }
}

static void* rows_thread(void* arg)
{
    run_rows((const rows_job*)arg);
    return NULL;
}

int rmsn_ref_rows_lanes(int dtype, const void* x, int64_t x_stride, const void* w,
                        void* y, int64_t y_stride, int64_t rows, int64_t n, float eps,
                        int lanes, int nthreads)
{
    if (!valid_lanes(lanes)) return 0;
    if (nthreads < 1) nthreads = 1;
    if ((int64_t)nthreads > rows) nthreads = (int)(rows > 0 ? rows : 1);
    rows_job base = {dtype, x, x_stride, w, y, y_stride, 0, rows, n, eps, lanes};
    if (nthreads == 1) {
        run_rows(&base);
        return 1;
    }
    rows_job* jobs = (rows_job*)calloc((size_t)nthreads, sizeof *jobs);
    pthread_t* tid = (pthread_t*)calloc((size_t)nthreads, sizeof *tid);
    int started = 0;
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = base;
        jobs[t].r0 = rows * t / nthreads;
        jobs[t].r1 = rows * (t + 1) / nthreads;
        if (pthread_create(&tid[t], NULL, rows_thread, &jobs[t]) == 0) {
            ++started;
        } else {
            run_rows(&jobs[t]);      /* no thread: do this block here */
            tid[t] = 0;
        }
    }
    for (int t = 0; t < nthreads; ++t)
        if (tid[t]) pthread_join(tid[t], NULL);
    free(jobs);
    free(tid);
    return started > 0 ? started : 1;
}

int rmsn_ref_rows(int dtype, const void* x, int64_t x_stride, const void* w,
                  void* y, int64_t y_stride, int64_t rows, int64_t n, float eps,
                  int nthreads)
{
    return rmsn_ref_rows_lanes(dtype, x, x_stride, w, y, y_stride, rows, n, eps, LANES,
                               nthreads);
}
