/*
 * rmsn_ref.h -- CPU oracle for the row-wise RMSNorm (test infrastructure).
 *
 * THIS IS TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT. Only the test suite,
 * the smoke check and the benchmark's CPU-baseline leg may load or call it.
 * It shares no code, header, table or helper with the HIP library.
 *
 * What it computes (Lecture 04 "Launch Geometry: Grids, Occupancy, and 327
 * Norms per Token", section 2 and 2.1): for one row of width n,
 *     ss  = sum over d of x[d]^2          (fixed association R256, below)
 *     inv = 1 / sqrt(ss / (float)n + eps)
 *     y[d] = (x[d] * inv) * w[d]
 * all in IEEE binary32, round-to-nearest-even, gradual underflow.
 *
 * The association of the sum of squares is part of the numerics (section 2.1
 * of the same lecture: the reduction width decides the bits, the apply width
 * does not). This library fixes it as "R256":
 *   1. 256 lane chains: p[l] = +0, then p[l] = fmaf(x[d], x[d], p[l]) for
 *      d = l, l+256, l+512, ... ascending while d < n.
 *   2. Four 64-lane trees, lanes 64w..64w+63, descending halving
 *      s = 32,16,8,4,2,1 with q[j] = q[j] + q[j+s] for j < s; W[w] = q[0].
 *   3. ss = (W[0] + W[2]) + (W[1] + W[3]).
 *   4. m = ss / (float)n       5. t = m + eps
 *   6. r = sqrtf(t)            7. inv = 1.0f / r      (each correctly rounded;
 *      the lecture's approximate reciprocal square root is replaced by two
 *      correctly rounded operations so a CPU can reproduce the bits)
 *   8. y[d] = (x[d] * inv) * w[d], left to right.
 * bf16 inputs are widened exactly; a bf16 output is rounded once, to nearest
 * even, from the binary32 y (NaN becomes the quiet NaN 0x7FC0 with its sign).
 *
 * Errors: none are reported; callers pass valid arguments (1 <= n <= 2^24,
 * non-null pointers). n above 2^24 would make (float)n inexact.
 */
#ifndef RMSN_REF_H
#define RMSN_REF_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { RMSN_REF_F32 = 0, RMSN_REF_BF16 = 1 };

/* Steps 1-3 on a binary32 row: the sum of squares under R256. */
float rmsn_ref_sumsq_f32(const float* x, int64_t n);
/* Steps 1-3 on a bf16 row (bit patterns), widened exactly to binary32. */
float rmsn_ref_sumsq_bf16(const uint16_t* x, int64_t n);
/* Steps 4-7: the inverse RMS from the sum of squares. */
float rmsn_ref_inv(float ss, int64_t n, float eps);
/* The four 64-lane tree totals W[0..3] of step 2 (for association probes). */
void rmsn_ref_wave_totals_f32(const float* x, int64_t n, float out_w[4]);

/* One full row, steps 1-8. */
void rmsn_ref_row_f32(const float* x, const float* w, float* y, int64_t n, float eps);
void rmsn_ref_row_bf16(const uint16_t* x, const uint16_t* w, uint16_t* y, int64_t n, float eps);

/* Many rows sharing one weight vector. Strides are in elements. nthreads <= 1
 * runs on the calling thread; otherwise rows are split into nthreads
 * contiguous blocks, one POSIX thread each. Returns the threads used. */
int rmsn_ref_rows(int dtype, const void* x, int64_t x_stride, const void* w,
                  void* y, int64_t y_stride, int64_t rows, int64_t n, float eps,
                  int nthreads);

/* The same definition with another lane count L (Lecture 04 section 2.1:
 * the reduction's thread count decides the bits; the lecture's kernel sums
 * on 128 threads). R_L: L lane chains as in step 1 with stride L; four
 * groups of L/4 lanes, each reduced by descending halving L/8, ..., 2, 1;
 * ss = (W[0] + W[2]) + (W[1] + W[3]); steps 4-8 unchanged. L = 256 is R256;
 * L = 128 is the four 32-lane groups of the lecture's 128-thread sum.
 * Other L: the sum returns NaN and the rows call returns 0 having done
 * nothing. */
float rmsn_ref_sumsq_lanes(int dtype, const void* x, int64_t n, int lanes);
int rmsn_ref_rows_lanes(int dtype, const void* x, int64_t x_stride, const void* w,
                        void* y, int64_t y_stride, int64_t rows, int64_t n, float eps,
                        int lanes, int nthreads);

/* Exact bf16 widening and the round-to-nearest-even narrowing of step 8. */
float rmsn_ref_bf16_to_f32(uint16_t b);
uint16_t rmsn_ref_f32_to_bf16(float v);
/* The narrowing over `count` consecutive binary32 bit patterns from
 * first_bits: out[i] = rmsn_ref_f32_to_bf16(bits first_bits + i). */
void rmsn_ref_f32_to_bf16_range(uint32_t first_bits, int64_t count, uint16_t* out);

#ifdef __cplusplus
}
#endif
#endif
