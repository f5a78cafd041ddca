// rmsn_kernels.hip -- row-wise RMSNorm kernels for CDNA4 (gfx950).
//
// What is computed (Lecture 04 "Launch Geometry: Grids, Occupancy, and 327
// Norms per Token", sections 2 and 2.1): per row, the sum of squares under
// one fixed association, inv = 1/sqrt(ss/(float)n + eps), y = (x*inv)*w.
// Section 2.1's rule decides the design: the association of the reduction is
// part of the numerics and stays fixed; the elementwise apply is laid out
// however the hardware likes. The association ("R256"):
//   lane chains  p[l] = fmaf(x[d], x[d], p[l]), d = l, l+256, ... ascending
//   group trees  four 64-lane groups, descending halving 32,16,8,4,2,1
//   combine      ss = (G0 + G2) + (G1 + G3)
// Every kernel below evaluates exactly these operations in this order; the
// row layouts only decide which hardware lane holds which chain. Steps 4-7,
// element and quad access and the bf16 narrowing are shared with the other
// builds (rmsn_common.h).
//
// Layouts (all rows are independent; one row never spans workgroups):
//   WAVE   one wavefront per row. Lane t holds elements 256k + 4t + {0..3}
//          of every 256-element chunk k -- one 16-byte (binary32) or 8-byte
//          (bf16) load per chunk -- so its four registers ARE the chains of
//          lanes 4t..4t+3. Group g is lanes 16g..16g+15 of the wavefront; the
//          halving steps 32/16/8/4 are DPP row shifts by 8/4/2/1 inside each
//          16-lane row, steps 2/1 are adds between a lane's own registers, and
//          the combine reads lanes 0/16/32/48. No LDS, no barrier; HBM is read
//          once and the row lives in VGPRs between the reduction and the apply.
//   BLOCK  four wavefronts (256 threads) per row. Thread l is chain l; wave g
//          is group g and reduces it with two cross-row shuffles and four DPP
//          row shifts; the four group totals meet in 16 bytes of LDS across
//          one barrier. Element loads are 4/2 bytes, so any element-aligned
//          pointer works; the row stays in VGPRs (n <= 256 * chunks).
//   (STREAM and WIDE, for rows too wide to hold in registers, are in
//   rmsn_wide.hip; the descriptor kernels and the persistent walk stream a row
//   that leaves their register bucket with BLOCK's mapping, row_block<T, 0>.)
//   GROUP  BLOCK's mapping of chains to threads, but wavefront g reads its
//          group's 64 elements of four chunks with one 16-byte (binary32) /
//          8-byte (bf16) load per lane and a 4x4 register transpose (32- and
//          16-lane swaps) gives each lane one chain over those four chunks:
//          a quarter of the load instructions of BLOCK.
//   SPLIT  one workgroup of S wavefronts per row, the row cut into 1 KB slices
//          (one 16-byte load per lane). Wavefront s holds U consecutive
//          slices; it continues the 256 lane chains from where wavefront s-1
//          left them (1 KB of LDS, one barrier per hand-off), and the last
//          wavefront runs the group trees. Every wavefront issues all of its
//          loads at once, so the whole row is in flight from the start.
// The descriptor kernels, which run one row read from a device table, are in
// rmsn_desc.hip. The layouts' device code is in rmsn_rows.h; the persistent
// launch, which walks a whole table in one kernel, is in rmsn_persistent.hip.
//
// Floating point: contraction is off for this file; the one fused operation
// of the association is written as fmaf. '/' and sqrtf are the correctly
// rounded sequences HIP generates by default for binary32 (no approximate
// reciprocal square root); f32 denormals are preserved.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rmsn_common.h"
#include "rmsn_group.h"
#include "rmsn_launch.h"
#include "rmsn_rows.h"

#pragma clang fp contract(off)

namespace rmsn {
namespace {

// ---------------------------------------------------------------------------
// Kernels.

// WAVE layout: RPB rows per workgroup, one per wavefront (EXACT: n is exactly
// 256 * NCH, so no chunk is partial; NT: streaming hints). The workgroup first
// stages the shared weight row in LDS (dynamic LDS of (n/4) quads), so each
// row reads x from HBM and w from LDS instead of every row re-reading w
// through L2.
template <typename T, int NCH, int RPB, bool EXACT, bool NT>
__global__ __launch_bounds__(64 * RPB, (wave_occupancy<T, NCH, EXACT>())) void k_rows_wave(
    const T* x, int64_t xs, const T* __restrict__ w, T* y, int64_t ys, int64_t rows, int n,
    float eps) {
    using Q = Quad<T>;
    extern __shared__ __align__(16) unsigned char wave_smem[];
    typename Q::raw* wl = reinterpret_cast<typename Q::raw*>(wave_smem);
    const int nq = n >> 2;  // complete quads of the weight row
    for (int q = threadIdx.x; q < nq; q += 64 * RPB) wl[q] = Q::load(w + (q << 2));
    __syncthreads();
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t r = (int64_t)blockIdx.x * RPB + wave;
    if (r >= rows) return;
    const int lane = threadIdx.x & 63;
    WaveRow<T, NCH, EXACT, NT> row;
    row.load(x + r * xs, n, lane);
    row.finish(w, wl, y + r * ys, n, eps, lane);
}

// SPLIT layout: one row per workgroup of blockDim.x / 64 wavefronts, U slices
// each (EXACT: the row is exactly 64 * U * wavefronts vectors). Wavefront s waits for its turn (barrier s), takes the lane chains
// from LDS, extends them over its slices and passes them on; the last
// wavefront finishes the sum and publishes inv for the apply.
template <typename T, int U, bool EXACT, bool NT>
__global__ __launch_bounds__(1024) void k_rows_split(const T* x, int64_t xs,
                                                     const T* __restrict__ w, T* y, int64_t ys,
                                                     int n, float eps) {
    __shared__ f32x4 hand[64];
    __shared__ float inv_shared;
    const int waves = blockDim.x >> 6;
    const int s = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int64_t r = blockIdx.x;
    const uint32_t nvec = (uint32_t)n * (uint32_t)sizeof(T) / 16u;
    SplitPart<T, U, EXACT, NT> part;
    part.load(scalar_gptr(reinterpret_cast<const char*>(x + r * xs)),
              scalar_gptr(reinterpret_cast<const char*>(w)), s, lane, nvec);
    for (int h = 0; h < waves; ++h) {
        if (h == s) {
            // the turn is the row's critical path: let this wavefront's
            // instructions go first on its SIMD
            __builtin_amdgcn_s_setprio(3);
            float p[4] = {0.0f, 0.0f, 0.0f, 0.0f};
            if (s > 0) {
                const f32x4 q = hand[lane];
                p[0] = q.x; p[1] = q.y; p[2] = q.z; p[3] = q.w;
            }
            part.chains(p, nvec);
            if (s + 1 < waves) {
                f32x4 q;
                q.x = p[0]; q.y = p[1]; q.z = p[2]; q.w = p[3];
                hand[lane] = q;
            } else {
                const float inv = inverse_rms(split_sumsq(p, lane, T()), n, eps);
                if (lane == 0) inv_shared = inv;
            }
            __builtin_amdgcn_s_setprio(0);
        }
        __syncthreads();
    }
    part.apply(inv_shared, scalar_gptr(reinterpret_cast<char*>(y + r * ys)), s, lane, nvec);
}

template <typename T, int Q>
__global__ __launch_bounds__(256) void k_rows_group(const T* x, int64_t xs,
                                                    const T* __restrict__ w, T* y, int64_t ys,
                                                    int n, float eps) {
    __shared__ float lds4[4];
    const int64_t r = blockIdx.x;
    row_group<T, Q>(x + r * xs, w, y + r * ys, n, eps, lds4);
}

// REPLICA layout: `parts` workgroups per row (blockIdx = row * parts + part),
// each the GROUP layout over the whole row's x -- the same sum, so the same
// inv in every workgroup -- applying and storing only its share of the
// row's 1024-element blocks. No workgroup reads what another writes; x is
// read `parts` times (from the caches after the first), w and y once.
template <typename T, int Q>
__global__ __launch_bounds__(256) void k_rows_replica(const T* x, int64_t xs,
                                                      const T* __restrict__ w, T* y, int64_t ys,
                                                      int n, float eps, uint32_t parts) {
    __shared__ float lds4[4];
    const uint32_t b = blockIdx.x;
    const int64_t r = b / parts;
    const int part = (int)(b - (uint32_t)r * parts);
    const int m0 = (part * Q) / (int)parts, m1 = ((part + 1) * Q) / (int)parts;
    row_group<T, Q>(x + r * xs, w, y + r * ys, n, eps, lds4, m0, m1);
}

template <typename T, int NCH>
__global__ __launch_bounds__(256) void k_rows_block(const T* x, int64_t xs,
                                                    const T* __restrict__ w, T* y, int64_t ys,
                                                    int n, float eps) {
    __shared__ float lds4[4];
    const int64_t r = blockIdx.x;
    row_block<T, NCH>(x + r * xs, w, y + r * ys, n, eps, lds4);
}

// ---------------------------------------------------------------------------
// Instance selection (the bucket lists are in rmsn_rows.h).

template <typename T>
hipError_t launch_wave_t(const Plan& p, const void* x, int64_t xs, const void* w, void* y,
                         int64_t ys, int64_t rows, int n, float eps, hipStream_t s) {
    const T* xp = static_cast<const T*>(x);
    const T* wp = static_cast<const T*>(w);
    T* yp = static_cast<T*>(y);
    const dim3 grid((unsigned)p.grid), block((unsigned)p.block);
    const size_t lds = (size_t)(n >> 2) * sizeof(typename Quad<T>::raw);
    const bool exact = n == 256 * p.chunks;
#define RMSN_RPB(C, R)                                                                        \
    if (exact && p.streaming)                                                                 \
        hipLaunchKernelGGL((k_rows_wave<T, C, R, true, true>), grid, block, lds, s, xp, xs,   \
                           wp, yp, ys, rows, n, eps);                                         \
    else if (exact)                                                                           \
        hipLaunchKernelGGL((k_rows_wave<T, C, R, true, false>), grid, block, lds, s, xp, xs,  \
                           wp, yp, ys, rows, n, eps);                                         \
    else if (p.streaming)                                                                     \
        hipLaunchKernelGGL((k_rows_wave<T, C, R, false, true>), grid, block, lds, s, xp, xs,  \
                           wp, yp, ys, rows, n, eps);                                         \
    else                                                                                      \
        hipLaunchKernelGGL((k_rows_wave<T, C, R, false, false>), grid, block, lds, s, xp, xs, \
                           wp, yp, ys, rows, n, eps)
#define RMSN_CASE(C)                                                   \
    case C:                                                            \
        switch (p.rows_per_block) {                                    \
            case 8: RMSN_RPB(C, 8); break;                             \
            case 4: RMSN_RPB(C, 4); break;                             \
            default: return hipErrorInvalidValue;                      \
        }                                                              \
        break;
    switch (p.chunks) {
        RMSN_FOR_BUCKETS(RMSN_CASE)
        default: return hipErrorInvalidValue;
    }
#undef RMSN_CASE
#undef RMSN_RPB
    return hipGetLastError();
}

template <typename T>
hipError_t launch_split_t(const Plan& p, const void* x, int64_t xs, const void* w, void* y,
                          int64_t ys, int n, float eps, hipStream_t s) {
    const T* xp = static_cast<const T*>(x);
    const T* wp = static_cast<const T*>(w);
    T* yp = static_cast<T*>(y);
    const dim3 grid((unsigned)p.grid), block((unsigned)p.block);
    const bool exact = (int64_t)n * (int64_t)sizeof(T) == (int64_t)p.loads * p.block * 16;
#define RMSN_LAUNCH(U, E, NT)                                                                  \
    hipLaunchKernelGGL((k_rows_split<T, U, E, NT>), grid, block, 0, s, xp, xs, wp, yp, ys, n, eps)
#define RMSN_CASE(U)                                                                           \
    case U:                                                                                    \
        if (exact && p.streaming) RMSN_LAUNCH(U, true, true);                                  \
        else if (exact) RMSN_LAUNCH(U, true, false);                                           \
        else if (p.streaming) RMSN_LAUNCH(U, false, true);                                     \
        else RMSN_LAUNCH(U, false, false);                                                     \
        break;
    switch (p.loads) {
        RMSN_CASE(1)
        RMSN_CASE(2)
        RMSN_CASE(4)
        RMSN_CASE(8)
        default: return hipErrorInvalidValue;
    }
#undef RMSN_CASE
#undef RMSN_LAUNCH
    return hipGetLastError();
}

template <typename T>
hipError_t launch_group_t(const Plan& p, const void* x, int64_t xs, const void* w, void* y,
                          int64_t ys, int n, float eps, hipStream_t s) {
    const T* xp = static_cast<const T*>(x);
    const T* wp = static_cast<const T*>(w);
    T* yp = static_cast<T*>(y);
    const dim3 grid((unsigned)p.grid), block(256);
#define RMSN_CASE(Q)                                                                          \
    case Q:                                                                                   \
        hipLaunchKernelGGL((k_rows_group<T, Q>), grid, block, 0, s, xp, xs, wp, yp, ys, n,   \
                           eps);                                                              \
        break;
    switch (p.loads) {
        RMSN_FOR_GROUP_BLOCKS(RMSN_CASE)
        default: return hipErrorInvalidValue;
    }
#undef RMSN_CASE
    return hipGetLastError();
}

template <typename T>
hipError_t launch_replica_t(const Plan& p, const void* x, int64_t xs, const void* w, void* y,
                            int64_t ys, int n, float eps, hipStream_t s) {
    const T* xp = static_cast<const T*>(x);
    const T* wp = static_cast<const T*>(w);
    T* yp = static_cast<T*>(y);
    const dim3 grid((unsigned)p.grid), block(256);
    const uint32_t parts = (uint32_t)p.parts;
#define RMSN_CASE(Q)                                                                          \
    case Q:                                                                                   \
        hipLaunchKernelGGL((k_rows_replica<T, Q>), grid, block, 0, s, xp, xs, wp, yp, ys, n, \
                           eps, parts);                                                       \
        break;
    switch (p.loads) {
        RMSN_FOR_GROUP_BLOCKS(RMSN_CASE)
        default: return hipErrorInvalidValue;
    }
#undef RMSN_CASE
    return hipGetLastError();
}

template <typename T>
hipError_t launch_block_t(const Plan& p, const void* x, int64_t xs, const void* w, void* y,
                          int64_t ys, int n, float eps, hipStream_t s) {
    const T* xp = static_cast<const T*>(x);
    const T* wp = static_cast<const T*>(w);
    T* yp = static_cast<T*>(y);
    const dim3 grid((unsigned)p.grid), block(256);
#define RMSN_CASE(C)                                                                          \
    case C:                                                                                   \
        hipLaunchKernelGGL((k_rows_block<T, C>), grid, block, 0, s, xp, xs, wp, yp, ys, n,   \
                           eps);                                                              \
        break;
    switch (p.chunks) {
        RMSN_FOR_BUCKETS(RMSN_CASE)
        default: return hipErrorInvalidValue;
    }
#undef RMSN_CASE
    return hipGetLastError();
}

}  // namespace

hipError_t launch_rows(const Plan& p, const void* x, int64_t xs, const void* w, void* y,
                       int64_t ys, int64_t rows, int n, float eps, hipStream_t stream) {
    if (p.grid < 1 || p.grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    if (p.path == RMSN_PATH_WAVE) {
        // the WAVE kernels rely on the plan's bucket choice for this n
        if (p.chunks != chunk_bucket(n)) return hipErrorInvalidValue;
        return p.dtype == RMSN_F32
                   ? launch_wave_t<float>(p, x, xs, w, y, ys, rows, n, eps, stream)
                   : launch_wave_t<uint16_t>(p, x, xs, w, y, ys, rows, n, eps, stream);
    }
    if (p.path == RMSN_PATH_SPLIT) {
        // the SPLIT kernel relies on the plan's geometry for this n: whole
        // 16-byte vectors, one wavefront per `loads` slices
        const int64_t waves = (split_slices(p.dtype, n) + p.loads - 1) / (p.loads > 0 ? p.loads : 1);
        if (p.loads < 1 || ((int64_t)n * elem_bytes(p.dtype)) % 16 != 0 ||
            waves > kMaxSplitWaves || p.block != kWave * waves || p.grid != rows)
            return hipErrorInvalidValue;
        return p.dtype == RMSN_F32
                   ? launch_split_t<float>(p, x, xs, w, y, ys, n, eps, stream)
                   : launch_split_t<uint16_t>(p, x, xs, w, y, ys, n, eps, stream);
    }
    if (p.path == RMSN_PATH_GROUP) {
        // the GROUP kernels rely on the plan's block count and a width of whole quads
        if ((n & 3) != 0 || p.loads != (n + 1023) / 1024 || p.block != kBlockThreads ||
            p.grid != rows)
            return hipErrorInvalidValue;
        return p.dtype == RMSN_F32 ? launch_group_t<float>(p, x, xs, w, y, ys, n, eps, stream)
                                   : launch_group_t<uint16_t>(p, x, xs, w, y, ys, n, eps, stream);
    }
    if (p.path == RMSN_PATH_REPLICA) {
        // each of the plan's `parts` workgroups per row takes at least one
        // of the row's blocks
        const int q = (n + 1023) / 1024;
        if ((n & 3) != 0 || p.loads != q || p.block != kBlockThreads ||
            p.parts < 1 || p.parts > q || p.grid != rows * p.parts)
            return hipErrorInvalidValue;
        return p.dtype == RMSN_F32
                   ? launch_replica_t<float>(p, x, xs, w, y, ys, n, eps, stream)
                   : launch_replica_t<uint16_t>(p, x, xs, w, y, ys, n, eps, stream);
    }
    if (p.path == RMSN_PATH_STREAM)
        return launch_stream_rows(p, x, xs, w, y, ys, rows, n, eps, stream);
    return p.dtype == RMSN_F32 ? launch_block_t<float>(p, x, xs, w, y, ys, n, eps, stream)
                               : launch_block_t<uint16_t>(p, x, xs, w, y, ys, n, eps, stream);
}

}  // namespace rmsn
