// rmsn_wide.hip -- rows too wide to hold in registers, for CDNA4 (gfx950).
//
// The association (R256, Lecture 04 "Launch Geometry: Grids, Occupancy, and
// 327 Norms per Token", sections 2 and 2.1) makes each of its 256 lane chains
// a sequence of n/256 dependent fused multiply-adds, so the sum of squares of
// one row can occupy at most 256 lanes -- four wavefronts, one per group --
// while the apply is elementwise and can spread over the whole chip. Rows
// beyond the register-resident layouts (more than 8192 elements, or more than
// the SPLIT layout's 128 KB) are streamed:
//
//   group chain  wavefront g runs the 64 chains of group g in the GROUP
//                placement (rmsn_group.h): lane 16q + t is association lane
//                64g + 4t + q. With x quad-aligned, each complete 1024-element
//                block is one 16-byte (binary32) / 8-byte (bf16) load per lane
//                and a 4x4 transpose; the chunks after the last complete
//                block, and every chunk of a row whose x is not quad-aligned,
//                are one element load per lane and chunk. Loads go through a
//                buffer resource ranged to the row (or to its complete blocks):
//                past it they return +0, which leaves a chain unchanged
//                (fmaf(0, 0, p) == p for p >= +0), so every batch issues the
//                same loads, and one batch is in flight while the previous
//                one is summed.
//   STREAM       one workgroup of four wavefronts per row: the four group
//                chains, the combine through LDS, then the apply streamed by
//                the whole workgroup, kSpan elements at a time.
//   WIDE         two launches. The first runs one wavefront per (row, group)
//                -- four CUs per row for the sum -- and writes the four group
//                totals to a caller's workspace; the second runs
//                ceil(n / kSpan) workgroups per row, each combining the four
//                totals in the association's order, (G0 + G2) + (G1 + G3), and
//                applying its kSpan elements. The kernel boundary orders the
//                totals' stores before their loads.
//
// Floating point: contraction is off; '/' and sqrtf are HIP's correctly
// rounded binary32 sequences (steps 4-7 in rmsn_common.h).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rmsn_common.h"
#include "rmsn_group.h"
#include "rmsn_launch.h"

#pragma clang fp contract(off)

namespace rmsn {
namespace {

typedef __amdgpu_buffer_rsrc_t brsrc;

// Loads in flight while a wavefront sums: one batch is summed while the next
// is loaded -- 1024-element blocks with quad loads, 256-element chunks with
// element loads. (Measured on MI355X: keeping 16 to 48 blocks in flight,
// refilled one block or eight at a time, changes nothing; the sum is bound by
// the chain of dependent multiply-adds, not by memory.)
constexpr int kBatch = 16;
constexpr int kEBatch = 24;

// A buffer resource for `bytes` bytes at p (raw, stride 0; the third word is
// the gfx9-family untyped format). Offsets at or past `bytes` read +0 and
// drop stores. p must be wave-uniform.
__device__ __forceinline__ brsrc wide_rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes,
                                             0x00020000);
}

// Four consecutive elements through a buffer resource.
template <typename T> struct BQuad;
template <> struct BQuad<float> {
    typedef u32x4 raw;
    static __device__ __forceinline__ raw load(brsrc r, uint32_t off) {
        return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    }
    static __device__ __forceinline__ void unpack(raw q, float v[4]) {
        v[0] = __uint_as_float(q.x); v[1] = __uint_as_float(q.y);
        v[2] = __uint_as_float(q.z); v[3] = __uint_as_float(q.w);
    }
    static __device__ __forceinline__ void store(brsrc r, uint32_t off, const float v[4]) {
        u32x4 q;
        q.x = __float_as_uint(v[0]); q.y = __float_as_uint(v[1]);
        q.z = __float_as_uint(v[2]); q.w = __float_as_uint(v[3]);
        __builtin_amdgcn_raw_buffer_store_b128(q, r, off, 0, 0);
    }
};
template <> struct BQuad<uint16_t> {
    typedef u32x2 raw;
    static __device__ __forceinline__ raw load(brsrc r, uint32_t off) {
        return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    }
    static __device__ __forceinline__ void unpack(raw q, float v[4]) {
        v[0] = lo_bf16(q.x); v[1] = hi_bf16(q.x); v[2] = lo_bf16(q.y); v[3] = hi_bf16(q.y);
    }
    static __device__ __forceinline__ void store(brsrc r, uint32_t off, const float v[4]) {
        u32x2 q;
        q.x = bf16_pair(v[0], v[1]);
        q.y = bf16_pair(v[2], v[3]);
        __builtin_amdgcn_raw_buffer_store_b64(q, r, off, 0, 0);
    }
};

// One element through a buffer resource.
template <typename T> struct BElem;
template <> struct BElem<float> {
    typedef uint32_t raw;
    static __device__ __forceinline__ raw load(brsrc r, uint32_t off) {
        return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
    }
    static __device__ __forceinline__ float value(raw b) { return __uint_as_float(b); }
    static __device__ __forceinline__ void store(brsrc r, uint32_t off, float v) {
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, off, 0, 0);
    }
};
template <> struct BElem<uint16_t> {
    typedef uint32_t raw;
    static __device__ __forceinline__ raw load(brsrc r, uint32_t off) {
        return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
    }
    static __device__ __forceinline__ float value(raw b) { return __uint_as_float(b << 16); }
    static __device__ __forceinline__ void store(brsrc r, uint32_t off, float v) {
        __builtin_amdgcn_raw_buffer_store_b16((unsigned short)bf16_bits(v), r, off, 0, 0);
    }
};

// ---------------------------------------------------------------------------
// The chains of one group.

// Blocks m0 .. m0 + kBatch - 1 (quad loads; lane offset `off` in a block).
template <typename T>
__device__ __forceinline__ void issue_blocks(typename BQuad<T>::raw (&b)[kBatch], brsrc r,
                                             uint32_t off, uint32_t m0) {
#pragma unroll
    for (int i = 0; i < kBatch; ++i) b[i] = BQuad<T>::load(r, (m0 + i) * 1024u * sizeof(T) + off);
}

// The chains through those blocks, chunks in ascending order: lane 16q + t
// loaded elements 256(4m + q) + 64g + 4t + {0..3}; after the transpose its
// v[k] is chain 64g + 4t + q in chunk 4m + k.
template <typename T>
__device__ __forceinline__ void chain_blocks(const typename BQuad<T>::raw (&b)[kBatch], float& p) {
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
        float v[4];
        BQuad<T>::unpack(b[i], v);
        transpose4(v);
        p = fmaf(v[0], v[0], p);
        p = fmaf(v[1], v[1], p);
        p = fmaf(v[2], v[2], p);
        p = fmaf(v[3], v[3], p);
    }
}

// Chunks c0 .. c0 + kEBatch - 1 (element loads; lane offset `off` in a chunk).
template <typename T>
__device__ __forceinline__ void issue_chunks(typename BElem<T>::raw (&b)[kEBatch], brsrc r,
                                             uint32_t off, uint32_t c0) {
#pragma unroll
    for (int i = 0; i < kEBatch; ++i) b[i] = BElem<T>::load(r, (c0 + i) * 256u * sizeof(T) + off);
}

template <typename T>
__device__ __forceinline__ void chain_chunks(const typename BElem<T>::raw (&b)[kEBatch], float& p) {
#pragma unroll
    for (int i = 0; i < kEBatch; ++i) {
        const float v = BElem<T>::value(b[i]);
        p = fmaf(v, v, p);
    }
}

// Group g's total for a row of width n at x (x and g wave-uniform): the
// finished chain of association lane 64g + 4t + q in lane 16q + t, then the
// group tree. Every lane returns the total.
template <typename T>
__device__ __forceinline__ float group_total(const T* x, uint32_t n, uint32_t g) {
    constexpr uint32_t es = sizeof(T);
    const uint32_t lane = threadIdx.x & 63;
    const uint32_t q = lane >> 4, t = lane & 15;
    const uint32_t eoff = (g * 64u + t * 4u + q) * es;  // this lane's element of a chunk
    const uint32_t nc = (n + 255u) >> 8;                // chunks, the last maybe partial
    float p = 0.0f;
    uint32_t c = 0;                                     // first chunk left for element loads
    if (reinterpret_cast<uintptr_t>(x) % (4u * es) == 0) {
        const uint32_t nb = n >> 10;                    // complete blocks
        if (nb > 0) {
            const brsrc r = wide_rsrc(x, nb * 1024u * es);
            const uint32_t off = (q * 256u + g * 64u + t * 4u) * es;
            typename BQuad<T>::raw a[kBatch], b[kBatch];
            issue_blocks<T>(a, r, off, 0);
            for (uint32_t m = 0; m < nb; m += 2 * kBatch) {
                issue_blocks<T>(b, r, off, m + kBatch);
                __builtin_amdgcn_sched_barrier(0);
                chain_blocks<T>(a, p);
                __builtin_amdgcn_sched_barrier(0);
                issue_blocks<T>(a, r, off, m + 2 * kBatch);
                __builtin_amdgcn_sched_barrier(0);
                chain_blocks<T>(b, p);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        c = nb * 4u;
        // at most four chunks remain, the last maybe partial
        const brsrc r = wide_rsrc(x, n * es);
        typename BElem<T>::raw e[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) e[i] = BElem<T>::load(r, (c + i) * 256u * es + eoff);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float v = BElem<T>::value(e[i]);
            p = fmaf(v, v, p);
        }
    } else if (c < nc) {
        const brsrc r = wide_rsrc(x, n * es);
        typename BElem<T>::raw a[kEBatch], b[kEBatch];
        issue_chunks<T>(a, r, eoff, 0);
        for (; c < nc; c += 2 * kEBatch) {
            issue_chunks<T>(b, r, eoff, c + kEBatch);
            __builtin_amdgcn_sched_barrier(0);
            chain_chunks<T>(a, p);
            __builtin_amdgcn_sched_barrier(0);
            issue_chunks<T>(a, r, eoff, c + 2 * kEBatch);
            __builtin_amdgcn_sched_barrier(0);
            chain_chunks<T>(b, p);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    return group_sumsq(p);
}

// ---------------------------------------------------------------------------
// The apply: y[d] = (x[d] * inv) * w[d] for d in [e0, e0 + kSpan) of a row, by
// 256 threads. QUADS (x, w, y quad-aligned and n a multiple of 4): thread i
// takes the quads at e0 + 1024j + 4i; otherwise the elements e0 + 256j + i.
// Accesses past the row read +0 and drop their stores (ranged resources), so
// a span may run past the row's end.

constexpr uint32_t kSpan = 4096;

struct RowRsrc {
    brsrc x, w, y;
};

template <typename T>
__device__ __forceinline__ RowRsrc row_rsrcs(const T* x, const T* w, T* y, uint32_t n) {
    const uint32_t bytes = n * (uint32_t)sizeof(T);
    return RowRsrc{wide_rsrc(x, bytes), wide_rsrc(w, bytes), wide_rsrc(y, bytes)};
}

template <typename T, bool QUADS> struct Span;

template <typename T> struct Span<T, true> {
    static constexpr int J = kSpan / 1024;
    typename BQuad<T>::raw x[J], w[J];
    __device__ __forceinline__ static uint32_t off(uint32_t e0, int j) {
        return (e0 + 1024u * j + 4u * threadIdx.x) * (uint32_t)sizeof(T);
    }
    __device__ __forceinline__ void load(const RowRsrc& r, uint32_t e0) {
#pragma unroll
        for (int j = 0; j < J; ++j) x[j] = BQuad<T>::load(r.x, off(e0, j));
#pragma unroll
        for (int j = 0; j < J; ++j) w[j] = BQuad<T>::load(r.w, off(e0, j));
    }
    __device__ __forceinline__ void store(const RowRsrc& r, uint32_t e0, float inv) const {
#pragma unroll
        for (int j = 0; j < J; ++j) {
            float a[4], b[4], o[4];
            BQuad<T>::unpack(x[j], a);
            BQuad<T>::unpack(w[j], b);
#pragma unroll
            for (int k = 0; k < 4; ++k) o[k] = (a[k] * inv) * b[k];
            BQuad<T>::store(r.y, off(e0, j), o);
        }
    }
};

template <typename T> struct Span<T, false> {
    static constexpr int J = kSpan / 256;
    typename BElem<T>::raw x[J], w[J];
    __device__ __forceinline__ static uint32_t off(uint32_t e0, int j) {
        return (e0 + 256u * j + threadIdx.x) * (uint32_t)sizeof(T);
    }
    __device__ __forceinline__ void load(const RowRsrc& r, uint32_t e0) {
#pragma unroll
        for (int j = 0; j < J; ++j) x[j] = BElem<T>::load(r.x, off(e0, j));
#pragma unroll
        for (int j = 0; j < J; ++j) w[j] = BElem<T>::load(r.w, off(e0, j));
    }
    __device__ __forceinline__ void store(const RowRsrc& r, uint32_t e0, float inv) const {
#pragma unroll
        for (int j = 0; j < J; ++j)
            BElem<T>::store(r.y, off(e0, j), (BElem<T>::value(x[j]) * inv) * BElem<T>::value(w[j]));
    }
};

// The whole row, two spans in flight: span s + 1 is loaded before span s is
// applied and stored (its elements are other elements, so an in-place row is
// safe), and a span's loads are issued before the stores of the span before
// it, so waiting for them never waits for those stores.
template <typename T, bool QUADS>
__device__ __forceinline__ void apply_row(const RowRsrc& r, uint32_t n, float inv) {
    Span<T, QUADS> a, b;
    a.load(r, 0);
    __builtin_amdgcn_sched_barrier(0);
    for (uint32_t e0 = 0; e0 < n; e0 += 2 * kSpan) {
        b.load(r, e0 + kSpan);
        __builtin_amdgcn_sched_barrier(0);
        a.store(r, e0, inv);
        __builtin_amdgcn_sched_barrier(0);
        a.load(r, e0 + 2 * kSpan);
        __builtin_amdgcn_sched_barrier(0);
        b.store(r, e0 + kSpan, inv);
        __builtin_amdgcn_sched_barrier(0);
    }
}

__device__ __forceinline__ bool quad_rows(const void* x, const void* w, const void* y,
                                          uint32_t n, uint32_t es) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(w) |
                        reinterpret_cast<uintptr_t>(y);
    return n % 4u == 0 && a % (4u * es) == 0;
}

// ---------------------------------------------------------------------------
// Kernels.

// STREAM: one row per workgroup of four wavefronts.
template <typename T>
__global__ __launch_bounds__(256) void k_rows_stream(const T* x, int64_t xs, const T* w, T* y,
                                                     int64_t ys, int n, float eps) {
    __shared__ float lds4[4];
    const int64_t r = blockIdx.x;
    const T* xr = x + r * xs;
    T* yr = y + r * ys;
    const uint32_t g = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const float gt = group_total<T>(xr, (uint32_t)n, g);
    if ((threadIdx.x & 63) == 0) lds4[g] = gt;
    __syncthreads();
    const float inv = inverse_rms((lds4[0] + lds4[2]) + (lds4[1] + lds4[3]), n, eps);
    const RowRsrc rr = row_rsrcs<T>(xr, w, yr, (uint32_t)n);
    if (quad_rows(xr, w, yr, (uint32_t)n, sizeof(T)))
        apply_row<T, true>(rr, (uint32_t)n, inv);
    else
        apply_row<T, false>(rr, (uint32_t)n, inv);
}

// WIDE, first launch: group blockIdx % 4 of row blockIdx / 4; lane 0 writes
// the group total to ws[4 * row + group].
template <typename T>
__global__ __launch_bounds__(64) void k_wide_sum(const T* x, int64_t xs, int n, float* ws) {
    const int64_t r = blockIdx.x >> 2;
    const uint32_t g = blockIdx.x & 3u;
    const float gt = group_total<T>(x + r * xs, (uint32_t)n, g);
    if (threadIdx.x == 0) ws[4 * r + g] = gt;
}

// WIDE, second launch: span blockIdx % spans of row blockIdx / spans.
template <typename T>
__global__ __launch_bounds__(256) void k_wide_apply(const T* x, int64_t xs, const T* w, T* y,
                                                    int64_t ys, int n, float eps, const float* ws,
                                                    uint32_t spans) {
    const uint32_t b = blockIdx.x;
    const int64_t r = b / spans;
    const uint32_t s = b - (uint32_t)r * spans;
    const float* gt = ws + 4 * r;
    const float inv = inverse_rms((gt[0] + gt[2]) + (gt[1] + gt[3]), n, eps);
    const T* xr = x + r * xs;
    T* yr = y + r * ys;
    const RowRsrc rr = row_rsrcs<T>(xr, w, yr, (uint32_t)n);
    if (quad_rows(xr, w, yr, (uint32_t)n, sizeof(T))) {
        Span<T, true> sp;
        sp.load(rr, s * kSpan);
        sp.store(rr, s * kSpan, inv);
    } else {
        Span<T, false> sp;
        sp.load(rr, s * kSpan);
        sp.store(rr, s * kSpan, inv);
    }
}

template <typename T>
hipError_t launch_stream_t(const Plan& p, const void* x, int64_t xs, const void* w, void* y,
                           int64_t ys, int n, float eps, hipStream_t s) {
    hipLaunchKernelGGL(k_rows_stream<T>, dim3((unsigned)p.grid), dim3(256), 0, s,
                       static_cast<const T*>(x), xs, static_cast<const T*>(w),
                       static_cast<T*>(y), ys, n, eps);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_wide_t(const Plan& p, const void* x, int64_t xs, const void* w, void* y,
                         int64_t ys, int64_t rows, int n, float eps, float* ws, hipStream_t s) {
    hipLaunchKernelGGL(k_wide_sum<T>, dim3((unsigned)(rows * 4)), dim3(64), 0, s,
                       static_cast<const T*>(x), xs, n, ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_wide_apply<T>, dim3((unsigned)(rows * p.loads)), dim3(256), 0, s,
                       static_cast<const T*>(x), xs, static_cast<const T*>(w),
                       static_cast<T*>(y), ys, n, eps, static_cast<const float*>(ws),
                       (uint32_t)p.loads);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_stream_rows(const Plan& p, const void* x, int64_t xs, const void* w, void* y,
                              int64_t ys, int64_t rows, int n, float eps, hipStream_t stream) {
    if (p.block != 256 || p.grid != rows || n < 1 || n > RMSN_MAX_N)
        return hipErrorInvalidValue;
    return p.dtype == RMSN_F32 ? launch_stream_t<float>(p, x, xs, w, y, ys, n, eps, stream)
                               : launch_stream_t<uint16_t>(p, x, xs, w, y, ys, n, eps, stream);
}

hipError_t launch_wide_rows(const Plan& p, const void* x, int64_t xs, const void* w, void* y,
                            int64_t ys, int64_t rows, int n, float eps, float* ws,
                            hipStream_t stream) {
    // the kernels rely on the plan's geometry for this n: four wavefronts per
    // row for the sum, one workgroup per kSpan elements for the apply
    if (p.path != RMSN_PATH_WIDE || n < 1 || n > RMSN_MAX_N || ws == nullptr ||
        p.grid != rows * 4 || p.loads != (int)(((uint32_t)n + kSpan - 1) / kSpan))
        return hipErrorInvalidValue;
    return p.dtype == RMSN_F32
               ? launch_wide_t<float>(p, x, xs, w, y, ys, rows, n, eps, ws, stream)
               : launch_wide_t<uint16_t>(p, x, xs, w, y, ys, rows, n, eps, ws, stream);
}

}  // namespace rmsn
