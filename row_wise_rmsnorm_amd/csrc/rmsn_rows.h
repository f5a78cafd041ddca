// rmsn_rows.h -- the row layouts of the association's lanes, as device code
// shared by the batched-row and descriptor kernels (rmsn_kernels.hip) and the
// persistent launch (rmsn_persistent.hip). Each layout evaluates the same
// operations in the same order (R256: 256 fmaf lane chains, four 64-lane
// descending-halving trees, (G0 + G2) + (G1 + G3), steps 4-7, (x * inv) * w);
// they differ only in which hardware lane holds which chain (see
// rmsn_kernels.hip for the layouts).
//
// Floating point: contraction is off; the one fused operation of the
// association is written as fmaf.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rmsn_common.h"
#include "rmsn_group.h"

#pragma clang fp contract(off)

namespace rmsn {
namespace {

// ---------------------------------------------------------------------------
// WAVE layout: one wavefront per row, lane t holds chains 4t..4t+3.

// Group trees and combine for the WAVE layout. On entry lane t's p[e] is the
// finished chain of association lane 4t+e; group g = lanes 16g..16g+15, where
// association lane 64g+j sits in wavefront lane 16g + j/4, register j%4.
__device__ __forceinline__ float wave_sumsq(float p0, float p1, float p2, float p3) {
    // halving s = 32, 16, 8, 4: partner j+s is s/4 wavefront lanes further
    p0 += row_shl<8>(p0); p1 += row_shl<8>(p1); p2 += row_shl<8>(p2); p3 += row_shl<8>(p3);
    p0 += row_shl<4>(p0); p1 += row_shl<4>(p1); p2 += row_shl<4>(p2); p3 += row_shl<4>(p3);
    p0 += row_shl<2>(p0); p1 += row_shl<2>(p1); p2 += row_shl<2>(p2); p3 += row_shl<2>(p3);
    p0 += row_shl<1>(p0); p1 += row_shl<1>(p1); p2 += row_shl<1>(p2); p3 += row_shl<1>(p3);
    // halving s = 2 and 1 inside the lane
    const float g = (p0 + p2) + (p1 + p3);
    // group totals sit in lanes 0, 16, 32, 48
    const float g0 = lane_value(g, 0), g1 = lane_value(g, 16);
    const float g2 = lane_value(g, 32), g3 = lane_value(g, 48);
    return (g0 + g2) + (g1 + g3);
}

// Chunks a kernel instance may assume complete: the plan picks the smallest
// bucket holding the row, so a row using bucket NCH has more than
// 256 * (previous bucket) elements.
constexpr int prev_bucket(int nch) {
    return nch <= 1 ? 0 : nch <= 2 ? 1 : nch <= 4 ? 2 : nch <= 6 ? 4 : nch <= 8 ? 6
         : nch <= 12 ? 8 : nch <= 16 ? 12 : nch <= 20 ? 16 : nch <= 24 ? 20 : nch <= 28 ? 24 : 28;
}

// Resident wavefronts per SIMD the WAVE kernels are compiled for: the row's
// registers (4 values per chunk; bf16 packed two per VGPR), the ragged-tail
// chunk unless the width is exactly 256 * NCH, and a few for chains,
// addresses and temporaries, out of 512 VGPRs per SIMD lane.
template <typename T, int NCH, bool EXACT>
constexpr int wave_occupancy() {
    constexpr int q = sizeof(T) == 4 ? 4 : 2;
    constexpr int regs = NCH * q + (EXACT ? 0 : q) + 16 + (sizeof(T) == 4 ? 8 : 0);
    constexpr int w = 512 / ((regs + 7) / 8 * 8);
    return w > 8 ? 8 : (w < 1 ? 1 : w);
}

// One row held by one wavefront: load() issues every load of the row, finish()
// reduces, normalises and stores it. NT: non-temporal (streaming) hints on the
// row's loads and stores, for batches too large for the caches to help.
// Requires 256 * prev_bucket(NCH) < n <= 256 * NCH, and n == 256 * NCH when
// EXACT (both guaranteed by the plan).
template <typename T, int NCH, bool EXACT, bool NT>
struct WaveRow {
    using Q = Quad<T>;
    static constexpr int MINF = EXACT ? NCH : prev_bucket(NCH);
    // Addresses are a scalar base per 4 KB of the row (the reach of the
    // instruction's immediate offset) plus an unsigned per-lane byte offset, so
    // every load and store uses the scalar-base addressing mode instead of a
    // 64-bit address pair per lane.
    static constexpr uint32_t chunk_bytes = 256u * sizeof(T);
    static constexpr int per_base = 4096 / chunk_bytes;

    typename Q::raw xr[NCH];
    typename Q::raw xt;

    // Chunks [0, full) are complete; chunk `full` is the ragged tail when n is
    // not a multiple of 256. `full` is wave-uniform, so the tests are scalar
    // branches; chunks below MINF need none (none at all when EXACT).
    static __device__ __forceinline__ int full_chunks(int n) { return EXACT ? NCH : (n >> 8); }

    __device__ __forceinline__ void load(const T* x, int n, int lane) {
        const int full = full_chunks(n);
        const uint32_t lane_bytes = (uint32_t)lane * (uint32_t)(4 * sizeof(T));
#pragma unroll
        for (int k = 0; k < NCH; ++k) {
            if (k < MINF || k < full) {
                gptr_c base =
                    scalar_gptr(reinterpret_cast<const char*>(x) + (k / per_base) * 4096);
                xr[k] = Q::template gload<NT>(base + lane_bytes +
                                              (uint32_t)(k % per_base) * chunk_bytes);
            }
        }
        xt = Q::zero();
        if (!EXACT && (n & 255)) xt = Q::load_tail(x, (full << 8) + (lane << 2), n);
    }

    // wl: the weight row staged in LDS as quads (quad q = elements 4q..4q+3);
    // w: the same row in global memory, read only for the ragged tail.
    __device__ __forceinline__ void finish(const T* __restrict__ w,
                                           const typename Q::raw* wl, T* y, int n, float eps,
                                           int lane) {
        const int full = full_chunks(n);
        const uint32_t lane_bytes = (uint32_t)lane * (uint32_t)(4 * sizeof(T));
        // Lane chains in ascending chunk order; the tail chunk comes last and
        // reads +0 past the row (fmaf(0, 0, p) == p for p >= +0). The per-chunk
        // scheduling barriers keep each chunk's widening next to its four fmas,
        // so widened copies of later chunks are never live with the packed row.
        __builtin_amdgcn_sched_barrier(0);
        float p0 = 0.0f, p1 = 0.0f, p2 = 0.0f, p3 = 0.0f;
#pragma unroll
        for (int k = 0; k < NCH; ++k) {
            if (k < MINF || k < full) {
                float v[4];
                Q::unpack(xr[k], v);
                p0 = fmaf(v[0], v[0], p0);
                p1 = fmaf(v[1], v[1], p1);
                p2 = fmaf(v[2], v[2], p2);
                p3 = fmaf(v[3], v[3], p3);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        if (!EXACT) {
            float v[4];
            Q::unpack(xt, v);
            p0 = fmaf(v[0], v[0], p0);
            p1 = fmaf(v[1], v[1], p1);
            p2 = fmaf(v[2], v[2], p2);
            p3 = fmaf(v[3], v[3], p3);
        }
        const float inv = inverse_rms(wave_sumsq(p0, p1, p2, p3), n, eps);
#pragma unroll
        for (int k = 0; k < NCH; ++k)
            if (k < MINF || k < full) opaque(xr[k]);
        // Apply two chunks at a time. The scheduling barrier stops the compiler
        // from hoisting every LDS weight read to the top (LDS cannot alias the
        // global stores), which would hold the whole weight row in registers.
#pragma unroll
        for (int k0 = 0; k0 < NCH; k0 += 2) {
#pragma unroll
            for (int k = k0; k < k0 + 2 && k < NCH; ++k) {
                if (k < MINF || k < full) {
                    float v[4], wv[4], o[4];
                    Q::unpack(xr[k], v);
                    Q::unpack(wl[(k << 6) + lane], wv);
#pragma unroll
                    for (int i = 0; i < 4; ++i) o[i] = (v[i] * inv) * wv[i];
                    gptr base = scalar_gptr(reinterpret_cast<char*>(y) + (k / per_base) * 4096);
                    Q::template gstore<NT>(base + lane_bytes +
                                               (uint32_t)(k % per_base) * chunk_bytes, o);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        if (!EXACT && (n & 255)) {
            const int et = (full << 8) + (lane << 2);
            float v[4];
            Q::unpack(xt, v);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (et + i < n) put(y + et + i, (v[i] * inv) * widen(w[et + i]));
        }
    }
};

// ---------------------------------------------------------------------------
// SPLIT layout: a row is a sequence of 1 KB slices; lane t of a wavefront
// loads bytes 16t..16t+15 of a slice. A binary32 slice is one 256-element
// chunk and lane t's four values are the chains 4t..4t+3, as on the WAVE
// path. A bf16 slice is two chunks: lane t < 32 loads elements 8t..8t+7 of
// the first, lane t + 32 the same elements of the second. One 32-lane swap
// per register pair regroups them so that every lane holds the same four
// chains of both chunks: lane t < 32 chains 8t..8t+3, lane t + 32 chains
// 8t+4..8t+7.

template <bool NT>
__device__ __forceinline__ u32x4 gload16(gptr_c p) {
    auto* a = reinterpret_cast<const __attribute__((address_space(1))) u32x4*>(p);
    return NT ? __builtin_nontemporal_load(a) : *a;
}
template <bool NT>
__device__ __forceinline__ void gstore16(gptr p, u32x4 v) {
    auto* a = reinterpret_cast<__attribute__((address_space(1))) u32x4*>(p);
    if (NT) __builtin_nontemporal_store(v, a);
    else *a = v;
}


__device__ __forceinline__ void chain4(float p[4], float v0, float v1, float v2, float v3) {
    p[0] = fmaf(v0, v0, p[0]);
    p[1] = fmaf(v1, v1, p[1]);
    p[2] = fmaf(v2, v2, p[2]);
    p[3] = fmaf(v3, v3, p[3]);
}

// One slice into the lane chains, chunks in ascending order.
__device__ __forceinline__ void slice_chains(float p[4], u32x4 v, float) {
    chain4(p, __uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z),
           __uint_as_float(v.w));
}
__device__ __forceinline__ void slice_chains(float p[4], u32x4 v, uint16_t) {
    // first chunk: dwords x, y of the lower half-wave; second chunk: the same
    // dwords of the upper half-wave (see swap32)
    const SwapPair a = swap32(v.x, v.z);
    const SwapPair b = swap32(v.y, v.w);
    chain4(p, lo_bf16(a.first), hi_bf16(a.first), lo_bf16(b.first), hi_bf16(b.first));
    chain4(p, lo_bf16(a.second), hi_bf16(a.second), lo_bf16(b.second), hi_bf16(b.second));
}

// Group trees and combine for the SPLIT layout.
__device__ __forceinline__ float split_sumsq(const float p[4], int, float) {
    return wave_sumsq(p[0], p[1], p[2], p[3]);  // binary32: the WAVE layout
}
// bf16: group g is lanes 8g..8g+7 and 8g+32..8g+39; association lane 64g+j
// sits in lane 8g + (j/8) + 32*((j/4)&1), register j%4.
__device__ __forceinline__ float split_sumsq(const float p[4], int lane, uint16_t) {
    float q[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        // halving s = 32, 16, 8: partner j+s is s/8 lanes further
        q[e] = p[e] + row_shl<4>(p[e]);
        q[e] = q[e] + row_shl<2>(q[e]);
        q[e] = q[e] + row_shl<1>(q[e]);
    }
    // j = e sits in lane 8g, j = 4+e in lane 8g+32. Halving s = 4 pairs the
    // two: the lower lane adds registers 0 and 2, the upper lane 1 and 3.
    const SwapPair s01 = swap32(__float_as_uint(q[0]), __float_as_uint(q[1]));
    const SwapPair s23 = swap32(__float_as_uint(q[2]), __float_as_uint(q[3]));
    const bool low = lane < 32;
    const float a0 = low ? q[0] : __uint_as_float(s01.first);   // j = e (e = 0 or 1)
    const float a4 = low ? __uint_as_float(s01.second) : q[1];  // j = e + 4
    const float c0 = low ? q[2] : __uint_as_float(s23.first);   // j = e + 2
    const float c4 = low ? __uint_as_float(s23.second) : q[3];  // j = e + 6
    // s = 2 in the lane; s = 1 between lane 8g (e = 0) and lane 8g+32 (e = 1)
    const float t = (a0 + a4) + (c0 + c4);
    const float g0 = lane_value(t, 0) + lane_value(t, 32);
    const float g1 = lane_value(t, 8) + lane_value(t, 40);
    const float g2 = lane_value(t, 16) + lane_value(t, 48);
    const float g3 = lane_value(t, 24) + lane_value(t, 56);
    return (g0 + g2) + (g1 + g3);
}

// y = (x * inv) * w for one slice, packed back into 16 bytes.
__device__ __forceinline__ u32x4 slice_apply(u32x4 x, u32x4 w, float inv, float) {
    u32x4 o;
    o.x = __float_as_uint((__uint_as_float(x.x) * inv) * __uint_as_float(w.x));
    o.y = __float_as_uint((__uint_as_float(x.y) * inv) * __uint_as_float(w.y));
    o.z = __float_as_uint((__uint_as_float(x.z) * inv) * __uint_as_float(w.z));
    o.w = __float_as_uint((__uint_as_float(x.w) * inv) * __uint_as_float(w.w));
    return o;
}
__device__ __forceinline__ uint32_t apply_pair(uint32_t x, uint32_t w, float inv) {
    const float lo = (lo_bf16(x) * inv) * lo_bf16(w);
    const float hi = (hi_bf16(x) * inv) * hi_bf16(w);
    return bf16_pair(lo, hi);
}
__device__ __forceinline__ u32x4 slice_apply(u32x4 x, u32x4 w, float inv, uint16_t) {
    u32x4 o;
    o.x = apply_pair(x.x, w.x, inv);
    o.y = apply_pair(x.y, w.y, inv);
    o.z = apply_pair(x.z, w.z, inv);
    o.w = apply_pair(x.w, w.w, inv);
    return o;
}

// The U slices wavefront s of a row owns: slices s*U .. s*U+U-1. nvec is the
// row's length in 16-byte vectors (the plan makes n * sizeof(T) a multiple of
// 16); vector v*64 + lane of the row is this lane's part of slice v. EXACT:
// every slice of every wavefront is complete (nvec == 64 * U * wavefronts).
// Otherwise vectors past the row are loaded from the row's last vector (an
// in-row address, so no load needs a branch), count as +0 in the chains and
// are not stored.
template <typename T, int U, bool EXACT, bool NT>
struct SplitPart {
    u32x4 xr[U], wr[U];
    uint32_t vi0;  // this lane's vector index in its first slice

    // A scalar base per 4 slices keeps each load's offset in the immediate field.
    static __device__ __forceinline__ uint32_t base_bytes(int s, int u) {
        return (uint32_t)(s * U + (u & ~3)) * 1024u;
    }
    static __device__ __forceinline__ uint32_t lane_bytes(int lane, int u) {
        return (uint32_t)lane * 16u + (uint32_t)(u & 3) * 1024u;
    }
    __device__ __forceinline__ bool in_row(int u, uint32_t nvec) const {
        return EXACT || vi0 + 64u * (uint32_t)u < nvec;
    }

    __device__ __forceinline__ void load(gptr_c x, gptr_c w, int s, int lane, uint32_t nvec) {
        load_x(x, s, lane, nvec);
        load_w(w, s, lane, nvec);
    }
    // The two halves of load(), for callers that issue w's loads earlier.
    __device__ __forceinline__ void load_x(gptr_c x, int s, int lane, uint32_t nvec) {
        vi0 = (uint32_t)(s * U) * 64u + (uint32_t)lane;
        if (EXACT) {
#pragma unroll
            for (int u = 0; u < U; ++u)
                xr[u] = gload16<NT>(scalar_gptr(x + base_bytes(s, u)) + lane_bytes(lane, u));
        } else {
            const uint32_t last = nvec - 1u;
#pragma unroll
            for (int u = 0; u < U; ++u)
                xr[u] = gload16<NT>(x + min(vi0 + 64u * (uint32_t)u, last) * 16u);
        }
    }
    __device__ __forceinline__ void load_w(gptr_c w, int s, int lane, uint32_t nvec) {
        const uint32_t v0 = (uint32_t)(s * U) * 64u + (uint32_t)lane;
        if (EXACT) {
#pragma unroll
            for (int u = 0; u < U; ++u)
                wr[u] = gload16<false>(scalar_gptr(w + base_bytes(s, u)) + lane_bytes(lane, u));
        } else {
            const uint32_t last = nvec - 1u;
#pragma unroll
            for (int u = 0; u < U; ++u)
                wr[u] = gload16<false>(w + min(v0 + 64u * (uint32_t)u, last) * 16u);
        }
    }

    __device__ __forceinline__ void chains(float p[4], uint32_t nvec) const {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const u32x4 v = in_row(u, nvec) ? xr[u] : u32x4{0u, 0u, 0u, 0u};
            slice_chains(p, v, T());
        }
    }

    __device__ __forceinline__ void apply(float inv, gptr y, int s, int lane, uint32_t nvec) const {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const u32x4 o = slice_apply(xr[u], wr[u], inv, T());
            if (EXACT)
                gstore16<NT>(scalar_gptr(y + base_bytes(s, u)) + lane_bytes(lane, u), o);
            else if (in_row(u, nvec))
                gstore16<NT>(y + (vi0 + 64u * (uint32_t)u) * 16u, o);
        }
    }
};

// Register buckets of the WAVE and BLOCK instances (chunks of 256 elements per
// lane); the list matches kChunkBuckets in rmsn_plan.h.
#define RMSN_FOR_BUCKETS(X) X(1) X(2) X(4) X(6) X(8) X(12) X(16) X(20) X(24) X(28) X(32)

// ---------------------------------------------------------------------------
// GROUP layout: 256 threads per row; wavefront g owns association group g.
// Instances: Q = 1..8 blocks of 1024 elements (rows up to 8192).
#define RMSN_FOR_GROUP_BLOCKS(X) X(1) X(2) X(3) X(4) X(5) X(6) X(7) X(8)

// One row on the GROUP layout, Q blocks of 1024 elements: requires
// 1024 (Q-1) < n <= 1024 Q, n a multiple of 4 and x, w, y aligned to a quad
// (16 B binary32, 8 B bf16). Blocks below Q-1 are complete; in the last one,
// quads past the row are loaded from the row's last quad (an in-row address)
// and masked to +0 after every load has been issued.
//
// m0, m1: the blocks [m0, m1) this workgroup applies and stores (wave-uniform;
// the whole row by default). Every call reads the whole of x and computes the
// whole row's sum, so a row may be applied by several workgroups, each taking
// a block range (REPLICA), with every workgroup's inv bit-identical.
template <typename T, int Q>
__device__ __forceinline__ void row_group(const T* x, const T* __restrict__ w, T* y, int n,
                                          float eps, float* lds4, int m0 = 0, int m1 = Q) {
    using QD = Quad<T>;
    constexpr uint32_t es = sizeof(T);
    const int g = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const uint32_t off = (uint32_t)((lane >> 4) * 256 + g * 64 + (lane & 15) * 4);  // elements
    const uint32_t last = (uint32_t)n - 4u;
    const bool exact = n == 1024 * Q;
    typename QD::raw xr[Q], wr[Q];
    gptr_c xg = scalar_gptr(reinterpret_cast<const char*>(x));
    gptr_c wg = scalar_gptr(reinterpret_cast<const char*>(w));
#pragma unroll
    for (int m = 0; m < Q; ++m) {
        const uint32_t e = m + 1 < Q || exact ? 1024u * m + off : min(1024u * m + off, last);
        xr[m] = QD::template gload<false>(xg + e * es);
    }
#pragma unroll
    for (int m = 0; m < Q; ++m) {
        const uint32_t e = m + 1 < Q || exact ? 1024u * m + off : min(1024u * m + off, last);
        if (m >= m0 && m < m1) wr[m] = QD::template gload<false>(wg + e * es);
        else wr[m] = QD::zero();
    }
    __builtin_amdgcn_sched_barrier(0);
    const bool tail_in = exact || 1024u * (Q - 1) + off < (uint32_t)n;
    float p = 0.0f;
#pragma unroll
    for (int m = 0; m < Q; ++m) {
        float v[4];
        QD::unpack(xr[m], v);
        if (m + 1 == Q && !tail_in) v[0] = v[1] = v[2] = v[3] = 0.0f;
        transpose4(v);
        p = fmaf(v[0], v[0], p);  // chunks 4m, 4m+1, 4m+2, 4m+3 of chain 64g + 4t + q
        p = fmaf(v[1], v[1], p);
        p = fmaf(v[2], v[2], p);
        p = fmaf(v[3], v[3], p);
    }
    const float gt = group_sumsq(p);
    if (lane == 0) lds4[g] = gt;
    __syncthreads();
    const float inv = inverse_rms((lds4[0] + lds4[2]) + (lds4[1] + lds4[3]), n, eps);
    gptr yg = scalar_gptr(reinterpret_cast<char*>(y));
#pragma unroll
    for (int m = 0; m < Q; ++m) {
        if (m < m0 || m >= m1) continue;
        if (m + 1 == Q && !tail_in) continue;
        float v[4], wv[4], o[4];
        QD::unpack(xr[m], v);
        QD::unpack(wr[m], wv);
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = (v[i] * inv) * wv[i];
        QD::template gstore<false>(yg + (1024u * m + off) * es, o);
    }
}


// ---------------------------------------------------------------------------
// BLOCK / STREAM layout: 256 threads per row, thread l = chain l, wave g = group g.

// Descending halving over the 64 lanes of this wavefront; the total lands in lane 0.
__device__ __forceinline__ float group_tree(float v) {
    v += __shfl_down(v, 32, 64);
    v += __shfl_down(v, 16, 64);
    v += row_shl<8>(v);
    v += row_shl<4>(v);
    v += row_shl<2>(v);
    v += row_shl<1>(v);
    return v;
}

// Group trees, the combine through LDS, and steps 4-7. Every thread of the
// block calls this once per row with its finished chain p.
__device__ __forceinline__ float block_inverse(float p, int n, float eps, float* lds4) {
    const float g = group_tree(p);
    if ((threadIdx.x & 63) == 0) lds4[threadIdx.x >> 6] = g;
    __syncthreads();
    const float ss = (lds4[0] + lds4[2]) + (lds4[1] + lds4[3]);
    return inverse_rms(ss, n, eps);
}

// NCH > 0: rows with 256 * prev_bucket(NCH) < n <= 256 * NCH are held in
// registers; any other n (possible for descriptor rows rewritten between graph
// replays) is streamed. NCH == 0: always streamed. x, w, y are global memory.
template <typename T, int NCH>
__device__ __forceinline__ void row_block(const T* x, const T* __restrict__ w, T* y, int n,
                                          float eps, float* lds4) {
    using E = Elem<T>;
    constexpr int MINF = prev_bucket(NCH);
    const uint32_t l = threadIdx.x;  // association lane 0..255
    const int full = n >> 8;         // complete 256-element chunks (wave-uniform)
    gptr_c xg = scalar_gptr(x);
    gptr_c wg = scalar_gptr(w);
    gptr yg = scalar_gptr(y);
    float p = 0.0f;
    if (NCH > 0 && full >= MINF && full + ((n & 255) != 0) <= NCH) {
        constexpr int R = NCH > 0 ? NCH : 1;
        // a scalar base per 4 KB of the row keeps every chunk's offset in the
        // instruction's immediate field
        constexpr uint32_t per_base = 4096 / (256 * sizeof(T));
        // Chunks below MINF are complete. The others (the bucket's top chunks:
        // complete, ragged or past the row) are loaded from a clamped, in-row
        // index without branches and masked to +0 past the row only after every
        // load of x and w has been issued (the scheduling barrier keeps the
        // compiler from waiting for x before issuing w).
        typename E::raw_t xr[R], wr[R];
#pragma unroll
        for (int k = 0; k < R; ++k) {
            const uint32_t kb = (uint32_t)(k / per_base) * 4096u;
            const uint32_t d = (uint32_t)(k % per_base) * 256u + l;
            if (k < MINF)
                xr[k] = E::raw(scalar_gptr(xg + kb), d);
            else
                xr[k] = E::raw(xg, min(((uint32_t)k << 8) + l, (uint32_t)n - 1u));
        }
#pragma unroll
        for (int k = 0; k < R; ++k) {
            const uint32_t kb = (uint32_t)(k / per_base) * 4096u;
            const uint32_t d = (uint32_t)(k % per_base) * 256u + l;
            if (k < MINF)
                wr[k] = E::raw(scalar_gptr(wg + kb), d);
            else
                wr[k] = E::raw(wg, min(((uint32_t)k << 8) + l, (uint32_t)n - 1u));
        }
        __builtin_amdgcn_sched_barrier(0);
        float xv[R], wv[R];
#pragma unroll
        for (int k = 0; k < R; ++k) {
            xv[k] = E::value(xr[k]);
            wv[k] = E::value(wr[k]);
            if (k >= MINF && ((uint32_t)k << 8) + l >= (uint32_t)n) xv[k] = 0.0f;
            p = fmaf(xv[k], xv[k], p);  // +0 past the row: no change
        }
        const float inv = block_inverse(p, n, eps, lds4);
#pragma unroll
        for (int k = 0; k < R; ++k) {
            const float v = (xv[k] * inv) * wv[k];
            if (k < MINF) {
                const uint32_t kb = (uint32_t)(k / per_base) * 4096u;
                E::store(scalar_gptr(yg + kb), (uint32_t)(k % per_base) * 256u + l, v);
            } else if (((uint32_t)k << 8) + l < (uint32_t)n) {
                E::store(yg, ((uint32_t)k << 8) + l, v);
            }
        }
    } else {
        for (uint32_t d = l; d < (uint32_t)n; d += 256) {
            const float v = E::load(xg, d);
            p = fmaf(v, v, p);
        }
        const float inv = block_inverse(p, n, eps, lds4);
        for (uint32_t d = l; d < (uint32_t)n; d += 256)
            E::store(yg, d, (E::load(xg, d) * inv) * E::load(wg, d));
    }
}

}  // namespace
}  // namespace rmsn
