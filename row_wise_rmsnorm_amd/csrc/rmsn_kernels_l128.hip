// rmsn_kernels_l128.hip -- the row kernels of the 128-lane build.
//
// Lecture 04 "Launch Geometry: Grids, Occupancy, and 327 Norms per Token",
// section 2.1: the kernel's sum of squares runs on exactly 128 threads, the
// elementwise apply on the whole (wider) block, and only the first of the two
// decides the bits. This library variant computes that association ("R128"):
//   lane chains  p[l] = fmaf(x[d], x[d], p[l]), d = l, l+128, ... (l < 128)
//   group trees  four 32-lane groups (the lecture's four warps), descending
//                halving 16, 8, 4, 2, 1
//   combine      ss = (G0 + G2) + (G1 + G3)
// and steps 4-8 as in every build. One workgroup of B threads per row
// (B = 128, 256, 512 or 1024: the apply width): threads 0..127 are the
// chains, wavefront w holding groups 2w and 2w+1 (lanes 0..31 and 32..63);
// every thread then applies. The row is streamed: read once for the sum and
// once more for the apply (quads when x, w and y are quad-aligned and n is a
// multiple of 4, elements otherwise), the second read mostly from L2.
#include "rmsn_common.h"

namespace rmsn {
namespace {

// Descending halving over each 32-lane half of the wavefront: 16 across the
// half's two DPP rows, then 8/4/2/1 inside them; totals land in lanes 0 and 32.
__device__ __forceinline__ float half_wave_tree(float v) {
    v += __shfl_down(v, 16, 32);
    v += row_shl<8>(v);
    v += row_shl<4>(v);
    v += row_shl<2>(v);
    v += row_shl<1>(v);
    return v;
}

template <typename T>
__device__ __forceinline__ void row_narrow(const T* x, const T* __restrict__ w, T* y, int n,
                                           float eps, float* lds4) {
    using E = Elem<T>;
    using Q = Quad<T>;
    const uint32_t t = threadIdx.x;
    gptr_c xg = scalar_gptr(x);
    gptr_c wg = scalar_gptr(w);
    gptr yg = scalar_gptr(y);
    if (t < 128) {  // wavefronts 0 and 1: the narrow reduction
        float p = 0.0f;
        for (uint32_t d = t; d < (uint32_t)n; d += 128) {
            const float v = E::load(xg, d);
            p = fmaf(v, v, p);
        }
        const float g = half_wave_tree(p);
        if ((t & 31) == 0) lds4[t >> 5] = g;
    }
    __syncthreads();
    const float inv = inverse_rms((lds4[0] + lds4[2]) + (lds4[1] + lds4[3]), n, eps);
    // the wide apply: every thread of the block
    const uint32_t B = blockDim.x;
    const uintptr_t a = reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(w) |
                        reinterpret_cast<uintptr_t>(y);
    if ((n & 3) == 0 && a % (4 * sizeof(T)) == 0) {
        for (uint32_t q = t; q < (uint32_t)n >> 2; q += B) {
            const uint32_t off = q * 4u * (uint32_t)sizeof(T);
            float v[4], wv[4], o[4];
            Q::unpack(Q::template gload<false>(xg + off), v);
            Q::unpack(Q::template gload<false>(wg + off), wv);
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = (v[i] * inv) * wv[i];
            Q::template gstore<false>(yg + off, o);
        }
    } else {
        for (uint32_t d = t; d < (uint32_t)n; d += B)
            E::store(yg, d, (E::load(xg, d) * inv) * E::load(wg, d));
    }
}

template <typename T>
__global__ __launch_bounds__(1024) void k_rows_narrow(const T* x, int64_t xs,
                                                     const T* __restrict__ w, T* y, int64_t ys,
                                                     int n, float eps) {
    __shared__ float lds4[4];
    const int64_t r = blockIdx.x;
    row_narrow<T>(x + r * xs, w, y + r * ys, n, eps, lds4);
}

template <typename T, bool POS>
__global__ __launch_bounds__(1024) void k_desc_narrow(const rmsn_desc* __restrict__ d, float eps,
                                                     PosArgs pa) {
    __shared__ float lds4[4];
    uint64_t pos;
    const rmsn_desc dd = desc_load<POS>(d, pa, &pos);
    const int64_t n = dd.n;
    if (n < 1 || n > RMSN_MAX_N) return;
    const T* x;
    T* y;
    desc_row<T, POS>(dd, pos, pa, x, y);
    row_narrow<T>(x, static_cast<const T*>(dd.w), y, (int)n, eps, lds4);
}

// The whole sequence in one launch of one workgroup, rows in table order
// (the same contract as the default build's persistent kernel).
template <typename T, bool POS>
__global__ __launch_bounds__(1024) void k_sequence_narrow(const rmsn_desc* __restrict__ d,
                                                         int32_t count, float eps, PosArgs pa) {
    __shared__ float lds4[4];
    uint64_t pos;
    rmsn_desc next = desc_load<POS>(d, pa, &pos);
    for (int32_t i = 0; i < count; ++i) {
        const rmsn_desc cur = next;
        if (i + 1 < count) {
            uint64_t unused;
            next = desc_load<false>(d + i + 1, pa, &unused);
        }
        const int64_t n = cur.n;
        if (n >= 1 && n <= RMSN_MAX_N) {
            const T* x;
            T* y;
            desc_row<T, POS>(cur, pos, pa, x, y);
            row_narrow<T>(x, static_cast<const T*>(cur.w), y, (int)n, eps, lds4);
        }
        __syncthreads();
    }
    if (POS && threadIdx.x == 0) {
        const uint64_t per = (uint64_t)pa.period;
        const uint64_t p = pos < per ? pos : pos % per;
        const_cast<int64_t*>(pa.d_pos)[0] = (int64_t)(p + 1 == per ? 0 : p + 1);
    }
}

bool narrow_block(const Plan& p) {
    return p.path == RMSN_PATH_BLOCK &&
           (p.block == 128 || p.block == 256 || p.block == 512 || p.block == 1024);
}

}  // namespace

hipError_t launch_rows(const Plan& p, const void* x, int64_t xs, const void* w, void* y,
                       int64_t ys, int64_t rows, int n, float eps, hipStream_t stream) {
    if (!narrow_block(p) || p.grid != rows || p.grid < 1 || p.grid > 0x7FFFFFFF)
        return hipErrorInvalidValue;
    const dim3 grid((unsigned)p.grid), block((unsigned)p.block);
    if (p.dtype == RMSN_F32)
        hipLaunchKernelGGL(k_rows_narrow<float>, grid, block, 0, stream,
                           static_cast<const float*>(x), xs, static_cast<const float*>(w),
                           static_cast<float*>(y), ys, n, eps);
    else
        hipLaunchKernelGGL(k_rows_narrow<uint16_t>, grid, block, 0, stream,
                           static_cast<const uint16_t*>(x), xs, static_cast<const uint16_t*>(w),
                           static_cast<uint16_t*>(y), ys, n, eps);
    return hipGetLastError();
}

// One build of the descriptor kernel here: eager launches and the launches a
// graph records share it.
hipError_t launch_desc_plain(const Plan& p, const rmsn_desc* d, float eps, const PosArgs* pos,
                             hipStream_t stream) {
    if (!narrow_block(p)) return hipErrorInvalidValue;
    const dim3 block((unsigned)p.block);
    const PosArgs none{nullptr, 0, 0, 1};
    if (p.dtype == RMSN_F32) {
        if (pos) hipLaunchKernelGGL((k_desc_narrow<float, true>), dim3(1), block, 0, stream, d, eps, *pos);
        else hipLaunchKernelGGL((k_desc_narrow<float, false>), dim3(1), block, 0, stream, d, eps, none);
    } else {
        if (pos) hipLaunchKernelGGL((k_desc_narrow<uint16_t, true>), dim3(1), block, 0, stream, d, eps, *pos);
        else hipLaunchKernelGGL((k_desc_narrow<uint16_t, false>), dim3(1), block, 0, stream, d, eps, none);
    }
    return hipGetLastError();
}

hipError_t launch_desc_preloaded(const Plan& p, const rmsn_desc* d, float eps, const PosArgs* pos,
                             hipStream_t stream) {
    return launch_desc_plain(p, d, eps, pos, stream);
}

// The WIDE path splits R256's four groups over workgroups; this build's plan
// never takes it.
hipError_t launch_wide_rows(const Plan&, const void*, int64_t, const void*, void*, int64_t,
                            int64_t, int, float, float*, hipStream_t) {
    return hipErrorInvalidValue;
}

// This build's persistent launch walks one workgroup row after row with
// barriers and never polls: it has no timeouts to count.
hipError_t walk_timeouts(uint32_t* out, bool) {
    *out = 0;
    return hipSuccess;
}

hipError_t launch_sequence_persistent(int dtype, const rmsn_desc* d, int32_t count, float eps,
                                     const PosArgs* pos, hipStream_t stream) {
    const int b = option_apply_threads();
    const dim3 grid(1), block((unsigned)(b == 0 ? 1024 : b));
    const PosArgs none{nullptr, 0, 0, 1};
    if (dtype == RMSN_F32) {
        if (pos) hipLaunchKernelGGL((k_sequence_narrow<float, true>), grid, block, 0, stream, d, count, eps, *pos);
        else hipLaunchKernelGGL((k_sequence_narrow<float, false>), grid, block, 0, stream, d, count, eps, none);
    } else {
        if (pos) hipLaunchKernelGGL((k_sequence_narrow<uint16_t, true>), grid, block, 0, stream, d, count, eps, *pos);
        else hipLaunchKernelGGL((k_sequence_narrow<uint16_t, false>), grid, block, 0, stream, d, count, eps, none);
    }
    return hipGetLastError();
}

}  // namespace rmsn
