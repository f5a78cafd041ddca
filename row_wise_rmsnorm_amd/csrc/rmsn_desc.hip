// rmsn_desc.hip -- the descriptor kernels: one row whose pointers and width
// are read from a device-resident table when the kernel runs, for the
// decode-step sequence run eagerly or replayed from a captured graph (Lecture
// 08 "Graph-resident decode", sections 1 and 2).
//
// This file is compiled twice, with the same device code:
//   RMSN_DESC_PRELOADED=1  kernel arguments preloaded into SGPRs by the
//                          dispatcher (launch_desc_preloaded);
//   RMSN_DESC_PRELOADED=0  the kernel loads its arguments itself
//                          (launch_desc_plain).
// Measured on MI355X (327-norm decode step): preloading takes about 0.15 us
// off each node of a captured graph (the kernel's first scalar load is gone)
// but adds about 0.17 us to each launch enqueued one by one while the HIP
// runtime keeps those launches' arguments in device memory (its default
// here); with the arguments in host memory (HIP_FORCE_DEV_KERNARG=0) the
// preloaded build is the faster one for those launches too. The bits are the
// same either way.
//
// Floating point as in rmsn_kernels.hip: contraction off, the one fused
// operation written as fmaf, correctly rounded '/' and sqrtf.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rmsn_common.h"
#include "rmsn_group.h"
#include "rmsn_launch.h"
#include "rmsn_rows.h"

#pragma clang fp contract(off)

#ifndef RMSN_DESC_PRELOADED
#error "rmsn_desc.hip is built with RMSN_DESC_PRELOADED=0 and =1"
#endif
#if RMSN_DESC_PRELOADED
#define RMSN_DESC_NS desc_preloaded
#define RMSN_DESC_LAUNCH launch_desc_preloaded
#else
#define RMSN_DESC_NS desc_loaded
#define RMSN_DESC_LAUNCH launch_desc_plain
#endif

namespace rmsn {
namespace RMSN_DESC_NS {
namespace {

// GROUP-layout descriptor row: the captured instance Q is used when the row
// read at run time fits it (width in (1024 (Q-1), 1024 Q], a multiple of 4,
// quad-aligned pointers); any other row is streamed with BLOCK's mapping.
template <typename T, int Q, bool POS>
__global__ __launch_bounds__(256) void k_desc_group(const rmsn_desc* __restrict__ d, float eps,
                                                    PosArgs pa) {
    __shared__ float lds4[4];
    uint64_t pos;
    const rmsn_desc dd = desc_load<POS>(d, pa, &pos);
    const int64_t n = dd.n;
    if (n < 1 || n > RMSN_MAX_N) return;
    const T* x;
    T* y;
    desc_row<T, POS>(dd, pos, pa, x, y);
    const T* w = static_cast<const T*>(dd.w);
    const uintptr_t a = reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(w) |
                        reinterpret_cast<uintptr_t>(y);
    if ((n & 3) == 0 && n > 1024 * (Q - 1) && n <= 1024 * Q && a % (4 * sizeof(T)) == 0)
        row_group<T, Q>(x, w, y, (int)n, eps, lds4);
    else
        row_block<T, 0>(x, w, y, (int)n, eps, lds4);
}

// One row whose pointers and width are read from device memory when the
// kernel runs (Lecture 08 "Graph-resident decode", section 2: a value used
// only as a loop bound can live in device memory; the launch geometry comes
// from the capture-time width).
template <typename T, int NCH, bool POS>
__global__ __launch_bounds__(256) void k_desc_block(const rmsn_desc* __restrict__ d, float eps,
                                                    PosArgs pa) {
    __shared__ float lds4[4];
    uint64_t pos;
    const rmsn_desc dd = desc_load<POS>(d, pa, &pos);
    const int64_t n = dd.n;
    if (n < 1 || n > RMSN_MAX_N) return;
    const T* x;
    T* y;
    desc_row<T, POS>(dd, pos, pa, x, y);
    row_block<T, NCH>(x, static_cast<const T*>(dd.w), y, (int)n, eps, lds4);
}

template <typename T, bool POS>
hipError_t launch_desc_t(const Plan& p, const rmsn_desc* d, float eps, const PosArgs& pa,
                         hipStream_t s) {
    if (p.path == RMSN_PATH_GROUP) {
#define RMSN_CASE(Q)                                                                          \
    case Q:                                                                                   \
        hipLaunchKernelGGL((k_desc_group<T, Q, POS>), dim3(1), dim3(256), 0, s, d, eps, pa);  \
        break;
        switch (p.loads) {
            RMSN_FOR_GROUP_BLOCKS(RMSN_CASE)
            default: return hipErrorInvalidValue;
        }
#undef RMSN_CASE
        return hipGetLastError();
    }
#define RMSN_CASE(C)                                                                          \
    case C:                                                                                   \
        hipLaunchKernelGGL((k_desc_block<T, C, POS>), dim3(1), dim3(256), 0, s, d, eps, pa);  \
        break;
    switch (p.chunks) {
        RMSN_CASE(0)
        RMSN_FOR_BUCKETS(RMSN_CASE)
        default: return hipErrorInvalidValue;
    }
#undef RMSN_CASE
    return hipGetLastError();
}

}  // namespace
}  // namespace RMSN_DESC_NS

hipError_t RMSN_DESC_LAUNCH(const Plan& p, const rmsn_desc* d, float eps, const PosArgs* pos,
                          hipStream_t stream) {
    using RMSN_DESC_NS::launch_desc_t;
    if (p.path == RMSN_PATH_WAVE || p.path == RMSN_PATH_SPLIT)
        return hipErrorInvalidValue;  // descriptors use GROUP, BLOCK or STREAM
    if (pos)
        return p.dtype == RMSN_F32 ? launch_desc_t<float, true>(p, d, eps, *pos, stream)
                                   : launch_desc_t<uint16_t, true>(p, d, eps, *pos, stream);
    const PosArgs none{nullptr, 0, 0, 1};
    return p.dtype == RMSN_F32 ? launch_desc_t<float, false>(p, d, eps, none, stream)
                               : launch_desc_t<uint16_t, false>(p, d, eps, none, stream);
}

}  // namespace rmsn
