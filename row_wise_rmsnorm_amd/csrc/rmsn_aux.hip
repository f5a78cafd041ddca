// rmsn_aux.hip -- the small kernels every build of the library carries: the
// position update of a positioned sequence, the diagnostics that run the
// row kernels' own steps 4-7 and bf16 narrowing over bit-pattern ranges, and
// a plain streaming copy that measures what the memory system gives a pure
// copy of the same bytes (the ceiling the row kernels are compared with).
#include "rmsn_common.h"

namespace rmsn {
namespace {

// The state update of a positioned sequence, its last launch (captured as
// the graph's last node): the next launch of the sequence normalises the rows
// of the next position, p + 1 wrapped to [0, period). One thread, a
// vector-memory read-modify-write.
__global__ __launch_bounds__(64) void k_advance(int64_t* d_pos, int64_t period) {
    if (threadIdx.x != 0) return;
    const uint64_t pos = (uint64_t)d_pos[0];
    const uint64_t per = (uint64_t)period;
    const uint64_t p = pos < per ? pos : pos % per;
    d_pos[0] = (int64_t)(p + 1 == per ? 0 : p + 1);
}

// The bf16 narrowing of the row kernels over consecutive bit patterns, two per
// thread through the packed conversion the stores use.
__global__ __launch_bounds__(256) void k_diag_bf16(uint32_t first, int64_t count, uint16_t* out) {
    const int64_t i = 2 * ((int64_t)blockIdx.x * blockDim.x + threadIdx.x);
    if (i >= count) return;
    const float a = __uint_as_float(first + (uint32_t)i);
    if (i + 1 < count) {
        const uint32_t p = bf16_pair(a, __uint_as_float(first + (uint32_t)i + 1u));
        out[i] = (uint16_t)p;
        out[i + 1] = (uint16_t)(p >> 16);
    } else {
        out[i] = (uint16_t)bf16_bits(a);
    }
}

__global__ __launch_bounds__(256) void k_diag_inverse(uint32_t first, int64_t count, int n,
                                                      float eps, float* r_out, float* inv_out) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= count) return;
    const float ss = __uint_as_float(first + (uint32_t)i);
    const float r = mean_eps_root(ss, n, eps);
    r_out[i] = r;
    inv_out[i] = reciprocal(r);
}

// Copy of nvec 16-byte vectors: workgroup b takes V * blockDim.x consecutive
// vectors, lane t vectors t, t + blockDim.x, ... of them; non-temporal loads
// and stores (the streaming hints the prefill kernel uses).
template <int V>
__global__ void k_diag_copy(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                            uint64_t nvec) {
    const uint64_t base = (uint64_t)blockIdx.x * blockDim.x * V + threadIdx.x;
    u32x4 v[V];
#pragma unroll
    for (int k = 0; k < V; ++k) {
        const uint64_t i = base + (uint64_t)k * blockDim.x;
        if (i < nvec) v[k] = __builtin_nontemporal_load(src + i);
    }
#pragma unroll
    for (int k = 0; k < V; ++k) {
        const uint64_t i = base + (uint64_t)k * blockDim.x;
        if (i < nvec) __builtin_nontemporal_store(v[k], dst + i);
    }
}

}  // namespace

hipError_t launch_diag_copy(const void* src, void* dst, int64_t bytes, int vectors, int block,
                            hipStream_t stream) {
    const uint64_t nvec = (uint64_t)bytes / 16u;
    const uint64_t per = (uint64_t)block * (uint64_t)vectors;
    const uint64_t groups = (nvec + per - 1) / per;
    if (groups > 0x7FFFFFFFull || groups * (uint64_t)block > 0xFFFFFFFFull)
        return hipErrorInvalidConfiguration;
    const u32x4* a = static_cast<const u32x4*>(src);
    u32x4* b = static_cast<u32x4*>(dst);
    const dim3 grid((unsigned)groups), blk((unsigned)block);
    switch (vectors) {
        case 1: hipLaunchKernelGGL(k_diag_copy<1>, grid, blk, 0, stream, a, b, nvec); break;
        case 2: hipLaunchKernelGGL(k_diag_copy<2>, grid, blk, 0, stream, a, b, nvec); break;
        case 4: hipLaunchKernelGGL(k_diag_copy<4>, grid, blk, 0, stream, a, b, nvec); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_advance(int64_t* d_pos, int64_t period, hipStream_t stream) {
    hipLaunchKernelGGL(k_advance, dim3(1), dim3(64), 0, stream, d_pos, period);
    return hipGetLastError();
}

hipError_t launch_diag_bf16(uint32_t first_bits, int64_t count, uint16_t* out,
                            hipStream_t stream) {
    if (count <= 0) return hipSuccess;
    const int64_t blocks = (count + 511) / 512;
    // a dispatch counts its grid in work-items as a 32-bit number
    if (blocks * 256 > 0xFFFFFFFFll) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(k_diag_bf16, dim3((unsigned)blocks), dim3(256), 0, stream, first_bits, count,
                       out);
    return hipGetLastError();
}

hipError_t launch_diag_inverse(uint32_t first_bits, int64_t count, int n, float eps, float* r_out,
                               float* inv_out, hipStream_t stream) {
    if (count <= 0) return hipSuccess;
    const int64_t blocks = (count + 255) / 256;
    if (blocks * 256 > 0xFFFFFFFFll) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(k_diag_inverse, dim3((unsigned)blocks), dim3(256), 0, stream, first_bits,
                       count, n, eps, r_out, inv_out);
    return hipGetLastError();
}

}  // namespace rmsn
