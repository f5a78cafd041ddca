// rmsn_aux.hip -- the small kernels every build of the library carries: the
// position update of a positioned sequence and the diagnostics that run the
// row kernels' own steps 4-7 and bf16 narrowing over bit-pattern ranges.
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

}  // namespace

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
