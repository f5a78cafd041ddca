// rmsn_launch.h -- host-side launchers of the gfx950 kernels (rmsn_kernels.hip,
// rmsn_desc.hip, rmsn_persistent.hip, rmsn_wide.hip, rmsn_aux.hip).
// Each enqueues on `stream` and returns the launch's hipError_t; none
// allocates or synchronises.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "rmsn_plan.h"
#include "rmsnorm.h"

namespace rmsn {

// `rows` rows, one per wavefront, with the geometry of plan `p`.
hipError_t launch_rows(const Plan& p, const void* x, int64_t xs, const void* w, void* y,
                       int64_t ys, int64_t rows, int n, float eps, hipStream_t stream);

// STREAM path (rmsn_wide.hip): one 256-thread workgroup per row, the row
// streamed twice.
hipError_t launch_stream_rows(const Plan& p, const void* x, int64_t xs, const void* w, void* y,
                              int64_t ys, int64_t rows, int n, float eps, hipStream_t stream);

// WIDE path (rmsn_wide.hip): two launches, the group totals of `rows` rows
// through ws (4 floats per row, device memory).
hipError_t launch_wide_rows(const Plan& p, const void* x, int64_t xs, const void* w, void* y,
                            int64_t ys, int64_t rows, int n, float eps, float* ws,
                            hipStream_t stream);

// The position of a positioned sequence, passed by value to its kernels: the
// position itself is device memory, read when the kernels run.
struct PosArgs {
    const int64_t* d_pos;
    int64_t x_pitch;  // bytes
    int64_t y_pitch;  // bytes
    int64_t period;   // >= 1
};

// One row described by the device-resident descriptor `d` (read when the
// kernel runs); plan `p` was made for the capture-time width. pos: NULL, or
// the row is taken at the sequence's device-resident position. Two builds of
// the same kernels (rmsn_desc.hip): launch_desc_preloaded, arguments
// preloaded into SGPRs by the dispatcher (the launches a sequence graph
// records), and launch_desc_plain, where the kernel loads its arguments
// (eager launches, unless the runtime keeps their arguments in host memory;
// rmsn_api.hip).
hipError_t launch_desc_plain(const Plan& p, const rmsn_desc* d, float eps, const PosArgs* pos,
                             hipStream_t stream);
hipError_t launch_desc_preloaded(const Plan& p, const rmsn_desc* d, float eps,
                                 const PosArgs* pos, hipStream_t stream);

// All `count` rows of a descriptor table, in order, in one launch of one
// workgroup; pos: NULL, or the rows are taken at the device-resident position
// and the position is advanced after the last row.
hipError_t launch_sequence_persistent(int dtype, const rmsn_desc* d, int32_t count, float eps,
                                     const PosArgs* pos, hipStream_t stream);

// Timeouts of the persistent launch's ordered waits since the last reset
// (the library's device counter; synchronous copies), and reset it if asked.
hipError_t walk_timeouts(uint32_t* out, bool reset);

// *d_pos = (*d_pos mod period + 1) mod period on the device (the state
// update of a positioned sequence).
hipError_t launch_advance(int64_t* d_pos, int64_t period, hipStream_t stream);

// A streaming copy of `bytes` (a multiple of 16) with `vectors` 16-byte
// vectors per lane in workgroups of `block` threads (diagnostic).
hipError_t launch_diag_copy(const void* src, void* dst, int64_t bytes, int vectors, int block,
                            hipStream_t stream);

// Step 8's bf16 narrowing over consecutive bit patterns (diagnostic).
hipError_t launch_diag_bf16(uint32_t first_bits, int64_t count, uint16_t* out,
                            hipStream_t stream);

// Steps 4-7 over consecutive bit patterns (diagnostic).
hipError_t launch_diag_inverse(uint32_t first_bits, int64_t count, int n, float eps, float* r_out,
                               float* inv_out, hipStream_t stream);

}  // namespace rmsn
