// rmsn_plan.h -- launch planning and argument validation (pure host C++, no
// HIP). One function decides every launch, so an eager call, a graph capture
// and a plan query can never disagree (Lecture 08 "Graph-resident decode",
// section 2: the capture check and the launcher call the same plan function).
#pragma once

#include <stdint.h>

#include "rmsnorm.h"

// Lane chains of the association this library variant computes: 256 (R256), or 128 for
// the build that reproduces the 128-thread sum of Lecture 04 section 2.1
// (compiled with -DRMSN_LANES=128; its only layout is one workgroup per row
// whose first 128 threads sum and whose every thread applies).
#ifndef RMSN_LANES
#define RMSN_LANES 256
#endif

namespace rmsn {

constexpr int kAssocLanes = RMSN_LANES;
static_assert(kAssocLanes == 256 || kAssocLanes == 128, "RMSN_LANES must be 256 or 128");

constexpr int kLanes = 256;      // lane chains of R256 (chunk width of its layouts)
constexpr int kWave = 64;        // CDNA wavefront width
constexpr int kBlockThreads = 256;
constexpr int kMaxChunks = 32;   // largest row held in registers: 32 * 256 = 8192
// Register-resident kernel instances: a lane keeps `chunks` values (BLOCK
// path) or groups of four values (WAVE path), one per 256 elements of the row.
constexpr int kChunkBuckets[] = {1, 2, 4, 6, 8, 12, 16, 20, 24, 28, 32};
constexpr int kNumBuckets = sizeof(kChunkBuckets) / sizeof(kChunkBuckets[0]);
// Row counts from which the WAVE path is chosen automatically: below it a row
// gets a whole workgroup (four wavefronts) so its loads spread over four SIMDs.
constexpr int64_t kWaveMinRows = 1024;
// Launch footprints (x read + y written) from which the WAVE path streams with
// non-temporal hints: far beyond the 32 MB of L2 and a large share of the
// 256 MB last-level cache, where keeping the rows cached cannot pay.
constexpr int64_t kStreamBytes = 64ll << 20;
// SPLIT path: a row is cut into 1 KB slices (one 16-byte load per lane of a
// wavefront); a workgroup of up to 16 wavefronts holds one row, each
// wavefront `loads` consecutive slices. Rows up to 128 slices (128 KB).
constexpr int kSliceBytes = 1024;
constexpr int kMaxSplitWaves = 16;
constexpr int kSplitLoads[] = {1, 2, 4, 8};
constexpr int kNumSplitLoads = sizeof(kSplitLoads) / sizeof(kSplitLoads[0]);

struct Plan {
    int dtype;           // RMSN_F32 / RMSN_BF16
    int path;            // RMSN_PATH_WAVE / _BLOCK / _STREAM / _SPLIT / _GROUP
    int chunks;          // kernel instance: a bucket, or 0 for streaming; SPLIT:
                         // 256-element chunks one wavefront holds
    int rows_per_block;  // wavefronts (= rows) per workgroup on the WAVE path, else 1
    int streaming;       // WAVE / SPLIT: non-temporal loads of x and stores of y
    int block;           // threads per workgroup
    int64_t grid;        // workgroups
    int loads;           // SPLIT: 16-byte loads per lane (slices per wavefront);
                         // GROUP, REPLICA: loads per lane (1024-element blocks);
                         // WIDE: apply workgroups per row; else 0
    int parts;           // REPLICA: workgroups per row, each applying a share of
                         // the row's blocks; else 1
};

inline int elem_bytes(int dtype) { return dtype == RMSN_F32 ? 4 : 2; }
// Rows one launch of plan p can hold. A dispatch counts its grid in
// work-items as a 32-bit number, so workgroups * block stays below 2^32 (and
// workgroups below 2^31); a batch beyond this goes as consecutive launches.
inline int64_t rows_per_launch(const Plan& p) {
    if (p.path == RMSN_PATH_WIDE)  // per row: 4 x 64 threads, then `loads` x 256
        return 0xFFFFFFFFll / (256ll * (p.loads > 1 ? p.loads : 1));
    int64_t groups = 0xFFFFFFFFll / (p.block > 0 ? p.block : 1);
    if (groups > 0x7FFFFFFFll) groups = 0x7FFFFFFFll;
    if (p.path == RMSN_PATH_REPLICA) return groups / (p.parts > 0 ? p.parts : 1);
    return groups * (p.rows_per_block > 0 ? p.rows_per_block : 1);
}
// Bytes one lane loads per 256-element chunk on the WAVE path: four elements.
inline int vec_bytes(int dtype) { return 4 * elem_bytes(dtype); }
// 1 KB slices of a row of width n (the last one may be partial).
inline int64_t split_slices(int dtype, int64_t n) {
    return (n * elem_bytes(dtype) + kSliceBytes - 1) / kSliceBytes;
}

// Smallest bucket holding ceil(n/256) chunks, or 0 if n needs more than kMaxChunks.
int chunk_bucket(int64_t n);

// Rows per workgroup and the streaming choice on the WAVE path, automatic.
int auto_rows_per_block(int64_t rows);
bool auto_streaming(int dtype, int64_t rows, int64_t n);
// Slices per wavefront on the SPLIT path for a row of `slices` slices (0 if
// the row is too long for kMaxSplitWaves wavefronts): 1, 2 or 4 by row
// length, as measured; 8 only where 4 would need more than 16 wavefronts.
int auto_split_loads(int64_t slices);

// Plan a launch of `rows` rows of width n. `align`: a byte alignment shared by
// every row start of x and y and by w (the largest power of two dividing it
// counts, up to 16; values 0 .. element size mean element alignment), or
// kAlignAtRunTime for descriptor rows, whose kernels check the pointers they
// read (only the GROUP path does, falling back to streaming when they do not
// fit). Returns RMSN_OK or RMSN_EINVAL (bad dtype, rows < 1, n outside
// [1, 2^24]).
// workspace: the launch may use one (rmsnorm_batched_rows_ws), which makes
// the WIDE path available. in_place: y == x; such a launch never takes
// REPLICA, whose workgroups read the whole row while their siblings store
// their shares of it.
constexpr int kAlignAtRunTime = -1;
int make_plan(int dtype, int64_t rows, int64_t n, int align, Plan* out, bool workspace = false,
              bool in_place = false);
// Elements one workgroup of the WIDE path's second launch applies.
constexpr int64_t kWideSpan = 4096;
// Rows of at least kWideMinBytes in batches of at most kWideMaxRows rows take
// the WIDE path when a workspace is available (measured on MI355X: below
// 64 KB a row is faster on SPLIT's one workgroup, whose loads are all in
// flight at once, than on two launches).
constexpr int64_t kWideMinBytes = 64 * 1024;
constexpr int64_t kWideMaxRows = 64;
// REPLICA path: workgroups per row when not set by option (capped at the
// row's block count).
constexpr int kReplicaParts = 4;

// Process-wide options (rmsnorm_set_option); read lazily from the environment.
int option_path();            // -1 automatic, else an RMSN_PATH_* value
int option_rows_per_block();  // 0 automatic, else 4 or 8
int option_streaming();       // -1 automatic, 0 off, 1 on
int option_split_loads();     // 0 automatic, else 1, 2, 4 or 8
int option_apply_threads();   // 128-lane build: 0 (= 1024) or 128, 256, 512, 1024
int option_persistent_workgroups();  // 0 automatic, 1 one workgroup
int option_replica_parts();   // 0 automatic, else 1..8 workgroups per row
int option_walk_spin_cap();   // 0 default, else polls per ordered wait (>= 1)
int set_option(int key, int value);
int get_option(int key, int* value);

// Argument checks shared by the entry points. Each returns RMSN_OK or
// RMSN_EINVAL and, on failure, sets the thread's last-error message.
int check_eps(float eps);
int check_row_args(int dtype, const void* x, int64_t xs, const void* w, const void* y, int64_t ys,
                   int64_t rows, int64_t n);
int check_sequence_args(int dtype, const rmsn_desc* d_table, const int64_t* h_widths,
                        int32_t count, float eps);
// Bytes of workspace plan p needs for `rows` rows (the four group totals of
// each row on the WIDE path, else none).
inline int64_t workspace_bytes(const Plan& p, int64_t rows) {
    return p.path == RMSN_PATH_WIDE ? rows * 4 * (int64_t)sizeof(float) : 0;
}
// A WIDE launch's workspace: non-null, 4-byte aligned, at least
// workspace_bytes, and overlapping none of x, w, y (arguments as
// check_row_args, which must have passed).
int check_workspace(int dtype, const void* x, int64_t xs, const void* w, const void* y,
                    int64_t ys, int64_t rows, int64_t n, const void* ws, int64_t ws_bytes);

void set_error(const char* fmt, ...);
void clear_error();
const char* last_error();

}  // namespace rmsn
