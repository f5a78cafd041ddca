/*
 * rmsnorm.h -- C ABI of the MI355X (gfx950) row-wise RMSNorm library.
 *
 * Operation (Lecture 04 "Launch Geometry: Grids, Occupancy, and 327 Norms per
 * Token", section 2 and 2.1): for each row of width n,
 *     inv  = 1 / sqrt( (sum_d x[d]^2) / (float)n + eps )
 *     y[d] = (x[d] * inv) * w[d]
 * in IEEE binary32. The sum of squares uses one fixed association ("R256"),
 * which is part of the result's bits (section 2.1: the reduction's width is
 * part of the numerics, the elementwise apply's width is not):
 *   1. 256 lane chains: lane l = fmaf(x[d], x[d], lane l) for d = l, l+256, ...
 *      ascending, starting from +0;
 *   2. each 64-lane group reduced by descending halving (j + 32, 16, 8, 4, 2, 1);
 *   3. ss = (G0 + G2) + (G1 + G3);
 *   4-7. m = ss / (float)n; t = m + eps; r = sqrtf(t); inv = 1.0f / r, every
 *      operation correctly rounded (no approximate reciprocal square root);
 *   8. y = (x * inv) * w, left to right; bf16 outputs are rounded once to
 *      nearest even from the binary32 value.
 * Every entry point and every internal code path (register-resident rows,
 * streaming rows, any rows-per-workgroup, eager, graph or persistent replay,
 * any pointer alignment) gives the same bits. Denormals are preserved, NaN/Inf
 * propagate per IEEE (bf16 NaN outputs are quiet NaNs; payloads are not
 * specified). A second build of this same ABI computes the lecture's own
 * 128-thread sum instead of R256 (see rmsnorm_association_lanes).
 *
 * Conventions for every call:
 *  - Tensor pointers are DEVICE pointers owned by the caller. The library
 *    never allocates, frees or synchronises inside rmsnorm_f32, rmsnorm_bf16,
 *    rmsnorm_batched_rows(_ws, _noalloc), rmsnorm_sequence_eager(_positioned),
 *    rmsnorm_sequence_persistent or rmsnorm_sequence_graph_launch, so each of
 *    them may itself be captured into a caller's HIP graph. Only the graph
 *    creation and update calls create HIP objects; they also allocate a
 *    256-byte device row for the pre-warm launches and synchronise their own
 *    private stream, and free the row before they return.
 *  - `stream` is a hipStream_t (NULL = the default stream). Work is enqueued
 *    asynchronously; the return value reports argument and launch errors
 *    only. A fault inside a kernel surfaces at the caller's next
 *    synchronisation.
 *  - Return value: an rmsn_status. On failure nothing is enqueued and
 *    rmsnorm_last_error() describes the reason (per calling thread).
 *  - RMSN_EINVAL: a null pointer, n < 1 or n > 2^24 ((float)n must be exact),
 *    rows < 1, a row stride < n, eps negative / NaN / infinite, a pointer not
 *    aligned to its element size (4 B binary32, 2 B bf16), or overlapping
 *    x / y ranges other than exact in-place use (y == x with equal strides),
 *    or w overlapping y. No HIP call is made before these checks pass.
 *  - In-place (y == x) is allowed: each row is read completely before any of
 *    its outputs is written.
 *  - bf16 values are passed as their 16-bit patterns (uint16_t).
 *  - Threads: every entry point may be called from several host threads at
 *    once; the error message is per thread and the options are process-wide.
 *    One graph handle must not be updated, launched or destroyed by two
 *    threads at the same time (the handle is not locked).
 */
#ifndef RMSNORM_H
#define RMSNORM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    RMSN_OK = 0,
    RMSN_EINVAL = 1,   /* invalid argument; nothing enqueued                        */
    RMSN_EHIP = 2,     /* a HIP runtime call failed; message names the call and code */
    RMSN_ECAPTURE = 3, /* graph capture failed; the handle replays eagerly instead   */
    RMSN_ENOMEM = 4    /* host or device allocation in graph creation failed         */
} rmsn_status;

typedef enum { RMSN_F32 = 0, RMSN_BF16 = 1 } rmsn_dtype;

#define RMSN_MAX_N (1 << 24)
#define RMSN_MAX_SEQUENCE 65536

/* One row of a sequence, stored in DEVICE memory (32 bytes, 8-byte aligned).
 * x, w, y: device pointers with the element type of the sequence; n: width.
 * Kernels read the descriptor when they run, so rewriting a table entry
 * between graph replays changes what the next replay normalises
 * (Lecture 08 "Graph-resident decode", section 2: values that vary per replay
 * live in device memory and are read by the kernel). n is used only as a loop
 * bound: any n in [1, 2^24] gives the exact result on replay, whatever width
 * the node was captured with (only speed depends on it); n outside that range
 * makes the node write nothing. Pointer alignment rules are as above. */
typedef struct rmsn_desc {
    const void* x;
    const void* w;
    void* y;
    int64_t n;
} rmsn_desc;

/* Opaque handle of a captured sequence (host memory owned by the library). */
typedef struct rmsn_graph rmsn_graph;

/* One binary32 row: y[0..n) from x[0..n) and w[0..n). Lecture 04 section 2. */
int rmsnorm_f32(const float* x, const float* w, float* y, int64_t n, float eps, void* stream);

/* One bf16 row (bit patterns); binary32 arithmetic, one rounding at the store.
 * The operation is Lecture 04 section 2's; the pages' kernel is binary32 only
 * (rms_norm_f32), so the bf16 storage format -- exact widening of x and w,
 * binary32 arithmetic, one round-to-nearest-even narrowing of y -- is taken
 * from this library's bf16 workloads (the 64 x 7168 and 8192 x 7168 batches),
 * not from the pages. */
int rmsnorm_bf16(const uint16_t* x, const uint16_t* w, uint16_t* y, int64_t n, float eps,
                 void* stream);

/* `rows` rows of width n sharing one weight row. Row r of x starts at
 * x + r * x_row_stride elements, row r of y at y + r * y_row_stride.
 * dtype is an rmsn_dtype. The layout is chosen per launch from measurements
 * on MI355X (Lecture 04 section 1: match the grid to the machine; see
 * rmsnorm_plan_query and the RMSN_PATH_* list): fewer than 1024 rows run one
 * 256-thread workgroup per row (GROUP); many rows of at least 4 KB whose x + y
 * stay under 64 MiB too, and a workgroup of several wavefronts per row with
 * 16-byte loads (SPLIT) from 64 MiB; rows under 1 KB run one wavefront per
 * row (WAVE); rows of 1-4 KB run WAVE under 32 MiB and SPLIT from there.
 * Rows that are not vector-aligned run BLOCK / STREAM. All give the same
 * bits. A dispatch counts its grid in work-items as a 32-bit number, so a
 * batch needing more than 2^32 - 1 threads (from about 4 million rows) is
 * issued as consecutive launches of the same layout on `stream`. */
int rmsnorm_batched_rows(int dtype, const void* x, int64_t x_row_stride, const void* w, void* y,
                         int64_t y_row_stride, int64_t rows, int64_t n, float eps, void* stream);

/* rmsnorm_batched_rows with a caller-provided device workspace, which lets
 * few wide rows (at most 64 rows of at least 64 KB) spread over many CUs:
 * RMSN_PATH_WIDE, two launches on `stream`, the group totals of the
 * association passing through the workspace (Lecture 04 section 1: match the
 * grid to the machine; section 2.1: the association, and so the bits, stay
 * those of every other path). Any other batch runs exactly as
 * rmsnorm_batched_rows and leaves the workspace untouched. workspace: DEVICE memory of at least the bytes
 * rmsnorm_workspace_query reports, 4-byte aligned, overlapping none of x, w,
 * y; its contents on entry do not matter and on return are unspecified. Calls
 * that may overlap in time need distinct workspaces. Errors as
 * rmsnorm_batched_rows, plus RMSN_EINVAL for a workspace the launch needs
 * that is NULL, too small, misaligned or overlapping the rows. */
int rmsnorm_batched_rows_ws(int dtype, const void* x, int64_t x_row_stride, const void* w,
                            void* y, int64_t y_row_stride, int64_t rows, int64_t n, float eps,
                            void* workspace, int64_t workspace_bytes, void* stream);

/* rmsnorm_batched_rows_ws for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same plan, kernels and bits, with the WIDE path's group
 * totals in a workspace the library holds instead of the caller's. That
 * workspace is a fixed 64 KB device array, one per GPU, kept until the
 * process ends; it holds the totals of at most 4096 rows, so a launch whose
 * plan would need more (only possible with RMSN_OPT_PATH forced to
 * RMSN_PATH_WIDE) is refused with RMSN_EINVAL before anything is enqueued.
 * Nothing is allocated, freed or synchronised; the first call on a device
 * looks up that device's copy of the array (hipGetSymbolAddress), so make
 * one call outside any capture first. Every call on a GPU shares that GPU's
 * array and leaves its last contents there: calls that may overlap in time
 * on one GPU (other streams, other host threads) race and must not be
 * issued. Errors as rmsnorm_batched_rows_ws, without the caller workspace's
 * checks. */
int rmsnorm_batched_rows_noalloc(int dtype, const void* x, int64_t x_row_stride, const void* w,
                                 void* y, int64_t y_row_stride, int64_t rows, int64_t n,
                                 float eps, void* stream);

/* The norms of a decode step, in order, issued as `count` dependent launches
 * on `stream` (the eager arm). d_table: DEVICE array of count descriptors.
 * h_widths: HOST array of count widths that size each launch (the same plan
 * function sizes graph nodes, so both arms launch the same kernels; the
 * graph's are a build with their arguments preloaded into SGPRs, these load
 * their own, which is faster for launches enqueued one by one while the HIP
 * runtime keeps their arguments in device memory (its default; with
 * HIP_FORCE_DEV_KERNARG=0 in the environment they take the preloaded build
 * too): same device code, same bits).
 * Lecture 08 "Graph-resident decode", section 1: the eager decode step pays
 * one host submission per kernel, the launch bill the graph removes; section
 * 4: the eager result is what every replay is compared against. Lecture 04
 * section 6: both arms live in one binary. */
int rmsnorm_sequence_eager(int dtype, const rmsn_desc* d_table, const int64_t* h_widths,
                           int32_t count, float eps, void* stream);

/* Capture the same `count` launches into one HIP graph and instantiate it
 * (Lecture 08 "Graph-resident decode", sections 1-3). Every kernel variant is
 * run once on a private scratch row before capture so that no lazy
 * initialisation happens inside it. On success *out is a new handle and
 * RMSN_OK is returned. If capture or instantiation fails, the partial graph is
 * destroyed, *out is still a valid handle in eager-fallback mode (launch then
 * issues the eager sequence: slower, same bits), and RMSN_ECAPTURE is
 * returned. d_table must stay valid until the handle is destroyed; h_widths
 * is copied. On RMSN_EINVAL / RMSN_ENOMEM / RMSN_EHIP, *out is NULL. */
int rmsnorm_sequence_graph_create(int dtype, const rmsn_desc* d_table, const int64_t* h_widths,
                                  int32_t count, float eps, rmsn_graph** out);

/* Replay the whole sequence with one graph launch on `stream` (Lecture 08
 * "Graph-resident decode", section 1: one submission replays every captured
 * node). On an eager-fallback handle (RMSN_ECAPTURE at creation) the same
 * launches are issued one by one instead (section 3: degrade, do not fail).
 * RMSN_EINVAL for a NULL handle; RMSN_EHIP if the launch fails. */
int rmsnorm_sequence_graph_launch(rmsn_graph* g, void* stream);

/* Release the graph and the handle. NULL is accepted. Does not synchronise:
 * the caller makes sure no launch of it is still pending. Lecture 08
 * "Graph-resident decode", sections 1-2: the executable graph is a per-process
 * object owned by whoever captured it; the device descriptor table it reads
 * stays the caller's. */
int rmsnorm_sequence_graph_destroy(rmsn_graph* g);

/* ---- positioned sequences: the step's state update inside the graph ------ */

/* A decode step is replayed once per token, and each token's rows differ.
 * Lecture 08 "Graph-resident decode", section 2: promote the varying value to
 * device memory, compute the address on the device, and run the state update
 * itself inside the captured region. A positioned sequence does exactly that:
 * its kernels read the device-resident position *d_pos when they run and take
 * entry i's rows at
 *     x_i + p * x_pitch,  y_i + p * y_pitch   (bytes),  p = (*d_pos) mod period,
 * (w_i does not move), and its last launch stores (p + 1) mod period in
 * *d_pos (so after the first step *d_pos stays in [0, period) and the kernels
 * need no division). Replaying it walks `period` rows per norm, one per
 * replay, with no host work between replays. */
typedef struct rmsn_position {
    int64_t* d_pos;   /* DEVICE int64, >= 0, 8-byte aligned, caller-owned; must
                         outlive the handle and hold no other data           */
    int64_t x_pitch;  /* bytes between consecutive positions' x rows, >= 0, a
                         multiple of the element size                         */
    int64_t y_pitch;  /* the same for y                                       */
    int64_t period;   /* positions before p wraps to 0, >= 1                  */
} rmsn_position;

/* The eager arm of a positioned sequence: count norm launches at the current
 * position, then the position update, all on `stream`. Arguments as for
 * rmsnorm_sequence_eager; RMSN_EINVAL also for a null position, d_pos null or
 * not 8-byte aligned, period < 1, negative or misaligned pitches, or
 * period * pitch overflowing. Lecture 08 "Graph-resident decode", section 2:
 * a value that changes from one step to the next (here the position) lives in
 * device memory and the sequence itself updates it. */
int rmsnorm_sequence_eager_positioned(int dtype, const rmsn_desc* d_table,
                                      const int64_t* h_widths, int32_t count, float eps,
                                      const rmsn_position* pos, void* stream);

/* Capture a positioned sequence: count norm nodes and a last node that moves
 * *d_pos to the next position (count + 1 nodes). Pre-warm runs every kernel variant, the
 * update included, on a private row and a private position: neither the
 * caller's rows nor *d_pos change before the first launch. Otherwise as
 * rmsnorm_sequence_graph_create (a capture failure leaves *d_pos untouched
 * and the handle replays eagerly, position update included). Lecture 08
 * "Graph-resident decode", section 2 (the state update captured inside the
 * graph, so replays differ with no host work) and section 3 (warm every
 * variant before capture; degrade to eager, do not fail). */
int rmsnorm_sequence_graph_create_positioned(int dtype, const rmsn_desc* d_table,
                                             const int64_t* h_widths, int32_t count, float eps,
                                             const rmsn_position* pos, rmsn_graph** out);

/* New capture-time widths for an existing handle (count must equal the
 * handle's). Widths are a capture key only through the launch plan
 * (Lecture 08 section 2: a value that decides the grid or the kernel cannot
 * be promoted to device memory; re-capture when the plan moves, with the
 * check and the launcher calling the same plan function). The sequence is
 * planned again with the function every launch uses; if each node's launch
 * (kernel instance, block, grid) is unchanged the executable graph is kept,
 * else the sequence is pre-warmed and captured again and the old graph is
 * released. *recaptured (may be NULL) is 1 if a new graph (or, on capture
 * failure, the eager fallback with the new plans: RMSN_ECAPTURE) replaced the
 * old one, else 0. On RMSN_EINVAL / RMSN_EHIP the handle is unchanged. Must not
 * overlap a pending launch of the handle. */
int rmsnorm_sequence_graph_update(rmsn_graph* g, const int64_t* h_widths, int32_t count,
                                  int* recaptured);

/* ---- the whole step in one launch ------------------------------------------- */

/* The sequence's count norms in ONE kernel launch that walks the descriptor
 * table (Lecture 08 "Graph-resident decode", further reading: a persistent
 * kernel as the endpoint of capturing many); the bits equal
 * rmsnorm_sequence_eager's. Rows that share no memory with any other row
 * (their reads and output meet no other row's output, their output no other
 * row's reads) cannot observe the order and run in parallel over up to 252
 * workgroups. The others ("bound") keep table order, so a table in which a
 * later x is an earlier y (y_i == x_j, i < j) computes exactly what the
 * launch sequence computes. They fall into components (rows that share
 * memory directly or through other bound rows); the first four workgroups
 * each take whole components, in table order within each:
 *  - when every row of a workgroup's components is at most 8192 elements, a
 *    multiple of 4, quad-aligned, and its rows share memory only at ranges
 *    a multiple of 1024 elements apart, the workgroup's four wavefronts share
 *    each row in a fixed mapping (every address is then read and written by
 *    one thread) and the next rows' loads are issued early; a row whose x is
 *    exactly the previous row's output takes it from registers;
 *  - else, when every such row is a whole number of 16-byte vectors,
 *    16-byte aligned and at most 8192 elements, the four wavefronts take one
 *    row each and a row starts only once every earlier row it shares memory
 *    with has finished (its stores complete), found among the 64 rows before
 *    it; these waits are bounded (RMSN_OPT_WALK_SPIN_CAP), and a wait that
 *    runs out is counted (rmsnorm_diag_walk_timeouts);
 *  - otherwise row after row, each row's stores ordered before the next
 *    row's loads by a workgroup barrier.
 * Tables of more than 1024 rows, and RMSN_OPT_PERSISTENT_WORKGROUPS = 1,
 * keep every row in one workgroup.
 * Widths come from the table (any n in [1, 2^24], any element alignment); no
 * host widths are needed. No row may write into the descriptor table itself.
 * pos: NULL, or the rows are taken at the position as in
 * rmsnorm_sequence_eager_positioned and the position is advanced after the
 * last row (when the rows are spread over workgroups, by a second, one-thread
 * launch on the same stream, so that every workgroup reads the same
 * position). Nothing is allocated or synchronised, so the call may itself be
 * captured into a caller's graph. RMSN_EINVAL: bad dtype, d_table null or not
 * 8-byte aligned, count outside [1, RMSN_MAX_SEQUENCE], bad eps or
 * position. */
int rmsnorm_sequence_persistent(int dtype, const rmsn_desc* d_table, int32_t count, float eps,
                                const rmsn_position* pos, void* stream);

/* Number of nodes in the captured graph (0 in eager-fallback mode): count,
 * plus one for a positioned sequence's update. Lecture 08 "Graph-resident
 * decode", section 1 reports its graph by node count (4,257 per rank); this
 * is the same figure for a captured norm sequence. RMSN_EINVAL for a NULL
 * handle or output. */
int rmsnorm_graph_node_count(const rmsn_graph* g, int64_t* out);

/* 1 if the handle replays eagerly because capture failed, else 0 (Lecture 08
 * "Graph-resident decode", section 3: a capture that fails falls back to
 * eager launches, and the fallback must be visible, not silent). */
int rmsnorm_graph_is_fallback(const rmsn_graph* g, int* out);

/* Human-readable reason for the last failure on this thread ("" if none).
 * Lecture 08 "Graph-resident decode", section 3: an error raised inside a
 * capture (or by a kernel) surfaces later and elsewhere, so each failing call
 * records which call and which HIP error it was, and the status code alone
 * never has to be decoded. The string is owned by the library and valid until
 * the thread's next call into it. */
const char* rmsnorm_last_error(void);

/* ---- launch planning (host only, no HIP call) ---------------------------- */

/* Code paths. All give identical bits; they differ in how rows are mapped to
 * the hardware (Lecture 04 section 2.1: the apply may be laid out freely once
 * the reduction's association is fixed).
 *   RMSN_PATH_WAVE:   one 64-lane wavefront per row, the row held in
 *                     registers, 16-byte (binary32) / 8-byte (bf16) loads;
 *                     needs vector-aligned rows and n <= 8192.
 *   RMSN_PATH_BLOCK:  one 256-thread workgroup per row, wavefront g holding
 *                     the 64 lane chains of group g in registers; any element
 *                     alignment, n <= 8192.
 *   RMSN_PATH_STREAM: one 256-thread workgroup per row that streams it twice:
 *                     wavefront g runs the 64 chains of group g with one
 *                     16-byte (binary32) / 8-byte (bf16) load per lane and
 *                     1024 elements when x is quad-aligned (element loads
 *                     otherwise), 16 such loads in flight behind the ones
 *                     being summed; then the whole workgroup applies the row.
 *                     Any alignment, any n up to 2^24.
 *   RMSN_PATH_SPLIT:  one workgroup of up to 16 wavefronts per row (Lecture 04
 *                     section 1.1: widen the block until the row's width is
 *                     the parallelism). The row is cut into 1 KB slices, one
 *                     16-byte load per lane; each wavefront holds `loads`
 *                     consecutive slices and continues the 256 lane chains
 *                     where the previous wavefront left them (handed over
 *                     through LDS), so the association is unchanged. Needs
 *                     16-byte aligned rows and w, n * element size a multiple
 *                     of 16, and rows of at most 128 KB.
 *   RMSN_PATH_GROUP:  BLOCK's chains-to-threads mapping, but wavefront g reads
 *                     its group's 64 elements of four consecutive 256-element
 *                     chunks with one 16-byte (binary32) / 8-byte (bf16) load
 *                     per lane and transposes them in registers: a quarter of
 *                     BLOCK's load instructions. Needs quad-aligned pointers
 *                     (16 B / 8 B), n a multiple of 4 and n <= 8192.
 *   RMSN_PATH_WIDE:   rmsnorm_batched_rows_ws only: the sum of each row split
 *                     over four one-wavefront workgroups, one per association
 *                     group (so four CUs per row; the association allows no
 *                     more lanes), writing the group totals to the caller's
 *                     workspace; then a second launch of ceil(n / 4096)
 *                     workgroups per row combines the totals in the
 *                     association's order and applies 4096 elements each.
 *                     Chosen for at most 64 rows of at least 64 KB.
 *   RMSN_PATH_REPLICA: one launch of `parts` GROUP workgroups per row (Lecture
 *                     04 section 1: fill the machine; section 2.1: only the
 *                     apply may be spread, the sum keeps its association).
 *                     Each workgroup reads the whole row's x and computes the
 *                     whole sum -- the same bits in every workgroup, no
 *                     exchange between them -- and applies and stores only
 *                     its share of the row's 1024-element blocks, loading w
 *                     for those blocks only. Same conditions as GROUP; parts
 *                     from RMSN_OPT_REPLICA_PARTS (at most the row's blocks).
 *                     In-place launches (y == x) never take it: a workgroup
 *                     still reading the row would see its siblings' stores. */
enum {
    RMSN_PATH_WAVE = 0,
    RMSN_PATH_BLOCK = 1,
    RMSN_PATH_STREAM = 2,
    RMSN_PATH_SPLIT = 3,
    RMSN_PATH_GROUP = 4,
    RMSN_PATH_WIDE = 5,
    RMSN_PATH_REPLICA = 6
};

typedef struct rmsn_plan_info {
    int32_t path;            /* one of RMSN_PATH_*                                */
    int32_t chunks;          /* 256-element chunks a lane's registers hold (0:
                                streaming); SPLIT: chunks one wavefront holds     */
    int32_t rows_per_block;  /* rows (wavefronts) per workgroup on WAVE, else 1   */
    int32_t block;           /* threads per workgroup                             */
    int64_t grid;            /* workgroups of the whole batch (beyond 2^32 - 1
                                threads it goes as several launches)              */
    int32_t streaming;       /* WAVE / SPLIT: 1 = non-temporal loads of x and
                                stores of y                                       */
    int32_t loads;           /* SPLIT: 16-byte loads per lane (1 KB slices per
                                wavefront); GROUP, REPLICA: loads per lane
                                (1024-element blocks); WIDE: apply workgroups per
                                row; else 0                                       */
    int32_t parts;           /* REPLICA: workgroups per row; else 1              */
} rmsn_plan_info;

/* The launch the library would use for `rows` rows of width n whose row starts
 * (x and y) and weight all share the byte alignment `align` (the largest power
 * of two dividing it counts, up to 16; 0 or anything below the element size
 * means element alignment only; -1 plans a descriptor row of a sequence,
 * whose pointers the kernel checks when it runs). Same function the launches
 * use (Lecture 08 "Graph-resident decode", section 2: the capture-time check
 * and the launcher call one plan function; Lecture 04 section 1: the grid and
 * block a launch gets). Returns RMSN_EINVAL for an invalid dtype, rows or n. */
int rmsnorm_plan_query(int dtype, int64_t rows, int64_t n, int align, rmsn_plan_info* out);

/* The plan rmsnorm_batched_rows_ws would use for `rows` rows of width n at
 * alignment `align` (as rmsnorm_plan_query), and in *bytes the workspace it
 * needs (16 bytes per row on RMSN_PATH_WIDE, else 0). plan may be NULL.
 * Lecture 04 section 1: a few rows on a chip of 256 CUs leave most of it idle
 * unless a row is split over several of them. */
int rmsnorm_workspace_query(int dtype, int64_t rows, int64_t n, int align, rmsn_plan_info* plan,
                            int64_t* bytes);

/* Process-wide overrides, for proving that code paths give identical bits
 * (Lecture 04 section 6: one binary, switchable arms). Defaults come from the
 * environment at first use, else automatic.
 *   RMSN_OPT_PATH:           -1 automatic, or an RMSN_PATH_* value; a path a
 *                            launch is not eligible for (WAVE on unaligned
 *                            rows or n > 8192, BLOCK with n > 8192, SPLIT or
 *                            GROUP outside their conditions above) falls back
 *                            to the automatic choice
 *   RMSN_OPT_ROWS_PER_BLOCK:  0 automatic, else 4 or 8 rows (wavefronts) per
 *                            workgroup sharing one LDS copy of w (WAVE path)
 *   RMSN_OPT_STREAMING:      -1 automatic (on when x + y of the launch reach
 *                            64 MiB), 0 off, 1 on: non-temporal loads of x and
 *                            stores of y (WAVE and SPLIT paths)
 *   RMSN_OPT_SPLIT_LOADS:     0 automatic, else 1, 2, 4 or 8 slices per
 *                            wavefront (SPLIT path; a value that would need
 *                            more than 16 wavefronts falls back to automatic)
 *   RMSN_OPT_APPLY_THREADS:   128-lane build only (RMSN_EINVAL in the default
 *                            build): threads per row for the elementwise
 *                            apply, 0 (= 1024), 128, 256, 512 or 1024; the sum
 *                            always runs on the first 128
 *   RMSN_OPT_PERSISTENT_WORKGROUPS: rmsnorm_sequence_persistent, 0 automatic
 *                            (rows that share no memory with any other row
 *                            spread over many workgroups), 1 one workgroup
 *                            walking the whole table (the 128-lane build
 *                            always uses one)
 *   RMSN_OPT_REPLICA_PARTS:   RMSN_PATH_REPLICA, 0 automatic (4), else 1..8
 *                            workgroups per row (capped at the row's
 *                            1024-element blocks)
 *   RMSN_OPT_WALK_SPIN_CAP:   rmsnorm_sequence_persistent, 0 default (2^22),
 *                            else 1..2^30: polls one wait of the ordered walk
 *                            may take before it gives up ordering the rest of
 *                            the launch and counts a timeout (see
 *                            rmsnorm_diag_walk_timeouts). A wait can always
 *                            end, so the default is never reached; a cap of
 *                            1 forces timeouts, for testing that path.
 * Returns RMSN_EINVAL for an unknown key or value. Not synchronised with
 * launches on other threads. Environment: RMSN_PATH, RMSN_ROWS_PER_BLOCK,
 * RMSN_STREAMING, RMSN_SPLIT_LOADS, RMSN_APPLY_THREADS,
 * RMSN_PERSISTENT_WORKGROUPS, RMSN_REPLICA_PARTS, RMSN_WALK_SPIN_CAP. */
enum {
    RMSN_OPT_PATH = 1,
    RMSN_OPT_ROWS_PER_BLOCK = 2,
    RMSN_OPT_STREAMING = 3,
    RMSN_OPT_SPLIT_LOADS = 4,
    RMSN_OPT_APPLY_THREADS = 5,
    RMSN_OPT_PERSISTENT_WORKGROUPS = 6,
    RMSN_OPT_REPLICA_PARTS = 7,
    RMSN_OPT_WALK_SPIN_CAP = 8
};
int rmsnorm_set_option(int key, int value);
int rmsnorm_get_option(int key, int* value);

/* ---- the association a build computes ---------------------------------------- */

/* Lane chains of the association this library computes: 256 (R256, every
 * statement above) for the default build librmsnorm_amd.so; 128 for the
 * reference-compatibility build librmsnorm_amd_l128.so, which sums the row on
 * 128 threads as Lecture 04 section 2.1's kernel does -- 128 lane chains
 * (stride 128), four 32-lane groups each reduced by descending halving
 * 16..1, combine (G0 + G2) + (G1 + G3), steps 4-8 unchanged -- and applies it
 * on the whole block (RMSN_OPT_APPLY_THREADS). That build has the same entry
 * points; every launch runs one workgroup per row (plan path RMSN_PATH_BLOCK,
 * chunks 0, block = the apply width) and RMSN_OPT_PATH, RMSN_OPT_ROWS_PER_BLOCK,
 * RMSN_OPT_STREAMING and RMSN_OPT_SPLIT_LOADS do not change its launches. The
 * two builds give different bits (the lane count is part of the numerics);
 * the apply width of the 128-lane build does not. */
int rmsnorm_association_lanes(void);

/* ---- diagnostics ----------------------------------------------------------- */

/* Runs the kernels' own steps 4-7 (the device functions every row kernel
 * calls) on count consecutive binary32 bit patterns starting at first_bits,
 * taken as ss, with the given n and eps: r_out[i] = sqrtf(ss/(float)n + eps),
 * inv_out[i] = 1.0f / r_out[i]. Device output arrays of count floats. Used to
 * check the device square root and division against a CPU exhaustively: the
 * epilogue of Lecture 04 section 2.1 (mean, eps, root, inverse), computed here
 * with a correctly rounded root and a correctly rounded division. */
int rmsnorm_diag_inverse(uint32_t first_bits, int64_t count, int64_t n, float eps, float* r_out,
                         float* inv_out, void* stream);

/* Runs the kernels' own binary32 -> bf16 narrowing of step 8 (the device
 * function every bf16 store calls) on count consecutive bit patterns starting
 * at first_bits: out[i] = bf16(pattern first_bits + i), a DEVICE array of count
 * uint16. Used to check the hardware conversion against a CPU for every
 * binary32 pattern. RMSN_EINVAL if the range leaves 32 bits or out is null or
 * odd. The bf16 output format is this library's (see rmsnorm_bf16), not the
 * pages'. */
int rmsnorm_diag_bf16(uint32_t first_bits, int64_t count, uint16_t* out, void* stream);

/* A plain streaming copy of `bytes` bytes from src to dst (DEVICE memory, not
 * overlapping, both 16-byte aligned, bytes a positive multiple of 16) on
 * `stream`: each lane loads and stores `vectors` 16-byte vectors (1, 2 or 4)
 * with non-temporal hints, in workgroups of `block` threads (a multiple of
 * 64, at most 1024), workgroup b taking the next vectors * block vectors.
 * It moves the same bytes as a norm of rows of that size and does nothing
 * else, so its time bounds what a row kernel's access pattern can reach on
 * this memory system (Lecture 04 section 3.1: compare the measured time with
 * the floor the bytes set). RMSN_EINVAL for a null, misaligned or
 * overlapping pointer, a bad size, vector count or block. */
int rmsnorm_diag_copy(const void* src, void* dst, int64_t bytes, int vectors, int block,
                      void* stream);

/* Waits of rmsnorm_sequence_persistent's ordered walk that ran out of polls
 * (RMSN_OPT_WALK_SPIN_CAP) on the current device since the last reset: *out
 * (host). A launch in which a wait timed out stops ordering its rows, so its
 * outputs are not to be trusted; the count is the device-side error flag of
 * that walk (Lecture 08 "Graph-resident decode", section 3: an error raised
 * inside the step surfaces later, so it must be recorded where it happened).
 * reset != 0 sets the counter to 0 after reading it. Synchronous (device to
 * host copy): call it between launches, not inside a capture. RMSN_EINVAL for
 * a null out. */
int rmsnorm_diag_walk_timeouts(uint32_t* out, int reset);

#ifdef __cplusplus
}
#endif
#endif /* RMSNORM_H */
