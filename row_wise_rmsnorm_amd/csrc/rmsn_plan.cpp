// rmsn_plan.cpp -- launch planning, options and argument validation.
// Pure host C++: nothing here touches the HIP runtime, so every check can run
// (and is tested) on a machine without a GPU.
#include "rmsn_plan.h"

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>

namespace rmsn {

namespace {

thread_local char g_err[512] = "";

std::atomic<int> g_path{-2};   // -2 = not yet read from the environment
std::atomic<int> g_rpb{-2};
std::atomic<int> g_stream{-2};
std::atomic<int> g_split{-2};
std::atomic<int> g_apply{-2};
std::atomic<int> g_pwg{-2};
std::atomic<int> g_parts{-2};
std::atomic<int> g_spin{-1};

int env_int(const char* name, int dflt) {
    const char* s = std::getenv(name);
    if (!s || !*s) return dflt;
    char* end = nullptr;
    long v = std::strtol(s, &end, 10);
    if (end == s) return dflt;
    return (int)v;
}

bool valid_path(int v) {
    return v == -1 || v == RMSN_PATH_WAVE || v == RMSN_PATH_BLOCK || v == RMSN_PATH_STREAM ||
           v == RMSN_PATH_SPLIT || v == RMSN_PATH_GROUP || v == RMSN_PATH_WIDE ||
           v == RMSN_PATH_REPLICA;
}
bool valid_split_loads(int v) { return v == 0 || v == 1 || v == 2 || v == 4 || v == 8; }
bool valid_apply_threads(int v) { return v == 0 || v == 128 || v == 256 || v == 512 || v == 1024; }
bool valid_rpb(int v) { return v == 0 || v == 4 || v == 8; }
bool valid_streaming(int v) { return v == -1 || v == 0 || v == 1; }
bool valid_persistent_wg(int v) { return v == 0 || v == 1; }
bool valid_parts(int v) { return v >= 0 && v <= 8; }
bool valid_spin_cap(int v) { return v >= 0 && v <= (1 << 30); }

// Byte ranges [a, a+la) and [b, b+lb) intersect.
bool overlaps(uintptr_t a, uint64_t la, uintptr_t b, uint64_t lb) {
    return a < b + lb && b < a + la;
}

}  // namespace

void set_error(const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
}

void clear_error() { g_err[0] = '\0'; }
const char* last_error() { return g_err; }

int option_path() {
    int v = g_path.load(std::memory_order_relaxed);
    if (v == -2) {
        v = env_int("RMSN_PATH", -1);
        if (!valid_path(v)) v = -1;
        g_path.store(v, std::memory_order_relaxed);
    }
    return v;
}

int option_rows_per_block() {
    int v = g_rpb.load(std::memory_order_relaxed);
    if (v == -2) {
        v = env_int("RMSN_ROWS_PER_BLOCK", 0);
        if (!valid_rpb(v)) v = 0;
        g_rpb.store(v, std::memory_order_relaxed);
    }
    return v;
}

int option_streaming() {
    int v = g_stream.load(std::memory_order_relaxed);
    if (v == -2) {
        v = env_int("RMSN_STREAMING", -1);
        if (!valid_streaming(v)) v = -1;
        g_stream.store(v, std::memory_order_relaxed);
    }
    return v;
}

int option_split_loads() {
    int v = g_split.load(std::memory_order_relaxed);
    if (v == -2) {
        v = env_int("RMSN_SPLIT_LOADS", 0);
        if (!valid_split_loads(v)) v = 0;
        g_split.store(v, std::memory_order_relaxed);
    }
    return v;
}

int option_apply_threads() {
    int v = g_apply.load(std::memory_order_relaxed);
    if (v == -2) {
        v = env_int("RMSN_APPLY_THREADS", 0);
        if (!valid_apply_threads(v)) v = 0;
        g_apply.store(v, std::memory_order_relaxed);
    }
    return v;
}

int option_persistent_workgroups() {
    int v = g_pwg.load(std::memory_order_relaxed);
    if (v == -2) {
        v = env_int("RMSN_PERSISTENT_WORKGROUPS", 0);
        if (!valid_persistent_wg(v)) v = 0;
        g_pwg.store(v, std::memory_order_relaxed);
    }
    return v;
}

int option_replica_parts() {
    int v = g_parts.load(std::memory_order_relaxed);
    if (v == -2) {
        v = env_int("RMSN_REPLICA_PARTS", 0);
        if (!valid_parts(v)) v = 0;
        g_parts.store(v, std::memory_order_relaxed);
    }
    return v;
}

int option_walk_spin_cap() {
    int v = g_spin.load(std::memory_order_relaxed);
    if (v == -1) {
        v = env_int("RMSN_WALK_SPIN_CAP", 0);
        if (!valid_spin_cap(v)) v = 0;
        g_spin.store(v, std::memory_order_relaxed);
    }
    return v;
}

int set_option(int key, int value) {
    if (key == RMSN_OPT_PATH) {
        if (!valid_path(value)) {
            set_error("rmsnorm_set_option: path must be -1 (automatic) or 0..6, got %d", value);
            return RMSN_EINVAL;
        }
        g_path.store(value, std::memory_order_relaxed);
        return RMSN_OK;
    }
    if (key == RMSN_OPT_ROWS_PER_BLOCK) {
        if (!valid_rpb(value)) {
            set_error("rmsnorm_set_option: rows per block must be 0, 4 or 8, got %d", value);
            return RMSN_EINVAL;
        }
        g_rpb.store(value, std::memory_order_relaxed);
        return RMSN_OK;
    }
    if (key == RMSN_OPT_STREAMING) {
        if (!valid_streaming(value)) {
            set_error("rmsnorm_set_option: streaming must be -1, 0 or 1, got %d", value);
            return RMSN_EINVAL;
        }
        g_stream.store(value, std::memory_order_relaxed);
        return RMSN_OK;
    }
    if (key == RMSN_OPT_SPLIT_LOADS) {
        if (!valid_split_loads(value)) {
            set_error("rmsnorm_set_option: split loads must be 0, 1, 2, 4 or 8, got %d", value);
            return RMSN_EINVAL;
        }
        g_split.store(value, std::memory_order_relaxed);
        return RMSN_OK;
    }
    if (key == RMSN_OPT_APPLY_THREADS) {
        if (kAssocLanes != 128) {
            set_error("rmsnorm_set_option: the apply width is an option of the 128-lane build "
                      "only (this library computes %d lanes)", kAssocLanes);
            return RMSN_EINVAL;
        }
        if (!valid_apply_threads(value)) {
            set_error("rmsnorm_set_option: apply threads must be 0, 128, 256, 512 or 1024, got %d",
                      value);
            return RMSN_EINVAL;
        }
        g_apply.store(value, std::memory_order_relaxed);
        return RMSN_OK;
    }
    if (key == RMSN_OPT_PERSISTENT_WORKGROUPS) {
        if (!valid_persistent_wg(value)) {
            set_error("rmsnorm_set_option: persistent workgroups must be 0 (automatic) or 1, got %d",
                      value);
            return RMSN_EINVAL;
        }
        g_pwg.store(value, std::memory_order_relaxed);
        return RMSN_OK;
    }
    if (key == RMSN_OPT_REPLICA_PARTS) {
        if (!valid_parts(value)) {
            set_error("rmsnorm_set_option: replica parts must be 0 (automatic) or 1..8, got %d",
                      value);
            return RMSN_EINVAL;
        }
        g_parts.store(value, std::memory_order_relaxed);
        return RMSN_OK;
    }
    if (key == RMSN_OPT_WALK_SPIN_CAP) {
        if (!valid_spin_cap(value)) {
            set_error("rmsnorm_set_option: walk spin cap must be 0 (default) or 1..2^30, got %d",
                      value);
            return RMSN_EINVAL;
        }
        g_spin.store(value, std::memory_order_relaxed);
        return RMSN_OK;
    }
    set_error("rmsnorm_set_option: unknown key %d", key);
    return RMSN_EINVAL;
}

int get_option(int key, int* value) {
    if (!value) {
        set_error("rmsnorm_get_option: null output pointer");
        return RMSN_EINVAL;
    }
    if (key == RMSN_OPT_PATH) { *value = option_path(); return RMSN_OK; }
    if (key == RMSN_OPT_ROWS_PER_BLOCK) { *value = option_rows_per_block(); return RMSN_OK; }
    if (key == RMSN_OPT_STREAMING) { *value = option_streaming(); return RMSN_OK; }
    if (key == RMSN_OPT_SPLIT_LOADS) { *value = option_split_loads(); return RMSN_OK; }
    if (key == RMSN_OPT_APPLY_THREADS) {
        *value = kAssocLanes == 128 ? option_apply_threads() : 0;
        return RMSN_OK;
    }
    if (key == RMSN_OPT_PERSISTENT_WORKGROUPS) { *value = option_persistent_workgroups(); return RMSN_OK; }
    if (key == RMSN_OPT_REPLICA_PARTS) { *value = option_replica_parts(); return RMSN_OK; }
    if (key == RMSN_OPT_WALK_SPIN_CAP) { *value = option_walk_spin_cap(); return RMSN_OK; }
    set_error("rmsnorm_get_option: unknown key %d", key);
    return RMSN_EINVAL;
}

int chunk_bucket(int64_t n) {
    const int64_t need = (n + kLanes - 1) / kLanes;
    for (int i = 0; i < kNumBuckets; ++i)
        if (kChunkBuckets[i] >= need) return kChunkBuckets[i];
    return 0;
}

int auto_rows_per_block(int64_t rows) {
    // The workgroup's wavefronts share one LDS copy of the weight row: eight
    // for large batches, four while eight would leave CUs without a
    // workgroup (fewer than 256 * 8 rows).
    return rows >= 8 * 256 ? 8 : 4;
}

// x + y bytes of a launch reach `bytes` (no overflow for any valid rows, n).
static bool footprint_at_least(int dtype, int64_t rows, int64_t n, int64_t bytes) {
    const int64_t per_row = n * 2 * elem_bytes(dtype);  // n <= 2^24: no overflow
    return rows >= (bytes + per_row - 1) / per_row;
}

bool auto_streaming(int dtype, int64_t rows, int64_t n) {
    return footprint_at_least(dtype, rows, n, kStreamBytes);
}

int auto_split_loads(int64_t slices) {
    // Measured on MI355X (rows of 256..8192 elements, 240 MB launches): one
    // slice per wavefront for a one-slice row, two for rows of 2..15 slices,
    // four from 16 slices on (fewer chain hand-offs once a row would need
    // more than 8 wavefronts); eight only where four would exceed 16.
    int u = slices <= 1 ? 1 : slices < 16 ? 2 : 4;
    while ((slices + u - 1) / u > kMaxSplitWaves && u < 8) u *= 2;
    return (slices + u - 1) / u <= kMaxSplitWaves ? u : 0;
}

int make_plan(int dtype, int64_t rows, int64_t n, int align, Plan* out, bool workspace,
              bool in_place) {
    if (dtype != RMSN_F32 && dtype != RMSN_BF16) {
        set_error("unknown dtype %d", dtype);
        return RMSN_EINVAL;
    }
    if (rows < 1) {
        set_error("rows must be >= 1, got %lld", (long long)rows);
        return RMSN_EINVAL;
    }
    if (n < 1 || n > RMSN_MAX_N) {
        set_error("n must be in [1, %d], got %lld", RMSN_MAX_N, (long long)n);
        return RMSN_EINVAL;
    }
    if (kAssocLanes == 128) {
        // The 128-lane build: one workgroup per row, 128 threads sum and the
        // whole block (the apply width) applies; any n, any alignment.
        const int b = option_apply_threads();
        Plan p{};
        p.dtype = dtype;
        p.parts = 1;
        p.path = RMSN_PATH_BLOCK;
        p.chunks = 0;
        p.rows_per_block = 1;
        p.streaming = 0;
        p.block = b == 0 ? 1024 : b;
        p.grid = rows;
        p.loads = 0;
        *out = p;
        return RMSN_OK;
    }
    // the power of two (at most 16) that `align` guarantees
    const bool run_time = align == kAlignAtRunTime;
    int a = 16;
    while (a > 1 && (align <= 0 || align % a)) a >>= 1;
    const int es = elem_bytes(dtype);
    const int bucket = chunk_bucket(n);
    const int64_t slices = split_slices(dtype, n);
    const int split_auto = auto_split_loads(slices);
    const bool can_split = a >= 16 && (n * es) % 16 == 0 && split_auto != 0;
    const bool can_wave = bucket != 0 && a >= vec_bytes(dtype);
    const bool can_block = bucket != 0;
    const bool can_group = bucket != 0 && n % 4 == 0 && (run_time || a >= vec_bytes(dtype));
    const bool can_wide = workspace && !run_time;
    int path;
    switch (option_path()) {
        case RMSN_PATH_WAVE: path = can_wave ? RMSN_PATH_WAVE : -1; break;
        case RMSN_PATH_BLOCK: path = can_block ? RMSN_PATH_BLOCK : -1; break;
        case RMSN_PATH_STREAM: path = RMSN_PATH_STREAM; break;
        case RMSN_PATH_SPLIT: path = can_split ? RMSN_PATH_SPLIT : -1; break;
        case RMSN_PATH_GROUP: path = can_group ? RMSN_PATH_GROUP : -1; break;
        case RMSN_PATH_WIDE: path = can_wide ? RMSN_PATH_WIDE : -1; break;
        case RMSN_PATH_REPLICA:
            path = can_group && !run_time && !in_place ? RMSN_PATH_REPLICA : -1;
            break;
        default: path = -1; break;
    }
    if (path < 0) {
        // Measured on MI355X (graph-captured launches, widths 256..8192, 16 to
        // 252 MB, 64 to 245,760 rows): few rows are latency-bound and take
        // GROUP; many rows of at least 4 KB take GROUP while x + y stay under
        // 64 MiB and SPLIT beyond; rows under 1 KB take WAVE; rows of 1-4 KB
        // take WAVE under 32 MiB and SPLIT from there. Descriptor rows keep
        // BLOCK: the GROUP descriptor kernel, which also carries the
        // streaming fallback, measured slower in the decode step.
        const bool many = rows >= kWaveMinRows;
        const bool big = footprint_at_least(dtype, rows, n, kStreamBytes);
        const bool mid = footprint_at_least(dtype, rows, n, kStreamBytes / 2);
        const int64_t row_bytes = n * es;
        if (run_time) path = can_block ? RMSN_PATH_BLOCK : RMSN_PATH_STREAM;
        else if (can_wide && n * es >= kWideMinBytes && rows <= kWideMaxRows)
            path = RMSN_PATH_WIDE;
        else if (!many && can_group) path = RMSN_PATH_GROUP;
        else if (many && !big && row_bytes >= 4096 && can_group) path = RMSN_PATH_GROUP;
        else if (many && row_bytes < 1024 && can_wave) path = RMSN_PATH_WAVE;
        else if (many && row_bytes < 4096 && !mid && can_wave) path = RMSN_PATH_WAVE;
        else if (many && can_split) path = RMSN_PATH_SPLIT;
        else if (many && can_wave) path = RMSN_PATH_WAVE;
        else if (can_group) path = RMSN_PATH_GROUP;
        else if (can_block) path = RMSN_PATH_BLOCK;
        else if (can_split) path = RMSN_PATH_SPLIT;
        else path = RMSN_PATH_STREAM;
    }
    Plan p{};
    p.dtype = dtype;
    p.path = path;
    p.parts = 1;
    const int st = option_streaming();
    if (path == RMSN_PATH_WAVE) {
        int rpb = option_rows_per_block();
        if (rpb == 0) rpb = auto_rows_per_block(rows);
        p.chunks = bucket;
        p.rows_per_block = rpb;
        p.streaming = st < 0 ? (auto_streaming(dtype, rows, n) ? 1 : 0) : st;
        p.block = kWave * rpb;
        p.grid = (rows + rpb - 1) / rpb;
    } else if (path == RMSN_PATH_SPLIT) {
        int u = option_split_loads();
        if (u == 0 || (slices + u - 1) / u > kMaxSplitWaves) u = split_auto;
        p.loads = u;
        p.chunks = u * (kSliceBytes / (kLanes * es));
        p.rows_per_block = 1;
        p.streaming = st < 0 ? (auto_streaming(dtype, rows, n) ? 1 : 0) : st;
        p.block = kWave * (int)((slices + u - 1) / u);
        p.grid = rows;
    } else if (path == RMSN_PATH_WIDE) {
        // four one-wavefront workgroups per row (one per group), then
        // ceil(n / kWideSpan) workgroups of 256 per row for the apply
        p.loads = (int)((n + kWideSpan - 1) / kWideSpan);
        p.chunks = 0;
        p.rows_per_block = 1;
        p.streaming = 0;
        p.block = kWave;
        p.grid = 4 * rows;
    } else if (path == RMSN_PATH_GROUP) {
        p.loads = (int)((n + 1023) / 1024);
        p.chunks = 4 * p.loads;
        p.rows_per_block = 1;
        p.streaming = 0;
        p.block = kBlockThreads;
        p.grid = rows;
    } else if (path == RMSN_PATH_REPLICA) {
        // GROUP over the whole row in each of `parts` workgroups per row, each
        // applying a share of the row's blocks
        p.loads = (int)((n + 1023) / 1024);
        p.chunks = 4 * p.loads;
        p.rows_per_block = 1;
        p.streaming = 0;
        p.block = kBlockThreads;
        const int want = option_replica_parts() ? option_replica_parts() : kReplicaParts;
        p.parts = want < p.loads ? want : p.loads;
        p.grid = rows * p.parts;
    } else {
        p.chunks = path == RMSN_PATH_BLOCK ? bucket : 0;
        p.rows_per_block = 1;
        p.streaming = 0;
        p.block = kBlockThreads;
        p.grid = rows;
    }
    *out = p;
    return RMSN_OK;
}

int check_eps(float eps) {
    if (!std::isfinite(eps) || eps < 0.0f) {
        set_error("eps must be finite and >= 0, got %g", (double)eps);
        return RMSN_EINVAL;
    }
    return RMSN_OK;
}

int check_row_args(int dtype, const void* x, int64_t xs, const void* w, const void* y, int64_t ys,
                   int64_t rows, int64_t n) {
    if (dtype != RMSN_F32 && dtype != RMSN_BF16) {
        set_error("unknown dtype %d", dtype);
        return RMSN_EINVAL;
    }
    if (!x || !w || !y) {
        set_error("null pointer (x=%p w=%p y=%p)", x, w, y);
        return RMSN_EINVAL;
    }
    if (n < 1 || n > RMSN_MAX_N) {
        set_error("n must be in [1, %d], got %lld", RMSN_MAX_N, (long long)n);
        return RMSN_EINVAL;
    }
    if (rows < 1) {
        set_error("rows must be >= 1, got %lld", (long long)rows);
        return RMSN_EINVAL;
    }
    if (xs < n || ys < n) {
        set_error("row strides must be >= n (x stride %lld, y stride %lld, n %lld)",
                  (long long)xs, (long long)ys, (long long)n);
        return RMSN_EINVAL;
    }
    const int64_t es = elem_bytes(dtype);
    const int64_t lim = INT64_MAX / 4;
    if ((rows - 1) > (lim - n) / xs || (rows - 1) > (lim - n) / ys) {
        set_error("rows * stride overflows");
        return RMSN_EINVAL;
    }
    const uintptr_t px = (uintptr_t)x, pw = (uintptr_t)w, py = (uintptr_t)y;
    if ((px | pw | py) % (uintptr_t)es) {
        set_error("pointers must be aligned to the %lld-byte element size (x=%p w=%p y=%p)",
                  (long long)es, x, w, y);
        return RMSN_EINVAL;
    }
    const uint64_t lx = (uint64_t)(((rows - 1) * xs + n) * es);
    const uint64_t ly = (uint64_t)(((rows - 1) * ys + n) * es);
    const uint64_t lw = (uint64_t)(n * es);
    const bool in_place = px == py && xs == ys;
    if (!in_place && overlaps(px, lx, py, ly)) {
        set_error("x and y overlap without being the same rows (in-place needs y == x and equal strides)");
        return RMSN_EINVAL;
    }
    if (overlaps(pw, lw, py, ly)) {
        set_error("w overlaps y");
        return RMSN_EINVAL;
    }
    return RMSN_OK;
}

}  // namespace rmsn

namespace rmsn {

int check_sequence_args(int dtype, const rmsn_desc* d_table, const int64_t* h_widths,
                        int32_t count, float eps) {
    if (dtype != RMSN_F32 && dtype != RMSN_BF16) {
        set_error("unknown dtype %d", dtype);
        return RMSN_EINVAL;
    }
    if (!d_table || !h_widths) {
        set_error("null pointer (d_table=%p h_widths=%p)", (const void*)d_table,
                  (const void*)h_widths);
        return RMSN_EINVAL;
    }
    if ((uintptr_t)d_table % alignof(rmsn_desc)) {
        set_error("d_table must be %d-byte aligned", (int)alignof(rmsn_desc));
        return RMSN_EINVAL;
    }
    if (count < 1 || count > RMSN_MAX_SEQUENCE) {
        set_error("count must be in [1, %d], got %d", RMSN_MAX_SEQUENCE, (int)count);
        return RMSN_EINVAL;
    }
    for (int32_t i = 0; i < count; ++i) {
        if (h_widths[i] < 1 || h_widths[i] > RMSN_MAX_N) {
            set_error("width %d must be in [1, %d], got %lld", (int)i, RMSN_MAX_N,
                      (long long)h_widths[i]);
            return RMSN_EINVAL;
        }
    }
    return check_eps(eps);
}

int check_workspace(int dtype, const void* x, int64_t xs, const void* w, const void* y,
                    int64_t ys, int64_t rows, int64_t n, const void* ws, int64_t ws_bytes) {
    const int64_t need = rows * 4 * (int64_t)sizeof(float);
    if (!ws || (uintptr_t)ws % 4) {
        set_error("the launch needs a non-null, 4-byte aligned workspace (ws=%p)", ws);
        return RMSN_EINVAL;
    }
    if (ws_bytes < need) {
        set_error("workspace of %lld bytes, the launch needs %lld", (long long)ws_bytes,
                  (long long)need);
        return RMSN_EINVAL;
    }
    const int64_t es = elem_bytes(dtype);
    const uintptr_t pw = (uintptr_t)ws;
    if (overlaps(pw, (uint64_t)need, (uintptr_t)x, (uint64_t)(((rows - 1) * xs + n) * es)) ||
        overlaps(pw, (uint64_t)need, (uintptr_t)w, (uint64_t)(n * es)) ||
        overlaps(pw, (uint64_t)need, (uintptr_t)y, (uint64_t)(((rows - 1) * ys + n) * es))) {
        set_error("the workspace overlaps x, w or y");
        return RMSN_EINVAL;
    }
    return RMSN_OK;
}

}  // namespace rmsn
