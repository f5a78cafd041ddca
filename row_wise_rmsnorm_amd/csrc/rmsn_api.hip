// rmsn_api.hip -- the C ABI (include/rmsnorm.h): validation, planning,
// launches, and the captured decode-step sequence.
//
// Graph discipline follows Lecture 08 "Graph-resident decode": the values that
// change per replay (row pointers, widths) live in a device descriptor table
// the kernels read when they run (section 2); launch geometry is a capture key
// decided by the same plan function the eager path uses (section 2); every
// kernel variant runs once before capture so nothing initialises lazily inside
// it, and a failed capture degrades to eager replay instead of failing
// (section 3). A positioned sequence also carries its state update: a
// device-resident position the kernels read, advanced by the sequence's last
// launch, so the captured graph walks rows on its own (section 2); widths that
// change the launch plan are a capture key and trigger a re-capture through
// the same plan function (section 2).
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <vector>

#include "rmsn_launch.h"
#include "rmsn_plan.h"
#include "rmsnorm.h"

using namespace rmsn;

// The library's own workspace (rmsnorm_batched_rows_noalloc): the group
// totals of up to 4096 rows on the WIDE path, one copy per GPU.
constexpr int64_t kScratchBytes = 64 * 1024;
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

struct rmsn_graph {
    int dtype = RMSN_F32;
    float eps = 0.0f;
    const rmsn_desc* table = nullptr;
    std::vector<Plan> plans;
    bool positioned = false;
    PosArgs pos{nullptr, 0, 0, 1};
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
    int64_t nodes = 0;
    bool fallback = false;
};

namespace {

int hip_fail(const char* what, hipError_t e) {
    set_error("%s failed: %s (%d)", what, hipGetErrorString(e), (int)e);
    return RMSN_EHIP;
}

// The byte alignment (a power of two, at most 16) shared by every row start of
// x and y and by w.
int rows_alignment(int dtype, const void* x, int64_t xs, const void* w, const void* y,
                   int64_t ys) {
    const uint64_t es = (uint64_t)elem_bytes(dtype);
    const uint64_t bits = (uint64_t)(uintptr_t)x | (uint64_t)(uintptr_t)w |
                          (uint64_t)(uintptr_t)y | ((uint64_t)xs * es) | ((uint64_t)ys * es) | 16u;
    return (int)(bits & (~bits + 1));  // lowest set bit
}

// ---------------------------------------------------------------------------
// The library's own workspace, `scratch` above: every device that loads the
// library holds its own copy until the process ends. Host code never passes
// `scratch` itself to a kernel -- on the host that name is a stand-in, not a
// device address -- but the address hipGetSymbolAddress returns for the
// current device, looked up once per device on its first call.
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// The current device's copy of `scratch` (*out), looked up on its first use.
int scratch_address(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail("hipGetDevice", e);
    if (dev < 0 || dev >= kMaxDevices) {
        set_error("device %d is beyond the %d devices the library keeps a workspace for", dev,
                  kMaxDevices);
        return RMSN_EHIP;
    }
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return hip_fail("hipGetSymbolAddress (library workspace)", e);
            if (!p) {
                set_error("hipGetSymbolAddress returned a null library workspace");
                return RMSN_EHIP;
            }
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return RMSN_OK;
}

// Where a WIDE launch's group totals go: the caller's workspace
// (rmsnorm_batched_rows_ws), the library's own (rmsnorm_batched_rows_noalloc),
// or none (rmsnorm_batched_rows: the plan never takes WIDE).
enum class Ws { kNone, kCaller, kLibrary };

int run_rows(int dtype, const void* x, int64_t xs, const void* w, void* y, int64_t ys,
             int64_t rows, int64_t n, float eps, Ws ws_kind, void* ws, int64_t ws_bytes,
             void* stream) {
    clear_error();
    int st = check_row_args(dtype, x, xs, w, y, ys, rows, n);
    if (st != RMSN_OK) return st;
    if ((st = check_eps(eps)) != RMSN_OK) return st;
    Plan p;
    st = make_plan(dtype, rows, n, rows_alignment(dtype, x, xs, w, y, ys), &p,
                   ws_kind != Ws::kNone, x == y);
    if (st != RMSN_OK) return st;
    const bool wide = p.path == RMSN_PATH_WIDE;
    if (wide && ws_kind == Ws::kCaller &&
        (st = check_workspace(dtype, x, xs, w, y, ys, rows, n, ws, ws_bytes)) != RMSN_OK)
        return st;
    if (wide && ws_kind == Ws::kLibrary) {
        const int64_t need = workspace_bytes(p, rows);
        if (need > kScratchBytes) {
            set_error("the launch needs %lld bytes of workspace and the library holds %lld "
                      "(at most %lld rows on the WIDE path); use rmsnorm_batched_rows_ws",
                      (long long)need, (long long)kScratchBytes,
                      (long long)(kScratchBytes / 16));
            return RMSN_EINVAL;
        }
        if ((st = scratch_address(&ws)) != RMSN_OK) return st;
    }
    // A batch of more rows than one launch can hold goes as consecutive
    // launches of the plan's layout (a row's bits do not depend on the launch
    // it is in). Each piece starts a whole number of rows further on, which
    // keeps the alignment the plan assumed.
    const int64_t es = elem_bytes(dtype);
    const int64_t most = rows_per_launch(p);
    for (int64_t r0 = 0; r0 < rows; r0 += most) {
        const int64_t piece = rows - r0 < most ? rows - r0 : most;
        Plan q = p;
        const void* xq = static_cast<const char*>(x) + r0 * xs * es;
        void* yq = static_cast<char*>(y) + r0 * ys * es;
        hipError_t e;
        if (wide) {
            q.grid = 4 * piece;
            e = launch_wide_rows(q, xq, xs, w, yq, ys, piece, (int)n, eps,
                                 static_cast<float*>(ws) + 4 * r0,
                                 static_cast<hipStream_t>(stream));
        } else {
            q.grid = p.path == RMSN_PATH_REPLICA
                         ? piece * p.parts
                         : (piece + p.rows_per_block - 1) / p.rows_per_block;
            e = launch_rows(q, xq, xs, w, yq, ys, piece, (int)n, eps,
                            static_cast<hipStream_t>(stream));
        }
        if (e != hipSuccess) return hip_fail("kernel launch", e);
    }
    return RMSN_OK;
}

int plan_sequence(int dtype, const int64_t* widths, int32_t count, std::vector<Plan>* plans) {
    plans->resize((size_t)count);
    for (int32_t i = 0; i < count; ++i) {
        // Descriptor rows may have any element alignment: GROUP (whose kernel
        // checks the pointers it reads), BLOCK or STREAM.
        const int st = make_plan(dtype, 1, widths[i], kAlignAtRunTime, &(*plans)[(size_t)i]);
        if (st != RMSN_OK) return st;
    }
    return RMSN_OK;
}

// Which build of the descriptor kernels eager launches take. The HIP runtime
// keeps the arguments of launches enqueued one by one in device memory by
// default here; then the build whose kernels load their own arguments is the
// faster (327-norm step 958 against 1003 us). With HIP_FORCE_DEV_KERNARG=0 it
// keeps them in host memory, and the preloaded build is the faster (872
// against 1100 us). Read once per process.
bool eager_desc_preloaded() {
    static const bool host_kernargs = [] {
        const char* v = std::getenv("HIP_FORCE_DEV_KERNARG");
        return v && v[0] == '0' && v[1] == '\0';
    }();
    return host_kernargs;
}

// The sequence's launches on `s`; a positioned sequence ends with its
// position update.
int enqueue_sequence(const std::vector<Plan>& plans, const rmsn_desc* table, float eps,
                     const PosArgs* pos, hipStream_t s) {
    const bool preloaded = eager_desc_preloaded();
    for (size_t i = 0; i < plans.size(); ++i) {
        const hipError_t e = preloaded ? launch_desc_preloaded(plans[i], table + i, eps, pos, s)
                                       : launch_desc_plain(plans[i], table + i, eps, pos, s);
        if (e != hipSuccess) return hip_fail("sequence kernel launch", e);
    }
    if (pos) {
        const hipError_t e = launch_advance(const_cast<int64_t*>(pos->d_pos), pos->period, s);
        if (e != hipSuccess) return hip_fail("position update launch", e);
    }
    return RMSN_OK;
}

int check_position(int dtype, const rmsn_position* pos, PosArgs* out) {
    if (!pos || !pos->d_pos) {
        set_error("null position (pos=%p)", (const void*)pos);
        return RMSN_EINVAL;
    }
    if ((uintptr_t)pos->d_pos % 8) {
        set_error("d_pos must be 8-byte aligned");
        return RMSN_EINVAL;
    }
    const int64_t es = elem_bytes(dtype);
    if (pos->period < 1 || pos->x_pitch < 0 || pos->y_pitch < 0 || pos->x_pitch % es ||
        pos->y_pitch % es) {
        set_error("position: period must be >= 1 and pitches >= 0 multiples of %lld bytes "
                  "(period %lld, x_pitch %lld, y_pitch %lld)",
                  (long long)es, (long long)pos->period, (long long)pos->x_pitch,
                  (long long)pos->y_pitch);
        return RMSN_EINVAL;
    }
    const int64_t lim = INT64_MAX / 4;
    if ((pos->x_pitch && pos->period - 1 > lim / pos->x_pitch) ||
        (pos->y_pitch && pos->period - 1 > lim / pos->y_pitch)) {
        set_error("position: period * pitch overflows");
        return RMSN_EINVAL;
    }
    *out = PosArgs{pos->d_pos, pos->x_pitch, pos->y_pitch, pos->period};
    return RMSN_OK;
}

// Run every distinct kernel variant the graph records (the preloaded-argument
// build of the descriptor kernels) once on a private 1-element
// row (and, for a positioned sequence, a private position), so module loading
// and any other first-use work happen before capture. The caller's rows and
// position are not touched.
int prewarm(const std::vector<Plan>& plans, int dtype, float eps, bool positioned,
            hipStream_t s) {
    void* scratch = nullptr;
    hipError_t e = hipMalloc(&scratch, 256);
    if (e != hipSuccess) return hip_fail("hipMalloc (pre-warm row)", e);
    char* base = static_cast<char*>(scratch);
    rmsn_desc h{base + 64, base + 128, base + 192, 1};
    int64_t* own_pos = reinterpret_cast<int64_t*>(base + 224);
    const PosArgs own{own_pos, 0, 0, 1};
    const int64_t zero = 0;
    int st = RMSN_OK;
    const uint32_t one_f32 = 0x3F800000u;
    const uint16_t one_bf16 = 0x3F80u;
    const void* one = dtype == RMSN_F32 ? (const void*)&one_f32 : (const void*)&one_bf16;
    const size_t es = (size_t)elem_bytes(dtype);
    if ((e = hipMemcpyAsync(base, &h, sizeof h, hipMemcpyHostToDevice, s)) != hipSuccess ||
        (e = hipMemcpyAsync(base + 64, one, es, hipMemcpyHostToDevice, s)) != hipSuccess ||
        (e = hipMemcpyAsync(base + 128, one, es, hipMemcpyHostToDevice, s)) != hipSuccess ||
        (e = hipMemcpyAsync(own_pos, &zero, sizeof zero, hipMemcpyHostToDevice, s)) != hipSuccess) {
        st = hip_fail("hipMemcpyAsync (pre-warm row)", e);
    }
    std::vector<int> seen;  // kernel variants already run: path * 256 + chunks
    for (size_t i = 0; st == RMSN_OK && i < plans.size(); ++i) {
        const int key = plans[i].path * 256 + plans[i].chunks;
        bool dup = false;
        for (int c : seen) dup = dup || c == key;
        if (dup) continue;
        seen.push_back(key);
        e = launch_desc_preloaded(plans[i], reinterpret_cast<const rmsn_desc*>(base), eps,
                        positioned ? &own : nullptr, s);
        if (e != hipSuccess) st = hip_fail("pre-warm launch", e);
    }
    if (st == RMSN_OK && positioned) {
        e = launch_advance(own_pos, 1, s);
        if (e != hipSuccess) st = hip_fail("pre-warm launch", e);
    }
    e = hipStreamSynchronize(s);
    if (st == RMSN_OK && e != hipSuccess) st = hip_fail("hipStreamSynchronize (pre-warm)", e);
    e = hipFree(scratch);
    if (st == RMSN_OK && e != hipSuccess) st = hip_fail("hipFree (pre-warm row)", e);
    return st;
}

bool env_flag(const char* name) {
    const char* v = std::getenv(name);
    return v && v[0] == '1' && v[1] == '\0';
}

// Records the sequence on `s` into g->graph and instantiates it. On any
// failure the capture is ended, partial objects are destroyed, and an error
// status is returned with the message set.
int capture(rmsn_graph* g, hipStream_t s) {
    hipError_t e = hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal);
    if (e != hipSuccess) return hip_fail("hipStreamBeginCapture", e);
    int st = RMSN_OK;
    const PosArgs* pos = g->positioned ? &g->pos : nullptr;
    for (size_t i = 0; i < g->plans.size() && st == RMSN_OK; ++i) {
        e = launch_desc_preloaded(g->plans[i], g->table + i, g->eps, pos, s);
        if (e != hipSuccess) st = hip_fail("captured launch", e);
        // Test hook: a synchronisation is not allowed while capturing, which
        // makes the capture fail the way a forgotten lazy initialisation would.
        if (st == RMSN_OK && i == 0 && env_flag("RMSN_TEST_BREAK_CAPTURE")) {
            e = hipStreamSynchronize(s);
            st = hip_fail("hipStreamSynchronize inside capture (RMSN_TEST_BREAK_CAPTURE)",
                          e == hipSuccess ? hipErrorStreamCaptureUnsupported : e);
        }
    }
    if (st == RMSN_OK && pos) {
        e = launch_advance(const_cast<int64_t*>(pos->d_pos), pos->period, s);
        if (e != hipSuccess) st = hip_fail("captured position update", e);
    }
    hipGraph_t graph = nullptr;
    e = hipStreamEndCapture(s, &graph);
    if (st == RMSN_OK && e != hipSuccess) st = hip_fail("hipStreamEndCapture", e);
    if (st == RMSN_OK && graph == nullptr) {
        set_error("hipStreamEndCapture returned no graph");
        st = RMSN_EHIP;
    }
    if (st != RMSN_OK) {
        if (graph) (void)hipGraphDestroy(graph);
        (void)hipGetLastError();  // do not leave the capture's error sticky
        return st;
    }
    hipGraphExec_t exec = nullptr;
    e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
    if (e != hipSuccess) {
        (void)hipGraphDestroy(graph);
        (void)hipGetLastError();
        return hip_fail("hipGraphInstantiate", e);
    }
    size_t nodes = 0;
    e = hipGraphGetNodes(graph, nullptr, &nodes);
    if (e != hipSuccess) {
        (void)hipGraphExecDestroy(exec);
        (void)hipGraphDestroy(graph);
        return hip_fail("hipGraphGetNodes", e);
    }
    g->graph = graph;
    g->exec = exec;
    g->nodes = (int64_t)nodes;
    return RMSN_OK;
}

// Pre-warm and capture g's sequence on a private stream. On success g holds
// the new graph and is not in fallback mode. On a capture failure the
// partial graph is gone, g->fallback is set (launches replay eagerly with the
// same kernels), the reason is logged when RMSN_LOG=1, and RMSN_ECAPTURE is
// returned. Other failures return their status with g unchanged.
int build_graph(rmsn_graph* g) {
    hipStream_t s = nullptr;
    hipError_t e = hipStreamCreateWithFlags(&s, hipStreamNonBlocking);
    if (e != hipSuccess) return hip_fail("hipStreamCreateWithFlags", e);
    int st = prewarm(g->plans, g->dtype, g->eps, g->positioned, s);
    if (st != RMSN_OK) {
        (void)hipStreamDestroy(s);
        return st;
    }
    st = capture(g, s);
    (void)hipStreamDestroy(s);
    if (st != RMSN_OK) {
        // Graceful downgrade: the handle stays usable and replays eagerly.
        // Capture executes nothing, so no device state needs restoring.
        g->fallback = true;
        g->graph = nullptr;
        g->exec = nullptr;
        g->nodes = 0;
        if (env_flag("RMSN_LOG"))
            std::fprintf(stderr, "[rmsnorm] graph capture failed, eager fallback: %s\n",
                         last_error());
        return RMSN_ECAPTURE;
    }
    g->fallback = false;
    return RMSN_OK;
}

bool same_launches(const std::vector<Plan>& a, const std::vector<Plan>& b) {
    if (a.size() != b.size()) return false;
    for (size_t i = 0; i < a.size(); ++i) {
        const Plan& p = a[i];
        const Plan& q = b[i];
        if (p.path != q.path || p.chunks != q.chunks || p.loads != q.loads ||
            p.block != q.block || p.grid != q.grid || p.rows_per_block != q.rows_per_block ||
            p.streaming != q.streaming || p.parts != q.parts)
            return false;
    }
    return true;
}

int create_graph(int dtype, const rmsn_desc* d_table, const int64_t* h_widths, int32_t count,
                 float eps, const rmsn_position* position, rmsn_graph** out) {
    clear_error();
    if (!out) {
        set_error("null output handle pointer");
        return RMSN_EINVAL;
    }
    *out = nullptr;
    int st = check_sequence_args(dtype, d_table, h_widths, count, eps);
    if (st != RMSN_OK) return st;
    PosArgs pos{nullptr, 0, 0, 1};
    if (position && (st = check_position(dtype, position, &pos)) != RMSN_OK) return st;
    rmsn_graph* g = new (std::nothrow) rmsn_graph;
    if (!g) {
        set_error("out of host memory for the graph handle");
        return RMSN_ENOMEM;
    }
    g->dtype = dtype;
    g->eps = eps;
    g->table = d_table;
    g->positioned = position != nullptr;
    g->pos = pos;
    if ((st = plan_sequence(dtype, h_widths, count, &g->plans)) != RMSN_OK) {
        delete g;
        return st;
    }
    st = build_graph(g);
    if (st != RMSN_OK && st != RMSN_ECAPTURE) {
        delete g;
        return st;
    }
    *out = g;
    return st;
}

}  // namespace

extern "C" {

int rmsnorm_f32(const float* x, const float* w, float* y, int64_t n, float eps, void* stream) {
    return run_rows(RMSN_F32, x, n, w, y, n, 1, n, eps, Ws::kNone, nullptr, 0, stream);
}

int rmsnorm_bf16(const uint16_t* x, const uint16_t* w, uint16_t* y, int64_t n, float eps,
                 void* stream) {
    return run_rows(RMSN_BF16, x, n, w, y, n, 1, n, eps, Ws::kNone, nullptr, 0, stream);
}

int rmsnorm_batched_rows(int dtype, const void* x, int64_t x_row_stride, const void* w, void* y,
                         int64_t y_row_stride, int64_t rows, int64_t n, float eps, void* stream) {
    return run_rows(dtype, x, x_row_stride, w, y, y_row_stride, rows, n, eps, Ws::kNone, nullptr,
                    0, stream);
}

int rmsnorm_batched_rows_ws(int dtype, const void* x, int64_t x_row_stride, const void* w,
                            void* y, int64_t y_row_stride, int64_t rows, int64_t n, float eps,
                            void* workspace, int64_t workspace_bytes, void* stream) {
    return run_rows(dtype, x, x_row_stride, w, y, y_row_stride, rows, n, eps, Ws::kCaller,
                    workspace, workspace_bytes, stream);
}

int rmsnorm_batched_rows_noalloc(int dtype, const void* x, int64_t x_row_stride, const void* w,
                                 void* y, int64_t y_row_stride, int64_t rows, int64_t n,
                                 float eps, void* stream) {
    return run_rows(dtype, x, x_row_stride, w, y, y_row_stride, rows, n, eps, Ws::kLibrary,
                    nullptr, 0, stream);
}

int rmsnorm_sequence_eager(int dtype, const rmsn_desc* d_table, const int64_t* h_widths,
                           int32_t count, float eps, void* stream) {
    clear_error();
    int st = check_sequence_args(dtype, d_table, h_widths, count, eps);
    if (st != RMSN_OK) return st;
    std::vector<Plan> plans;
    if ((st = plan_sequence(dtype, h_widths, count, &plans)) != RMSN_OK) return st;
    return enqueue_sequence(plans, d_table, eps, nullptr, static_cast<hipStream_t>(stream));
}

int rmsnorm_sequence_eager_positioned(int dtype, const rmsn_desc* d_table,
                                      const int64_t* h_widths, int32_t count, float eps,
                                      const rmsn_position* position, void* stream) {
    clear_error();
    int st = check_sequence_args(dtype, d_table, h_widths, count, eps);
    if (st != RMSN_OK) return st;
    PosArgs pos;
    if ((st = check_position(dtype, position, &pos)) != RMSN_OK) return st;
    std::vector<Plan> plans;
    if ((st = plan_sequence(dtype, h_widths, count, &plans)) != RMSN_OK) return st;
    return enqueue_sequence(plans, d_table, eps, &pos, static_cast<hipStream_t>(stream));
}

int rmsnorm_sequence_persistent(int dtype, const rmsn_desc* d_table, int32_t count, float eps,
                                const rmsn_position* position, void* stream) {
    clear_error();
    if (dtype != RMSN_F32 && dtype != RMSN_BF16) {
        set_error("unknown dtype %d", dtype);
        return RMSN_EINVAL;
    }
    if (!d_table || (uintptr_t)d_table % alignof(rmsn_desc)) {
        set_error("d_table must be a non-null, %d-byte aligned device pointer",
                  (int)alignof(rmsn_desc));
        return RMSN_EINVAL;
    }
    if (count < 1 || count > RMSN_MAX_SEQUENCE) {
        set_error("count must be in [1, %d], got %d", RMSN_MAX_SEQUENCE, (int)count);
        return RMSN_EINVAL;
    }
    int st = check_eps(eps);
    if (st != RMSN_OK) return st;
    PosArgs pos;
    if (position && (st = check_position(dtype, position, &pos)) != RMSN_OK) return st;
    const hipError_t e = launch_sequence_persistent(dtype, d_table, count, eps,
                                                    position ? &pos : nullptr,
                                                    static_cast<hipStream_t>(stream));
    return e == hipSuccess ? RMSN_OK : hip_fail("persistent sequence launch", e);
}

int rmsnorm_sequence_graph_create(int dtype, const rmsn_desc* d_table, const int64_t* h_widths,
                                  int32_t count, float eps, rmsn_graph** out) {
    return create_graph(dtype, d_table, h_widths, count, eps, nullptr, out);
}

int rmsnorm_sequence_graph_create_positioned(int dtype, const rmsn_desc* d_table,
                                             const int64_t* h_widths, int32_t count, float eps,
                                             const rmsn_position* position, rmsn_graph** out) {
    if (!position) {
        clear_error();
        if (out) *out = nullptr;
        set_error("null position");
        return RMSN_EINVAL;
    }
    return create_graph(dtype, d_table, h_widths, count, eps, position, out);
}

int rmsnorm_sequence_graph_update(rmsn_graph* g, const int64_t* h_widths, int32_t count,
                                  int* recaptured) {
    clear_error();
    if (recaptured) *recaptured = 0;
    if (!g) {
        set_error("null graph handle");
        return RMSN_EINVAL;
    }
    if ((size_t)count != g->plans.size()) {
        set_error("count %d differs from the handle's %d norms", (int)count, (int)g->plans.size());
        return RMSN_EINVAL;
    }
    int st = check_sequence_args(g->dtype, g->table, h_widths, count, g->eps);
    if (st != RMSN_OK) return st;
    std::vector<Plan> plans;
    if ((st = plan_sequence(g->dtype, h_widths, count, &plans)) != RMSN_OK) return st;
    // Same launches: the captured graph already runs exactly these kernels
    // (widths are loop bounds read from the table when they run).
    if (same_launches(plans, g->plans) && !g->fallback) return RMSN_OK;
    rmsn_graph next = *g;
    next.plans = plans;
    next.graph = nullptr;
    next.exec = nullptr;
    next.nodes = 0;
    st = build_graph(&next);
    if (st != RMSN_OK && st != RMSN_ECAPTURE) return st;  // g unchanged
    // Swap in the new graph (or the eager fallback with the new plans).
    if (g->exec) (void)hipGraphExecDestroy(g->exec);
    if (g->graph) (void)hipGraphDestroy(g->graph);
    *g = next;
    if (recaptured) *recaptured = 1;
    return st;
}

int rmsnorm_sequence_graph_launch(rmsn_graph* g, void* stream) {
    clear_error();
    if (!g) {
        set_error("null graph handle");
        return RMSN_EINVAL;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (g->fallback)
        return enqueue_sequence(g->plans, g->table, g->eps, g->positioned ? &g->pos : nullptr, s);
    const hipError_t e = hipGraphLaunch(g->exec, s);
    return e == hipSuccess ? RMSN_OK : hip_fail("hipGraphLaunch", e);
}

int rmsnorm_sequence_graph_destroy(rmsn_graph* g) {
    clear_error();
    if (!g) return RMSN_OK;
    int st = RMSN_OK;
    if (g->exec) {
        const hipError_t e = hipGraphExecDestroy(g->exec);
        if (e != hipSuccess) st = hip_fail("hipGraphExecDestroy", e);
    }
    if (g->graph) {
        const hipError_t e = hipGraphDestroy(g->graph);
        if (e != hipSuccess && st == RMSN_OK) st = hip_fail("hipGraphDestroy", e);
    }
    delete g;
    return st;
}

int rmsnorm_graph_node_count(const rmsn_graph* g, int64_t* out) {
    clear_error();
    if (!g || !out) {
        set_error("null argument");
        return RMSN_EINVAL;
    }
    *out = g->nodes;
    return RMSN_OK;
}

int rmsnorm_graph_is_fallback(const rmsn_graph* g, int* out) {
    clear_error();
    if (!g || !out) {
        set_error("null argument");
        return RMSN_EINVAL;
    }
    *out = g->fallback ? 1 : 0;
    return RMSN_OK;
}

const char* rmsnorm_last_error(void) { return last_error(); }

int rmsnorm_association_lanes(void) { return kAssocLanes; }

static void plan_info(const Plan& p, rmsn_plan_info* out) {
    out->path = p.path;
    out->chunks = p.chunks;
    out->rows_per_block = p.rows_per_block;
    out->parts = p.parts;
    out->block = p.block;
    out->grid = p.grid;
    out->streaming = p.streaming;
    out->loads = p.loads;
}

int rmsnorm_plan_query(int dtype, int64_t rows, int64_t n, int align, rmsn_plan_info* out) {
    clear_error();
    if (!out) {
        set_error("null output pointer");
        return RMSN_EINVAL;
    }
    Plan p;
    const int st = make_plan(dtype, rows, n, align, &p);
    if (st != RMSN_OK) return st;
    plan_info(p, out);
    return RMSN_OK;
}

int rmsnorm_workspace_query(int dtype, int64_t rows, int64_t n, int align, rmsn_plan_info* plan,
                            int64_t* bytes) {
    clear_error();
    if (!bytes) {
        set_error("null output pointer");
        return RMSN_EINVAL;
    }
    Plan p;
    const int st = make_plan(dtype, rows, n, align, &p, true);
    if (st != RMSN_OK) return st;
    if (plan) plan_info(p, plan);
    *bytes = workspace_bytes(p, rows);
    return RMSN_OK;
}

int rmsnorm_set_option(int key, int value) {
    clear_error();
    return set_option(key, value);
}

int rmsnorm_get_option(int key, int* value) {
    clear_error();
    return get_option(key, value);
}

int rmsnorm_diag_copy(const void* src, void* dst, int64_t bytes, int vectors, int block,
                      void* stream) {
    clear_error();
    const uintptr_t a = (uintptr_t)src, b = (uintptr_t)dst;
    if (!src || !dst || (a | b) % 16) {
        set_error("src and dst must be non-null and 16-byte aligned (src=%p dst=%p)", src, dst);
        return RMSN_EINVAL;
    }
    if (bytes <= 0 || bytes % 16) {
        set_error("bytes must be a positive multiple of 16, got %lld", (long long)bytes);
        return RMSN_EINVAL;
    }
    if (a < b + (uint64_t)bytes && b < a + (uint64_t)bytes) {
        set_error("src and dst overlap");
        return RMSN_EINVAL;
    }
    if ((vectors != 1 && vectors != 2 && vectors != 4) || block < 64 || block > 1024 ||
        block % 64) {
        set_error("vectors must be 1, 2 or 4 and block a multiple of 64 up to 1024 (got %d, %d)",
                  vectors, block);
        return RMSN_EINVAL;
    }
    const hipError_t e = launch_diag_copy(src, dst, bytes, vectors, block,
                                          static_cast<hipStream_t>(stream));
    return e == hipSuccess ? RMSN_OK : hip_fail("diagnostic copy launch", e);
}

int rmsnorm_diag_walk_timeouts(uint32_t* out, int reset) {
    clear_error();
    if (!out) {
        set_error("null output pointer");
        return RMSN_EINVAL;
    }
    const hipError_t e = walk_timeouts(out, reset != 0);
    return e == hipSuccess ? RMSN_OK : hip_fail("reading the walk timeout counter", e);
}

int rmsnorm_diag_bf16(uint32_t first_bits, int64_t count, uint16_t* out, void* stream) {
    clear_error();
    if (!out) {
        set_error("null output pointer");
        return RMSN_EINVAL;
    }
    if (count < 0 || (uint64_t)first_bits + (uint64_t)count > 0x100000000ull) {
        set_error("bit-pattern range [%u, %u + %lld) leaves 32 bits", first_bits, first_bits,
                  (long long)count);
        return RMSN_EINVAL;
    }
    if ((uintptr_t)out % 2) {
        set_error("output must be 2-byte aligned");
        return RMSN_EINVAL;
    }
    const hipError_t e = launch_diag_bf16(first_bits, count, out, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? RMSN_OK : hip_fail("diagnostic launch", e);
}

int rmsnorm_diag_inverse(uint32_t first_bits, int64_t count, int64_t n, float eps, float* r_out,
                         float* inv_out, void* stream) {
    clear_error();
    if (!r_out || !inv_out) {
        set_error("null output pointer");
        return RMSN_EINVAL;
    }
    if (count < 0 || (uint64_t)first_bits + (uint64_t)count > 0x100000000ull) {
        set_error("bit-pattern range [%u, %u + %lld) leaves 32 bits", first_bits, first_bits,
                  (long long)count);
        return RMSN_EINVAL;
    }
    if (n < 1 || n > RMSN_MAX_N) {
        set_error("n must be in [1, %d], got %lld", RMSN_MAX_N, (long long)n);
        return RMSN_EINVAL;
    }
    int st = check_eps(eps);
    if (st != RMSN_OK) return st;
    if (((uintptr_t)r_out | (uintptr_t)inv_out) % 4) {
        set_error("outputs must be 4-byte aligned");
        return RMSN_EINVAL;
    }
    const hipError_t e = launch_diag_inverse(first_bits, count, (int)n, eps, r_out, inv_out,
                                             static_cast<hipStream_t>(stream));
    return e == hipSuccess ? RMSN_OK : hip_fail("diagnostic launch", e);
}

}  // extern "C"
