// rmsn_api.hip -- the C ABI (include/rmsnorm.h): validation, planning,
// launches, and the captured decode-step sequence.
//
// Graph discipline follows Lecture 08 "Graph-resident decode": the values that
// change per replay (row pointers, widths) live in a device descriptor table
// the kernels read when they run (section 2); launch geometry is a capture key
// decided by the same plan function the eager path uses (section 2); every
// kernel variant runs once before capture so nothing initialises lazily inside
// it, and a failed capture degrades to eager replay instead of failing
// (section 3).
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <vector>

#include "rmsn_launch.h"
#include "rmsn_plan.h"
#include "rmsnorm.h"

using namespace rmsn;

struct rmsn_graph {
    int dtype = RMSN_F32;
    float eps = 0.0f;
    const rmsn_desc* table = nullptr;
    std::vector<Plan> plans;
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

int run_rows(int dtype, const void* x, int64_t xs, const void* w, void* y, int64_t ys,
             int64_t rows, int64_t n, float eps, void* stream) {
    clear_error();
    int st = check_row_args(dtype, x, xs, w, y, ys, rows, n);
    if (st != RMSN_OK) return st;
    if ((st = check_eps(eps)) != RMSN_OK) return st;
    Plan p;
    st = make_plan(dtype, rows, n, rows_alignment(dtype, x, xs, w, y, ys), &p);
    if (st != RMSN_OK) return st;
    const hipError_t e =
        launch_rows(p, x, xs, w, y, ys, rows, (int)n, eps, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? RMSN_OK : hip_fail("kernel launch", e);
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

int enqueue_sequence(const std::vector<Plan>& plans, const rmsn_desc* table, float eps,
                     hipStream_t s) {
    for (size_t i = 0; i < plans.size(); ++i) {
        const hipError_t e = launch_desc(plans[i], table + i, eps, s);
        if (e != hipSuccess) return hip_fail("sequence kernel launch", e);
    }
    return RMSN_OK;
}

// Run every distinct kernel variant of the sequence once on a private 1-element
// row, so module loading and any other first-use work happen before capture.
int prewarm(const std::vector<Plan>& plans, int dtype, float eps, hipStream_t s) {
    void* scratch = nullptr;
    hipError_t e = hipMalloc(&scratch, 256);
    if (e != hipSuccess) return hip_fail("hipMalloc (pre-warm row)", e);
    char* base = static_cast<char*>(scratch);
    rmsn_desc h{base + 64, base + 128, base + 192, 1};
    int st = RMSN_OK;
    const uint32_t one_f32 = 0x3F800000u;
    const uint16_t one_bf16 = 0x3F80u;
    const void* one = dtype == RMSN_F32 ? (const void*)&one_f32 : (const void*)&one_bf16;
    const size_t es = (size_t)elem_bytes(dtype);
    if ((e = hipMemcpyAsync(base, &h, sizeof h, hipMemcpyHostToDevice, s)) != hipSuccess ||
        (e = hipMemcpyAsync(base + 64, one, es, hipMemcpyHostToDevice, s)) != hipSuccess ||
        (e = hipMemcpyAsync(base + 128, one, es, hipMemcpyHostToDevice, s)) != hipSuccess) {
        st = hip_fail("hipMemcpyAsync (pre-warm row)", e);
    }
    std::vector<int> seen;  // kernel variants already run: path * 256 + chunks
    for (size_t i = 0; st == RMSN_OK && i < plans.size(); ++i) {
        const int key = plans[i].path * 256 + plans[i].chunks;
        bool dup = false;
        for (int c : seen) dup = dup || c == key;
        if (dup) continue;
        seen.push_back(key);
        e = launch_desc(plans[i], reinterpret_cast<const rmsn_desc*>(base), eps, s);
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
    for (size_t i = 0; i < g->plans.size() && st == RMSN_OK; ++i) {
        e = launch_desc(g->plans[i], g->table + i, g->eps, s);
        if (e != hipSuccess) st = hip_fail("captured launch", e);
        // Test hook: a synchronisation is not allowed while capturing, which
        // makes the capture fail the way a forgotten lazy initialisation would.
        if (st == RMSN_OK && i == 0 && env_flag("RMSN_TEST_BREAK_CAPTURE")) {
            e = hipStreamSynchronize(s);
            st = hip_fail("hipStreamSynchronize inside capture (RMSN_TEST_BREAK_CAPTURE)",
                          e == hipSuccess ? hipErrorStreamCaptureUnsupported : e);
        }
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

}  // namespace

extern "C" {

int rmsnorm_f32(const float* x, const float* w, float* y, int64_t n, float eps, void* stream) {
    return run_rows(RMSN_F32, x, n, w, y, n, 1, n, eps, stream);
}

int rmsnorm_bf16(const uint16_t* x, const uint16_t* w, uint16_t* y, int64_t n, float eps,
                 void* stream) {
    return run_rows(RMSN_BF16, x, n, w, y, n, 1, n, eps, stream);
}

int rmsnorm_batched_rows(int dtype, const void* x, int64_t x_row_stride, const void* w, void* y,
                         int64_t y_row_stride, int64_t rows, int64_t n, float eps, void* stream) {
    return run_rows(dtype, x, x_row_stride, w, y, y_row_stride, rows, n, eps, stream);
}

int rmsnorm_sequence_eager(int dtype, const rmsn_desc* d_table, const int64_t* h_widths,
                           int32_t count, float eps, void* stream) {
    clear_error();
    int st = check_sequence_args(dtype, d_table, h_widths, count, eps);
    if (st != RMSN_OK) return st;
    std::vector<Plan> plans;
    if ((st = plan_sequence(dtype, h_widths, count, &plans)) != RMSN_OK) return st;
    return enqueue_sequence(plans, d_table, eps, static_cast<hipStream_t>(stream));
}

int rmsnorm_sequence_graph_create(int dtype, const rmsn_desc* d_table, const int64_t* h_widths,
                                  int32_t count, float eps, rmsn_graph** out) {
    clear_error();
    if (!out) {
        set_error("null output handle pointer");
        return RMSN_EINVAL;
    }
    *out = nullptr;
    int st = check_sequence_args(dtype, d_table, h_widths, count, eps);
    if (st != RMSN_OK) return st;
    rmsn_graph* g = new (std::nothrow) rmsn_graph;
    if (!g) {
        set_error("out of host memory for the graph handle");
        return RMSN_ENOMEM;
    }
    g->dtype = dtype;
    g->eps = eps;
    g->table = d_table;
    if ((st = plan_sequence(dtype, h_widths, count, &g->plans)) != RMSN_OK) {
        delete g;
        return st;
    }
    hipStream_t s = nullptr;
    hipError_t e = hipStreamCreateWithFlags(&s, hipStreamNonBlocking);
    if (e != hipSuccess) {
        delete g;
        return hip_fail("hipStreamCreateWithFlags", e);
    }
    st = prewarm(g->plans, dtype, eps, s);
    if (st != RMSN_OK) {
        (void)hipStreamDestroy(s);
        delete g;
        return st;
    }
    st = capture(g, s);
    (void)hipStreamDestroy(s);
    if (st != RMSN_OK) {
        // Graceful downgrade: the handle stays usable and replays eagerly.
        g->fallback = true;
        if (env_flag("RMSN_LOG"))
            std::fprintf(stderr, "[rmsnorm] graph capture failed, eager fallback: %s\n",
                         last_error());
        *out = g;
        return RMSN_ECAPTURE;
    }
    *out = g;
    return RMSN_OK;
}

int rmsnorm_sequence_graph_launch(rmsn_graph* g, void* stream) {
    clear_error();
    if (!g) {
        set_error("null graph handle");
        return RMSN_EINVAL;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (g->fallback) return enqueue_sequence(g->plans, g->table, g->eps, s);
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

int rmsnorm_plan_query(int dtype, int64_t rows, int64_t n, int align, rmsn_plan_info* out) {
    clear_error();
    if (!out) {
        set_error("null output pointer");
        return RMSN_EINVAL;
    }
    Plan p;
    const int st = make_plan(dtype, rows, n, align, &p);
    if (st != RMSN_OK) return st;
    out->path = p.path;
    out->chunks = p.chunks;
    out->rows_per_block = p.rows_per_block;
    out->block = p.block;
    out->grid = p.grid;
    out->streaming = p.streaming;
    out->loads = p.loads;
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
