// rmsn_persistent.hip -- the decode step's norms in one launch, for CDNA4
// (gfx950): a persistent kernel that walks a whole descriptor table and keeps
// the order of the table where it can be observed (Lecture 08
// "Graph-resident decode", further reading: a resident kernel as the
// endpoint of capturing many launches). Every row is computed by the row
// layouts of rmsn_rows.h, so its bits are those of the launch sequence.
//
// Floating point: contraction is off; '/' and sqrtf are HIP's correctly
// rounded binary32 sequences (steps 4-7 in rmsn_common.h).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <type_traits>

#include "rmsn_common.h"
#include "rmsn_group.h"
#include "rmsn_launch.h"
#include "rmsn_rows.h"

#pragma clang fp contract(off)

namespace rmsn {
namespace {

// The whole decode step in one launch (Lecture 08 "Graph-resident decode",
// further reading: a persistent kernel instead of many captured ones). One
// workgroup of four wavefronts walks the descriptor table, in one of three
// ways chosen when the launch starts (every thread checks some rows, then one
// barrier):
//  - round walk, when every row is a whole number of 16-byte vectors (at most
//    8192 elements, 16-byte aligned) and no row of an aligned group of 16 (or
//    at least of 4) consecutive rows reads or writes memory that another row
//    of the group writes: each wavefront takes a row of its own and holds it
//    whole, four rows at a time, and a workgroup barrier after each group
//    orders the group's stores before the next group's loads;
//  - pipelined, when every row fits the GROUP mapping (width a multiple of
//    4 and at most 8192, pointers quad-aligned) and no row reads memory that
//    one of the three rows before it writes, nor writes memory the row just
//    before it writes: the four wavefronts share each row, and the next row's
//    loads are issued before the current row is reduced;
//  - otherwise row after row, with a workgroup barrier after each row that
//    orders its stores before the next row's loads.
// All three compute what the launch sequence computes. With POS the rows are
// taken at the device-resident position, read once, and the last thread
// stores the next position after the last row (the same update as the
// sequence's last node).

// Row pointers of descriptor `dd` at position `pos`.
template <typename T, bool POS>
__device__ __forceinline__ void persistent_ptrs(const rmsn_desc& dd, uint64_t pos,
                                                const PosArgs& pa, const T*& x, const T*& w,
                                                T*& y) {
    desc_row<T, POS>(dd, pos, pa, x, y);
    w = static_cast<const T*>(dd.w);
}

template <typename T>
__device__ __forceinline__ bool group_fits(const T* x, const T* w, const T* y, int64_t n) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(w) |
                        reinterpret_cast<uintptr_t>(y);
    return n >= 1 && n <= 8192 && (n & 3) == 0 && a % (4 * sizeof(T)) == 0;
}

template <typename T>
__device__ __forceinline__ void persistent_row(const T* x, const T* w, T* y, int64_t n, float eps,
                                               float* lds4) {
    if (n < 1 || n > RMSN_MAX_N) return;
    if (group_fits<T>(x, w, y, n)) {
        switch ((int)((n + 1023) >> 10)) {
#define RMSN_CASE(Q) \
    case Q: row_group<T, Q>(x, w, y, (int)n, eps, lds4); break;
            RMSN_FOR_GROUP_BLOCKS(RMSN_CASE)
#undef RMSN_CASE
            default: break;
        }
    } else {
        row_block<T, 0>(x, w, y, (int)n, eps, lds4);
    }
}

// --- Pipelined walk. Every row takes the GROUP mapping at the table's widest
// block count (1024-element blocks) through buffer loads and stores whose
// range is the row's byte length: lanes past the row load +0
// (fmaf(0, 0, p) == p) and their stores are dropped by the hardware's range
// check, so every row issues the same instructions whatever its width and the
// compiler can wait for exactly the row it needs while the next one is in
// flight.

typedef __amdgpu_buffer_rsrc_t brsrc;

// A buffer resource for `bytes` bytes at p (raw, stride 0; the third word is
// the gfx9-family untyped format). Offsets at or past `bytes` are out of range.
__device__ __forceinline__ brsrc row_rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes,
                                             0x00020000);
}

template <typename T> struct PipeQuad;
template <> struct PipeQuad<float> {
    typedef u32x4 raw;
    static __device__ __forceinline__ raw load(brsrc r, uint32_t off) {
        return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    }
    static __device__ __forceinline__ void store(raw v, brsrc r, uint32_t off) {
        __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 0);
    }
    static __device__ __forceinline__ void unpack(raw q, float v[4]) {
        v[0] = __uint_as_float(q.x); v[1] = __uint_as_float(q.y);
        v[2] = __uint_as_float(q.z); v[3] = __uint_as_float(q.w);
    }
    static __device__ __forceinline__ raw apply(raw x, raw w, float inv) {
        return slice_apply(x, w, inv, 0.0f);
    }
};
template <> struct PipeQuad<uint16_t> {
    typedef u32x2 raw;
    static __device__ __forceinline__ raw load(brsrc r, uint32_t off) {
        return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    }
    static __device__ __forceinline__ void store(raw v, brsrc r, uint32_t off) {
        __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, 0);
    }
    static __device__ __forceinline__ void unpack(raw q, float v[4]) {
        v[0] = lo_bf16(q.x); v[1] = hi_bf16(q.x); v[2] = lo_bf16(q.y); v[3] = hi_bf16(q.y);
    }
    static __device__ __forceinline__ raw apply(raw x, raw w, float inv) {
        raw o;
        o.x = apply_pair(x.x, w.x, inv);
        o.y = apply_pair(x.y, w.y, inv);
        return o;
    }
};

struct PipeRow {
    brsrc x, w, y;
    int n;
};

template <typename T, int QM>
struct PipeBuf {
    typename PipeQuad<T>::raw x[QM], w[QM];
};

// Descriptor i of the table, or the last one past its end (only its base
// pointers are used then, with an empty range).
__device__ __forceinline__ rmsn_desc pipe_desc(const rmsn_desc* d, int32_t i, int32_t count) {
    return d[i < count ? i : count - 1];
}

// Buffer resources of a row; `real` false gives an empty range (every access
// out of range, no memory touched) on valid bases.
template <typename T, bool POS>
__device__ __forceinline__ PipeRow pipe_row_of(const rmsn_desc& dd, bool real, uint64_t pos,
                                               const PosArgs& pa) {
    const T* x;
    const T* w;
    T* y;
    persistent_ptrs<T, POS>(dd, pos, pa, x, w, y);
    const uint32_t bytes = real ? (uint32_t)dd.n * (uint32_t)sizeof(T) : 0u;
    return PipeRow{row_rsrc(x, bytes), row_rsrc(w, bytes), row_rsrc(y, bytes), (int)dd.n};
}

// This lane's byte offset in block m: GROUP's element 1024 m + 256 q + 64 g + 4 t.
template <typename T>
__device__ __forceinline__ uint32_t pipe_off(uint32_t lane_off, int m) {
    return lane_off + (uint32_t)m * 1024u * (uint32_t)sizeof(T);
}

template <typename T, int QM>
__device__ __forceinline__ void pipe_issue(PipeBuf<T, QM>& b, const PipeRow& r,
                                           uint32_t lane_off) {
#pragma unroll
    for (int m = 0; m < QM; ++m) b.x[m] = PipeQuad<T>::load(r.x, pipe_off<T>(lane_off, m));
#pragma unroll
    for (int m = 0; m < QM; ++m) b.w[m] = PipeQuad<T>::load(r.w, pipe_off<T>(lane_off, m));
}

// Workgroup barrier for LDS only: it does not wait for this wavefront's
// global loads and stores (a full barrier would wait for the next row's
// loads, in flight by design).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <typename T, int QM>
__device__ __forceinline__ void pipe_compute(const PipeBuf<T, QM>& b, const PipeRow& r,
                                             uint32_t lane_off, float eps, float* lds4, int g,
                                             int lane) {
    float p = 0.0f;
#pragma unroll
    for (int m = 0; m < QM; ++m) {
        float v[4];
        PipeQuad<T>::unpack(b.x[m], v);
        transpose4(v);
        p = fmaf(v[0], v[0], p);  // chunks 4m .. 4m+3 of chain 64g + 4t + q
        p = fmaf(v[1], v[1], p);
        p = fmaf(v[2], v[2], p);
        p = fmaf(v[3], v[3], p);
    }
    const float gt = group_sumsq(p);
    if (lane == 0) lds4[g] = gt;
    lds_barrier();
    const float inv = inverse_rms((lds4[0] + lds4[2]) + (lds4[1] + lds4[3]), r.n, eps);
#pragma unroll
    for (int m = 0; m < QM; ++m)
        PipeQuad<T>::store(PipeQuad<T>::apply(b.x[m], b.w[m], inv), r.y,
                           pipe_off<T>(lane_off, m));
}

// --- Round walk: one wavefront per row, the four wavefronts on four
// consecutive rows at a time (a round). A row is the SPLIT layout with a
// single wavefront: U 1 KB slices, one 16-byte load per lane each, so the
// wavefront holds the whole row and needs neither LDS nor a hand-off. Every
// row issues its own number of loads, and the four rows of a round are in
// flight together.

template <typename T, int U, bool EXACT>
__device__ __forceinline__ void wave_row_slices(const T* x, const T* w, T* y, int n, float eps,
                                                int lane) {
    const uint32_t nvec = (uint32_t)n * (uint32_t)sizeof(T) / 16u;
    SplitPart<T, U, EXACT, false> part;
    part.load(scalar_gptr(reinterpret_cast<const char*>(x)),
              scalar_gptr(reinterpret_cast<const char*>(w)), 0, lane, nvec);
    float p[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    part.chains(p, nvec);
    const float inv = inverse_rms(split_sumsq(p, lane, T()), n, eps);
    part.apply(inv, scalar_gptr(reinterpret_cast<char*>(y)), 0, lane, nvec);
}

// Slice buckets of the one-wavefront rows (rows of at most 8192 elements:
// 32 slices of binary32, 16 of bf16).
#define RMSN_FOR_ROUND_SLICES(X) X(1) X(2) X(3) X(4) X(6) X(8) X(12) X(16) X(20) X(24) X(28) X(32)

// One row of a round: 1 <= n <= 8192, n * sizeof(T) a multiple of 16, x, w, y
// 16-byte aligned (checked before the round walk is chosen).
template <typename T>
__device__ __forceinline__ void round_row(const T* x, const T* w, T* y, int n, float eps,
                                          int lane) {
    const int bytes = n * (int)sizeof(T);
    const int slices = (bytes + 1023) >> 10;
#define RMSN_CASE(U)                                                                   \
    if constexpr (U * 1024 <= 8192 * (int)sizeof(T)) {                                 \
        if (slices <= U) {                                                             \
            if (bytes == U * 1024) wave_row_slices<T, U, true>(x, w, y, n, eps, lane);  \
            else wave_row_slices<T, U, false>(x, w, y, n, eps, lane);                  \
            return;                                                                    \
        }                                                                              \
    }
    RMSN_FOR_ROUND_SLICES(RMSN_CASE)
#undef RMSN_CASE
}

// Rounds of four rows, a workgroup barrier after every K rounds: wavefront w
// takes rows 4q + w of each group of 4K rows, and the barrier orders the
// group's stores before the next group's loads.
template <typename T, bool POS, int K>
__device__ __forceinline__ void round_walk(const rmsn_desc* d, int32_t count, float eps,
                                           uint64_t pos, const PosArgs& pa) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    for (int32_t r = 0; r < count; r += 4 * K) {
        for (int q = 0; q < K; ++q) {
            const int32_t j = r + 4 * q + wave;
            if (j < count) {
                const rmsn_desc dd = d[j];
                const T* x;
                const T* w;
                T* y;
                persistent_ptrs<T, POS>(dd, pos, pa, x, w, y);
                round_row<T>(x, w, y, (int)dd.n, eps, lane);
            }
        }
        __syncthreads();  // the group's stores before the next group's loads
    }
}

// How the table is walked (see above): kRoundWalk16 or kRoundWalk4 (no row of
// an aligned group of 16 / 4 rows reads or writes what another row of the
// group writes), a block count 1..8 for the pipelined walk (the widest
// row's), or 0 for row after row. Every thread checks rows threadIdx.x,
// threadIdx.x + blockDim.x, ...; the answer is the workgroup's.
constexpr int kRoundWalk4 = 100;
constexpr int kRoundWalk16 = 101;
constexpr int kSpanRows = 1024;  // output ranges published in LDS (16 KB)
// Workgroups of the spread launch: kWalkers "walkers" that take the rows bound
// to table order (each walks whole components of them, see spread_on), then
// workers for the free rows -- one wave of workgroups on the 256 CUs (the
// kernel's registers allow one workgroup per CU).
constexpr int kWalkers = 4;
constexpr int kSpreadWorkers = 256 - kWalkers;

__device__ __forceinline__ bool ranges_meet(uintptr_t a, uintptr_t la, uintptr_t b, uintptr_t lb) {
    return a < b + lb && b < a + la;
}

// Row j's pointers as integers, its byte length, and what the walks need of it.
template <typename T, bool POS>
__device__ __forceinline__ void walk_row_facts(const rmsn_desc& dj, uint64_t pos,
                                               const PosArgs& pa, uintptr_t& bx, uintptr_t& bw,
                                               uintptr_t& by, uintptr_t& len, bool& fits,
                                               bool& vec) {
    const T* x;
    const T* w;
    T* y;
    persistent_ptrs<T, POS>(dj, pos, pa, x, w, y);
    bx = reinterpret_cast<uintptr_t>(x);
    bw = reinterpret_cast<uintptr_t>(w);
    by = reinterpret_cast<uintptr_t>(y);
    fits = group_fits<T>(x, w, y, dj.n);
    len = (uintptr_t)(dj.n < 0 ? 0 : dj.n) * sizeof(T);
    vec = fits && len % 16 == 0 && (bx | bw | by) % 16 == 0;
}

// What row j finds against row k (k != j): rules of the walks above.
__device__ __forceinline__ void walk_pair(int32_t j, int32_t k, uintptr_t bx, uintptr_t bw,
                                          uintptr_t by, uintptr_t len, uintptr_t ky,
                                          uintptr_t klen, bool& no_pipe, bool& no_round,
                                          bool& no_round16) {
    const bool reads = ranges_meet(bx, len, ky, klen) || ranges_meet(bw, len, ky, klen);
    const bool writes = ranges_meet(by, len, ky, klen);
    const int32_t r0 = j & ~3, g0 = j & ~15;
    if (k < j && j - k <= 3 && (reads || (writes && k == j - 1))) no_pipe = true;
    const bool meet = reads || (writes && k < j);
    if (k >= r0 && k < r0 + 4 && meet) no_round = true;
    if (k >= g0 && meet) no_round16 = true;
}

// How the table is walked (see above): kRoundWalk16 or kRoundWalk4, a block
// count 1..8 for the pipelined walk (the widest row's), or 0 for row after
// row. Every thread checks rows threadIdx.x, threadIdx.x + blockDim.x, ...
// against the rows of their windows (the three rows before, the other rows
// of their groups of 4 and 16); the answer is the workgroup's. Tables of up to
// kSpanRows rows first publish every row's output range in LDS, so a check
// reads 16 bytes of LDS instead of a descriptor from memory.
template <typename T, bool POS>
__device__ __forceinline__ int walk_mode(const rmsn_desc* d, int32_t count, uint64_t pos,
                                         const PosArgs& pa, int* lds_fold) {
    __shared__ uintptr_t yspan[kSpanRows][2];  // output start, byte length
    bool no_pipe = false, no_round = false, no_round16 = false;
    int blocks = 1;
    if (count <= kSpanRows) {
        // at most kSpanRows / 256 rows per thread: their facts stay in registers
        constexpr int R = kSpanRows / 256;
        uintptr_t bx[R], bw[R], by[R], len[R];
        bool live[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int32_t j = threadIdx.x + 256 * r;
            live[r] = j < count;
            bool fits = true, vec = true;
            if (live[r]) {
                const rmsn_desc dj = d[j];
                walk_row_facts<T, POS>(dj, pos, pa, bx[r], bw[r], by[r], len[r], fits, vec);
                yspan[j][0] = by[r];
                yspan[j][1] = len[r];
                blocks = max(blocks, (int)((dj.n + 1023) >> 10));
            }
            if (!fits) no_pipe = no_round = no_round16 = true;
            if (!vec) no_round = no_round16 = true;
        }
        __syncthreads();
#pragma unroll
        for (int r = 0; r < R; ++r) {
            if (!live[r]) continue;
            const int32_t j = threadIdx.x + 256 * r;
            const int32_t g0 = j & ~15;
            const int32_t k_end = min(count, g0 + 16);
#pragma unroll 4
            for (int32_t k = max(0, min(j - 3, g0)); k < k_end; ++k) {
                if (k == j) continue;
                walk_pair(j, k, bx[r], bw[r], by[r], len[r], yspan[k][0], yspan[k][1], no_pipe,
                          no_round, no_round16);
            }
        }
    } else {
        for (int32_t j = threadIdx.x; j < count; j += blockDim.x) {
            const rmsn_desc dj = d[j];
            uintptr_t bx, bw, by, len;
            bool fits, vec;
            walk_row_facts<T, POS>(dj, pos, pa, bx, bw, by, len, fits, vec);
            if (!fits) {
                no_pipe = no_round = no_round16 = true;
                break;
            }
            if (!vec) no_round = no_round16 = true;
            blocks = max(blocks, (int)((dj.n + 1023) >> 10));
            const int32_t g0 = j & ~15;
            const int32_t k_end = min(count, g0 + 16);
            for (int32_t k = max(0, min(j - 3, g0)); k < k_end; ++k) {
                if (k == j) continue;
                uintptr_t kx, kw, ky, klen;
                bool kf, kv;
                walk_row_facts<T, POS>(d[k], pos, pa, kx, kw, ky, klen, kf, kv);
                walk_pair(j, k, bx, bw, by, len, ky, klen, no_pipe, no_round, no_round16);
            }
        }
    }
    // One exchange for the workgroup: each wavefront folds its lanes (ballots
    // and a maximum), lane 0 publishes the result, one barrier, every thread
    // folds the four.
    const uint32_t flags = (__ballot(no_pipe) ? 1u : 0u) | (__ballot(no_round) ? 2u : 0u) |
                           (__ballot(no_round16) ? 4u : 0u);
    int wmax = blocks;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) wmax = max(wmax, __shfl_xor(wmax, o, 64));
    if ((threadIdx.x & 63) == 0) lds_fold[threadIdx.x >> 6] = (int)(flags << 8) | wmax;
    __syncthreads();
    uint32_t all_flags = 0;
    int all_blocks = 1;
    for (int wv = 0; wv < (int)(blockDim.x >> 6); ++wv) {
        all_flags |= (uint32_t)lds_fold[wv] >> 8;
        all_blocks = max(all_blocks, lds_fold[wv] & 0xFF);
    }
    if (!(all_flags & 4u)) return kRoundWalk16;
    if (!(all_flags & 2u)) return kRoundWalk4;
    if (!(all_flags & 1u)) return all_blocks;
    return 0;
}

template <typename T, bool POS, int QM>
__device__ __forceinline__ void pipelined_walk(const rmsn_desc* d, int32_t count, float eps,
                                               uint64_t pos, const PosArgs& pa,
                                               float (*lds8)[4]) {
    const int g = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const uint32_t lane_off =
        (uint32_t)((lane >> 4) * 256 + g * 64 + (lane & 15) * 4) * (uint32_t)sizeof(T);
    PipeBuf<T, QM> a, b;
    PipeRow cur = pipe_row_of<T, POS>(pipe_desc(d, 0, count), true, pos, pa);
    pipe_issue<T, QM>(a, cur, lane_off);
    // QM stores to an empty range (dropped by the range check): every row's
    // loads are then followed by the same QM stores, at the loop's entry as on
    // its back edge, so the compiler's wait for a row never covers the
    // previous row's stores.
    const brsrc none = row_rsrc(pipe_desc(d, 0, count).y, 0u);
#pragma unroll
    for (int m = 0; m < QM; ++m)
        PipeQuad<T>::store(typename PipeQuad<T>::raw{}, none, pipe_off<T>(lane_off, m));
    rmsn_desc ahead = pipe_desc(d, 1, count);  // descriptors are read one row ahead
    // Scheduling barriers keep each row's reduction below the next row's load
    // issue: the reduction waits for its own loads only.
    for (int32_t i = 0;;) {
        // row i is in a; row i + 1's loads go into b before row i is reduced
        PipeRow nxt = pipe_row_of<T, POS>(ahead, i + 1 < count, pos, pa);
        pipe_issue<T, QM>(b, nxt, lane_off);
        ahead = pipe_desc(d, i + 2, count);
        __builtin_amdgcn_sched_barrier(0);
        pipe_compute<T, QM>(a, cur, lane_off, eps, lds8[0], g, lane);
        __builtin_amdgcn_sched_barrier(0);
        if (++i >= count) break;
        cur = nxt;
        nxt = pipe_row_of<T, POS>(ahead, i + 1 < count, pos, pa);
        pipe_issue<T, QM>(a, nxt, lane_off);
        ahead = pipe_desc(d, i + 2, count);
        __builtin_amdgcn_sched_barrier(0);
        pipe_compute<T, QM>(b, cur, lane_off, eps, lds8[1], g, lane);
        __builtin_amdgcn_sched_barrier(0);
        if (++i >= count) break;
        cur = nxt;
    }
}

template <typename T, bool POS>
__device__ __forceinline__ void serial_walk(const rmsn_desc* d, int32_t count, float eps,
                                            uint64_t pos, const PosArgs& pa, float* lds4) {
    uint64_t unused;
    rmsn_desc next = desc_load<false>(d, pa, &unused);
    for (int32_t i = 0; i < count; ++i) {
        const rmsn_desc cur = next;
        if (i + 1 < count) next = desc_load<false>(d + i + 1, pa, &unused);
        const T* x;
        const T* w;
        T* y;
        persistent_ptrs<T, POS>(cur, pos, pa, x, w, y);
        persistent_row<T>(x, w, y, cur.n, eps, lds4);
        __syncthreads();  // this row's stores before the next row's loads; lds4 reused
    }
}

// --- Free rows over many workgroups. A row whose reads and output meet no
// other row's output, and whose output meets no other row's reads, can run at
// any time, in any workgroup: the order of the table cannot be observed on it.
// With more than one workgroup launched (tables of at most kSpanRows rows; a
// positioned table's rows taken at its position), workgroups W..G-1 take such
// "free" rows (row j in workgroup W + j mod (G-W)), while the first W
// workgroups (the walkers) run the others ("bound" rows) in table order. The
// bound rows fall into components, groups of rows that meet one another
// directly or through other rows; rows of different components share no
// memory, so each component only needs its own order, and the walkers take
// whole components each. Every workgroup decides from the same descriptors
// by the same rules, so every row is run exactly once; no workgroup waits for
// another.

struct RowSpan {
    uintptr_t x, w, y, len;  // addresses and byte length; 0 for a width the kernels skip
};

template <typename T, bool POS>
__device__ __forceinline__ RowSpan row_span(const rmsn_desc& dj, uint64_t pos, const PosArgs& pa) {
    const T* x;
    const T* w;
    T* y;
    persistent_ptrs<T, POS>(dj, pos, pa, x, w, y);  // the row where it is taken at this position
    const bool valid = dj.n >= 1 && dj.n <= RMSN_MAX_N;
    return RowSpan{reinterpret_cast<uintptr_t>(x), reinterpret_cast<uintptr_t>(w),
                   reinterpret_cast<uintptr_t>(y),
                   valid ? (uintptr_t)dj.n * sizeof(T) : (uintptr_t)0};
}

// Rows a and b (both non-empty) meet: one reads or writes memory the other
// writes. Branch-free (bitwise operators): a few compares on one LDS load of
// each row, not a chain of branches each waiting for its own load.
__device__ __forceinline__ bool rows_meet(const RowSpan& a, const RowSpan& b) {
    const uintptr_t ae = a.len, be = b.len;
    const bool xb = (a.x < b.y + be) & (b.y < a.x + ae);   // a reads b's output (x)
    const bool wb = (a.w < b.y + be) & (b.y < a.w + ae);   // a reads b's output (w)
    const bool yy = (a.y < b.y + be) & (b.y < a.y + ae);   // outputs overlap
    const bool xa = (b.x < a.y + ae) & (a.y < b.x + be);   // b reads a's output (x)
    const bool wa = (b.w < a.y + ae) & (a.y < b.w + be);   // b reads a's output (w)
    return (ae != 0) & (be != 0) & (xb | wb | yy | xa | wa);
}

// The same rows as 32-bit offsets from the table's lowest address with their
// ends, when every row lies within 4 GB of it (as rows from one allocator
// do): the test is then ten 32-bit compares. A row the kernels skip is all
// 0xFFFFFFFF, which meets nothing.
struct RowSpan32 {
    uint32_t x, xe, w, we, y, ye;
};

__device__ __forceinline__ RowSpan32 row_span32(const RowSpan& r, uintptr_t base) {
    if (r.len == 0) return RowSpan32{~0u, ~0u, ~0u, ~0u, ~0u, ~0u};
    const uint32_t x = (uint32_t)(r.x - base), w = (uint32_t)(r.w - base);
    const uint32_t y = (uint32_t)(r.y - base), l = (uint32_t)r.len;
    return RowSpan32{x, x + l, w, w + l, y, y + l};
}

// Row a's w range meets row b's output.
__device__ __forceinline__ bool w_meets_output(const RowSpan& a, const RowSpan& b) {
    return (a.len != 0) & (b.len != 0) & (a.w < b.y + b.len) & (b.y < a.w + a.len);
}
__device__ __forceinline__ bool w_meets_output(const RowSpan32& a, const RowSpan32& b) {
    return (a.w < b.ye) & (b.y < a.we);
}

__device__ __forceinline__ bool rows_meet(const RowSpan32& a, const RowSpan32& b) {
    return ((a.x < b.ye) & (b.y < a.xe)) | ((a.w < b.ye) & (b.y < a.we)) |
           ((a.y < b.ye) & (b.y < a.ye)) | ((b.x < a.ye) & (a.y < b.xe)) |
           ((b.w < a.ye) & (a.y < b.we));
}

// Whether two ranges that meet start a multiple of the run walk's period
// apart (1024 elements: `pmask` is its byte length less one), so that each
// address of both is taken by the same thread of that walk.
__device__ __forceinline__ bool off_period(uintptr_t a, uintptr_t b, uint32_t pmask) {
    return ((uint32_t)(a - b) & pmask) != 0;
}

// Rows a and b meet (rows_meet) at some pair of ranges whose starts are not a
// multiple of the period apart.
__device__ __forceinline__ bool rows_meet_off(const RowSpan& a, const RowSpan& b, uint32_t pmask) {
    const uintptr_t ae = a.len, be = b.len;
    const bool xb = (a.x < b.y + be) & (b.y < a.x + ae) & off_period(a.x, b.y, pmask);
    const bool wb = (a.w < b.y + be) & (b.y < a.w + ae) & off_period(a.w, b.y, pmask);
    const bool yy = (a.y < b.y + be) & (b.y < a.y + ae) & off_period(a.y, b.y, pmask);
    const bool xa = (b.x < a.y + ae) & (a.y < b.x + be) & off_period(b.x, a.y, pmask);
    const bool wa = (b.w < a.y + ae) & (a.y < b.w + be) & off_period(b.w, a.y, pmask);
    return (ae != 0) & (be != 0) & (xb | wb | yy | xa | wa);
}
__device__ __forceinline__ bool rows_meet_off(const RowSpan32& a, const RowSpan32& b,
                                              uint32_t pmask) {
    const bool xb = (a.x < b.ye) & (b.y < a.xe) & off_period(a.x, b.y, pmask);
    const bool wb = (a.w < b.ye) & (b.y < a.we) & off_period(a.w, b.y, pmask);
    const bool yy = (a.y < b.ye) & (b.y < a.ye) & off_period(a.y, b.y, pmask);
    const bool xa = (b.x < a.ye) & (a.y < b.xe) & off_period(b.x, a.y, pmask);
    const bool wa = (b.w < a.ye) & (a.y < b.we) & off_period(b.w, a.y, pmask);
    return xb | wb | yy | xa | wa;
}

// What the run walk reads of a span: byte length, addresses (the 32-bit
// offsets are from `base`), and the tests it makes against the row before.
__device__ __forceinline__ uint32_t span_bytes(const RowSpan& s) { return (uint32_t)s.len; }
__device__ __forceinline__ uint32_t span_bytes(const RowSpan32& s) { return s.xe - s.x; }
__device__ __forceinline__ void span_addrs(const RowSpan& s, uintptr_t, uintptr_t& x,
                                           uintptr_t& w, uintptr_t& y) {
    x = s.x;
    w = s.w;
    y = s.y;
}
__device__ __forceinline__ void span_addrs(const RowSpan32& s, uintptr_t base, uintptr_t& x,
                                           uintptr_t& w, uintptr_t& y) {
    x = base + s.x;
    w = base + s.w;
    y = base + s.y;
}
__device__ __forceinline__ bool x_meets_output(const RowSpan& a, const RowSpan& b) {
    return (a.len != 0) & (b.len != 0) & (a.x < b.y + b.len) & (b.y < a.x + a.len);
}
__device__ __forceinline__ bool x_meets_output(const RowSpan32& a, const RowSpan32& b) {
    return (a.x < b.ye) & (b.y < a.xe);
}
// a's x is exactly b's output
__device__ __forceinline__ bool x_is_output(const RowSpan& a, const RowSpan& b) {
    return a.len != 0 && a.x == b.y && a.len == b.len;
}
__device__ __forceinline__ bool x_is_output(const RowSpan32& a, const RowSpan32& b) {
    return a.x == b.y && a.xe == b.ye;
}
// a's w meets its own output at other than the same addresses
__device__ __forceinline__ bool w_off_own(const RowSpan& a, uint32_t pmask) {
    return (a.len != 0) & (a.w < a.y + a.len) & (a.y < a.w + a.len) & off_period(a.w, a.y, pmask);
}
__device__ __forceinline__ bool w_off_own(const RowSpan32& a, uint32_t pmask) {
    return (a.w < a.ye) & (a.y < a.we) & off_period(a.w, a.y, pmask);
}

// True in every thread when p holds in any thread of the workgroup (a ballot
// per wavefront, one LDS word each, one barrier; the answer is read into a
// scalar register). fold4 is free again when it returns.
__device__ __forceinline__ bool workgroup_any(bool p, int* fold4) {
    const int wave_any = __ballot(p) != 0;  // every lane takes part in the ballot
    if ((threadIdx.x & 63) == 0) fold4[threadIdx.x >> 6] = wave_any;
    __syncthreads();
    const int any = fold4[0] | fold4[1] | fold4[2] | fold4[3];
    __syncthreads();
    return __builtin_amdgcn_readfirstlane(any) != 0;
}

// Bit 0: a holds in some thread of the workgroup; bit 1: b does. As
// workgroup_any, one barrier to publish and one to free fold4.
__device__ __forceinline__ int workgroup_any2(bool a, bool b, int* fold4) {
    const int wave_any = (__ballot(a) != 0 ? 1 : 0) | (__ballot(b) != 0 ? 2 : 0);
    if ((threadIdx.x & 63) == 0) fold4[threadIdx.x >> 6] = wave_any;
    __syncthreads();
    const int any = fold4[0] | fold4[1] | fold4[2] | fold4[3];
    __syncthreads();
    return __builtin_amdgcn_readfirstlane(any);
}

// One row, its pointers taken from the descriptor (a wave-uniform load), not
// from the LDS copy used for the overlap tests.
template <typename T, bool POS>
__device__ __forceinline__ void spread_row(const rmsn_desc& dj, uint64_t pos, const PosArgs& pa,
                                           float eps, float* lds4) {
    const T* x;
    const T* w;
    T* y;
    persistent_ptrs<T, POS>(dj, pos, pa, x, w, y);
    persistent_row<T>(x, w, y, dj.n, eps, lds4);
}

// Which rows meet another one (rows_meet), found without testing every pair
// when the outputs are disjoint: the outputs are put in order of start
// address, and they are disjoint exactly when each one ends at or before the
// next one starts. Their ends are then in order as well, so for each x or w
// range the first output ending past its start is found by binary search, and
// the outputs meeting the range are that one and those after it that start
// before the range ends; both rows of every such pair (the row's own output,
// in place, aside) are bound. With disjoint outputs no other pair meets. The
// order is a rank sort of the unique keys start * 2^16 + row (quarter_ranks:
// each quarter ranked within itself, then merged by binary searches).
// Returns kNoneBound, kBoundMarked (bound[j] is 1
// exactly for the bound rows), or kBoundUnknown when outputs overlap or lie
// past 2^48 (beyond the key): the all-pairs test then decides.
// mine[r] is row threadIdx.x + 256 r. Every thread gets the same answer.
// Each meeting pair found is added to the edge list, and both its rows are
// marked in el.off when the ranges' starts are not a multiple of the run
// walk's period apart (off_period).
constexpr int kNoneBound = 0, kBoundMarked = 1, kBoundUnknown = 2;

// Ranks of the keys o_key[0..count) (unique), in two steps so that no lane
// compares its keys with all count of them: wavefront v ranks the keys of
// rows [v q, v q + n_v) (q = ceil(count / 4)) among themselves, each lane
// holding RE of them and reading the others as LDS broadcasts, and writes them
// in order into its quarter of `sorted` (P slots, the rest padded with the
// largest key); after a barrier each key's rank is its rank in its own
// quarter plus the keys below it in each other quarter, found by three
// branch-free binary searches side by side. rank_of[j] is row j's rank. P is
// a power of two, at least q.
template <int RE>
__device__ __forceinline__ void quarter_ranks(const uint64_t* o_key, int32_t count, int32_t q,
                                              int32_t P, uint64_t* sorted, uint16_t* rank_of) {
    const int32_t v = (int32_t)(threadIdx.x >> 6), lane = (int32_t)(threadIdx.x & 63);
    const int32_t q0 = v * q, qn = max(0, min(q, count - q0));
    uint64_t key[RE];
    int32_t rank[RE];
#pragma unroll
    for (int i = 0; i < RE; ++i) {
        key[i] = lane + 64 * i < qn ? o_key[q0 + lane + 64 * i] : ~0ull;
        rank[i] = 0;
    }
#pragma unroll 8
    for (int32_t t = 0; t < qn; ++t) {
        const uint64_t kk = o_key[q0 + t];  // the same word in every lane
#pragma unroll
        for (int i = 0; i < RE; ++i) rank[i] += kk < key[i] ? 1 : 0;
    }
#pragma unroll
    for (int i = 0; i < RE; ++i) {
        const int32_t idx = lane + 64 * i;
        if (idx < qn) sorted[v * P + rank[i]] = key[i];
        else if (idx < P) sorted[v * P + idx] = ~0ull;  // padding sorts after every key
    }
    for (int32_t idx = lane + 64 * RE; idx < P; idx += 64) sorted[v * P + idx] = ~0ull;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < RE; ++i) {
        // the other three quarters (this one's count is rank[i] already)
        int32_t at[3] = {0, 0, 0};  // keys below key[i] in each, before the last step
        for (int32_t step = P >> 1; step > 0; step >>= 1) {
#pragma unroll
            for (int u = 0; u < 3; ++u) {
                const int32_t b = ((v + 1 + u) & 3) * P;
                at[u] += sorted[b + at[u] + step - 1] < key[i] ? step : 0;
            }
        }
        int32_t total = rank[i];
#pragma unroll
        for (int u = 0; u < 3; ++u)
            total += at[u] + (sorted[((v + 1 + u) & 3) * P + at[u]] < key[i] ? 1 : 0);
        if (lane + 64 * i < qn) rank_of[q0 + lane + 64 * i] = (uint16_t)total;
    }
    __syncthreads();
}

// Pairs of rows that meet, for the components of the bound rows: (j << 16) | k,
// at most kMaxEdges of them (a count past it means the list is incomplete).
constexpr int kMaxEdges = 2048;

struct EdgeList {
    uint32_t* e;
    uint32_t* n;  // pairs appended (may pass kMaxEdges)
    uint8_t* off; // off[j]: row j meets a row at ranges whose starts are not a period apart
};

__device__ __forceinline__ void add_edge(const EdgeList& el, int32_t j, int32_t k) {
    const uint32_t at = atomicAdd(el.n, 1u);
    if (at < (uint32_t)kMaxEdges) el.e[at] = ((uint32_t)j << 16) | (uint32_t)k;
}

// The outputs that the x and w ranges of this thread's first RA rows meet,
// from the outputs in order of start (o_start, o_end, o_row: m slots, past
// count padded): every lane's 2 RA searches side by side, a branch-free lower
// bound with the same log2(m) steps for all, so their LDS reads are in flight
// together; then the outputs from the first one ending past the range's
// start to the last one starting before its end. Marks both rows of every
// such pair bound (the row's own output, in place, aside), adds the pair to
// the edge list and marks it in el.off when the starts are not a period
// apart. True when this thread found a pair.
template <int RA, int R>
__device__ __forceinline__ bool ranges_meeting_outputs(const RowSpan (&mine)[R], int32_t count,
                                                       int32_t m, const uint64_t* o_start,
                                                       const uint64_t* o_end,
                                                       const uint16_t* o_row, uint8_t* bound,
                                                       uint32_t pmask, const EdgeList& el) {
    constexpr int NQ = 2 * RA;
    uint64_t lo[NQ], hi[NQ];
    int32_t at[NQ];
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
        const RowSpan& rs = mine[i >> 1];
        lo[i] = (i & 1) ? (uint64_t)rs.w : (uint64_t)rs.x;
        hi[i] = lo[i] + rs.len;
        at[i] = 0;  // every output before at[i] ends at or before lo[i]
    }
    for (int32_t step = m >> 1; step > 0; step >>= 1) {
#pragma unroll
        for (int i = 0; i < NQ; ++i) at[i] += o_end[at[i] + step - 1] <= lo[i] ? step : 0;
    }
    bool meet = false;
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
        const int32_t j = threadIdx.x + 256 * (i >> 1);
        if (j >= count || mine[i >> 1].len == 0) continue;
        int32_t p = at[i] + (o_end[at[i]] <= lo[i] ? 1 : 0);  // first output ending past lo[i]
        for (; p < m && o_start[p] < hi[i]; ++p) {
            const int32_t o = o_row[p];
            if (o == j) continue;
            meet = true;
            bound[j] = 1;  // every writer stores the same value
            bound[o] = 1;
            add_edge(el, j, o);
            if (off_period(lo[i], o_start[p], pmask)) el.off[j] = el.off[o] = 1;
        }
    }
    return meet;
}

template <int R>
__device__ __forceinline__ int find_bound_rows(const RowSpan (&mine)[R], int32_t count,
                                               uint8_t* bound, int* fold4, uint32_t pmask,
                                               const EdgeList& el) {
    __shared__ uint64_t o_key[kSpanRows], o_start[kSpanRows], o_end[kSpanRows];
    __shared__ uint16_t o_row[kSpanRows];
    constexpr uint64_t kNoOutput = 0xFFFFFFFFFFFFull;  // the key's start for an empty row
    int32_t m = 2;
    while (m < count) m <<= 1;
    uint64_t key[R];
    int32_t rank[R];
    bool high = false;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int32_t j = threadIdx.x + 256 * r;
        const bool out = j < count && mine[r].len != 0;  // an empty row writes nothing
        high |= out && ((uint64_t)(mine[r].y + mine[r].len) >> 48) != 0;
        key[r] = ((out ? (uint64_t)mine[r].y : kNoOutput) << 16) | (uint64_t)j;
        rank[r] = 0;
        if (j < count) o_key[j] = key[r];
    }
    __syncthreads();  // o_key published
    {
        // the quarters' sorted keys go where the ordered starts are written
        // next (their last reads come before quarter_ranks' last barrier)
        __shared__ uint16_t rank_of[kSpanRows];
        const int32_t q = (count + 3) >> 2;
        int32_t P = 1;
        while (P < q) P <<= 1;
        switch ((q + 63) >> 6) {
            case 1: quarter_ranks<1>(o_key, count, q, P, o_start, rank_of); break;
            case 2: quarter_ranks<2>(o_key, count, q, P, o_start, rank_of); break;
            case 3: quarter_ranks<3>(o_key, count, q, P, o_start, rank_of); break;
            default: quarter_ranks<4>(o_key, count, q, P, o_start, rank_of); break;
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int32_t j = threadIdx.x + 256 * r;
            rank[r] = j < count ? (int32_t)rank_of[j] : 0;
        }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int32_t j = threadIdx.x + 256 * r;
        if (j >= m) continue;
        const bool out = j < count && mine[r].len != 0;
        const int32_t p = j < count ? rank[r] : j;  // padding sorts after every row
        o_start[p] = out ? (uint64_t)mine[r].y : ~0ull;
        o_end[p] = out ? (uint64_t)(mine[r].y + mine[r].len) : ~0ull;
        o_row[p] = (uint16_t)j;
    }
    for (int32_t j = threadIdx.x; j < count; j += 256) bound[j] = el.off[j] = 0;
    if (threadIdx.x == 0) *el.n = 0u;
    __syncthreads();
    // keys past 2^48 or overlapping outputs leave the answer unknown; the
    // searches below still stay in bounds (the ranks are a permutation), and
    // the all-pairs marking then rewrites every mark they made
    bool unknown = high;
    for (int32_t i = threadIdx.x; i + 1 < m; i += 256)
        unknown |= (o_start[i + 1] != ~0ull) & (o_end[i] > o_start[i + 1]);
    bool meet = false;
    switch ((count + 255) >> 8) {
        case 1: meet = ranges_meeting_outputs<1>(mine, count, m, o_start, o_end, o_row, bound, pmask, el); break;
        case 2: meet = ranges_meeting_outputs<2>(mine, count, m, o_start, o_end, o_row, bound, pmask, el); break;
        case 3: meet = ranges_meeting_outputs<3>(mine, count, m, o_start, o_end, o_row, bound, pmask, el); break;
        default: meet = ranges_meeting_outputs<4>(mine, count, m, o_start, o_end, o_row, bound, pmask, el); break;
    }
    // the barriers inside also publish bound[], the pairs and the marks
    const int any = workgroup_any2(unknown, meet, fold4);
    return (any & 1) ? kBoundUnknown : (any & 2) ? kBoundMarked : kNoneBound;
}

// --- Dependency walk: the bound rows in table order on four wavefronts,
// each row waiting only for the rows it depends on. Rows are the walk list
// lst[0..nb) (table indices). For each, dep is the latest earlier row of the
// list it meets (rows_meet: either reads what the other writes, or both write
// the same memory), found among the kDagWindow rows before it; if none of
// those meets it, every row before the window counts as a dependency. dep_w is
// the same for the earlier outputs that meet its w alone. Wavefront v takes
// list entries v, v + 4, ... in order, and next[v] is the entry it is on (past
// its last one when done): all entries up to d are complete exactly when every
// other wavefront's next is past d. A row issues its w loads once dep_w is
// complete, its x loads once dep is complete, then sums, applies and stores,
// waits for its stores and moves next[v] on. The wavefront holding the lowest
// pending entry always finds its dependencies complete, so the walk never
// stalls; every wait is still bounded by `cap` polls, after which the walk
// stops waiting (abort), counts the timeout in g_walk_timeouts and finishes
// its rows unordered. Every row is a whole number of 16-byte vectors, at most
// 8192 elements, 16-byte aligned (the round walk's one-wavefront rows).
constexpr int kDagWindow = 64;
constexpr uint32_t kDagSpinCap = 1u << 22;

__device__ unsigned int g_walk_timeouts;

// Wait until every list entry up to dep is complete (see above); false when
// the wait ran out of polls (the walk then aborts its ordering).
__device__ __forceinline__ bool dag_wait(const int* next, int* abort, int wave, int dep,
                                         uint32_t cap) {
    if (dep < 0) return true;
    for (uint32_t spin = 0;; ++spin) {
        const bool ok = __hip_atomic_load(abort, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) != 0;
        bool all = true;
#pragma unroll
        for (int v = 0; v < 4; ++v)
            all &= (v == wave) |
                   (__hip_atomic_load(next + v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) > dep);
        if (__builtin_amdgcn_readfirstlane((int)(ok | all))) break;
        if (spin >= cap) {
            if ((threadIdx.x & 63) == 0) {
                __hip_atomic_store(abort, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                __hip_atomic_fetch_add(&g_walk_timeouts, 1u, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
            }
            return false;
        }
        __builtin_amdgcn_s_sleep(1);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");  // the rows' stores before our loads
    return true;
}

template <typename T, int U, bool EXACT>
__device__ __forceinline__ void dag_row_slices(const T* x, const T* w, T* y, int n, float eps,
                                               int lane, const int* next, int* abort, int wave,
                                               int dep_w, int dep, uint32_t cap) {
    const uint32_t nvec = (uint32_t)n * (uint32_t)sizeof(T) / 16u;
    SplitPart<T, U, EXACT, false> part;
    dag_wait(next, abort, wave, dep_w, cap);
    part.load_w(scalar_gptr(reinterpret_cast<const char*>(w)), 0, lane, nvec);
    dag_wait(next, abort, wave, dep, cap);
    part.load_x(scalar_gptr(reinterpret_cast<const char*>(x)), 0, lane, nvec);
    float p[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    part.chains(p, nvec);
    const float inv = inverse_rms(split_sumsq(p, lane, T()), n, eps);
    part.apply(inv, scalar_gptr(reinterpret_cast<char*>(y)), 0, lane, nvec);
}

// One row of the dependency walk (the round walk's one-wavefront layout).
template <typename T>
__device__ __forceinline__ void dag_row(const T* x, const T* w, T* y, int n, float eps, int lane,
                                        const int* next, int* abort, int wave, int dep_w,
                                        int dep, uint32_t cap) {
    const int bytes = n * (int)sizeof(T);
    const int slices = (bytes + 1023) >> 10;
#define RMSN_CASE(U)                                                                          \
    if constexpr (U * 1024 <= 8192 * (int)sizeof(T)) {                                        \
        if (slices <= U) {                                                                    \
            if (bytes == U * 1024)                                                            \
                dag_row_slices<T, U, true>(x, w, y, n, eps, lane, next, abort, wave, dep_w,   \
                                           dep, cap);                                         \
            else                                                                              \
                dag_row_slices<T, U, false>(x, w, y, n, eps, lane, next, abort, wave, dep_w,  \
                                            dep, cap);                                        \
            return;                                                                           \
        }                                                                                     \
    }
    RMSN_FOR_ROUND_SLICES(RMSN_CASE)
#undef RMSN_CASE
}

template <typename T, bool POS, typename S>
__device__ __forceinline__ void dag_walk(const S* span, const uint16_t* lst, int32_t nb,
                                         const rmsn_desc* d, float eps, uint64_t pos,
                                         const PosArgs& pa, uint32_t cap) {
    __shared__ int16_t dep[kSpanRows], dep_w[kSpanRows];
    __shared__ int next[4];
    __shared__ int abort;
    for (int32_t i = threadIdx.x; i < nb; i += blockDim.x) {
        const S a = span[lst[i]];
        const int32_t lo = max(0, i - kDagWindow);
        int32_t da = -1, dw = -1;
        for (int32_t k = i - 1; k >= lo; --k) {
            const S b = span[lst[k]];
            if (da < 0 && rows_meet(a, b)) da = k;
            if (w_meets_output(a, b)) {
                dw = k;  // meeting w is meeting: da is set too
                break;
            }
        }
        dep[i] = (int16_t)(da >= 0 ? da : lo - 1);
        dep_w[i] = (int16_t)(dw >= 0 ? dw : lo - 1);
    }
    if (threadIdx.x < 4) next[threadIdx.x] = (int)threadIdx.x;
    if (threadIdx.x == 0) abort = 0;
    __syncthreads();
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int lane = threadIdx.x & 63;
    for (int32_t i = wave; i < nb; i += 4) {
        const rmsn_desc dd = d[lst[i]];
        const T* x;
        const T* w;
        T* y;
        persistent_ptrs<T, POS>(dd, pos, pa, x, w, y);
        dag_row<T>(x, w, y, (int)dd.n, eps, lane, next, &abort, wave, dep_w[i], dep[i], cap);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");  // our stores before the mark
        if (lane == 0)
            __hip_atomic_store(next + wave, (int)(i + 4), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    if (lane == 0)
        __hip_atomic_store(next + wave, 0x7FFFFFFF, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// --- Run walk: the bound rows in table order, each one shared by the four
// wavefronts in the pipelined walk's mapping, so that element e of every row
// is taken by the same thread (the one for e mod 1024). It is chosen when
// every pair of rows that meet, meets at ranges whose starts are a multiple
// of 1024 elements apart: each address is then read and written by one
// thread only, whichever row touches it, and a thread's own loads and stores
// to one address take effect in program order, so the table's order holds
// with no wait between threads. For the same reason a row's own w may meet
// its output only at the same addresses; its x may meet it anywhere (every
// thread has its x before the row's barrier, and the stores come after it).
//  - Each row's stored values stay in registers until the next row is done.
//    When entry j's x is exactly entry j - 1's output (same range), those
//    values are its x ("forwarded") and x is not loaded.
//  - Entry j is "ahead" when its w, and its x unless forwarded, meet none of
//    the outputs of the kRunDepth entries before it: its loads may be issued
//    before those entries store.
//  - A run is a stretch of entries each ahead but the first. At the start of
//    a run (after every store before it) the loads of its first kRunDepth
//    entries are issued; while entry i is reduced, entry i + kRunDepth's loads
//    are in flight, issued before entry i + 1 stores. An entry that is not
//    ahead starts a new run.
//  - A stretch of at least kFwdRun consecutive entries, each ahead and
//    forwarded from the entry just before, is a run of its own (a "forward
//    run", as a chain of rows each reading the one before): it loads w only.
//    Other runs issue x and w loads for every entry (x over an empty range
//    when forwarded), so that each loop issues the same instructions on
//    every pass and the compiler's waits stay exact.
// A later row's stores over what an earlier row c reads are ordered by the
// rows' barriers: every thread has used its loads of row c before it
// reaches row c + 1's barrier, and each row stores after its own barrier.
// Every row has the walk's block count QM (lanes past the row take empty
// ranges, as in the pipelined walk), 1 <= n <= 8192, n a multiple of 4,
// pointers quad-aligned. No thread waits for a flag: the only waits are the
// rows' barriers, which every thread reaches in the same order.
constexpr int kRunDepth = 2;  // entries whose loads are in flight beyond the one reduced
constexpr int kFwdRun = 4;    // shortest forward run
// entry flags: ahead, deep (loads kRunDepth entries early), forwarded, in a
// forward run, continues the run of the entry before
constexpr uint8_t kRunAhead = 1, kRunDeep = 2, kRunFwd = 4, kRunFwdRun = 8, kRunCont = 16;

// Buffer resources of list entry i (the last entry's bases with empty ranges
// past the end); x and w get their range only when `what` asks for them
// (bit 0: x, bit 1: w).
template <typename T, typename S>
__device__ __forceinline__ PipeRow run_row(const S* span, const uint16_t* lst, int32_t i,
                                           int32_t nb, uintptr_t base, unsigned what) {
    const bool real = i < nb;
    const S s = span[lst[real ? i : nb - 1]];
    uintptr_t x, w, y;
    span_addrs(s, base, x, w, y);
    const uint32_t bytes = real ? __builtin_amdgcn_readfirstlane(span_bytes(s)) : 0u;
    // the addresses come from LDS: wave-uniform values, taken into scalar registers
    const auto sp = [](uintptr_t p) {
        return reinterpret_cast<const void*>(
            reinterpret_cast<uint64_t>(scalar_gptr(reinterpret_cast<const void*>(p))));
    };
    return PipeRow{row_rsrc(sp(x), (what & 1u) ? bytes : 0u), row_rsrc(sp(w), (what & 2u) ? bytes : 0u),
                   row_rsrc(sp(y), bytes), (int)(bytes / (uint32_t)sizeof(T))};
}

// The loads entry i takes (w, and x unless forwarded), or none when `issue`
// is false or the list has ended.
__device__ __forceinline__ unsigned run_loads(const uint8_t* flag, int32_t i, int32_t nb,
                                              bool issue) {
    if (!issue || i >= nb) return 0u;
    return (flag[i] & kRunFwd) ? 2u : 3u;
}

template <typename T, int QM>
struct RunPrev {
    typename PipeQuad<T>::raw v[QM];  // the stored values of the row just done
};

// Row r: x from buffer b, or the stored values of the row just before when
// forwarded (FWD: always, and b holds w only); reduce, apply, store; prev
// then holds this row's stored values.
template <bool FWD, typename T, int QM>
__device__ __forceinline__ void run_compute(PipeBuf<T, QM>& b, const PipeRow& r, bool fwd,
                                            RunPrev<T, QM>& prev, uint32_t lane_off, float eps,
                                            float* lds4, int g, int lane) {
    typedef typename PipeQuad<T>::raw raw;
    raw x[QM];
    if (FWD || fwd) {
        const uint32_t bytes = (uint32_t)r.n * (uint32_t)sizeof(T);
#pragma unroll
        for (int m = 0; m < QM; ++m)  // lanes past the row load zeros
            x[m] = pipe_off<T>(lane_off, m) < bytes ? prev.v[m] : raw{};
    } else {
#pragma unroll
        for (int m = 0; m < QM; ++m) x[m] = b.x[m];
    }
    float p = 0.0f;
#pragma unroll
    for (int m = 0; m < QM; ++m) {
        float v[4];
        PipeQuad<T>::unpack(x[m], v);
        transpose4(v);
        p = fmaf(v[0], v[0], p);  // chunks 4m .. 4m+3 of chain 64g + 4t + q
        p = fmaf(v[1], v[1], p);
        p = fmaf(v[2], v[2], p);
        p = fmaf(v[3], v[3], p);
    }
    const float gt = group_sumsq(p);
    if (lane == 0) lds4[g] = gt;
    lds_barrier();
    const float inv = inverse_rms((lds4[0] + lds4[2]) + (lds4[1] + lds4[3]), r.n, eps);
#pragma unroll
    for (int m = 0; m < QM; ++m) {
        prev.v[m] = PipeQuad<T>::apply(x[m], b.w[m], inv);
        PipeQuad<T>::store(prev.v[m], r.y, pipe_off<T>(lane_off, m));
    }
}

// Steps P, P + 1, ... NB - 1 of the unrolled run loop, each with its buffer
// index fixed at compile time; false as soon as one ends the run.
template <int P, int NB>
struct RunSteps {
    template <typename F>
    __device__ __forceinline__ static bool go(F& step) {
        return step(std::integral_constant<int, P>{}) && RunSteps<P + 1, NB>::go(step);
    }
};
template <int NB>
struct RunSteps<NB, NB> {
    template <typename F>
    __device__ __forceinline__ static bool go(F&) { return true; }
};

// This entry's loads into b: x (unless FWD) and w.
template <bool FWD, typename T, int QM>
__device__ __forceinline__ void run_issue(PipeBuf<T, QM>& b, const PipeRow& r, uint32_t lane_off) {
    if (!FWD) {
#pragma unroll
        for (int m = 0; m < QM; ++m) b.x[m] = PipeQuad<T>::load(r.x, pipe_off<T>(lane_off, m));
    }
#pragma unroll
    for (int m = 0; m < QM; ++m) b.w[m] = PipeQuad<T>::load(r.w, pipe_off<T>(lane_off, m));
}

// One run from entry i (its first entry), leaving i at the next run's first.
template <bool FWD, typename T, int QM, typename S>
__device__ __forceinline__ void run_one(const S* span, const uint16_t* lst, const uint8_t* flag,
                                        int32_t nb, uintptr_t base, float eps, float (*lds8)[4],
                                        RunPrev<T, QM>& prev, int32_t& i, uint32_t lane_off, int g,
                                        int lane) {
    constexpr int NB = kRunDepth + 1;  // entries i .. i + kRunDepth
    PipeBuf<T, QM> buf[NB];
    // the run's first kRunDepth entries load now (after every store before
    // them). Each entry's loads are followed by QM stores to an empty range,
    // as on the loop's back edge each entry's loads are followed by a row's
    // stores: the compiler's waits for an entry then cover that entry's loads
    // only, at the loop's entry as on its back edge.
    const PipeRow none = run_row<T, S>(span, lst, nb, nb, base, 0u);
    bool chain = true;
#pragma unroll
    for (int m = 0; m < kRunDepth; ++m) {
        chain = chain && (m == 0 || (i + m < nb && (flag[i + m] & kRunCont)));
        const unsigned what = FWD ? (chain && i + m < nb ? 2u : 0u) : run_loads(flag, i + m, nb, chain);
        run_issue<FWD, T, QM>(buf[m], run_row<T, S>(span, lst, i + m, nb, base, what), lane_off);
#pragma unroll
        for (int q = 0; q < QM; ++q)
            PipeQuad<T>::store(typename PipeQuad<T>::raw{}, none.y, pipe_off<T>(lane_off, q));
    }
    // entry i is in buf[p]; entry i + kRunDepth's loads go into the buffer
    // entry i - 1 used, when every entry up to it continues the run
    auto step = [&](auto pc) -> bool {
        constexpr int p = decltype(pc)::value;
        const uint8_t fi = __builtin_amdgcn_readfirstlane(flag[i]);
        const int32_t j = i + kRunDepth;
        const bool deep = j < nb && (flag[j] & kRunDeep);
        const unsigned what = FWD ? (deep ? 2u : 0u) : run_loads(flag, j, nb, deep);
        run_issue<FWD, T, QM>(buf[(p + kRunDepth) % NB], run_row<T, S>(span, lst, j, nb, base, what),
                              lane_off);
        const PipeRow cur = run_row<T, S>(span, lst, i, nb, base, 0u);
        __builtin_amdgcn_sched_barrier(0);
        run_compute<FWD, T, QM>(buf[p], cur, (fi & kRunFwd) != 0, prev, lane_off, eps,
                                lds8[i & 1], g, lane);
        __builtin_amdgcn_sched_barrier(0);
        ++i;
        return i < nb && (__builtin_amdgcn_readfirstlane(flag[i]) & kRunCont);
    };
    while (RunSteps<0, NB>::go(step)) {
    }
}

template <typename T, int QM, typename S>
__device__ __forceinline__ void run_walk(const S* span, const uint16_t* lst, const uint8_t* flag,
                                         int32_t nb, uintptr_t base, float eps,
                                         float (*lds8)[4]) {
    const int g = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const uint32_t lane_off =
        (uint32_t)((lane >> 4) * 256 + g * 64 + (lane & 15) * 4) * (uint32_t)sizeof(T);
    RunPrev<T, QM> prev;
#pragma unroll
    for (int m = 0; m < QM; ++m) prev.v[m] = {};
    for (int32_t i = 0; i < nb;) {
        if (__builtin_amdgcn_readfirstlane(flag[i]) & kRunFwdRun)
            run_one<true, T, QM, S>(span, lst, flag, nb, base, eps, lds8, prev, i, lane_off, g,
                                    lane);
        else
            run_one<false, T, QM, S>(span, lst, flag, nb, base, eps, lds8, prev, i, lane_off, g,
                                     lane);
    }
}

// Components of the bound rows under rows_meet, from the edge list: label[j]
// ends as the least row of j's component (rows in different components share
// no memory, so their order cannot be observed). Each round hooks, for every
// pair whose labels differ, the greater label to the lesser (labels only
// decrease and label[j] <= j, so they form a forest whose roots are the
// least rows), then every row follows its labels to their root; the rounds
// end when no pair has two labels. False when the edge list overflowed or
// kMaxRounds rounds did not settle it: the caller then keeps every bound row
// in one walk.
constexpr int kMaxRounds = 24;

__device__ __forceinline__ bool components(const EdgeList& el, int32_t count, uint32_t* label,
                                           int* fold4) {
    const uint32_t ne = *el.n;  // published by a barrier before: the same in every thread
    if (ne > (uint32_t)kMaxEdges) return false;
    for (int32_t j = threadIdx.x; j < count; j += blockDim.x) label[j] = (uint32_t)j;
    __syncthreads();
    for (int round = 0; round < kMaxRounds; ++round) {
        bool hooked = false;
        for (uint32_t e = threadIdx.x; e < ne; e += blockDim.x) {
            const uint32_t a = el.e[e] >> 16, b = el.e[e] & 0xFFFFu;
            const uint32_t la = label[a], lb = label[b];
            if (la != lb) {
                atomicMin(&label[max(la, lb)], min(la, lb));
                hooked = true;
            }
        }
        if (!workgroup_any(hooked, fold4)) return true;
        // each row follows its labels to their root; the other threads' writes
        // only shorten the way (every label is an ancestor, and decreases)
        for (int32_t j = threadIdx.x; j < count; j += blockDim.x) {
            uint32_t r = label[j];
            while (label[r] != r) r = label[r];
            label[j] = r;
        }
        __syncthreads();
    }
    return false;
}

// The free rows and the bound rows of a spread launch, on spans of type S in
// LDS (RowSpan or RowSpan32).
//  - Workers (blockIdx >= walkers) test their rows against every row, 256 at
//    a time, and run those that meet none.
//  - Every walker finds the same bound rows (marked from the ordered outputs,
//    `marked`, else by testing all pairs: wavefront v decides rows v, v + 4,
//    ..., its lanes test 64 rows at a time and a ballot gives the answer), the
//    meeting pairs among them, and from those the components. Components, in
//    order of their least row, go round-robin to the walkers; each walker
//    walks its components' rows in table order: by the run walk when they fit
//    its mapping and meet only a multiple of its period apart (no row marked
//    in el.off, no row's w meeting its own output elsewhere), else by the
//    dependency walk when every row fits the one-wavefront layout, else row
//    after row.
// Returns as spread_rows does.
constexpr uint8_t kFitVec = 1, kFitGroup = 2;  // row fits: one-wavefront layout, GROUP mapping

template <typename T, bool POS, typename S>
__device__ __forceinline__ bool spread_on(const S* span, uint8_t* bound, const uint8_t* rfit,
                                          bool marked, const EdgeList& el, uintptr_t base,
                                          const rmsn_desc* d, int32_t count, float eps,
                                          uint64_t pos, const PosArgs& pa, float* lds4,
                                          float (*lds8)[4], int* fold4, uint32_t cap) {
    const int32_t walkers = min(kWalkers, (int32_t)gridDim.x - 1);
    if ((int32_t)blockIdx.x >= walkers) {
        const int32_t workers = (int32_t)gridDim.x - walkers;
        for (int32_t j = (int32_t)blockIdx.x - walkers; j < count; j += workers) {
            const S sj = span[j];
            bool meet = false;
            for (int32_t k = threadIdx.x; k < count; k += blockDim.x)
                meet |= (k != j) & rows_meet(sj, span[k]);
            if (workgroup_any(meet, fold4)) continue;  // bound: a walker runs it in order
            spread_row<T, POS>(d[j], pos, pa, eps, lds4);
            __syncthreads();  // lds4 is reused by the next row
        }
        return true;
    }
    constexpr uint32_t pmask = 1024u * (uint32_t)sizeof(T) - 1u;
    const int32_t wave = (int32_t)(threadIdx.x >> 6), lane = (int32_t)(threadIdx.x & 63);
    for (int32_t j = marked ? count : wave; j < count; j += 4) {
        const S sj = span[j];
        bool meet = false, off = false;
#pragma unroll 4
        for (int32_t k = lane; k < count; k += 64) {
            const S sk = span[k];
            const bool m = (k != j) & rows_meet(sj, sk);
            meet |= m;
            off |= m & rows_meet_off(sj, sk, pmask);
            if (m & (k < j)) add_edge(el, j, k);
        }
        const bool any = __ballot(meet) != 0;
        const bool any_off = __ballot(off) != 0;
        if (lane == 0) {
            bound[j] = any;
            if (any_off) el.off[j] = 1;  // the pair's other row marks itself in its turn
        }
    }
    __syncthreads();
    // components, and the walker of each: rank of its least row among the
    // components' least rows, modulo the walkers
    __shared__ uint32_t label[kSpanRows];
    __shared__ uint16_t crank[kSpanRows];
    const bool split = components(el, count, label, fold4);
    if (wave == 0) {
        int32_t nc = 0;
        for (int32_t j0 = 0; j0 < count; j0 += 64) {
            const int32_t j = j0 + lane;
            const bool root = j < count && bound[j] != 0 && label[j] == (uint32_t)j;
            const unsigned long long roots = __ballot(root);
            if (root) crank[j] = (uint16_t)(nc + __builtin_popcountll(roots & ((1ull << lane) - 1ull)));
            nc += __builtin_popcountll(roots);
        }
    }
    __syncthreads();
    const auto mine = [&](int32_t j) {
        return bound[j] != 0 &&
               (split ? (int32_t)crank[label[j]] % walkers : 0) == (int32_t)blockIdx.x;
    };
    // this walker's rows in table order, 64 at a time by a ballot
    __shared__ uint16_t lst[kSpanRows];
    __shared__ uint8_t flag[kSpanRows], flag2[kSpanRows];
    __shared__ int32_t nb_shared;
    if (wave == 0) {
        int32_t nb = 0;
        for (int32_t j0 = 0; j0 < count; j0 += 64) {
            const bool b = j0 + lane < count && mine(j0 + lane);
            const unsigned long long marks = __ballot(b);
            if (b) lst[nb + __builtin_popcountll(marks & ((1ull << lane) - 1ull))] =
                (uint16_t)(j0 + lane);
            nb += __builtin_popcountll(marks);
        }
        if (lane == 0) nb_shared = nb;
    }
    __syncthreads();
    const int32_t nb = nb_shared;
    // which walk takes them, and the run walk's block count
    __shared__ int qm4[4];
    bool not_vec = false, not_group = false;
    int blocks = 1;
    for (int32_t i = threadIdx.x; i < nb; i += blockDim.x) {
        const int32_t j = lst[i];
        const S sj = span[j];
        not_vec |= !(rfit[j] & kFitVec);
        not_group |= !(rfit[j] & kFitGroup) || el.off[j] || w_off_own(sj, pmask);
        blocks = max(blocks, (int)((span_bytes(sj) / (uint32_t)sizeof(T) + 1023u) >> 10));
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) blocks = max(blocks, __shfl_xor(blocks, o, 64));
    if (lane == 0) qm4[wave] = blocks;
    const int fits = workgroup_any2(not_vec, not_group, fold4);  // its barriers publish qm4
    if (nb == 0) return true;
    if (!(fits & 2)) {
        // each entry against the kRunDepth before it: forwarded (its x is
        // exactly the output of the entry just before), ahead (w, and x
        // unless forwarded, meet none of their outputs); entry 0 starts the
        // first run
        for (int32_t i = threadIdx.x; i < nb; i += blockDim.x) {
            const S a = span[lst[i]];
            bool fwd = false, xnear = false, wnear = false;
#pragma unroll
            for (int k = 1; k <= kRunDepth; ++k) {
                if (i - k < 0) break;
                const S b = span[lst[i - k]];
                if (k == 1) fwd = x_is_output(a, b);
                xnear |= x_meets_output(a, b);
                wnear |= w_meets_output(a, b);
            }
            // a forwarded x is not loaded: whatever earlier outputs wrote
            // under it, the output just before has overwritten all of it
            xnear = fwd ? false : xnear;
            const bool ahead = i > 0 && !wnear && !xnear;
            flag[i] = (uint8_t)((ahead ? kRunAhead : 0) | (fwd ? kRunFwd : 0));
        }
        __syncthreads();
        // forward runs: stretches of at least kFwdRun entries each ahead and
        // forwarded from the entry just before (counted up to kFwdRun - 1 on
        // each side of the entry)
        const auto chained = [&](int32_t k) {
            return k > 0 && k < nb && (flag[k] & kRunAhead) && (flag[k] & kRunFwd);
        };
        for (int32_t i = threadIdx.x; i < nb; i += blockDim.x) {
            int len = 0;
            if (chained(i)) {
                len = 1;
                for (int k = 1; k < kFwdRun && chained(i - k); ++k) ++len;
                for (int k = 1; k < kFwdRun && chained(i + k); ++k) ++len;
            }
            flag2[i] = flag[i] | (len >= kFwdRun ? kRunFwdRun : 0);
        }
        __syncthreads();
        // cont: ahead and of the same kind of run as the entry before; deep:
        // this entry and the kRunDepth - 1 before it all continue the run
        const auto cont = [&](int32_t k) {
            return k > 0 && (flag2[k] & kRunAhead) &&
                   ((flag2[k] ^ flag2[k - 1]) & kRunFwdRun) == 0;
        };
        for (int32_t i = threadIdx.x; i < nb; i += blockDim.x) {
            bool deep = i >= kRunDepth;
#pragma unroll
            for (int k = 0; k < kRunDepth; ++k) deep = deep && cont(i - k);
            flag[i] = flag2[i] | (cont(i) ? kRunCont : 0) | (deep ? kRunDeep : 0);
        }
        __syncthreads();
        const int qm = max(max(qm4[0], qm4[1]), max(qm4[2], qm4[3]));
        switch (qm) {
#define RMSN_CASE(Q) \
    case Q: run_walk<T, Q, S>(span, lst, flag, nb, base, eps, lds8); break;
            RMSN_FOR_GROUP_BLOCKS(RMSN_CASE)
#undef RMSN_CASE
            default: break;
        }
        return true;
    }
    if (!(fits & 1)) {
        dag_walk<T, POS, S>(span, lst, nb, d, eps, pos, pa, cap);
        return true;
    }
    // every bound row in this walker and no row free: the ordered walks of
    // the whole table (workgroup 0 only; it is then the only walker with rows)
    if (blockIdx.x == 0 && nb == count) return false;
    // row after row, in table order
    for (int32_t i = 0; i < nb; ++i) {
        spread_row<T, POS>(d[lst[i]], pos, pa, eps, lds4);
        __syncthreads();  // this row's stores before the next row's loads
    }
    return true;
}

// Returns true when this workgroup's part of the table is done, false (in
// workgroup 0 only) when no row is free, so the ordered walk takes the whole
// table. (No row writes into the table itself: the walks read descriptors as
// they go, and this step reads them all first.)
template <typename T, bool POS>
__device__ __forceinline__ bool spread_rows(const rmsn_desc* d, int32_t count, float eps,
                                            uint64_t pos, const PosArgs& pa, float* lds4,
                                            float (*lds8)[4], int* fold4, uint32_t cap) {
    __shared__ RowSpan span[kSpanRows];   // 64-bit spans, or RowSpan32 in the same bytes
    __shared__ uint8_t bound[kSpanRows];
    __shared__ uint8_t rfit[kSpanRows];   // the layouts the row fits (kFitVec, kFitGroup)
    __shared__ unsigned long long lo_hi[2];
    constexpr int R = kSpanRows / 256;     // rows per thread (blockDim.x == 256)
    RowSpan mine[R];
    uint64_t lo = ~0ull, hi = 0ull;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int32_t j = threadIdx.x + 256 * r;
        mine[r] = j < count ? row_span<T, POS>(d[j], pos, pa) : RowSpan{0, 0, 0, 0};
        if (mine[r].len != 0) {
            lo = min(lo, (uint64_t)min(mine[r].x, min(mine[r].w, mine[r].y)));
            hi = max(hi, (uint64_t)max(mine[r].x, max(mine[r].w, mine[r].y)) + mine[r].len);
        }
    }
    __shared__ uint32_t edges[kMaxEdges], n_edges;
    __shared__ uint8_t off[kSpanRows];
    const EdgeList el{edges, &n_edges, off};
    if ((int32_t)blockIdx.x >= min(kWalkers, (int32_t)gridDim.x - 1)) {
        // a worker tests each of its rows against every row on the 64-bit spans
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int32_t j = threadIdx.x + 256 * r;
            if (j < count) span[j] = mine[r];
        }
        __syncthreads();
        return spread_on<T, POS>(static_cast<const RowSpan*>(span), bound, rfit, false, el, 0, d,
                                 count, eps, pos, pa, lds4, lds8, fold4, cap);
    }
    // no row meets another (the usual table): the workers run every row
    if (threadIdx.x == 0) {
        lo_hi[0] = ~0ull;  // published by the barriers of the search
        lo_hi[1] = 0ull;
    }
    const int found =
        find_bound_rows(mine, count, bound, fold4, 1024u * (uint32_t)sizeof(T) - 1u, el);
    if (found == kNoneBound) return true;
    // lowest and highest address: within the wavefront, then one LDS atomic each
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        lo = min(lo, (uint64_t)__shfl_xor((unsigned long long)lo, o, 64));
        hi = max(hi, (uint64_t)__shfl_xor((unsigned long long)hi, o, 64));
    }
    if ((threadIdx.x & 63) == 0) {
        atomicMin(&lo_hi[0], (unsigned long long)lo);
        atomicMax(&lo_hi[1], (unsigned long long)hi);
    }
    __syncthreads();
    const uintptr_t base = (uintptr_t)lo_hi[0];
    const bool narrow = lo_hi[1] <= lo_hi[0] || lo_hi[1] - lo_hi[0] < 0xFFFFFFFFull;
    RowSpan32* span32 = reinterpret_cast<RowSpan32*>(span);
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int32_t j = threadIdx.x + 256 * r;
        if (j >= count) continue;
        const RowSpan& m = mine[r];
        const bool in = m.len != 0 && m.len <= 8192 * sizeof(T);
        const bool vec = in && m.len % 16 == 0 && ((m.x | m.w | m.y) & 15) == 0;
        const bool quad = in && m.len % (4 * sizeof(T)) == 0 &&
                          ((m.x | m.w | m.y) & (4 * sizeof(T) - 1)) == 0;
        rfit[j] = (vec ? kFitVec : 0) | (quad ? kFitGroup : 0);
        if (narrow) span32[j] = row_span32(m, base);
        else span[j] = m;
    }
    __syncthreads();
    const bool marked = found == kBoundMarked;
    return narrow ? spread_on<T, POS>(span32, bound, rfit, marked, el, base, d, count, eps, pos,
                                      pa, lds4, lds8, fold4, cap)
                  : spread_on<T, POS>(static_cast<const RowSpan*>(span), bound, rfit, marked, el,
                                      base, d, count, eps, pos, pa, lds4, lds8, fold4, cap);
}

template <typename T, bool POS>
__global__ __launch_bounds__(256) void k_sequence_persistent(const rmsn_desc* __restrict__ d,
                                                             int32_t count, float eps,
                                                             PosArgs pa, uint32_t cap) {
    __shared__ float lds4[4];
    __shared__ float lds8[2][4];
    __shared__ int lds_fold[4];
    uint64_t pos = 0;
    if (POS) {
        const uint64_t per = (uint64_t)pa.period;
        const uint64_t raw = (uint64_t)*pa.d_pos;
        pos = raw < per ? raw : raw % per;
    }
    // the launcher gives more than one workgroup only to tables of at most
    // kSpanRows rows
    if (gridDim.x > 1 && spread_rows<T, POS>(d, count, eps, pos, pa, lds4, lds8, lds_fold, cap)) return;
    switch (walk_mode<T, POS>(d, count, pos, pa, lds_fold)) {
        case kRoundWalk16: round_walk<T, POS, 4>(d, count, eps, pos, pa); break;
        case kRoundWalk4: round_walk<T, POS, 1>(d, count, eps, pos, pa); break;
#define RMSN_CASE(Q) \
    case Q: pipelined_walk<T, POS, Q>(d, count, eps, pos, pa, lds8); break;
        RMSN_FOR_GROUP_BLOCKS(RMSN_CASE)
#undef RMSN_CASE
        default: serial_walk<T, POS>(d, count, eps, pos, pa, lds4); break;
    }
    // with more than one workgroup the launcher advances the position in a
    // launch of its own, once every workgroup has read it
    if (POS && gridDim.x == 1 && threadIdx.x == 0) {
        const uint64_t per = (uint64_t)pa.period;
        const_cast<int64_t*>(pa.d_pos)[0] = (int64_t)(pos + 1 == per ? 0 : pos + 1);
    }
}

}  // namespace

hipError_t launch_sequence_persistent(int dtype, const rmsn_desc* d, int32_t count, float eps,
                                     const PosArgs* pos, hipStream_t stream) {
    const PosArgs none{nullptr, 0, 0, 1};
    // the walkers plus one worker per row (at most kSpreadWorkers) for free rows
    const bool spread = count > 1 && count <= kSpanRows && option_persistent_workgroups() == 0;
    const dim3 grid(spread ? (unsigned)(kWalkers + std::min(count, kSpreadWorkers)) : 1u),
        block(kBlockThreads);
    const int opt_cap = option_walk_spin_cap();
    const uint32_t cap = opt_cap > 0 ? (uint32_t)opt_cap : kDagSpinCap;
    if (dtype == RMSN_F32) {
        if (pos)
            hipLaunchKernelGGL((k_sequence_persistent<float, true>), grid, block, 0, stream, d,
                               count, eps, *pos, cap);
        else
            hipLaunchKernelGGL((k_sequence_persistent<float, false>), grid, block, 0, stream, d,
                               count, eps, none, cap);
    } else {
        if (pos)
            hipLaunchKernelGGL((k_sequence_persistent<uint16_t, true>), grid, block, 0, stream, d,
                               count, eps, *pos, cap);
        else
            hipLaunchKernelGGL((k_sequence_persistent<uint16_t, false>), grid, block, 0, stream,
                               d, count, eps, none, cap);
    }
    const hipError_t e = hipGetLastError();
    // the rows of every workgroup are taken at the position read when the
    // kernel starts; it is advanced after all of them, by the next launch
    if (e != hipSuccess || !spread || pos == nullptr) return e;
    return launch_advance(const_cast<int64_t*>(pos->d_pos), pos->period, stream);
}

hipError_t walk_timeouts(uint32_t* out, bool reset) {
    hipError_t e = hipMemcpyFromSymbol(out, HIP_SYMBOL(g_walk_timeouts), sizeof(uint32_t), 0,
                                       hipMemcpyDeviceToHost);
    if (e != hipSuccess || !reset) return e;
    const uint32_t zero = 0;
    return hipMemcpyToSymbol(HIP_SYMBOL(g_walk_timeouts), &zero, sizeof zero, 0,
                             hipMemcpyHostToDevice);
}

}  // namespace rmsn
