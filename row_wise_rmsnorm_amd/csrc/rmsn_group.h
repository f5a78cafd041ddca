// rmsn_group.h -- the GROUP placement of the association's lanes, shared by the
// GROUP kernels and the wide-row kernels: wavefront g holds group g, and lane
// 16q + t of it holds association lane 64g + 4t + q. Register transposes for
// loads that cover four chunks at once, and the group tree for this placement.
#pragma once

#include "rmsn_common.h"

#pragma clang fp contract(off)

namespace rmsn {
namespace {

// Lanes 0..31 keep their own a and receive b's upper half; lanes 32..63 keep
// their own b and receive a's lower half -- as (r.first, r.second):
//   lane i < 32:  first = a[i],      second = a[i + 32]
//   lane i >= 32: first = b[i - 32], second = b[i]
struct SwapPair { uint32_t first, second; };
__device__ __forceinline__ SwapPair swap32(uint32_t a, uint32_t b) {
    const auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
    return {r[0], r[1]};
}

// One load per lane covers the group's 64 elements in four consecutive
// 256-element chunks: lane 16q + t reads elements 256(4m+q) + 64g + 4t + {0..3}
// of block m (1024 elements). A 4x4 transpose between the lane's 16-lane row
// q and its register index then leaves lane 16q + t holding chain
// 64g + 4t + q for chunks 4m .. 4m+3, in order.

// Lanes 0..15 / 32..47 keep their own a and receive b's rows 0 / 2; lanes
// 16..31 / 48..63 keep their own b and receive a's rows 1 / 3:
//   first  = a with its odd 16-lane rows replaced by b's even rows
//   second = b with its even 16-lane rows replaced by a's odd rows
__device__ __forceinline__ SwapPair swap16(uint32_t a, uint32_t b) {
    const auto r = __builtin_amdgcn_permlane16_swap(a, b, false, false);
    return {r[0], r[1]};
}

// v[e] of lane 16q + t is X[q][e] (row q, register e); afterwards v[k] of that
// lane is X[k][q].
__device__ __forceinline__ void transpose4(float v[4]) {
    const SwapPair a = swap32(__float_as_uint(v[0]), __float_as_uint(v[2]));
    const SwapPair b = swap32(__float_as_uint(v[1]), __float_as_uint(v[3]));
    // rows 0,1 of registers 2,3 moved to rows 2,3 of registers 0,1 and back
    const SwapPair c = swap16(a.first, b.first);
    const SwapPair d = swap16(a.second, b.second);
    v[0] = __uint_as_float(c.first);
    v[1] = __uint_as_float(c.second);
    v[2] = __uint_as_float(d.first);
    v[3] = __uint_as_float(d.second);
}

// Group tree of the GROUP layout: association lane 64g + 4t + q sits in lane
// 16q + t. Halving 32/16/8/4 moves t by 8/4/2/1 (DPP row shifts); halving 2
// and 1 move q by 2 and 1, i.e. lanes 0/32 and 16/48.
__device__ __forceinline__ float group_sumsq(float p) {
    p += row_shl<8>(p);
    p += row_shl<4>(p);
    p += row_shl<2>(p);
    p += row_shl<1>(p);
    return (lane_value(p, 0) + lane_value(p, 32)) + (lane_value(p, 16) + lane_value(p, 48));
}


}  // namespace
}  // namespace rmsn
