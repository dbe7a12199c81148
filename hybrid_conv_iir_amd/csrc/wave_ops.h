// Wave-wide collectives for 64-lane waves on the vector ALU: values move between
// lanes by DPP (quad permutations, row mirrors, row shifts), the gfx950 row
// swaps (v_permlane16_swap / v_permlane32_swap) and lane reads, never through the
// LDS crossbar.  The all-reduce steps pair lanes symmetrically (each pair combines
// the same two values, in either order), so a commutative operation leaves the
// same bits on every lane.  Every function must be called by all 64 lanes of the
// wave (uniform control flow): a lane outside the exec mask would supply stale
// data to its partner.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hci {

// lane i receives lane sel(i)'s v; lanes whose source lies outside their 16-lane row read 0
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
    const uint64_t b = (uint64_t)__double_as_longlong(v);
    const uint64_t lo = dpp_u32<CTRL>((uint32_t)b), hi = dpp_u32<CTRL>((uint32_t)(b >> 32));
    return __longlong_as_double((long long)((hi << 32) | lo));
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __uint_as_float(dpp_u32<CTRL>(__float_as_uint(v)));
}

constexpr int kQuadSwap1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kQuadSwap2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kHalfMirror = 0x141;    // lane i <-> 7 - i within each 8-lane half row
constexpr int kRowMirror = 0x140;     // lane i <-> 15 - i within each 16-lane row
constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;

// the pair (own, partner) for the lane of the neighbouring 16-lane row (rows 0<->1, 2<->3;
// first = rows32 ? 32-lane halves swapped); the two come back in either order
template <bool ROWS32>
__device__ __forceinline__ void swap_pair(uint32_t v, uint32_t& a, uint32_t& b) {
    if constexpr (ROWS32) {
        const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        a = r[0]; b = r[1];
    } else {
        const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        a = r[0]; b = r[1];
    }
}

template <bool ROWS32, typename Op>
__device__ __forceinline__ double swap_op_f64(double v, Op op) {
    const uint64_t x = (uint64_t)__double_as_longlong(v);
    uint32_t l0, l1, h0, h1;
    swap_pair<ROWS32>((uint32_t)x, l0, l1);
    swap_pair<ROWS32>((uint32_t)(x >> 32), h0, h1);
    return op(__longlong_as_double((long long)(((uint64_t)h0 << 32) | l0)),
              __longlong_as_double((long long)(((uint64_t)h1 << 32) | l1)));
}

template <bool ROWS32, typename Op>
__device__ __forceinline__ int swap_op_i32(int v, Op op) {
    uint32_t a, b;
    swap_pair<ROWS32>((uint32_t)v, a, b);
    return op((int)a, (int)b);
}

// all-reduce of a commutative, associative-in-effect operation; the same bits on every lane
template <typename Op>
__device__ __forceinline__ double wave_allreduce_f64(double v, Op op) {
    v = op(v, dpp_f64<kQuadSwap1>(v));
    v = op(v, dpp_f64<kQuadSwap2>(v));
    v = op(v, dpp_f64<kHalfMirror>(v));
    v = op(v, dpp_f64<kRowMirror>(v));
    v = swap_op_f64<false>(v, op);
    return swap_op_f64<true>(v, op);
}

template <typename Op>
__device__ __forceinline__ int wave_allreduce_i32(int v, Op op) {
    v = op(v, (int)dpp_u32<kQuadSwap1>((uint32_t)v));
    v = op(v, (int)dpp_u32<kQuadSwap2>((uint32_t)v));
    v = op(v, (int)dpp_u32<kHalfMirror>((uint32_t)v));
    v = op(v, (int)dpp_u32<kRowMirror>((uint32_t)v));
    v = swap_op_i32<false>(v, op);
    return swap_op_i32<true>(v, op);
}

__device__ __forceinline__ double wave_sum_f64(double v) {
    return wave_allreduce_f64(v, [](double a, double b) { return a + b; });
}
__device__ __forceinline__ double wave_max_f64(double v) {
    return wave_allreduce_f64(v, [](double a, double b) { return fmax(a, b); });
}
__device__ __forceinline__ double wave_min_f64(double v) {
    return wave_allreduce_f64(v, [](double a, double b) { return fmin(a, b); });
}
__device__ __forceinline__ int wave_min_i32(int v) {
    return wave_allreduce_i32(v, [](int a, int b) { return a < b ? a : b; });
}
__device__ __forceinline__ int wave_max_i32(int v) {
    return wave_allreduce_i32(v, [](int a, int b) { return a > b ? a : b; });
}

__device__ __forceinline__ double readlane_f64(double v, int lane) {
    const uint64_t b = (uint64_t)__double_as_longlong(v);
    const uint64_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, lane);
    const uint64_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), lane);
    return __longlong_as_double((long long)((hi << 32) | lo));
}

// inclusive prefix sum over the lanes in a fixed order: a shift-and-add scan inside each
// 16-lane row, then the row totals (lanes 15, 31, 47) added row by row.  *total = the sum
// over all 64 lanes, formed as lane 63's scan value.
__device__ __forceinline__ double wave_incl_scan_f64(double v, int lane, double* total = nullptr) {
    v += dpp_f64<kRowShr1>(v);
    v += dpp_f64<kRowShr2>(v);
    v += dpp_f64<kRowShr4>(v);
    v += dpp_f64<kRowShr8>(v);
    const double r0 = readlane_f64(v, 15), r1 = readlane_f64(v, 31), r2 = readlane_f64(v, 47);
    const double o1 = r0, o2 = r0 + r1, o3 = o2 + r2;
    const int row = lane >> 4;
    if (row == 1) v += o1;
    else if (row == 2) v += o2;
    else if (row == 3) v += o3;
    if (total) *total = readlane_f64(v, 63);
    return v;
}

// x / T, as a multiplication by the exact reciprocal when T is a normal power of two (then
// both are the same correctly rounded value), else a division.  T is uniform across the wave.
__device__ __forceinline__ double over_T(double x, double T) {
    const uint64_t b = (uint64_t)__double_as_longlong(T);
    const uint32_t e = (uint32_t)(b >> 52) & 0x7FF;
    if ((b & 0xFFFFFFFFFFFFFull) == 0 && e >= 1 && e <= 2045) {
        const double inv = __longlong_as_double((long long)(((uint64_t)(2046 - e) << 52) | (b & (1ull << 63))));
        return x * inv;
    }
    return x / T;
}

}  // namespace hci
