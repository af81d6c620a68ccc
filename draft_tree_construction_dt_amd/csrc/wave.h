// Wave64 reductions for gfx950: a DPP butterfly inside each 16-lane row
// (quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror:
// every step pairs lanes holding disjoint partial results), then the four
// row results read into scalar registers and combined.  Every lane gets the
// same (wave-uniform) result.  Max, min and integer sums are exact; a
// floating-point sum is taken in this fixed order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dt {

// (every step reads a lane of its own row, so no lane is out of bounds and
// the moves need no initial value)
__device__ __forceinline__ int dpp_step(int v, int ctrl) {
    switch (ctrl) {
    case 0: return __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
    case 1: return __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
    case 2: return __builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, false);  // row_half_mirror
    default: return __builtin_amdgcn_mov_dpp(v, 0x140, 0xF, 0xF, false); // row_mirror
    }
}

// min / max by compare and select: the operands are never NaN here, and the
// library's fmin/fmax would first canonicalise both (two more instructions)
__device__ __forceinline__ double min_d(double a, double b) { return b < a ? b : a; }
__device__ __forceinline__ double max_d(double a, double b) { return b > a ? b : a; }
__device__ __forceinline__ float min_f(float a, float b) { return b < a ? b : a; }
__device__ __forceinline__ float max_f(float a, float b) { return b > a ? b : a; }

__device__ __forceinline__ uint64_t dpp_step64(uint64_t v, int ctrl) {
    const uint32_t lo = (uint32_t)dpp_step((int)(uint32_t)v, ctrl);
    const uint32_t hi = (uint32_t)dpp_step((int)(uint32_t)(v >> 32), ctrl);
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint64_t readlane64(uint64_t v, int l) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), l);
    return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
    for (int s = 0; s < 4; ++s) v = max_f(v, __int_as_float(dpp_step(__float_as_int(v), s)));
    const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return max_f(max_f(a, b), max_f(c, d));
}

__device__ __forceinline__ float wave_min_f32(float v) {
#pragma unroll
    for (int s = 0; s < 4; ++s) v = min_f(v, __int_as_float(dpp_step(__float_as_int(v), s)));
    const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return min_f(min_f(a, b), min_f(c, d));
}

__device__ __forceinline__ double wave_max_f64(double v) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
        v = max_d(v, __longlong_as_double((long long)dpp_step64((uint64_t)__double_as_longlong(v), s)));
    const uint64_t u = (uint64_t)__double_as_longlong(v);
    const double a = __longlong_as_double((long long)readlane64(u, 0));
    const double b = __longlong_as_double((long long)readlane64(u, 16));
    const double c = __longlong_as_double((long long)readlane64(u, 32));
    const double d = __longlong_as_double((long long)readlane64(u, 48));
    return max_d(max_d(a, b), max_d(c, d));
}

__device__ __forceinline__ double wave_min_f64(double v) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
        v = min_d(v, __longlong_as_double((long long)dpp_step64((uint64_t)__double_as_longlong(v), s)));
    const uint64_t u = (uint64_t)__double_as_longlong(v);
    const double a = __longlong_as_double((long long)readlane64(u, 0));
    const double b = __longlong_as_double((long long)readlane64(u, 16));
    const double c = __longlong_as_double((long long)readlane64(u, 32));
    const double d = __longlong_as_double((long long)readlane64(u, 48));
    return min_d(min_d(a, b), min_d(c, d));
}

__device__ __forceinline__ double wave_add_f64(double v) {
#pragma unroll
    for (int s = 0; s < 4; ++s) v += __longlong_as_double((long long)dpp_step64((uint64_t)__double_as_longlong(v), s));
    const uint64_t u = (uint64_t)__double_as_longlong(v);
    const double a = __longlong_as_double((long long)readlane64(u, 0));
    const double b = __longlong_as_double((long long)readlane64(u, 16));
    const double c = __longlong_as_double((long long)readlane64(u, 32));
    const double d = __longlong_as_double((long long)readlane64(u, 48));
    return (a + b) + (c + d);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const uint64_t o = dpp_step64(v, s);
        v = o > v ? o : v;
    }
    uint64_t r = readlane64(v, 0);
    const uint64_t b = readlane64(v, 16), c = readlane64(v, 32), d = readlane64(v, 48);
    r = b > r ? b : r;
    r = c > r ? c : r;
    return d > r ? d : r;
}

__device__ __forceinline__ uint64_t wave_min_u64(uint64_t v) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const uint64_t o = dpp_step64(v, s);
        v = o < v ? o : v;
    }
    uint64_t r = readlane64(v, 0);
    const uint64_t b = readlane64(v, 16), c = readlane64(v, 32), d = readlane64(v, 48);
    r = b < r ? b : r;
    r = c < r ? c : r;
    return d < r ? d : r;
}

// minimum over the wave, left in every lane's register: the row butterfly,
// then the two row-swapping permutes of gfx950 (rows r and r^1, then r and
// r^2), so no value goes through a scalar register
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const uint32_t o = (uint32_t)dpp_step((int)v, s);
        v = o < v ? o : v;
    }
    const auto q16 = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    v = q16[0] < q16[1] ? q16[0] : q16[1];
    const auto q32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return q32[0] < q32[1] ? q32[0] : q32[1];
}

// The same reductions with the result left in every lane's register: the
// row butterfly, then the two row-swapping permutes (rows r and r^1, then r
// and r^2).  Each permute pairs one row's partial with its partner's in the
// same order in both rows, so every lane ends with the same value.
__device__ __forceinline__ uint32_t swap_rows16(uint32_t v, uint32_t* other) {
    const auto q = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    *other = q[1];
    return q[0];
}
__device__ __forceinline__ uint32_t swap_rows32(uint32_t v, uint32_t* other) {
    const auto q = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    *other = q[1];
    return q[0];
}

__device__ __forceinline__ float wave_max_f32_all(float v) {
#pragma unroll
    for (int s = 0; s < 4; ++s) v = max_f(v, __int_as_float(dpp_step(__float_as_int(v), s)));
    uint32_t o;
    float a = __uint_as_float(swap_rows16(__float_as_uint(v), &o));
    v = max_f(a, __uint_as_float(o));
    a = __uint_as_float(swap_rows32(__float_as_uint(v), &o));
    return max_f(a, __uint_as_float(o));
}

// 64-bit values move as two words
__device__ __forceinline__ uint64_t swap_rows16_64(uint64_t v, uint64_t* other) {
    uint32_t ol, oh;
    const uint32_t l = swap_rows16((uint32_t)v, &ol), h = swap_rows16((uint32_t)(v >> 32), &oh);
    *other = ((uint64_t)oh << 32) | ol;
    return ((uint64_t)h << 32) | l;
}
__device__ __forceinline__ uint64_t swap_rows32_64(uint64_t v, uint64_t* other) {
    uint32_t ol, oh;
    const uint32_t l = swap_rows32((uint32_t)v, &ol), h = swap_rows32((uint32_t)(v >> 32), &oh);
    *other = ((uint64_t)oh << 32) | ol;
    return ((uint64_t)h << 32) | l;
}

__device__ __forceinline__ double wave_add_f64_all(double v) {
#pragma unroll
    for (int s = 0; s < 4; ++s) v += __longlong_as_double((long long)dpp_step64((uint64_t)__double_as_longlong(v), s));
    uint64_t o;
    double a = __longlong_as_double((long long)swap_rows16_64((uint64_t)__double_as_longlong(v), &o));
    v = a + __longlong_as_double((long long)o);
    a = __longlong_as_double((long long)swap_rows32_64((uint64_t)__double_as_longlong(v), &o));
    return a + __longlong_as_double((long long)o);
}

__device__ __forceinline__ uint64_t wave_max_u64_all(uint64_t v) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const uint64_t o = dpp_step64(v, s);
        v = o > v ? o : v;
    }
    uint64_t o;
    uint64_t a = swap_rows16_64(v, &o);
    v = o > a ? o : a;
    a = swap_rows32_64(v, &o);
    return o > a ? o : a;
}

__device__ __forceinline__ uint64_t wave_min_u64_all(uint64_t v) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const uint64_t o = dpp_step64(v, s);
        v = o < v ? o : v;
    }
    uint64_t o;
    uint64_t a = swap_rows16_64(v, &o);
    v = o < a ? o : a;
    a = swap_rows32_64(v, &o);
    return o < a ? o : a;
}

__device__ __forceinline__ int wave_add_i32_all(int v) {
#pragma unroll
    for (int s = 0; s < 4; ++s) v += dpp_step(v, s);
    uint32_t o;
    uint32_t a = swap_rows16((uint32_t)v, &o);
    v = (int)(a + o);
    a = swap_rows32((uint32_t)v, &o);
    return (int)(a + o);
}

__device__ __forceinline__ int wave_add_i32(int v) {
#pragma unroll
    for (int s = 0; s < 4; ++s) v += dpp_step(v, s);
    return (__builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16)) +
           (__builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48));
}

__device__ __forceinline__ int wave_min_i32(int v) {
#pragma unroll
    for (int s = 0; s < 4; ++s) v = min(v, dpp_step(v, s));
    return min(min(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
               min(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}

}  // namespace dt
