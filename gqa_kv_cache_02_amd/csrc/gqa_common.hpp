// gqa_common.hpp -- device helpers shared by the libgqa kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqa {

// log2(e): scores are pre-multiplied by scale * log2(e) so that softmax can
// use exp2, which maps to the hardware v_exp_f32.
constexpr float kLog2e = 1.4426950408889634f;

typedef __attribute__((__vector_size__(8 * sizeof(short)))) short bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

__device__ __forceinline__ float bf16_to_f32(uint16_t x) {
    return __uint_as_float(static_cast<uint32_t>(x) << 16);
}

// fp32 -> bf16, round to nearest even (hardware v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two floats -> packed bf16 pair (low half = a), one conversion instruction.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}

// 2^x with the bare hardware instruction; softmax never needs results in the
// denormal range to be accurate.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <typename T> struct Elem;
template <> struct Elem<float> {
    __device__ __forceinline__ static float load(const float *p) { return *p; }
    __device__ __forceinline__ static void store(float *p, float v) { *p = v; }
};
template <> struct Elem<uint16_t> {
    __device__ __forceinline__ static float load(const uint16_t *p) { return bf16_to_f32(*p); }
    __device__ __forceinline__ static void store(uint16_t *p, float v) { *p = f32_to_bf16(v); }
};

// Butterfly reductions over the whole 64-lane wavefront.
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1)
        x += __shfl_xor(x, m, 64);
    return x;
}
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1)
        x = fmaxf(x, __shfl_xor(x, m, 64));
    return x;
}

__device__ __forceinline__ int wave_min_i(int x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1)
        x = min(x, __shfl_xor(x, m, 64));
    return x;
}
__device__ __forceinline__ int wave_max_i(int x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1)
        x = max(x, __shfl_xor(x, m, 64));
    return x;
}

// Window lower bound for a query at cell t (segment start 0): the current
// cell plus at most window-1 earlier cells; window < 0 means none.
__device__ __forceinline__ int window_lo(int t, int window) {
    if (window < 0)
        return 0;
    int lo = t - (window - 1);
    return lo > 0 ? lo : 0;
}

// Lower bound of the permitted keys of a query at cell p whose segment
// starts at cell seg: the later of the segment start and the window start
// ("Share key/value heads and make context explicit", section "Intersect the
// window with the context already permitted").  -1 when the segment starts
// after the query (no permitted key).
__device__ __forceinline__ int segment_lo(int p, int seg, int window) {
    if (seg > p)
        return -1;
    const int w = window_lo(p, window);
    return seg > w ? seg : w;
}

} // namespace gqa
