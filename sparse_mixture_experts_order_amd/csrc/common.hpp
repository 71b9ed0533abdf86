// Device-side helpers shared by the Switch FFN layer kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace swmoe {

typedef uint16_t bf16_t;                                        // raw bf16 bits
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));      // MFMA A/B operand (8 x bf16)
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // 16-byte load/store unit (a native vector, kept in VGPRs)
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;

// Round-to-nearest-even float -> bf16 bits; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) | 0x40u) & 0xffffu;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) {
    return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) {
    bf16x8 r;
    __builtin_memcpy(&r, &v, sizeof(r));
    return r;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m);
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
    return v;
}

// Largest value, lowest index among equal values.
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        float ov = __shfl_xor(v, m);
        int oi = __shfl_xor(i, m);
        if (ov > v || (ov == v && oi < i)) { v = ov; i = oi; }
    }
}

// Map a linear block id to a logical tile id so that consecutive logical tiles
// run on the same XCD (the hardware deals workgroups round-robin over the 8
// XCDs, each with its own L2).  The grid is padded to a multiple of 8; the
// caller exits when the returned id is >= the real tile count.
__device__ __forceinline__ int xcd_swizzle(int bid, int grid_padded) {
    const int per_xcd = grid_padded >> 3;
    return (bid & 7) * per_xcd + (bid >> 3);
}

}  // namespace swmoe
