// Device helpers shared by the MegaMoE kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace megamoe {

constexpr int kWave = 64;

typedef int v4i __attribute__((ext_vector_type(4)));

// fp16 bits -> fp32 (exact).
__device__ __forceinline__ float h2f(uint16_t b) {
    return (float)__builtin_bit_cast(_Float16, b);
}

// fp32 -> fp16 bits, IEEE round to nearest even (hardware conversion).
__device__ __forceinline__ uint16_t f2h(float f) {
    return __builtin_bit_cast(uint16_t, (_Float16)f);
}

// Materialises an fp32 value as rounded fp32.  Without it the compiler folds
// "fp32 multiply, then convert to fp16" into one mixed-precision FMA that rounds
// once from the exact product; the dequant step rounds the fp32 product first.
__device__ __forceinline__ float keep_f32(float v) {
    asm volatile("" : "+v"(v));
    return v;
}

// fp32 -> bf16 bits, round to nearest even.  Adding 0x7fff plus the lowest kept
// bit and truncating rounds half-way cases to the even neighbour; overflow
// carries into the exponent and yields infinity.  NaNs stay quiet NaNs.
__device__ __forceinline__ uint32_t f2bf(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ float bf2f(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
    return v;
}

// Inclusive prefix sum across the 64 lanes of a wave.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        int t = __shfl_up(v, off, kWave);
        if (lane >= off) v += t;
    }
    return v;
}

}  // namespace megamoe
