// Device helpers shared by the MegaMoE kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace megamoe {

constexpr int kWave = 64;

typedef int v4i __attribute__((ext_vector_type(4)));

// 16-byte loads and stores with the non-temporal hint, for data that is
// read or written once per forward (streaming through the caches)
__device__ __forceinline__ uint4 load_nt16(const void *p) {
    const v4i v = __builtin_nontemporal_load(reinterpret_cast<const v4i *>(p));
    return make_uint4((uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3]);
}
__device__ __forceinline__ void store_nt16(void *p, uint4 v) {
    __builtin_nontemporal_store(v4i{(int)v.x, (int)v.y, (int)v.z, (int)v.w},
                                reinterpret_cast<v4i *>(p));
}

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

// Two fp32 values -> packed bf16 bits (a in the low half), round to nearest
// even, by the gfx950 conversion instruction v_cvt_pk_bf16_f32.  The unpermute's
// output is compared bit for bit with the oracle's own round-to-nearest-even
// conversion on every parity shape.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f2bf_pk(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}

// bf16 bits in the low / high half of a word -> fp32 (exact)
__device__ __forceinline__ float bf2f_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf2f_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

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
