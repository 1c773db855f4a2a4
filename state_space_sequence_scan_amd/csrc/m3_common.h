// m3_common.h -- shared device helpers for the Mamba-3 scan kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace m3 {

// bf16 is carried as its 16 raw bits.
struct bf16_t {
    uint16_t bits;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16, round to nearest, ties to even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x0040u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

// Loads / stores of the io dtype as fp32.
template <typename T> struct io;
template <> struct io<float> {
    __device__ __forceinline__ static float load(const float* p) { return *p; }
    __device__ __forceinline__ static void store(float* p, float v) { *p = v; }
};
template <> struct io<bf16_t> {
    __device__ __forceinline__ static float load(const bf16_t* p) { return bf16_to_f32(p->bits); }
    __device__ __forceinline__ static void store(bf16_t* p, float v) { p->bits = f32_to_bf16(v); }
};

// Accurate sin/cos of an angle of any size (chunk-local angle sums can reach
// hundreds of radians); the HIP library routine does the range reduction.
__device__ __forceinline__ void sincos_acc(float a, float* s, float* c) { sincosf(a, s, c); }

}  // namespace m3
