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

// Token span of sequence b.  A packed variable-length batch gives the starts
// (cu[b] .. cu[b+1]) in device memory; they are clamped to the T tokens present
// and to at most L tokens (the maximum length the launch was sized for), so
// that inconsistent offsets give wrong results but never an access out of
// bounds.  Without offsets every sequence is L tokens starting at b * L.
struct SeqSpan {
    int64_t start, len;
};
__device__ __forceinline__ SeqSpan seq_span(const int64_t* cu, int64_t b, int64_t L, int64_t T) {
    if (!cu) return SeqSpan{b * L, L};
    int64_t s = cu[b], e = cu[b + 1];
    s = s < 0 ? 0 : (s > T ? T : s);
    e = e < s ? s : (e > T ? T : e);
    return SeqSpan{s, e - s < L ? e - s : L};
}

// One state element of a state stored in fp32 or bf16 (chosen at run time).
__device__ __forceinline__ float state_load(const void* p, size_t i, bool bf16) {
    return bf16 ? bf16_to_f32(static_cast<const uint16_t*>(p)[i]) : static_cast<const float*>(p)[i];
}
__device__ __forceinline__ void state_store(void* p, size_t i, float v, bool bf16) {
    if (bf16)
        static_cast<uint16_t*>(p)[i] = f32_to_bf16(v);
    else
        static_cast<float*>(p)[i] = v;
}

// Four consecutive state values: fp32 (16 bytes) or bf16 (8 bytes, rounded to
// nearest even on store), streamed with non-temporal accesses.
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
template <typename S> struct state4;
template <> struct state4<float> {
    __device__ __forceinline__ static f32x4_t load(const float* p) {
        return __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
    }
    __device__ __forceinline__ static void store(float* p, f32x4_t v) {
        __builtin_nontemporal_store(v, reinterpret_cast<f32x4_t*>(p));
    }
};
template <> struct state4<bf16_t> {
    __device__ __forceinline__ static f32x4_t load(const bf16_t* p) {
        const u32x2_t w = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
        return f32x4_t{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                       __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u)};
    }
    __device__ __forceinline__ static void store(bf16_t* p, f32x4_t v) {
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        const bf16x2 lo = {static_cast<__bf16>(v.x), static_cast<__bf16>(v.y)};
        const bf16x2 hi = {static_cast<__bf16>(v.z), static_cast<__bf16>(v.w)};
        const u32x2_t w = {__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
        __builtin_nontemporal_store(w, reinterpret_cast<u32x2_t*>(p));
    }
};

// One DPP move of a float between lanes (control C: a quad permutation or a rotation
// within each row of 16 lanes); every source lane exists for these controls.
template <int C>
__device__ __forceinline__ float dpp_move(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), C, 0xf, 0xf, false));
}

// Sum over the 64 lanes of a wave, all of them active (every lane gets it): the lanes of
// each row of 16 are summed with DPP moves (swap neighbours, swap pairs, rotate by 4, by 8),
// then the four row sums are read into scalars and added.
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp_move<0xB1>(v);    // quad_perm [1, 0, 3, 2]
    v += dpp_move<0x4E>(v);    // quad_perm [2, 3, 0, 1]
    v += dpp_move<0x124>(v);   // row_ror 4
    v += dpp_move<0x128>(v);   // row_ror 8
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return (r0 + r1) + (r2 + r3);
}

// silu(v) = v / (1 + e^-v), the output gate's nonlinearity, with the hardware reciprocal
// (1 ulp) in place of an IEEE division: a dozen fewer instructions per gated output.
// Large negative v gives e^-v = inf, a reciprocal of 0 and silu = -0.
__device__ __forceinline__ float silu(float v) { return v * __builtin_amdgcn_rcpf(1.f + __expf(-v)); }

// Accurate sin/cos of an angle of any size (chunk-local angle sums can reach
// hundreds of radians); the HIP library routine does the range reduction.
__device__ __forceinline__ void sincos_acc(float a, float* s, float* c) { sincosf(a, s, c); }

}  // namespace m3
