// m3_mfma_common.h -- device helpers of the matrix-core prefill kernels (gfx950):
// bf16 MFMA wrappers, LDS access helpers (opaque per-lane bases, the transposing 64-bit
// read), the swizzled X tile layout, the XCD-aware workgroup order and the parameters
// of the scan kernels.
#pragma once

#include "m3_common.h"
#include "m3_internal.h"

namespace m3 {
namespace mf {

constexpr int N = 128;
constexpr int P = 64;
constexpr int KP = N / 2;
constexpr int NT = 256;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Transposing 64-bit LDS read (gfx950): within each group of 16 lanes, lane j
// receives element (j mod 4) of the 4-element segments addressed by lanes
// 4e + j/4, e = 0..3.  If lane s of a group addresses row r0 + s/4, columns
// c0 + 4(s mod 4) .. +3 of a row-major tile, lane j receives column c0 + j of
// rows r0 .. r0+3: a 4-row slice of the tile, transposed.
__device__ __forceinline__ s16x4 lds_read_tr4(const uint16_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4*)((__attribute__((address_space(3))) uint16_t*)(p)));
}

// Per-lane LDS byte address held opaque to the optimizer.  The tiles live above
// 64 KB of LDS, beyond the 16-bit immediate offset of LDS instructions; with the
// array's absolute address folded into every access the compiler keeps one
// address register per access pattern (and spills them).  From an opaque base,
// every access of a tile is base + immediate.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    uint32_t a = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const void*)(p)));
    asm volatile("" : "+v"(a));
    return a;
}
template <typename T>
__device__ __forceinline__ T lds_ld(uint32_t a) {
    return *(__attribute__((address_space(3))) const T*)(static_cast<uintptr_t>(a));
}
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void lds_st(uint32_t a, uint4 v) {
    *(__attribute__((address_space(3))) u32x4*)(static_cast<uintptr_t>(a)) = u32x4{v.x, v.y, v.z, v.w};
}
__device__ __forceinline__ void lds_st(uint32_t a, uint2 v) {
    *(__attribute__((address_space(3))) u32x2*)(static_cast<uintptr_t>(a)) = u32x2{v.x, v.y};
}
__device__ __forceinline__ s16x4 lds_tr4(uint32_t a) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(static_cast<uintptr_t>(a)));
}

// Global-memory view of a pointer chosen at run time (a select between two
// pointers hides their address space from the compiler).  Loads through it are
// global loads; a generic (flat) load would also count as a possible LDS access
// and make every LDS wait of the loop a full drain.
template <typename T>
__device__ __forceinline__ const __attribute__((address_space(1))) T* global_view(const T* p) {
    return (const __attribute__((address_space(1))) T*)(p);
}

__device__ __forceinline__ f32x4 mfma_k32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_k16(s16x4 a, s16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ __bf16 to_bf(float f) { return static_cast<__bf16>(f); }
__device__ __forceinline__ float from_bf(__bf16 b) { return static_cast<float>(b); }
__device__ __forceinline__ float bits_to_f(uint16_t u) { return __uint_as_float(static_cast<uint32_t>(u) << 16); }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 v = {to_bf(a), to_bf(b)};
    return __builtin_bit_cast(uint32_t, v);
}

struct ScanParams {
    const uint16_t* x;      // (b, L, H, R, P) bf16
    const float* dt;        // (b, L, H)
    const float* A;         // (H)
    const float* lam;       // (b, L, H)
    const float* D;         // (H)
    const uint8_t* prep;    // prepared operands, per (b, g, chunk)
    uint16_t* y;            // (b, L, H, R, P) bf16
    uint16_t* y_sink;       // 64 x 64 bf16 scratch: stores of rows past the sequence end land here
    const float* s_init;    // states entering the state-only pieces: (b, H, sinit_stride, N, P) fp32, or null;
                            // segment s of the output pass starts from entry sinit_step * s
    const void* h_in;       // used when s_init is null (nseg == 1): (b, H, N, P), may be null
    const uint16_t* bl_in;  // carry in (b, G, R, N), may be null
    const uint16_t* xl_in;  // carry in (b, H, R, P), may be null
    void* h_out;            // final state (b, H, N, P), may be null
    float* seg_state;       // state-only mode: (b, H, nseg-1, N, P)
    float* seg_decay;       // state-only mode: (b, H, nseg-1)
    float* seg_rot;         // state-only mode: (b, H, nseg-1, KP, 2)
    int64_t L;              // sequence length (the maximum one with cu)
    int H, G, nchunks, nseg, chunks_per_seg;
    int sinit_stride, sinit_step;
    int state_bf16;         // h_in and h_out hold bf16 (else fp32)
    const int64_t* cu;      // packed variable-length batch: sequence starts, or null
    int64_t T;              // tokens in the packed arrays
    const float* At;        // per-token decay rates (b, L, H) replacing A, or null
    const uint16_t* z;      // output gate input, laid out as y, or null
    const float* onw;       // output RMSNorm weight (H, P), or null
    float eps;              // its epsilon
    int Gt;                 // angle groups: the prepared operands are per (b, angle group, chunk)
    int seqs;               // sequences per workgroup of the output pass (equal lengths, whole chunks,
                            // one angle group, one segment): seqs * w .. + seqs - 1, one after another
    int batch;              // sequences in the batch
};

// Initial state of segment 0 when no segment pass ran: h_in plus the beta term
// the first token gives the carried previous input.
template <int R>
__device__ float initial_state(const ScanParams& p, int b, int h, int g, int n, int col, float c1) {
    float s = p.h_in ? state_load(p.h_in, (static_cast<size_t>(b) * p.H + h) * N * P + n * P + col, p.state_bf16)
                     : 0.f;
    if (p.bl_in && p.xl_in) {
        float u = 0.f;
#pragma unroll
        for (int r = 0; r < R; ++r)
            u += bits_to_f(p.bl_in[((static_cast<size_t>(b) * p.G + g) * R + r) * N + n]) *
                 bits_to_f(p.xl_in[((static_cast<size_t>(b) * p.H + h) * R + r) * P + col]);
        s += c1 * u;
    }
    return s;
}

// Element offset of (row, col) in a row-major [rows][P] bf16 LDS tile (P = 64: four
// 32-byte column groups per 128-byte row) whose groups are permuted by row: group g of
// row r is stored at position g ^ f(r), f(r) = (r ^ (r >> 2)) & 3.  LDS has 64 banks of
// 4 bytes and serves 32 lanes of a 64-bit read per clock; the transposing reads of these
// tiles cover 8 rows x one 32-byte group per 32 lanes, and rows 128 bytes apart repeat
// every other row on the same 32 banks.  With f the 8 rows land on 8 different sets of
// 8 banks.  f depends only on bits 0-3 of the row, so moving by a multiple of 16 rows is a
// constant offset.
__device__ __forceinline__ int xoff(int row, int col) {
    return row * P + ((((col >> 4) ^ row ^ (row >> 2)) & 3) << 4) + (col & 15);
}

// Swap a value with the neighbouring lane (lane ^ 1) through a DPP quad permutation.
__device__ __forceinline__ float swap_adjacent(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));
}

// Sum over each 16-lane row of a wave (DPP quad swaps, then rotations within the row, the
// first steps of wave_sum); every lane gets its row's sum.  The 16 lanes of a row must all
// be active.
__device__ __forceinline__ float row16_sum(float v) {
    v += dpp_move<0xB1>(v);    // quad_perm [1, 0, 3, 2]
    v += dpp_move<0x4E>(v);    // quad_perm [2, 3, 0, 1]
    v += dpp_move<0x124>(v);   // row_ror 4
    v += dpp_move<0x128>(v);   // row_ror 8
    return v;
}

// Workgroups are dispatched to the 8 XCDs round-robin by linear id, and each
// XCD has its own L2.  The heads of one (batch, segment) group read the same
// prepared Bt/Ct, so the linear id is permuted to place a group's heads on one
// XCD, one after another: the prepared operands are then fetched into one L2
// instead of eight.  Any id permutation is correct; this one only helps speed.
__device__ __forceinline__ void xcd_decode(int id, int total, int H, int nseg, int* b, int* h, int* seg) {
    int v = id;
    if ((total & 7) == 0) {
        const int per = total >> 3;
        v = (id & 7) * per + (id >> 3);
    }
    const int grp = v / H;
    *h = v - grp * H;
    *b = grp / nseg;
    *seg = grp - *b * nseg;
}

// Prefetched data is carried in vector-typed values (never addressable arrays)
// so that it stays in registers while the loads are in flight.
template <int K> using u32v = uint32_t __attribute__((ext_vector_type(K)));
template <int K> using bfv = __bf16 __attribute__((ext_vector_type(K)));

template <int K>
__device__ __forceinline__ uint4 quad(const u32v<K>& v, int i) {   // i: constant after unrolling
    return uint4{v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]};
}
template <int K>
__device__ __forceinline__ void set_quad(u32v<K>& v, int i, uint4 q) {
    v[4 * i] = q.x;
    v[4 * i + 1] = q.y;
    v[4 * i + 2] = q.z;
    v[4 * i + 3] = q.w;
}
template <int K>
__device__ __forceinline__ bf16x8 oct(const bfv<K>& v, int i) {
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = v[8 * i + e];
    return o;
}
template <int K>
__device__ __forceinline__ void set_oct(bfv<K>& v, int i, bf16x8 o) {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[8 * i + e] = o[e];
}

}  // namespace mf
}  // namespace m3
