// m3_decode.hip -- one decode step of the Mamba-3 scan (gfx950).
//
// Per (b, h), with the trapezoid carry U_prev = B_prev X_prev:
//   h <- alpha M (h + (1 - lambda) dt U_prev) + lambda dt U,   U = B_t X_t
//   y  = C_t^T h + D X_t
// (alpha M h + beta M U_prev + gamma U with beta = (1 - lambda) dt alpha, the
// exponential-trapezoidal step of the Mamba-3 paper note, "Solution 1", with the
// rotation of "Solution 2" and the rank-R input/read-out of "Solution 3").
//
// The step reads and writes the whole state (fp32 or bf16) and does little arithmetic
// per byte: it is bound by HBM bandwidth.  decode_fast (N = 128, P = 64 at R = 1, 2, 4,
// and N = P = 16 at R = 1) streams each (b, h) state slice once with non-temporal loads
// and stores, keeps every rotation pair (2k, 2k+1) inside one thread, and reduces the
// R x P read-out across lanes and then across waves through LDS; decode_generic handles
// any other shape.
#include <type_traits>

#include "m3_common.h"
#include "m3_internal.h"

namespace m3 {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// CW consecutive state values of one row: 16 bytes for CW = 4 fp32 or CW = 8 bf16
// (8 bytes for CW = 4 bf16), streamed with non-temporal accesses.
template <typename S, int CW> struct state_vec;
// Raw is the loaded form (kept in registers by the prefetching variant) and widen()
// turns it into fp32.
template <> struct state_vec<float, 4> {
    typedef float V __attribute__((ext_vector_type(4)));
    typedef V Raw;
    __device__ __forceinline__ static V load(const float* p) { return state4<float>::load(p); }
    __device__ __forceinline__ static Raw load_raw(const float* p) { return state4<float>::load(p); }
    __device__ __forceinline__ static V widen(Raw w) { return w; }
    __device__ __forceinline__ static void store(float* p, V v) { state4<float>::store(p, v); }
};
template <> struct state_vec<bf16_t, 4> {
    typedef float V __attribute__((ext_vector_type(4)));
    typedef u32x2_t Raw;
    __device__ __forceinline__ static V load(const bf16_t* p) { return state4<bf16_t>::load(p); }
    __device__ __forceinline__ static Raw load_raw(const bf16_t* p) {
        return __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
    }
    __device__ __forceinline__ static V widen(Raw w) {
        return V{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                 __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u)};
    }
    __device__ __forceinline__ static void store(bf16_t* p, V v) { state4<bf16_t>::store(p, v); }
};
template <> struct state_vec<bf16_t, 8> {
    typedef float V __attribute__((ext_vector_type(8)));
    typedef uint32_t W __attribute__((ext_vector_type(4)));
    __device__ __forceinline__ static V load(const bf16_t* p) {
        const W w = __builtin_nontemporal_load(reinterpret_cast<const W*>(p));
        return V{__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                 __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u),
                 __uint_as_float(w.z << 16), __uint_as_float(w.z & 0xffff0000u),
                 __uint_as_float(w.w << 16), __uint_as_float(w.w & 0xffff0000u)};
    }
    __device__ __forceinline__ static void store(bf16_t* p, V v) {
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        const bf16x2 a = {static_cast<__bf16>(v[0]), static_cast<__bf16>(v[1])};
        const bf16x2 b = {static_cast<__bf16>(v[2]), static_cast<__bf16>(v[3])};
        const bf16x2 c = {static_cast<__bf16>(v[4]), static_cast<__bf16>(v[5])};
        const bf16x2 d = {static_cast<__bf16>(v[6]), static_cast<__bf16>(v[7])};
        const W w = {__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b),
                     __builtin_bit_cast(uint32_t, c), __builtin_bit_cast(uint32_t, d)};
        __builtin_nontemporal_store(w, reinterpret_cast<W*>(p));
    }
};

// n consecutive values of T from p into fp32, with loads of up to 16 bytes, and the
// reverse.  (Global accesses need not be aligned to their width on this hardware; the
// callers' runs start at multiples of their own length.)
template <typename T, int n> struct run;
template <int n> struct run<bf16_t, n> {
    __device__ __forceinline__ static void load(const bf16_t* p, float* out) {
        if constexpr (n % 8 == 0) {
#pragma unroll
            for (int k = 0; k < n / 8; ++k) {
                const u32x4_t w = *reinterpret_cast<const u32x4_t*>(p + 8 * k);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    out[8 * k + 2 * j] = __uint_as_float(w[j] << 16);
                    out[8 * k + 2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
                }
            }
        } else if constexpr (n == 4) {
            const u32x2_t w = *reinterpret_cast<const u32x2_t*>(p);
            out[0] = __uint_as_float(w.x << 16);
            out[1] = __uint_as_float(w.x & 0xffff0000u);
            out[2] = __uint_as_float(w.y << 16);
            out[3] = __uint_as_float(w.y & 0xffff0000u);
        } else {
#pragma unroll
            for (int k = 0; k < n; ++k) out[k] = io<bf16_t>::load(p + k);
        }
    }
    __device__ __forceinline__ static void store(bf16_t* p, const float* v) {
        if constexpr (n % 4 == 0) {
#pragma unroll
            for (int k = 0; k < n / 4; ++k) {
                const u32x2_t w = {f32_to_bf16(v[4 * k]) | (static_cast<uint32_t>(f32_to_bf16(v[4 * k + 1])) << 16),
                                   f32_to_bf16(v[4 * k + 2]) | (static_cast<uint32_t>(f32_to_bf16(v[4 * k + 3])) << 16)};
                *reinterpret_cast<u32x2_t*>(p + 4 * k) = w;
            }
        } else {
#pragma unroll
            for (int k = 0; k < n; ++k) io<bf16_t>::store(p + k, v[k]);
        }
    }
};
template <int n> struct run<float, n> {
    __device__ __forceinline__ static void load(const float* p, float* out) {
        if constexpr (n % 4 == 0) {
#pragma unroll
            for (int k = 0; k < n / 4; ++k) {
                const f32x4_t w = *reinterpret_cast<const f32x4_t*>(p + 4 * k);
#pragma unroll
                for (int j = 0; j < 4; ++j) out[4 * k + j] = w[j];
            }
        } else {
#pragma unroll
            for (int k = 0; k < n; ++k) out[k] = p[k];
        }
    }
    __device__ __forceinline__ static void store(float* p, const float* v) {
        if constexpr (n % 4 == 0) {
#pragma unroll
            for (int k = 0; k < n / 4; ++k)
                *reinterpret_cast<f32x4_t*>(p + 4 * k) = f32x4_t{v[4 * k], v[4 * k + 1], v[4 * k + 2], v[4 * k + 3]};
        } else {
#pragma unroll
            for (int k = 0; k < n; ++k) p[k] = v[k];
        }
    }
};

// The fused prologue on the staged per-token operands: each of the R rows of B, C
// and the previous B (N values in LDS, fp32) through RMSNorm (weight (R, N)) and
// bias (R, N), then B and the previous B scaled by bscale and bpscale.  One wave
// per row at a time; the block has nt threads (one partial wave when nt < 64).
// Ends with a barrier.
// The RMSNorm scales of the 3R staged rows (B, C, previous B) into sScale[3R]; ends
// with a barrier when a norm weight is given.
__device__ __forceinline__ void bc_scales(const float* sB, const float* sC, const float* sBp, float* sScale,
                                          int R, int N, int nt, const Fusion& fu) {
    const int tid = threadIdx.x, width = nt < 64 ? nt : 64, lane = tid % width, wave = tid / width;
    const int nwaves = (nt + width - 1) / width;
    if (fu.bnw || fu.cnw) {
        for (int row = wave; row < 3 * R; row += nwaves) {
            const float* src = row < R ? sB + row * N : (row < 2 * R ? sC + (row - R) * N : sBp + (row - 2 * R) * N);
            float ss = 0.f;
            for (int n = lane; n < N; n += width) ss += src[n] * src[n];
            if (width == 64) {
                ss = wave_sum(ss);
            } else {
                for (int off = 1; off < width; off <<= 1) ss += __shfl_xor(ss, off, width);
            }
            if (lane == 0) sScale[row] = rsqrtf(ss / N + fu.eps);
        }
        __syncthreads();
    }
}

__device__ __forceinline__ void fuse_bc(float* sB, float* sC, float* sBp, float* sScale, int R, int N,
                                        int nt, const Fusion& fu, float bscale = 1.f, float bpscale = 1.f) {
    const int tid = threadIdx.x;
    bc_scales(sB, sC, sBp, sScale, R, N, nt, fu);
    for (int i = tid; i < R * N; i += nt) {
        const int r = i / N;
        float b = sB[i], c = sC[i], bp = sBp[i];
        if (fu.bnw) {
            b *= sScale[r] * fu.bnw[i];
            bp *= sScale[2 * R + r] * fu.bnw[i];
        }
        if (fu.cnw) c *= sScale[R + r] * fu.cnw[i];
        if (fu.bbias) {
            b += fu.bbias[i];
            bp += fu.bbias[i];
        }
        if (fu.cbias) c += fu.cbias[i];
        sB[i] = b * bscale;
        sC[i] = c;
        sBp[i] = bp * bpscale;
    }
    __syncthreads();
}

// Output RMSNorm scales: rows r < R of P values in sO (LDS, fp32) into
// sRs[r] = 1 / sqrt(mean(row^2) + eps), one wave (or the whole block when it has fewer
// than 64 threads) per row at a time.  Ends with a barrier.
__device__ __forceinline__ void row_rms(const float* sO, float* sRs, int R, int P, int nt, float eps) {
    const int tid = threadIdx.x, width = nt < 64 ? nt : 64, lane = tid % width, wave = tid / width;
    const int nwaves = (nt + width - 1) / width;
    for (int r = wave; r < R; r += nwaves) {
        float ss = 0.f;
        for (int q = lane; q < P; q += width) ss += sO[r * P + q] * sO[r * P + q];
        if (width == 64) {
            ss = wave_sum(ss);
        } else {
            for (int off = 1; off < width; off <<= 1) ss += __shfl_xor(ss, off, width);
        }
        if (lane == 0) sRs[r] = rsqrtf(ss / P + eps);
    }
    __syncthreads();
}

// Fast path.  One workgroup of NT threads per (b, h).  Thread tid owns the
// CW-column block c = tid % PC (PC = P/CW) and the rotation pairs
// k = kk + TPG * j (kk = tid / PC, j < PPT), i.e. 2 * PPT state rows x CW columns.
// FU: the fused prologue/epilogue may be present (its weights, biases and gate input are
// then loaded with the other small operands, ahead of the state stream).
// PACED: the per-token operands are loaded and staged in LDS in three dependent
// groups (B, C and the previous B; X and the previous X; the angles), and the state
// loads are issued after the last.  Measured at N = 128, P = 64, R = 4 with an fp32
// state (169 us per step at batch 256, H = 64), this is 4% faster than issuing the
// state loads right behind all the operand loads, and the variants that start the
// fp32 state stream earlier still (the operands staged in one group: 3% slower; the
// state loads first: 7% slower) lose too: the state streams of the resident workgroups
// are spread in time.  Without PACED the operands are loaded in one or two wide
// unconditional loads per array and the state loads issued right behind them, their
// staging under the state stream: with a bf16 state, whose single-wave workgroups
// carry more arithmetic per byte, that is 7% faster than operand loads that complete
// one after another (97 against 103 us).
template <typename T, typename S, int N, int P, int R, int NT, int CW, bool FU, bool PACED>
__global__ __launch_bounds__(NT) void decode_fast(
    S* __restrict__ h, const T* __restrict__ b_last, const T* __restrict__ x_last,
    const T* __restrict__ x_t, const float* __restrict__ dt_t, const float* __restrict__ A,
    const float* __restrict__ lam_t, const float* __restrict__ theta_t,
    const T* __restrict__ B_t, const T* __restrict__ C_t, const float* __restrict__ D,
    T* __restrict__ y_t, int H, int G, int has_carry, Fusion fu) {
    constexpr int KP = N / 2;
    constexpr int PC = P / CW;
    constexpr int TPG = NT / PC;
    constexpr int PPT = KP / TPG;
    constexpr int NW = (NT + 63) / 64;
    static_assert(P % CW == 0 && NT % PC == 0 && KP % TPG == 0 && PPT >= 1, "decode tiling");
    typedef state_vec<S, CW> SV;
    typedef typename SV::V fvec;
    typedef typename SV::Raw raw;

    const int tid = threadIdx.x;
    __builtin_assume(tid < NT);   // lets the element guards below fold away
    const int c = tid % PC;
    const int kk = tid / PC;

    __shared__ float sB[R][N], sC[R][N], sBp[R][N];
    __shared__ __align__(32) float sX[R][P];
    __shared__ __align__(32) float sXp[R][P];
    __shared__ float sCs[KP + 1], sSn[KP + 1];   // + a slot that threads past KP write
    __shared__ __align__(32) float sY[NW][R][P];

    constexpr int SPT = (R * N + NT - 1) / NT;
    constexpr int XPT = (R * P + NT - 1) / NT;
    constexpr int KPT = (KP + NT - 1) / NT;
    constexpr bool SRUN = !PACED && (R * N) % NT == 0, XRUN = !PACED && (R * P) % NT == 0;
    auto sidx = [&](int e) { return SRUN ? tid * SPT + e : tid + NT * e; };   // element of B/C
    auto xidx = [&](int e) { return XRUN ? tid * XPT + e : tid + NT * e; };   // element of X/Y

    const int bh = blockIdx.x;
    const int b = bh / H, hh = bh - b * H;
    const int g = hh / (H / G);
    const int Gt = fu.tgroups(G), gt = hh / (H / Gt);   // angle group

    // Without PACED the small per-token operands are loaded into registers here, the
    // state loads are issued, and then the operands are staged in LDS.  A thread's
    // elements are consecutive when the threads tile the array exactly (SRUN, XRUN: one
    // or two wide loads each), else strided, and every load is unconditional (a clamped
    // index or a valid stand-in array; unwanted values are dropped at staging), so that
    // the compiler has no branch join at which to wait for them.
    const size_t gofs = (static_cast<size_t>(b) * G + g) * R * N;
    const size_t hofs = static_cast<size_t>(bh) * R * P;
    const T* bl = has_carry ? b_last : B_t;   // without a carry its values are dropped
    const T* xl = has_carry ? x_last : x_t;
    constexpr int SR = PACED ? 1 : SPT, XR = PACED ? 1 : XPT, KR = PACED ? 1 : KPT;
    float vb[SR], vc[SR], vbp[SR], vx[XR], vxp[XR], vth[KR];
    if constexpr (!PACED) {
        if constexpr (SRUN) {
            run<T, SPT>::load(B_t + gofs + tid * SPT, vb);
            run<T, SPT>::load(C_t + gofs + tid * SPT, vc);
            run<T, SPT>::load(bl + gofs + tid * SPT, vbp);
        } else {
#pragma unroll
            for (int e = 0; e < SPT; ++e) {
                const int i = sidx(e), ic = i < R * N ? i : 0;
                vb[e] = io<T>::load(B_t + gofs + ic);
                vc[e] = io<T>::load(C_t + gofs + ic);
                vbp[e] = io<T>::load(bl + gofs + ic);
            }
        }
        if constexpr (XRUN) {
            run<T, XPT>::load(x_t + hofs + tid * XPT, vx);
            run<T, XPT>::load(xl + hofs + tid * XPT, vxp);
        } else {
#pragma unroll
            for (int e = 0; e < XPT; ++e) {
                const int i = xidx(e), ic = i < R * P ? i : 0;
                vx[e] = io<T>::load(x_t + hofs + ic);
                vxp[e] = io<T>::load(xl + hofs + ic);
            }
        }
#pragma unroll
        for (int e = 0; e < KPT; ++e) {
            const int k = tid + NT * e;
            vth[e] = theta_t[(static_cast<size_t>(b) * Gt + gt) * KP + (k < KP ? k : 0)];
        }
    }
    // Fused pieces of this thread's elements: norm weights and biases of its B/C entries,
    // the gate input and output-norm weight of its outputs (absent ones read a stand-in
    // and are replaced by their neutral value at use).
    constexpr int FS = FU ? SPT : 1, FX = FU ? XPT : 1;
    float wbn[FS], wcn[FS], wbb[FS], wcb[FS], vz[FX], won[FX];
    if constexpr (FU) {
        const float* one = dt_t + bh;   // any valid element
#pragma unroll
        for (int e = 0; e < SPT; ++e) {
            const int i = sidx(e), ic = i < R * N ? i : 0;
            wbn[e] = *(fu.bnw ? fu.bnw + ic : one);
            wcn[e] = *(fu.cnw ? fu.cnw + ic : one);
            wbb[e] = *(fu.bbias ? fu.bbias + ic : one);
            wcb[e] = *(fu.cbias ? fu.cbias + ic : one);
        }
#pragma unroll
        for (int e = 0; e < XPT; ++e) {
            const int i = xidx(e), ic = i < R * P ? i : 0;
            vz[e] = io<T>::load((fu.z ? static_cast<const T*>(fu.z) : x_t) + hofs + ic);
            won[e] = *(fu.onw ? fu.onw + hh * P + ic % P : one);
        }
    }

    // Step scalars.  gamma = lambda dt is folded into the staged B, the carry weight
    // (1 - lambda) dt into the staged previous B (after BCNorm when that is fused:
    // the norm is applied to the raw rows), and alpha into the rotation, so that the
    // per-element work is R products for each of U_prev, U and the read-out plus two
    // for the rotation.
    const float dtv = dt_t[bh];
    const float lv = lam_t[bh];
    const float alpha = __expf(dtv * (fu.At ? fu.At[bh] : A[hh]));
    const float c1 = (1.f - lv) * dtv;   // (1 - lambda) dt : weight of the carry before the decay
    const float c2 = lv * dtv;           // gamma
    const bool fuse = FU && fu.bc();     // uniform across the grid
    const float bsc = fuse ? 1.f : c2, bpsc = fuse ? 1.f : c1;

    S* hp = h + static_cast<size_t>(bh) * N * P;
    raw s0[PPT], s1[PPT];
    auto load_state = [&]() {
#pragma unroll
        for (int j = 0; j < PPT; ++j) {
            const int k = kk + TPG * j;
            s0[j] = SV::load_raw(hp + (2 * k) * P + CW * c);
            s1[j] = SV::load_raw(hp + (2 * k + 1) * P + CW * c);
        }
    };
    if constexpr (PACED) {
        // Three dependent groups: each is staged before the next is issued (the
        // scheduling barriers keep the later loads behind the earlier LDS writes).
#pragma unroll
        for (int e = 0; e < SPT; ++e) {
            const int i = sidx(e), ic = i < R * N ? i : 0;
            const float vbe = io<T>::load(B_t + gofs + ic), vce = io<T>::load(C_t + gofs + ic);
            const float vbpe = io<T>::load(bl + gofs + ic);
            if (i < R * N) {
                (&sB[0][0])[i] = vbe * bsc;
                (&sC[0][0])[i] = vce;
                (&sBp[0][0])[i] = has_carry ? vbpe * bpsc : 0.f;
            }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int e = 0; e < XPT; ++e) {
            const int i = xidx(e), ic = i < R * P ? i : 0;
            const float vxe = io<T>::load(x_t + hofs + ic), vxpe = io<T>::load(xl + hofs + ic);
            if (i < R * P) {
                (&sX[0][0])[i] = vxe;
                (&sXp[0][0])[i] = has_carry ? vxpe : 0.f;
            }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int e = 0; e < KPT; ++e) {
            const int k = tid + NT * e, kw = k < KP ? k : KP;   // threads past KP write the spare slot
            float sn, cs;
            sincos_acc(theta_t[(static_cast<size_t>(b) * Gt + gt) * KP + (k < KP ? k : 0)], &sn, &cs);
            sCs[kw] = alpha * cs;
            sSn[kw] = alpha * sn;
        }
        __builtin_amdgcn_sched_barrier(0);
        load_state();
    } else {
        load_state();
        // Keep the staging below behind the state loads (the scheduler would otherwise
        // hoist it, and with it the wait for the small loads, ahead of them).
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int e = 0; e < SPT; ++e) {
            const int i = sidx(e);
            if (i < R * N) {
                (&sB[0][0])[i] = vb[e] * bsc;
                (&sC[0][0])[i] = vc[e];
                (&sBp[0][0])[i] = has_carry ? vbp[e] * bpsc : 0.f;
            }
        }
#pragma unroll
        for (int e = 0; e < XPT; ++e) {
            const int i = xidx(e);
            if (i < R * P) {
                (&sX[0][0])[i] = vx[e];
                (&sXp[0][0])[i] = has_carry ? vxp[e] : 0.f;
            }
        }
#pragma unroll
        for (int e = 0; e < KPT; ++e) {
            // every thread, without a branch, so that the angle load is not moved behind
            // the state loads; threads past KP write the spare slot
            const int k = tid + NT * e, kw = k < KP ? k : KP;
            float sn, cs;
            sincos_acc(vth[e], &sn, &cs);
            sCs[kw] = alpha * cs;
            sSn[kw] = alpha * sn;
        }
    }
    __syncthreads();
    if constexpr (FU) {
        if (fuse) {   // norm and bias of the staged rows with this thread's preloaded weights
            __shared__ float sScale[3 * R];
            bc_scales(&sB[0][0], &sC[0][0], &sBp[0][0], sScale, R, N, NT, fu);
            float* fB = &sB[0][0];
            float* fC = &sC[0][0];
            float* fBp = &sBp[0][0];
#pragma unroll
            for (int e = 0; e < SPT; ++e) {
                const int i = sidx(e);
                if (i < R * N) {
                    const int r = i / N;
                    const float sb = fu.bnw ? sScale[r] : 1.f, sbp = fu.bnw ? sScale[2 * R + r] : 1.f;
                    const float sc = fu.cnw ? sScale[R + r] : 1.f;
                    const float wb = fu.bnw ? wbn[e] : 1.f, wc = fu.cnw ? wcn[e] : 1.f;
                    const float bb = fu.bbias ? wbb[e] : 0.f, cb = fu.cbias ? wcb[e] : 0.f;
                    fB[i] = (fB[i] * (sb * wb) + bb) * c2;
                    fC[i] = fC[i] * (sc * wc) + cb;
                    fBp[i] = has_carry ? (fBp[i] * (sbp * wb) + bb) * c1 : 0.f;
                }
            }
            __syncthreads();
        }
    }

    fvec xv[R], xpv[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        xv[r] = reinterpret_cast<const fvec*>(sX[r])[c];
        xpv[r] = reinterpret_cast<const fvec*>(sXp[r])[c];
    }
    fvec yacc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) yacc[r] = fvec(0.f);

#pragma unroll
    for (int j = 0; j < PPT; ++j) {
        const int k = kk + TPG * j;
        const float cs = sCs[k], sn = sSn[k];   // alpha cos, alpha sin
        fvec v0 = SV::widen(s0[j]), v1 = SV::widen(s1[j]), n0 = fvec(0.f), n1 = n0;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            v0 += sBp[r][2 * k] * xpv[r];       // h + (1 - lambda) dt U_prev
            v1 += sBp[r][2 * k + 1] * xpv[r];
            n0 += sB[r][2 * k] * xv[r];         // gamma U
            n1 += sB[r][2 * k + 1] * xv[r];
        }
        n0 += cs * v0;   // one fused multiply-add each
        n0 -= sn * v1;
        n1 += sn * v0;
        n1 += cs * v1;
        SV::store(hp + (2 * k) * P + CW * c, n0);
        SV::store(hp + (2 * k + 1) * P + CW * c, n1);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            yacc[r] += sC[r][2 * k] * n0;
            yacc[r] += sC[r][2 * k + 1] * n1;
        }
    }

    // Sum the read-out over the threads that share column block c: first the
    // lanes of one wave (stride PC), then the waves through LDS.
#pragma unroll
    for (int off = PC; off < 64 && off < NT; off <<= 1) {
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int q = 0; q < CW; ++q) yacc[r][q] += __shfl_xor(yacc[r][q], off);
    }
    const int lane = tid & 63, wave = tid >> 6;
    if (lane < PC) {
#pragma unroll
        for (int r = 0; r < R; ++r) reinterpret_cast<fvec*>(sY[wave][r])[c] = yacc[r];
    }
    __syncthreads();
    const float dv = D[hh];
    float yo[XPT];
#pragma unroll
    for (int e = 0; e < XPT; ++e) {
        const int i = xidx(e);
        float acc = 0.f;
        if (i < R * P) {
#pragma unroll
            for (int w = 0; w < NW; ++w) acc += (&sY[w][0][0])[i];
            acc += dv * (&sX[0][0])[i];
            if constexpr (FU) {
                if (fu.z) acc *= silu(vz[e]);
            }
        }
        yo[e] = acc;
    }
    if constexpr (FU) {
        if (fu.onw) {   // output RMSNorm over each row of P outputs (uniform branch)
            __shared__ float sO[R * P];
            __shared__ float sRs[R];
#pragma unroll
            for (int e = 0; e < XPT; ++e) {
                const int i = xidx(e);
                if (i < R * P) sO[i] = yo[e];
            }
            __syncthreads();
            row_rms(sO, sRs, R, P, NT, fu.eps);
#pragma unroll
            for (int e = 0; e < XPT; ++e) {
                const int i = xidx(e);
                if (i < R * P) yo[e] *= sRs[i / P] * won[e];
            }
        }
    }
    if constexpr (XRUN) {
        run<T, XPT>::store(y_t + hofs + tid * XPT, yo);
    } else {
#pragma unroll
        for (int e = 0; e < XPT; ++e) {
            const int i = xidx(e);
            if (i < R * P) io<T>::store(y_t + hofs + i, yo[e]);
        }
    }
}

// Any shape: one workgroup per (b, h); each thread owns whole state columns p and
// walks the N/2 rotation pairs of that column.  R <= kMaxRankGeneric.
template <typename T, typename S>
__global__ __launch_bounds__(64) void decode_generic(
    S* __restrict__ h, const T* __restrict__ b_last, const T* __restrict__ x_last,
    const T* __restrict__ x_t, const float* __restrict__ dt_t, const float* __restrict__ A,
    const float* __restrict__ lam_t, const float* __restrict__ theta_t,
    const T* __restrict__ B_t, const T* __restrict__ C_t, const float* __restrict__ D,
    T* __restrict__ y_t, int H, int G, int N, int P, int R, int has_carry, Fusion fu) {
    extern __shared__ float smem[];
    const int KP = N / 2;
    float* sB = smem;               // R*N
    float* sC = sB + R * N;         // R*N
    float* sBp = sC + R * N;        // R*N
    float* sX = sBp + R * N;        // R*P
    float* sXp = sX + R * P;        // R*P
    float* sCs = sXp + R * P;       // KP
    float* sSn = sCs + KP;          // KP
    float* sScale = sSn + KP;       // 3R
    float* sO = sScale + 3 * R;     // R*P outputs (output norm only)
    float* sRs = sO + R * P;        // R

    const int bh = blockIdx.x;
    const int b = bh / H, hh = bh - b * H;
    const int g = hh / (H / G);
    const int Gt = fu.tgroups(G), gt = hh / (H / Gt);   // angle group
    const int tid = threadIdx.x;
    const size_t gofs = (static_cast<size_t>(b) * G + g) * R * N;
    const size_t hofs = static_cast<size_t>(bh) * R * P;
    for (int i = tid; i < R * N; i += blockDim.x) {
        sB[i] = io<T>::load(B_t + gofs + i);
        sC[i] = io<T>::load(C_t + gofs + i);
        sBp[i] = has_carry ? io<T>::load(b_last + gofs + i) : 0.f;
    }
    for (int i = tid; i < R * P; i += blockDim.x) {
        sX[i] = io<T>::load(x_t + hofs + i);
        sXp[i] = has_carry ? io<T>::load(x_last + hofs + i) : 0.f;
    }
    for (int k = tid; k < KP; k += blockDim.x) {
        float sn, cs;
        sincos_acc(theta_t[(static_cast<size_t>(b) * Gt + gt) * KP + k], &sn, &cs);
        sCs[k] = cs;
        sSn[k] = sn;
    }
    __syncthreads();
    if (fu.bc()) fuse_bc(sB, sC, sBp, sScale, R, N, blockDim.x, fu);
    const float dtv = dt_t[bh], lv = lam_t[bh];
    const float alpha = __expf(dtv * (fu.At ? fu.At[bh] : A[hh]));
    const float c1 = (1.f - lv) * dtv, c2 = lv * dtv;
    S* hp = h + static_cast<size_t>(bh) * N * P;
    for (int p = tid; p < P; p += blockDim.x) {
        float yacc[kMaxRankGeneric];
        for (int r = 0; r < R; ++r) yacc[r] = 0.f;
        for (int k = 0; k < KP; ++k) {
            float up0 = 0.f, up1 = 0.f, u0 = 0.f, u1 = 0.f;
            for (int r = 0; r < R; ++r) {
                up0 += sBp[r * N + 2 * k] * sXp[r * P + p];
                up1 += sBp[r * N + 2 * k + 1] * sXp[r * P + p];
                u0 += sB[r * N + 2 * k] * sX[r * P + p];
                u1 += sB[r * N + 2 * k + 1] * sX[r * P + p];
            }
            const float v0 = io<S>::load(hp + (2 * k) * P + p) + c1 * up0;
            const float v1 = io<S>::load(hp + (2 * k + 1) * P + p) + c1 * up1;
            const float n0 = alpha * (sCs[k] * v0 - sSn[k] * v1) + c2 * u0;
            const float n1 = alpha * (sSn[k] * v0 + sCs[k] * v1) + c2 * u1;
            io<S>::store(hp + (2 * k) * P + p, n0);
            io<S>::store(hp + (2 * k + 1) * P + p, n1);
            for (int r = 0; r < R; ++r) yacc[r] += sC[r * N + 2 * k] * n0 + sC[r * N + 2 * k + 1] * n1;
        }
        for (int r = 0; r < R; ++r) {
            float v = yacc[r] + D[hh] * sX[r * P + p];
            if (fu.z) v *= silu(io<T>::load(static_cast<const T*>(fu.z) + hofs + r * P + p));
            if (fu.onw)
                sO[r * P + p] = v;   // stored after the norm below
            else
                io<T>::store(y_t + hofs + r * P + p, v);
        }
    }
    if (fu.onw) {   // output RMSNorm over each row of P outputs
        __syncthreads();
        row_rms(sO, sRs, R, P, blockDim.x, fu.eps);
        for (int i = tid; i < R * P; i += blockDim.x)
            io<T>::store(y_t + hofs + i, sO[i] * sRs[i / P] * fu.onw[hh * P + i % P]);
    }
}

// Dynamic LDS of decode_generic: staged operands, scales, and the outputs of the norm.
static size_t generic_decode_lds(const DecodeArgs& a) {
    return sizeof(float) * (3 * a.R * a.N + 2 * a.R * a.P + a.N + 3 * a.R + a.R * a.P + a.R);
}

// Four columns per thread for either state dtype.  (Eight bf16 columns, for 16-byte
// accesses, measured slower at N = 128, P = 64, R = 4: with half the state bytes the
// step is limited by its fp32 arithmetic, and fewer rows per thread are in flight.)
template <typename T, typename S, int N, int P, int R, int NT, int CW = 4>
static hipError_t launch_fast(const DecodeArgs& a, hipStream_t st) {
    // the fused variant only when a norm, bias, gate or output norm is given (a per-token A
    // or angles per head alone are one scalar or one index per workgroup, read by both)
    const bool fused = a.fu.bc() || a.fu.z || a.fu.onw;
    constexpr bool PACED = std::is_same<S, float>::value;
    auto kernel = fused ? decode_fast<T, S, N, P, R, NT, CW, true, PACED> : decode_fast<T, S, N, P, R, NT, CW, false, PACED>;
    hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>(a.batch * a.H)),
                       dim3(NT), 0, st, static_cast<S*>(a.h), static_cast<const T*>(a.b_last),
                       static_cast<const T*>(a.x_last), static_cast<const T*>(a.x_t), a.dt_t, a.A,
                       a.lam_t, a.theta_t, static_cast<const T*>(a.B_t),
                       static_cast<const T*>(a.C_t), a.D, static_cast<T*>(a.y_t), a.H, a.G,
                       a.has_carry, a.fu);
    return hipGetLastError();
}

template <typename T, typename S>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t st) {
    if (a.N == 128 && a.P == 64) {
        switch (a.R) {
            case 1: return launch_fast<T, S, 128, 64, 1, 256>(a, st);
            case 2: return launch_fast<T, S, 128, 64, 2, 256>(a, st);
            case 4:
                // A bf16 state halves the bytes per element but not the arithmetic: one
                // wave per (b, h), with 16 rotation pairs per thread, spends the fewest
                // instructions outside the per-element work (measured 8% faster than
                // 256 threads; the fp32 state is faster with 256).
                if constexpr (std::is_same<S, bf16_t>::value) return launch_fast<T, S, 128, 64, 4, 64>(a, st);
                else return launch_fast<T, S, 128, 64, 4, 256>(a, st);
            default: break;
        }
    }
    if (a.N == 16 && a.P == 16 && a.R == 1) return launch_fast<T, S, 16, 16, 1, 32>(a, st);
    const size_t shm = generic_decode_lds(a);
    hipLaunchKernelGGL((decode_generic<T, S>), dim3(static_cast<unsigned>(a.batch * a.H)), dim3(64),
                       shm, st, static_cast<S*>(a.h), static_cast<const T*>(a.b_last),
                       static_cast<const T*>(a.x_last), static_cast<const T*>(a.x_t), a.dt_t, a.A,
                       a.lam_t, a.theta_t, static_cast<const T*>(a.B_t),
                       static_cast<const T*>(a.C_t), a.D, static_cast<T*>(a.y_t), a.H, a.G,
                       a.N, a.P, a.R, a.has_carry, a.fu);
    return hipGetLastError();
}

bool decode_supported(const DecodeArgs& a) {
    if (a.R > kMaxRankGeneric) return false;
    return generic_decode_lds(a) <= 64 * 1024;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t st) {
    if (a.state_bf16)
        return a.bf16 ? launch_decode_t<bf16_t, bf16_t>(a, st) : launch_decode_t<float, bf16_t>(a, st);
    return a.bf16 ? launch_decode_t<bf16_t, float>(a, st) : launch_decode_t<float, float>(a, st);
}

}  // namespace m3
