// m3_backward.hip -- backward pass (reverse-mode derivative) of the Mamba-3 scan
// on gfx950, for training.
//
// The forward recurrence is the one of the prefill kernels (Mamba-3 paper note,
// "Solution 1" exponential-trapezoidal update, "Solution 2" rotation of state
// pairs, "Solution 3" rank-R input and output).  Its derivative is taken by the
// adjoint method: with g_t = dLoss/dh_t and q_t = M_t^T g_t (M_t the rotation),
//   g_t  = C_t dy_t^T + alpha_{t+1} q_{t+1}           (the adjoint runs backwards)
//   dU_t = gamma_t g_t + beta_{t+1} q_{t+1}           (U_t = B_t X_t feeds h_t and h_{t+1})
// and every input gradient is a contraction of g_t, q_t, dU_t with the forward
// quantities (see m3_backward below).  The adjoint needs h_{t-1} and h_t at
// every step; they are not stored per token.  The reverse sweep takes segments of
// KS tokens last to first, recomputes each segment's states into LDS from the state
// before it, and walks them backwards.  The states before the segments come from
// checkpoints in two levels: a forward sweep keeps h after every group of `grp`
// segments in the workspace, and before a group is reversed the states after each
// of its segments are recomputed from the group's checkpoint into a per-workgroup
// scratch.  With grp = 1 (whenever a checkpoint after every segment fits the
// workspace budget) there is no second level; otherwise grp is about the square root
// of the segments of a part, which keeps the workspace near 2 sqrt(L / KS) states per
// (b, h) for one more forward pass.  The inputs of a segment's tokens (and of the
// token before it) are staged into LDS once per segment by the whole workgroup in
// 16-byte units, so the per-token steps read their operands from LDS, not from
// global memory.
//
// Sequence split.  Both recurrences are linear: over a piece of the sequence the
// state maps as h_end = e^{sum dt A} R(sum theta) h_start + (the piece's own end
// state from a zero start), and the adjoint at the piece's first token is the
// piece's own (from a zero cotangent) plus a decayed, counter-rotated copy of
// the adjoint entering from the right.  When few (batch, head) pairs would leave
// CUs idle, each sequence is cut into pieces of whole segments: a local pass
// gives every piece its two own terms and its sums of dt A and theta (in fp64,
// the angles reduced mod 2 pi), a combine pass chains them into the state and the
// adjoint each piece starts from, and the gradient pass runs every piece at once.
//
// One workgroup per (batch, head) and piece, 512 threads; thread t owns state rows
// 4 (t >> 4) .. +3 (two rotation pairs) and columns 4 (t & 15) .. +3, of h and of
// the adjoint, in registers.  Sums over columns (dB, dC, dtheta) are taken
// within the 16 lanes that share rows, by DPP lane exchanges; sums over rows
// (dX) and over the whole state (dalpha, dbeta, dgamma) go through LDS, one
// barrier per token.  Gradients of inputs shared by the heads of a group (B, C,
// theta, the carried B) are written per head and summed by a second kernel in a
// fixed order, so results do not depend on scheduling.  All gradients are fp32.
#include <cmath>

#include "m3_common.h"
#include "m3_internal.h"

namespace m3 {
namespace bw {

constexpr int N = 128;
constexpr int P = 64;
constexpr int NT = 512;
constexpr int KS = 3;           // tokens per recompute segment
constexpr int PS = P;           // row of a state in LDS (a 16-lane group reads or writes one row)

template <typename T> struct ld;
template <> struct ld<float> {
    __device__ __forceinline__ static void v4(const float* p, float* o) {
        const float4 v = *reinterpret_cast<const float4*>(p);
        o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
    }
};
template <> struct ld<bf16_t> {
    __device__ __forceinline__ static void v4(const bf16_t* p, float* o) {
        const uint2 v = *reinterpret_cast<const uint2*>(p);
        o[0] = __uint_as_float(v.x << 16); o[1] = __uint_as_float(v.x & 0xffff0000u);
        o[2] = __uint_as_float(v.y << 16); o[3] = __uint_as_float(v.y & 0xffff0000u);
    }
};

// Sum over the 16 lanes of a DPP row (the lanes that share state rows); every lane gets it.
__device__ __forceinline__ float sum16(float v) {
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));   // lane ^ 1
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true));   // lane ^ 2
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, true));  // half-row mirror
    v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x128, 0xF, 0xF, true));  // row rotate by 8
    return v;
}
// Sum over the 64 lanes of a wave; valid in lane 63.
__device__ __forceinline__ float sum64(float v) {
    v = sum16(v);
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xA, 0xF, false));  // row_bcast:15
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xC, 0xF, false));  // row_bcast:31
    return v;
}
// Sum over the 4 DPP rows of a wave (lanes 16 and 32 apart); every lane gets it.
__device__ __forceinline__ float sum_rows(float v) {
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    return v;
}

template <typename T> struct lds4;
template <> struct lds4<float> {
    __device__ __forceinline__ static void get(const float* p, float* o) {
        const float4 v = *reinterpret_cast<const float4*>(p);
        o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
    }
};
template <> struct lds4<bf16_t> {
    __device__ __forceinline__ static void get(const bf16_t* p, float* o) {
        const uint2 v = *reinterpret_cast<const uint2*>(p);
        o[0] = __uint_as_float(v.x << 16); o[1] = __uint_as_float(v.x & 0xffff0000u);
        o[2] = __uint_as_float(v.y << 16); o[3] = __uint_as_float(v.y & 0xffff0000u);
    }
};

// LOCAL: the first pass of a split sequence (see launch_backward): for one part, the
// forward sweep from a zero state and the adjoint sweep from a zero cotangent, with
// the part's sums of dt*A and of theta.  Otherwise the gradient pass over one part
// (the whole sequence when it is not split).
template <typename T, int R, bool LOCAL>
__global__ __launch_bounds__(NT) void bwd_scan(BwdArgs a) {
    const int64_t BH = a.batch * a.H;
    const int bh = static_cast<int>(blockIdx.x % BH), part = static_cast<int>(blockIdx.x / BH);
    const int b = bh / a.H, h = bh - b * a.H, g = h / (a.H / a.G);
    const int tid = threadIdx.x, cb = tid & 15, pb = tid >> 4, lane = tid & 63, wv = tid >> 6;
    const int r0 = 4 * pb, c0 = 4 * cb;   // state rows r0 .. r0+3 (two rotation pairs), columns c0 .. c0+3
    // This sequence's tokens: b * L .. + L, or those of packed sequence b (clamped as the
    // prefill clamps them)
    const SeqSpan span = seq_span(a.cu, b, a.L, a.T);
    const int64_t tb = span.start, L = span.len;
    const int H = a.H, G = a.G;
    const float Ah = a.At ? 0.f : a.A[h], Dh = a.D[h];   // Ah: the head's decay rate without At
    const int64_t nseg = (L + KS - 1) / KS;                    // segments of this sequence
    const int64_t s_lo = part * a.seg_per_part;
    const int64_t s_hi = s_lo + a.seg_per_part < nseg ? s_lo + a.seg_per_part : nseg;   // segments of this part
    const bool split = a.parts > 1;
    const size_t pidx = static_cast<size_t>(bh) * a.parts + part;
    const int64_t grp = a.grp, gpp = (a.seg_per_part + grp - 1) / grp;   // groups per part
    float* ck = a.ckpt + pidx * gpp * N * P;         // state after group u of this part: ck[u]
    float* scr = a.scratch + pidx * grp * N * P;     // state after segment i of the group being reversed
    const bool carry = a.bl && a.xl;
    const T* x = static_cast<const T*>(a.x);
    const T* dy = static_cast<const T*>(a.dy);
    const T* Bm = static_cast<const T*>(a.B);
    const T* Cm = static_cast<const T*>(a.C);
    const T* blp = static_cast<const T*>(a.bl);
    const T* xlp = static_cast<const T*>(a.xl);
    // group-shared gradients go to per-head rows when heads share a group
    const int gh = a.per_head ? h : g, GH = a.per_head ? H : G;

    __shared__ __align__(16) float sH[LOCAL ? 1 : KS][LOCAL ? 4 : N * PS];   // states h_{t0-1} .. h_{t0+len-2}
    __shared__ __align__(16) float sDX[2][NT / 64][LOCAL ? 4 : R * P];       // per-wave dX sums, by token parity
    __shared__ float sSc[2][NT / 64][4];                         // per-wave dalpha, dbeta, dgamma, dD
    // inputs of tokens t0-1 .. t0+KS-1 (slot k holds token t0 - 1 + k)
    __shared__ __align__(16) T sB[KS + 1][R * N];
    __shared__ __align__(16) T sC[KS + 1][R * N];
    __shared__ __align__(16) T sX[KS + 1][R * P];
    __shared__ __align__(16) T sDY[KS + 1][R * P];
    __shared__ __align__(16) float sTh[KS + 1][N / 2];
    __shared__ __align__(16) float sRot[KS + 1][N];             // cos, sin of each pair's angle
    __shared__ float sDt[KS + 1], sLam[KS + 1], sAt[KS + 1];   // sAt: decay rate of each token

    auto soff = [&](int64_t t) { return (tb + t) * H + h; };

    // Tokens t0-1 .. t0+len-1 into slots 0 .. len, in 16-byte units spread over the
    // workgroup; token -1 is the carried previous input (B and X only), or zeros.
    auto stage = [&](int64_t t0, int len, bool with_cdy, bool with_bx = true) {
        constexpr int E = 16 / static_cast<int>(sizeof(T));
        constexpr int uB = R * N / E, uX = R * P / E, uT = (N / 2) / 4;
        constexpr int upt = 2 * uB + 2 * uX + uT;
        const int total = upt * (len + 1);
        for (int u = tid; u < total; u += NT) {
            const int k = u / upt, w = u - k * upt;
            const int64_t t = t0 - 1 + k;
            uint4 v = {0u, 0u, 0u, 0u};
            void* dst;
            if (w < uB) {
                const int o = w * E;
                dst = &sB[k][o];
                if (t >= 0 && with_bx) v = *reinterpret_cast<const uint4*>(Bm + ((tb + t) * G + g) * (R * N) + o);
                else if (carry && with_bx) v = *reinterpret_cast<const uint4*>(blp + (static_cast<int64_t>(b) * G + g) * (R * N) + o);
            } else if (w < 2 * uB) {
                const int o = (w - uB) * E;
                dst = &sC[k][o];
                if (t >= 0 && with_cdy)
                    v = *reinterpret_cast<const uint4*>(Cm + ((tb + t) * G + g) * (R * N) + o);
            } else if (w < 2 * uB + uX) {
                const int o = (w - 2 * uB) * E;
                dst = &sX[k][o];
                if (t >= 0 && with_bx) v = *reinterpret_cast<const uint4*>(x + ((tb + t) * H + h) * (R * P) + o);
                else if (carry && with_bx) v = *reinterpret_cast<const uint4*>(xlp + (static_cast<int64_t>(b) * H + h) * (R * P) + o);
            } else if (w < 2 * uB + 2 * uX) {
                const int o = (w - 2 * uB - uX) * E;
                dst = &sDY[k][o];
                if (t >= 0 && with_cdy)
                    v = *reinterpret_cast<const uint4*>(dy + ((tb + t) * H + h) * (R * P) + o);
            } else {
                const int o = (w - 2 * uB - 2 * uX) * 4;
                dst = &sTh[k][o];
                if (t >= 0) v = *reinterpret_cast<const uint4*>(a.theta + ((tb + t) * G + g) * (N / 2) + o);
                // the rotation of these four pairs, once per token for the whole workgroup
                const float th[4] = {__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w)};
                float cs4[4], sn4[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) sincos_acc(th[e], &sn4[e], &cs4[e]);
                *reinterpret_cast<float4*>(&sRot[k][2 * o]) = float4{cs4[0], sn4[0], cs4[1], sn4[1]};
                *reinterpret_cast<float4*>(&sRot[k][2 * o + 4]) = float4{cs4[2], sn4[2], cs4[3], sn4[3]};
            }
            *reinterpret_cast<uint4*>(dst) = v;
        }
        if (tid <= len) {
            const int64_t t = t0 - 1 + tid;
            sDt[tid] = t >= 0 ? a.dt[soff(t)] : 0.f;
            sLam[tid] = t >= 0 ? a.lam[soff(t)] : 0.f;
            sAt[tid] = t >= 0 ? (a.At ? a.At[soff(t)] : Ah) : 0.f;
        }
    };
    // The staging of the forward sweeps (B, X and theta; C and dy are not read there) split
    // in two: fetch issues a segment's loads into registers, commit writes them to the
    // slots.  A sweep fetches the next segment before stepping through the current one, so
    // the loads are in flight during its steps.  Every load is unconditional (an index
    // clamped into the sequence; `use` says whether the value counts), so the compiler has
    // no branch join at which to wait for it.
    constexpr int kE = 16 / static_cast<int>(sizeof(T));
    constexpr int kuB = R * N / kE, kuX = R * P / kE, kuT = (N / 2) / 4;
    constexpr int kUF = kuB + kuX + kuT;                   // units per token
    constexpr int kUnits = (kUF * (KS + 1) + NT - 1) / NT; // units per thread
    struct Pref {
        uint4 v[kUnits];
        unsigned use;     // bit e: unit e holds a value (else zeros are staged)
        float dt, lam, at;
    };
    auto fetch = [&](int64_t t0, int len, Pref& pf) {
        const int total = kUF * (len + 1);
        pf.use = 0;
#pragma unroll
        for (int e = 0; e < kUnits; ++e) {
            const int u = tid + NT * e;
            const int uc = u < total ? u : 0;
            const int k = uc / kUF, w = uc - k * kUF;
            const int64_t t = t0 - 1 + k;
            const int64_t tc = t >= 0 ? t : 0;   // a token of this sequence (len >= 1)
            const bool from_carry = t < 0 && carry;
            const uint4* src;
            bool use;
            if (w < kuB) {
                const int o = w * kE;
                src = reinterpret_cast<const uint4*>(from_carry ? blp + (static_cast<int64_t>(b) * G + g) * (R * N) + o
                                                                : Bm + ((tb + tc) * G + g) * (R * N) + o);
                use = t >= 0 || carry;
            } else if (w < kuB + kuX) {
                const int o = (w - kuB) * kE;
                src = reinterpret_cast<const uint4*>(from_carry ? xlp + (static_cast<int64_t>(b) * H + h) * (R * P) + o
                                                                : x + ((tb + tc) * H + h) * (R * P) + o);
                use = t >= 0 || carry;
            } else {
                const int o = (w - kuB - kuX) * 4;
                src = reinterpret_cast<const uint4*>(a.theta + ((tb + tc) * G + g) * (N / 2) + o);
                use = t >= 0;
            }
            pf.v[e] = *src;
            if (use && u < total) pf.use |= 1u << e;
        }
        const int64_t t = t0 - 1 + (tid <= len ? tid : 0);
        const int64_t tc = t >= 0 ? t : 0;
        pf.dt = a.dt[soff(tc)];
        pf.lam = a.lam[soff(tc)];
        pf.at = a.At ? a.At[soff(tc)] : Ah;
        if (t < 0) pf.dt = pf.lam = pf.at = 0.f;
    };
    auto commit = [&](int len, const Pref& pf) {
        const int total = kUF * (len + 1);
#pragma unroll
        for (int e = 0; e < kUnits; ++e) {
            const int u = tid + NT * e;
            if (u >= total) continue;
            const int k = u / kUF, w = u - k * kUF;
            const uint4 v = (pf.use >> e) & 1u ? pf.v[e] : uint4{0u, 0u, 0u, 0u};
            void* dst;
            if (w < kuB) {
                dst = &sB[k][w * kE];
            } else if (w < kuB + kuX) {
                dst = &sX[k][(w - kuB) * kE];
            } else {
                const int o = (w - kuB - kuX) * 4;
                dst = &sTh[k][o];
                const float th[4] = {__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w)};
                float cs4[4], sn4[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) sincos_acc(th[q], &sn4[q], &cs4[q]);
                *reinterpret_cast<float4*>(&sRot[k][2 * o]) = float4{cs4[0], sn4[0], cs4[1], sn4[1]};
                *reinterpret_cast<float4*>(&sRot[k][2 * o + 4]) = float4{cs4[2], sn4[2], cs4[3], sn4[3]};
            }
            *reinterpret_cast<uint4*>(dst) = v;
        }
        if (tid <= len) {
            sDt[tid] = pf.dt;
            sLam[tid] = pf.lam;
            sAt[tid] = pf.at;
        }
    };
    auto slot_bx = [&](int k, float (&Bv)[R][4], float (&Xv)[R][4]) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            lds4<T>::get(&sB[k][r * N + r0], Bv[r]);
            lds4<T>::get(&sX[k][r * P + c0], Xv[r]);
        }
    };
    auto uval = [&](const float (&Bv)[R][4], const float (&Xv)[R][4], int i, int j) {
        float u = 0.f;
#pragma unroll
        for (int r = 0; r < R; ++r) u += Bv[r][i] * Xv[r][j];
        return u;
    };
    auto coeffs = [&](int k, float* al, float* be, float* ga, float* sn, float* cs) {
        const float dtv = sDt[k], lv = sLam[k];
        *al = __expf(dtv * sAt[k]);
        *be = (1.f - lv) * dtv * *al;
        *ga = lv * dtv;
        const float4 rot = *reinterpret_cast<const float4*>(&sRot[k][4 * pb]);   // pairs 2pb, 2pb+1
        cs[0] = rot.x;
        sn[0] = rot.y;
        cs[1] = rot.z;
        sn[1] = rot.w;
    };
    // one forward step on hs for the token in slot k: h <- M (alpha h + beta U_{t-1}) + gamma U_t
    auto fwd_step = [&](int k, float (&hs)[4][4]) {
        float Bp[R][4], Xp[R][4], Bv[R][4], Xv[R][4];
        slot_bx(k - 1, Bp, Xp);
        slot_bx(k, Bv, Xv);
        float al, be, ga, sn[2], cs[2];
        coeffs(k, &al, &be, &ga, sn, cs);
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float v0 = al * hs[2 * q][j] + be * uval(Bp, Xp, 2 * q, j);
                const float v1 = al * hs[2 * q + 1][j] + be * uval(Bp, Xp, 2 * q + 1, j);
                hs[2 * q][j] = cs[q] * v0 - sn[q] * v1 + ga * uval(Bv, Xv, 2 * q, j);
                hs[2 * q + 1][j] = sn[q] * v0 + cs[q] * v1 + ga * uval(Bv, Xv, 2 * q + 1, j);
            }
    };
    auto load_state = [&](float (&hs)[4][4], const float* src, int stride) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float4 u = *reinterpret_cast<const float4*>(src + (r0 + i) * stride + c0);
            hs[i][0] = u.x; hs[i][1] = u.y; hs[i][2] = u.z; hs[i][3] = u.w;
        }
    };
    auto store_state = [&](const float (&hs)[4][4], float* dst, int stride) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *reinterpret_cast<float4*>(dst + (r0 + i) * stride + c0) = float4{hs[i][0], hs[i][1], hs[i][2], hs[i][3]};
    };
    auto initial_state = [&](float (&hs)[4][4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                hs[i][j] = a.h0 ? state_load(a.h0, (static_cast<size_t>(bh) * N + r0 + i) * P + c0 + j, a.state_bf16)
                                : 0.f;
    };

    if constexpr (LOCAL) {
        // ---- forward sweep of the part from a zero state (the token before the part
        // still feeds its first update through U_{t-1})
        float hs[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) hs[i][j] = 0.f;
        double sum = 0.0;   // thread i < N/2: theta of pair i; thread N/2: dt * A (as the steps round it)
        auto seg_len = [&](int64_t s) { return static_cast<int>(L - s * KS < KS ? L - s * KS : KS); };
        Pref pf;
        if (s_lo < s_hi) fetch(s_lo * KS, seg_len(s_lo), pf);
        for (int64_t s = s_lo; s < s_hi; ++s) {
            const int len = seg_len(s);
            __syncthreads();
            commit(len, pf);
            __syncthreads();
            if (s + 1 < s_hi) fetch((s + 1) * KS, seg_len(s + 1), pf);   // in flight during the steps
            for (int j = 1; j <= len; ++j) fwd_step(j, hs);
            if (tid < N / 2) {
                for (int j = 1; j <= len; ++j) sum += static_cast<double>(sTh[j][tid]);
            } else if (tid == N / 2) {
                for (int j = 1; j <= len; ++j) sum += static_cast<double>(sDt[j] * sAt[j]);
            }
        }
        store_state(hs, a.hloc + pidx * N * P, P);
        constexpr double kTwoPi = 6.283185307179586;
        if (tid < N / 2) a.ang[pidx * (N / 2) + tid] = static_cast<float>(sum - kTwoPi * floor(sum / kTwoPi));
        else if (tid == N / 2) a.dec[pidx] = sum;
        // ---- adjoint sweep of the part from a zero cotangent: g_t = C_t dy_t^T + alpha_{t+1} q_{t+1},
        // q_t = M_t^T g_t; the result is the part's share of q at its first token
        float qs[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) qs[i][j] = 0.f;
        float an = 0.f;
        for (int64_t s = s_hi - 1; s >= s_lo; --s) {
            const int64_t t0 = s * KS;
            const int len = static_cast<int>(L - t0 < KS ? L - t0 : KS);
            __syncthreads();
            stage(t0, len, true, false);
            __syncthreads();
            for (int j = len - 1; j >= 0; --j) {
                const int k = j + 1;
                float al, be, ga, sn[2], cs[2];
                coeffs(k, &al, &be, &ga, sn, cs);
                float Cv[R][4], dyv[R][4];
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    lds4<T>::get(&sC[k][r * N + r0], Cv[r]);
                    lds4<T>::get(&sDY[k][r * P + c0], dyv[r]);
                }
#pragma unroll
                for (int q = 0; q < 2; ++q)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        float g0 = an * qs[2 * q][jj], g1 = an * qs[2 * q + 1][jj];
#pragma unroll
                        for (int r = 0; r < R; ++r) {
                            g0 += Cv[r][2 * q] * dyv[r][jj];
                            g1 += Cv[r][2 * q + 1] * dyv[r][jj];
                        }
                        qs[2 * q][jj] = cs[q] * g0 + sn[q] * g1;
                        qs[2 * q + 1][jj] = -sn[q] * g0 + cs[q] * g1;
                    }
                an = al;
            }
        }
        store_state(qs, a.qloc + pidx * N * P, P);
        return;
    }

    // ---- forward sweep: checkpoint after the last segment of every group (the last group's
    // end is never a starting point).  A part after the first starts from the state the
    // combine pass left for it.
    float hc[4][4];
    auto part_start = [&](float (&hs)[4][4]) {
        if (split) load_state(hs, a.hloc + pidx * N * P, P);
        else initial_state(hs);
    };
    part_start(hc);
    // forward steps of segments s0 .. s1-1 on hs; with `dst`, the state after segment s is
    // stored at dst[(s - s0 - 1 + off) ...] as described at the call
    auto seg_len = [&](int64_t s) { return static_cast<int>(L - s * KS < KS ? L - s * KS : KS); };
    auto sweep = [&](float (&hs)[4][4], int64_t s0, int64_t s1, auto&& after) {
        Pref pf;
        if (s0 < s1) fetch(s0 * KS, seg_len(s0), pf);
        for (int64_t s = s0; s < s1; ++s) {
            const int len = seg_len(s);
            __syncthreads();   // the previous segment's slots are read
            commit(len, pf);
            __syncthreads();
            if (s + 1 < s1) fetch((s + 1) * KS, seg_len(s + 1), pf);   // in flight during the steps
            for (int j = 1; j <= len; ++j) fwd_step(j, hs);
            after(s, hs);
        }
    };
    sweep(hc, s_lo, s_hi, [&](int64_t s, const float (&hs)[4][4]) {
        const int64_t i = s - s_lo;
        if (i % grp == grp - 1 && s + 1 < s_hi) store_state(hs, ck + (i / grp) * N * P, P);
    });

    // ---- reverse sweep.  q_{t+1}, alpha_{t+1}, beta_{t+1} belong to the token after; the
    // final-state cotangent enters as a token after the last one with alpha = 1, beta = 0 and
    // no rotation.  A part before the last starts from the q of the next part's first
    // token (left by the combine pass) and that token's alpha and beta.
    float qn[4][4];
    if (split) {
        load_state(qn, a.qloc + pidx * N * P, P);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                qn[i][j] = a.dh_out ? a.dh_out[(static_cast<size_t>(bh) * N + r0 + i) * P + c0 + j] : 0.f;
    }
    float an = 1.f, bn = 0.f;
    if (s_hi < nseg) {
        const int64_t tn = s_hi * KS;
        const float dtv = a.dt[soff(tn)], lv = a.lam[soff(tn)];
        an = __expf(dtv * (a.At ? a.At[soff(tn)] : Ah));
        bn = (1.f - lv) * dtv * an;
    }
    float dA_acc = 0.f, dD_acc = 0.f;   // thread 0

    const int64_t ngrp = (s_hi - s_lo + grp - 1) / grp;
    for (int64_t u = ngrp - 1; u >= 0; --u) {
    const int64_t g_lo = s_lo + u * grp, g_hi = g_lo + grp < s_hi ? g_lo + grp : s_hi;
    auto group_start = [&](float (&hs)[4][4]) {
        if (u > 0) load_state(hs, ck + (u - 1) * N * P, P);
        else part_start(hs);
    };
    if (g_hi - g_lo > 1) {   // the states after segments g_lo .. g_hi-2, into the scratch
        float hg[4][4];
        group_start(hg);
        sweep(hg, g_lo, g_hi - 1, [&](int64_t s, const float (&hs)[4][4]) { store_state(hs, scr + (s - g_lo) * N * P, P); });
    }
    for (int64_t s = g_hi - 1; s >= g_lo; --s) {
        const int64_t t0 = s * KS;
        const int len = static_cast<int>(L - t0 < KS ? L - t0 : KS);
        __syncthreads();   // the previous segment's readers are done with sH and the slots
        stage(t0, len, true);
        __syncthreads();
        {   // recompute h_{t0-1} .. h_{t0+len-2} into LDS
            float hr[4][4];
            if (s > g_lo) load_state(hr, scr + (s - 1 - g_lo) * N * P, P);
            else group_start(hr);
            store_state(hr, sH[0], PS);
            for (int j = 1; j < len; ++j) {
                fwd_step(j, hr);
                store_state(hr, sH[j], PS);
            }
        }
        __syncthreads();

        for (int j = len - 1; j >= 0; --j) {
            const int64_t t = t0 + j;
            const int par = static_cast<int>(t & 1);
            const int k = j + 1;   // slot of token t (slot j holds token t - 1)
            float al, be, ga, sn[2], cs[2];
            coeffs(k, &al, &be, &ga, sn, cs);
            float Bv[R][4], Xv[R][4];
            slot_bx(k, Bv, Xv);

            // (1) g_t = alpha_{t+1} q_{t+1} + C_t dy_t^T; dU_t; dgamma; dC_t = h_t dy_t; dD
            float gg[4][4], dU[4][4], dC[R][4];
            float dga = 0.f, dDp = 0.f;
            {
                float Cv[R][4], dyv[R][4];
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    lds4<T>::get(&sC[k][r * N + r0], Cv[r]);
                    lds4<T>::get(&sDY[k][r * P + c0], dyv[r]);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        float v = an * qn[i][jj];
#pragma unroll
                        for (int r = 0; r < R; ++r) v += Cv[r][i] * dyv[r][jj];
                        gg[i][jj] = v;
                        dU[i][jj] = ga * v + bn * qn[i][jj];
                        dga += v * uval(Bv, Xv, i, jj);
                    }
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        float c = 0.f;
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj) c += hc[i][jj] * dyv[r][jj];
                        dC[r][i] = c;
                    }
                if (pb == 0) {
#pragma unroll
                    for (int r = 0; r < R; ++r)
#pragma unroll
                        for (int jj = 0; jj < 4; ++jj) dDp += dyv[r][jj] * Xv[r][jj];
                }
            }
            // (2) q_t = M_t^T g_t; dalpha, dbeta, dtheta (needs h_{t-1} and U_{t-1})
            float dal = 0.f, dbe = 0.f, dth[2] = {0.f, 0.f};
            {
                float Bp[R][4], Xp[R][4];
                slot_bx(k - 1, Bp, Xp);
                load_state(hc, sH[j], PS);   // hc <- h_{t-1} (h_t is no longer needed)
#pragma unroll
                for (int q = 0; q < 2; ++q)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const float g0 = gg[2 * q][jj], g1 = gg[2 * q + 1][jj];
                        const float q0 = cs[q] * g0 + sn[q] * g1, q1 = -sn[q] * g0 + cs[q] * g1;
                        qn[2 * q][jj] = q0;
                        qn[2 * q + 1][jj] = q1;
                        const float h0v = hc[2 * q][jj], h1v = hc[2 * q + 1][jj];
                        const float u0 = uval(Bp, Xp, 2 * q, jj), u1 = uval(Bp, Xp, 2 * q + 1, jj);
                        dal += q0 * h0v + q1 * h1v;
                        dbe += q0 * u0 + q1 * u1;
                        const float v0 = al * h0v + be * u0, v1 = al * h1v + be * u1;
                        dth[q] += q1 * v0 - q0 * v1;
                    }
            }
            // (3) dB_t = dU_t X_t^T, dX_t = B_t^T dU_t
            float dB[R][4], dX[R][4];
#pragma unroll
            for (int r = 0; r < R; ++r) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float d = 0.f;
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) d += dU[i][jj] * Xv[r][jj];
                    dB[r][i] = d;
                }
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    float v = 0.f;
#pragma unroll
                    for (int i = 0; i < 4; ++i) v += Bv[r][i] * dU[i][jj];
                    dX[r][jj] = v;
                }
            }

            // sums over columns (the 16 lanes of a row): dB, dC, dtheta
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    dC[r][i] = sum16(dC[r][i]);
                    dB[r][i] = sum16(dB[r][i]);
                }
            dth[0] = sum16(dth[0]);
            dth[1] = sum16(dth[1]);
            {
                const int64_t go = ((tb + t) * GH + gh) * (R * N);
                float* dCo = a.per_head ? a.dC_part : a.dC;
                float* dBo = a.per_head ? a.dB_part : a.dB;
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        if (((r * 4 + i) & 15) == cb) {
                            dCo[go + r * N + r0 + i] = dC[r][i];
                            dBo[go + r * N + r0 + i] = dB[r][i];
                        }
                    }
                float* dTo = a.per_head ? a.dtheta_part : a.dtheta;
                if (cb < 2) dTo[((tb + t) * GH + gh) * (N / 2) + 2 * pb + cb] = cb ? dth[1] : dth[0];
            }
            // sums over rows: dX within the wave, then across waves through LDS; scalars per wave
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) dX[r][jj] = sum_rows(dX[r][jj]);
            if (lane < 16) {
#pragma unroll
                for (int r = 0; r < R; ++r)
                    *reinterpret_cast<float4*>(&sDX[par][wv][r * P + c0]) = float4{dX[r][0], dX[r][1], dX[r][2], dX[r][3]};
            }
            dal = sum64(dal);
            dbe = sum64(dbe);
            dga = sum64(dga);
            dDp = sum64(dDp);
            if (lane == 63) {
                sSc[par][wv][0] = dal;
                sSc[par][wv][1] = dbe;
                sSc[par][wv][2] = dga;
                sSc[par][wv][3] = dDp;
            }
            __syncthreads();
            for (int o = tid; o < R * P; o += NT) {
                float v = 0.f;
#pragma unroll
                for (int w2 = 0; w2 < NT / 64; ++w2) v += sDX[par][w2][o];
                const int64_t xi = ((tb + t) * H + h) * (R * P) + o;
                a.dx[xi] = v + Dh * io<T>::load(reinterpret_cast<const T*>(&sDY[k][o]));
            }
            if (tid == 0) {
                float sa = 0.f, sb = 0.f, sg = 0.f, sd = 0.f;
#pragma unroll
                for (int w2 = 0; w2 < NT / 64; ++w2) {
                    sa += sSc[par][w2][0];
                    sb += sSc[par][w2][1];
                    sg += sSc[par][w2][2];
                    sd += sSc[par][w2][3];
                }
                const float dtv = sDt[k], lv = sLam[k], av = sAt[k];
                a.ddt[soff(t)] = sa * av * al + sb * (1.f - lv) * (al + dtv * av * al) + sg * lv;
                a.dlam[soff(t)] = -sb * dtv * al + sg * dtv;
                const float dav = sa * dtv * al + sb * (1.f - lv) * dtv * dtv * al;
                if (a.At) a.dA[soff(t)] = dav;   // per-token rate: its own gradient
                else dA_acc += dav;
                dD_acc += sd;
            }
            an = al;
            bn = be;
        }
    }
    }

    // ---- h_0 and the carried previous input (dU_0 = beta_1 q_1): the first part only
    if (part == 0 && a.dh0) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) a.dh0[(static_cast<size_t>(bh) * N + r0 + i) * P + c0 + j] = an * qn[i][j];
    }
    if (part != 0) {
        // nothing before this part
    } else if (carry && (a.dbl || a.dxl)) {
        float Bv[R][4], Xv[R][4], dB[R][4], dX[R][4];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            ld<T>::v4(blp + ((static_cast<int64_t>(b) * G + g) * R + r) * N + r0, Bv[r]);
            ld<T>::v4(xlp + ((static_cast<int64_t>(b) * H + h) * R + r) * P + c0, Xv[r]);
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float d = 0.f;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) d += bn * qn[i][jj] * Xv[r][jj];
                dB[r][i] = sum16(d);
            }
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                float v = 0.f;
#pragma unroll
                for (int i = 0; i < 4; ++i) v += Bv[r][i] * bn * qn[i][jj];
                dX[r][jj] = sum_rows(v);
            }
        }
        if (a.dbl) {
            float* dBo = a.per_head ? a.dbl_part : a.dbl;
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (((r * 4 + i) & 15) == cb) dBo[((static_cast<int64_t>(b) * GH + gh) * R + r) * N + r0 + i] = dB[r][i];
        }
        __syncthreads();
        if (lane < 16) {
#pragma unroll
            for (int r = 0; r < R; ++r)
                *reinterpret_cast<float4*>(&sDX[0][wv][r * P + c0]) = float4{dX[r][0], dX[r][1], dX[r][2], dX[r][3]};
        }
        __syncthreads();
        if (a.dxl) {
            for (int o = tid; o < R * P; o += NT) {
                float v = 0.f;
#pragma unroll
                for (int w2 = 0; w2 < NT / 64; ++w2) v += sDX[0][w2][o];
                a.dxl[static_cast<size_t>(bh) * R * P + o] = v;
            }
        }
    } else if (a.dxl) {
        for (int o = tid; o < R * P; o += NT) a.dxl[static_cast<size_t>(bh) * R * P + o] = 0.f;
    }
    if (tid == 0) {
        a.dA_part[pidx] = dA_acc;
        a.dD_part[pidx] = dD_acc;
    }
}

// Combine pass of a split sequence, one workgroup per (b, h), same element ownership as
// bwd_scan.  The state after part p is e^{dec_p} R(ang_p) (state before it) plus the
// part's local end state; the q at the first token of part p is the part's local q plus
// (product of alpha over tokens T_p+1 .. T_{p+1}) R(-ang_p) (q at T_{p+1}), where the
// alpha after the last token is 1 and the final-state cotangent is the q there.  Each
// part's slots of hloc and qloc are overwritten with what it starts from: the state
// before its first token and the q of the token after its last.
__global__ __launch_bounds__(NT) void bwd_combine(BwdArgs a) {
    const int bh = blockIdx.x;
    const int b = bh / a.H, h = bh - b * a.H;
    const int tid = threadIdx.x, cb = tid & 15, pb = tid >> 4;
    const int r0 = 4 * pb, c0 = 4 * cb;
    const int S = a.parts;
    const float Ah = a.At ? 0.f : a.A[h];
    const int64_t tok_per_part = a.seg_per_part * KS;
    const SeqSpan span = seq_span(a.cu, b, a.L, a.T);   // a packed sequence may leave trailing parts empty
    auto dta = [&](int64_t t) {   // dt A at token t of the sequence; 0 (alpha = 1) past its end
        if (t >= span.len) return 0.0;
        const int64_t i = (span.start + t) * a.H + h;
        return static_cast<double>(a.dt[i] * (a.At ? a.At[i] : Ah));
    };
    auto slot = [&](float* base, int p) { return base + ((static_cast<size_t>(bh) * S + p) * N + r0) * P + c0; };
    auto ld16 = [&](const float* p, float (&v)[4][4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float4 u = *reinterpret_cast<const float4*>(p + i * P);
            v[i][0] = u.x; v[i][1] = u.y; v[i][2] = u.z; v[i][3] = u.w;
        }
    };
    auto st16 = [&](float* p, const float (&v)[4][4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) *reinterpret_cast<float4*>(p + i * P) = float4{v[i][0], v[i][1], v[i][2], v[i][3]};
    };

    float st[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            st[i][j] = a.h0 ? state_load(a.h0, (static_cast<size_t>(bh) * N + r0 + i) * P + c0 + j, a.state_bf16) : 0.f;
    for (int p = 0; p < S; ++p) {
        float* sp = slot(a.hloc, p);
        float hl[4][4];
        ld16(sp, hl);
        st16(sp, st);
        if (p + 1 == S) break;
        const float d = static_cast<float>(exp(a.dec[static_cast<size_t>(bh) * S + p]));
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            float sn, cs;
            sincos_acc(a.ang[(static_cast<size_t>(bh) * S + p) * (N / 2) + 2 * pb + q], &sn, &cs);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float v0 = st[2 * q][j], v1 = st[2 * q + 1][j];
                st[2 * q][j] = d * (cs * v0 - sn * v1) + hl[2 * q][j];
                st[2 * q + 1][j] = d * (sn * v0 + cs * v1) + hl[2 * q + 1][j];
            }
        }
    }

    float qs[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            qs[i][j] = a.dh_out ? a.dh_out[(static_cast<size_t>(bh) * N + r0 + i) * P + c0 + j] : 0.f;
    for (int p = S - 1; p >= 0; --p) {
        float* sp = slot(a.qloc, p);
        float ql[4][4];
        ld16(sp, ql);
        st16(sp, qs);
        if (p == 0) break;
        const int64_t tp = p * tok_per_part;   // first token of part p
        const double lq = a.dec[static_cast<size_t>(bh) * S + p] - dta(tp) + dta(tp + tok_per_part);
        const float d = static_cast<float>(exp(lq));
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            float sn, cs;
            sincos_acc(a.ang[(static_cast<size_t>(bh) * S + p) * (N / 2) + 2 * pb + q], &sn, &cs);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float g0 = qs[2 * q][j], g1 = qs[2 * q + 1][j];
                qs[2 * q][j] = ql[2 * q][j] + d * (cs * g0 + sn * g1);
                qs[2 * q + 1][j] = ql[2 * q + 1][j] + d * (-sn * g0 + cs * g1);
            }
        }
    }
}

// Sums of per-head gradient rows over the heads of each group, and of dA, dD over the batch.
__global__ __launch_bounds__(256) void bwd_group_sum(const float* __restrict__ part, float* __restrict__ out,
                                                     int64_t rows, int heads_per_group, int width) {
    // part: (rows * heads_per_group, width) -> out: (rows, width); rows index (outer, group)
    const int64_t n = rows * width;
    for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < n; i += static_cast<int64_t>(gridDim.x) * 256) {
        const int64_t row = i / width, c = i - row * width;
        float s = 0.f;
        for (int k = 0; k < heads_per_group; ++k) s += part[(row * heads_per_group + k) * width + c];
        out[i] = s;
    }
}

__global__ __launch_bounds__(256) void bwd_fill_zero(float* __restrict__ p, int64_t n) {
    for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < n; i += static_cast<int64_t>(gridDim.x) * 256) p[i] = 0.f;
}

__global__ __launch_bounds__(256) void bwd_head_sum(const float* __restrict__ dA_part, const float* __restrict__ dD_part,
                                                    float* __restrict__ dA, float* __restrict__ dD, int batch, int H,
                                                    int parts) {
    const int h = blockIdx.x * 256 + threadIdx.x;
    if (h >= H) return;
    float sa = 0.f, sd = 0.f;
    for (int b = 0; b < batch; ++b)   // fixed order
        for (int p = 0; p < parts; ++p) {
            sa += dA_part[(static_cast<size_t>(b) * H + h) * parts + p];
            sd += dD_part[(static_cast<size_t>(b) * H + h) * parts + p];
        }
    if (dA) dA[h] = sa;   // null with a per-token rate, whose dA the scan writes
    dD[h] = sd;
}

}  // namespace bw

bool backward_supported(const BwdShape& s) {
    return s.N == bw::N && s.P == bw::P && (s.R == 1 || s.R == 2 || s.R == 4);
}

// One workgroup per (b, h) and part, one workgroup per CU (its LDS and registers
// allow no second).  With few (b, h) most CUs would idle, so the sequence is split
// into S parts of whole segments when that shortens the run: the cost model counts
// rounds of workgroups over the CUs times the segments of a part, and charges
// the split its local and combine passes (about a third of the gradient pass).
// The CU count is MI355X's, fixed, so that the split (and with it the rounding of
// the results) depends on the shape alone.
void backward_parts(const BwdShape& s, int* parts, int64_t* seg_per_part) {
    constexpr int64_t kCUs = 256;
    constexpr double kSplitCost = 1.3;
    const int64_t nseg = (s.L + bw::KS - 1) / bw::KS;
    const int64_t bh = s.batch * s.H;
    auto rounds = [&](int64_t wgs) { return (wgs + kCUs - 1) / kCUs; };
    int best_s = 1;
    int64_t best_per = nseg;
    double best = static_cast<double>(rounds(bh)) * static_cast<double>(nseg);
    for (int64_t S = 2; S <= 64 && S <= nseg; ++S) {
        const int64_t per = (nseg + S - 1) / S;
        const int64_t used = (nseg + per - 1) / per;   // every part holds at least one segment
        const double cost = kSplitCost * static_cast<double>(rounds(bh * used)) * static_cast<double>(per);
        if (cost < 0.95 * best) {
            best = cost;
            best_s = static_cast<int>(used);
            best_per = per;
        }
    }
    *parts = best_s;
    *seg_per_part = best_per;
}

// Segments per checkpoint group at each checkpoint level: level 0 keeps a checkpoint after
// every segment; level 1 groups ceil(sqrt(segments of a part)) segments, which minimises
// checkpoints plus scratch (groups per part + segments per group states).  The grouping
// changes where states are kept, not how they are computed: the gradients are the same bits
// for every group size.
static int64_t checkpoint_group(int level, int64_t seg_per_part) {
    if (level == 0) return 1;
    int64_t g = static_cast<int64_t>(std::ceil(std::sqrt(static_cast<double>(seg_per_part))));
    return g < 1 ? 1 : g;
}

// Workspace: checkpoints (batch, H, parts, groups per part, N, P) fp32 and, with groups of
// more than one segment, a scratch of one group's states per (batch, head, part); per-head
// partials of the group-shared gradients when H > G; dA/dD per (batch, head, part); with a
// split, each part's local state and adjoint (N, P) and its decay and angle sums.
BwdLayout backward_layout(const BwdShape& s, int level) {
    BwdLayout l{};
    auto al = [](size_t v) { return (v + 255) & ~static_cast<size_t>(255); };
    backward_parts(s, &l.parts, &l.seg_per_part);
    l.grp = checkpoint_group(level, l.seg_per_part);
    const size_t units = static_cast<size_t>(s.batch) * s.H * l.parts;
    const size_t gpp = static_cast<size_t>((l.seg_per_part + l.grp - 1) / l.grp);
    size_t off = 0;
    l.ckpt = off;
    off += al(units * gpp * s.N * s.P * 4);
    l.scratch = off;
    if (l.grp > 1) off += al(units * static_cast<size_t>(l.grp) * s.N * s.P * 4);
    l.kept_bytes = off;
    l.per_head = s.H != s.G;
    if (l.per_head) {
        l.dB_part = off;
        off += al(static_cast<size_t>(s.batch) * s.L * s.H * s.R * s.N * 4);
        l.dC_part = off;
        off += al(static_cast<size_t>(s.batch) * s.L * s.H * s.R * s.N * 4);
        l.dtheta_part = off;
        off += al(static_cast<size_t>(s.batch) * s.L * s.H * (s.N / 2) * 4);
        l.dbl_part = off;
        off += al(static_cast<size_t>(s.batch) * s.H * s.R * s.N * 4);
    }
    l.dA_part = off;
    off += al(units * 4);
    l.dD_part = off;
    off += al(units * 4);
    if (l.parts > 1) {
        l.hloc = off;
        off += al(units * s.N * s.P * 4);
        l.qloc = off;
        off += al(units * s.N * s.P * 4);
        l.dec = off;
        off += al(units * 8);
        l.ang = off;
        off += al(units * (s.N / 2) * 4);
    }
    l.bytes = off;
    return l;
}

namespace {
template <bool LOCAL>
void launch_scan(const BwdArgs& a, dim3 grid, hipStream_t st) {
    if (a.bf16) {
        if (a.R == 1) bw::bwd_scan<bf16_t, 1, LOCAL><<<grid, bw::NT, 0, st>>>(a);
        if (a.R == 2) bw::bwd_scan<bf16_t, 2, LOCAL><<<grid, bw::NT, 0, st>>>(a);
        if (a.R == 4) bw::bwd_scan<bf16_t, 4, LOCAL><<<grid, bw::NT, 0, st>>>(a);
    } else {
        if (a.R == 1) bw::bwd_scan<float, 1, LOCAL><<<grid, bw::NT, 0, st>>>(a);
        if (a.R == 2) bw::bwd_scan<float, 2, LOCAL><<<grid, bw::NT, 0, st>>>(a);
        if (a.R == 4) bw::bwd_scan<float, 4, LOCAL><<<grid, bw::NT, 0, st>>>(a);
    }
}
}  // namespace

hipError_t launch_backward(BwdArgs a, const BwdLayout& l, hipStream_t st) {
    uint8_t* ws = static_cast<uint8_t*>(a.workspace);
    a.ckpt = reinterpret_cast<float*>(ws + l.ckpt);
    a.scratch = reinterpret_cast<float*>(ws + l.scratch);
    a.grp = l.grp;
    a.per_head = l.per_head;
    if (l.per_head) {
        a.dB_part = reinterpret_cast<float*>(ws + l.dB_part);
        a.dC_part = reinterpret_cast<float*>(ws + l.dC_part);
        a.dtheta_part = reinterpret_cast<float*>(ws + l.dtheta_part);
        a.dbl_part = reinterpret_cast<float*>(ws + l.dbl_part);
    }
    a.dA_part = reinterpret_cast<float*>(ws + l.dA_part);
    a.dD_part = reinterpret_cast<float*>(ws + l.dD_part);
    a.parts = l.parts;
    a.seg_per_part = l.seg_per_part;
    if (l.parts > 1) {
        a.hloc = reinterpret_cast<float*>(ws + l.hloc);
        a.qloc = reinterpret_cast<float*>(ws + l.qloc);
        a.dec = reinterpret_cast<double*>(ws + l.dec);
        a.ang = reinterpret_cast<float*>(ws + l.ang);
    }
    const dim3 grid(static_cast<unsigned>(a.batch * a.H * l.parts));
    if (l.parts > 1) {   // local pass of every part, then the combine over parts
        launch_scan<true>(a, grid, st);
        bw::bwd_combine<<<static_cast<unsigned>(a.batch * a.H), bw::NT, 0, st>>>(a);
    }
    launch_scan<false>(a, grid, st);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_backward_sums(a, l, st);
}

hipError_t launch_backward_sums(const BwdArgs& a, const BwdLayout& l, hipStream_t st) {
    hipError_t e;
    if (l.per_head) {
        const int hpg = a.H / a.G;
        auto sum = [&](const float* part, float* out, int64_t rows, int width) {
            const int64_t n = rows * width;
            const unsigned blocks = static_cast<unsigned>(n / 256 + 1 < 65536 ? n / 256 + 1 : 65536);
            bw::bwd_group_sum<<<blocks, 256, 0, st>>>(part, out, rows, hpg, width);
        };
        const int64_t tokens = a.cu ? a.T : a.batch * a.L;
        if (tokens > 0) {
            sum(a.dB_part, a.dB, tokens * a.G, a.R * a.N);
            sum(a.dC_part, a.dC, tokens * a.G, a.R * a.N);
            sum(a.dtheta_part, a.dtheta, tokens * a.G, a.N / 2);
        }
        if (a.dbl && a.bl && a.xl) sum(a.dbl_part, a.dbl, a.batch * a.G, a.R * a.N);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (a.dbl && !(a.bl && a.xl)) {   // no carried input: its gradient is zero
        const int64_t n = a.batch * a.G * a.R * a.N;
        bw::bwd_fill_zero<<<static_cast<unsigned>(n / 256 + 1 < 4096 ? n / 256 + 1 : 4096), 256, 0, st>>>(a.dbl, n);
    }
    bw::bwd_head_sum<<<(a.H + 255) / 256, 256, 0, st>>>(a.dA_part, a.dD_part, a.At ? nullptr : a.dA, a.dD, static_cast<int>(a.batch), a.H,
                                                      l.parts);
    return hipGetLastError();
}

}  // namespace m3
