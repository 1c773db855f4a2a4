// m3_backward_generic.hip -- backward pass of the Mamba-3 scan for shapes off the fast
// kernel's (any even state size N and head dim P with N * P <= 8192, N and P <= 256,
// rank 1..8), on gfx950, fp32 arithmetic, fp32 or bf16 io.
//
// The recurrence and its adjoint are those of m3_backward.hip (Mamba-3 paper note,
// "Solution 1" exponential-trapezoidal update, "Solution 2" rotation of state pairs,
// "Solution 3" rank-R input and output):
//   h_t  = M_t (alpha_t h_{t-1} + beta_t U_{t-1}) + gamma_t U_t,   U_t = B_t^T X_t
//   g_t  = C_t^T dy_t + alpha_{t+1} q_{t+1},   q_t = M_t^T g_t
//   dU_t = gamma_t g_t + beta_{t+1} q_{t+1}
// and the input gradients are contractions of g, q, dU with the forward quantities.
//
// One workgroup of 256 threads per (b, h); thread t owns the element pairs
// e = t + 256 i (rotation pair k = e / P, column p = e % P) of h and of the adjoint, in
// registers, for the whole sequence.  While they fit the checkpoint budget, the forward
// sweep keeps every state in the workspace and the reverse sweep reads them back; else it
// keeps the state before every segment of `ks` tokens, and the reverse sweep takes the
// segments last to first, recomputes a segment's states into a per-(b, h) scratch (each
// thread its own pairs, so no synchronisation is needed for them) and walks its tokens
// backwards.
// Per token, the sums over columns (dB, dC, dtheta), over state rows (dX) and over the
// whole state (dalpha, dbeta, dgamma, dD) are taken from LDS copies of h_t, dU_t and the
// per-pair angle terms in a fixed order, so results do not depend on scheduling.  Group-
// shared gradients are written per head when H > G and summed afterwards, as in the fast
// kernel.  The inputs of up to 16 tokens are staged into LDS at once.  The adjoint of a
// pair needs nothing from other threads, so in the reverse sweep each thread steps its
// pairs through a batch of up to 16 staged tokens before one barrier, and the batch's sums
// follow together: two barriers per batch.  The block and batch sizes are those with the
// fewest barriers per token whose LDS fits in 128 KB.  Each token's gradients are
// collected in LDS and a block's are written out together by the whole workgroup, in
// coalesced runs.  This path is for the small and
// unusual shapes; N = 128, P = 64 run the fast kernel.
#include <cmath>

#include "m3_common.h"
#include "m3_internal.h"

namespace m3 {
namespace bg {

constexpr int NT = 256;
constexpr int kMaxR = 8;
constexpr int kMaxEPT = 16;      // element pairs per thread: (N / 2) * P <= NT * kMaxEPT
constexpr int kMaxDim = 256;

// Dynamic LDS layout (floats), sized for this launch's N, P, R, TB tokens per staged block
// and TS tokens per batch of sums.  Slot j of B and X holds token t0 - 1 + j (slot 0: the
// token before the block, the carry, or zeros); slot j of the others holds token t0 + j.
struct Lds {
    int b, x, c, dy, cs, sn, sc, hL, dUL, thc, red, ob, ow, total;
    __host__ __device__ Lds(int N, int P, int R, int TB, int TS) {
        int o = 0;
        b = o;  o += (TB + 1) * R * N;
        x = o;  o += (TB + 1) * R * P;
        c = o;  o += TB * R * N;
        dy = o; o += TB * R * P;
        cs = o; o += TB * (N / 2);    // cos, sin of each token's pair angles
        sn = o; o += TB * (N / 2);
        sc = o; o += TB * 4;          // dt, lambda, decay rate of each token
        hL = o; o += (TS + 1) * N * P;   // h_t of each token of a batch and h_{t-1} of its last, (n, p) row-major
        dUL = o; o += TS * N * P;     // dU_t
        thc = o; o += TS * (N / 2) * P;   // per (pair, column) terms of dtheta
        red = o; o += TS * 3 * (NT / 64);   // per-wave sums of dalpha, dbeta, dgamma
        ow = 2 * R * N + N / 2 + R * P + 4;   // one token's outputs: dC, dB, dtheta, dx, ddt, dlambda, dA
        ob = o; o += TB * ow;         // the block's outputs, written out once per block
        total = o;
    }
};

template <typename T>
__device__ __forceinline__ float ldv(const T* p, int64_t i) { return io<T>::load(p + i); }

// floor(u / d) for 0 <= u < 8192 and 1 <= d <= 256, from inv = 1/d in fp32: (u + 1/2) / d
// lies at least 1/512 from an integer, and the two roundings move it by at most
// u * 2^-23 < 2^-10, so the truncation is exact.
__device__ __forceinline__ int fdiv(int u, float inv) {
    return static_cast<int>((static_cast<float>(u) + 0.5f) * inv);
}

// ks: tokens per recompute segment, a multiple of TB (tokens staged per block); TS: tokens
// per batch of sums, dividing TB.  EPT: element pairs per thread, the smallest power of two
// that covers N / 2 * P.
template <typename T, int EPT>
__global__ __launch_bounds__(NT) void bwd_generic(BwdArgs a, int64_t ks, int TB, int TS) {
    extern __shared__ __align__(16) float lds[];
    const int N = a.N, P = a.P, R = a.R, KP = N / 2, E = KP * P, RN = R * N, RP = R * P;
    const float invN = 1.f / N, invP = 1.f / P;   // for the task indices (fdiv)
    // the per-token sums as tasks of 4 lanes each, each kind from a multiple of 16 tasks (a
    // wave): dC (RN), dB (RN), dtheta (KP), dX (RP); ntask: the tasks' count (and the offset
    // of the scalars in a token's outputs).  The whole-state sums go to the wave where the
    // dtheta tasks (the fewest) start.
    auto up16 = [](int v) { return (v + 15) & ~15; };
    const int t1 = up16(RN), t2 = t1 + up16(RN), t3 = t2 + up16(KP), tspan = t3 + up16(RP);
    const int ntask = 2 * RN + KP + RP;
    const int sw = ((t2 * 4) / 64) % (NT / 64);   // the scalar wave
    const Lds lay(N, P, R, TB, TS);
    float* sB = lds + lay.b;
    float* sX = lds + lay.x;
    float* sC = lds + lay.c;
    float* sDY = lds + lay.dy;
    float* sCs = lds + lay.cs;
    float* sSn = lds + lay.sn;
    float* sSc = lds + lay.sc;
    float* sHL = lds + lay.hL;
    float* sDU = lds + lay.dUL;
    float* sTh = lds + lay.thc;
    float* sRed = lds + lay.red;
    float* sOut = lds + lay.ob;
    const int OW = lay.ow;
    __shared__ float kOne;   // the stride-0 operand of the dtheta sums (set before the first barrier)

    const int bh = blockIdx.x;
    const int b = bh / a.H, h = bh - b * a.H, g = h / (a.H / a.G);
    const int tid = threadIdx.x, lane = tid & 63;
    if (tid == 0) kOne = 1.f;
    const int H = a.H, G = a.G;
    const SeqSpan span = seq_span(a.cu, b, a.L, a.T);
    const int64_t tb = span.start, L = span.len;
    const int64_t nseg = (L + ks - 1) / ks;
    const float Ah = a.At ? 0.f : a.A[h], Dh = a.D[h];
    const bool carry = a.bl && a.xl;
    const T* x = static_cast<const T*>(a.x);
    const T* dy = static_cast<const T*>(a.dy);
    const T* Bm = static_cast<const T*>(a.B);
    const T* Cm = static_cast<const T*>(a.C);
    const T* blp = static_cast<const T*>(a.bl);
    const T* xlp = static_cast<const T*>(a.xl);
    const int gh = a.per_head ? h : g, GH = a.per_head ? H : G;
    // per-(b, h) workspace: the state before each segment, then one segment's states
    // (h_{t0-1} .. h_{t0+len-1}); a state is stored as E float2 pairs, pair e at e
    float2* ck = reinterpret_cast<float2*>(a.ckpt) + static_cast<size_t>(bh) * a.seg_per_part * E;
    float2* scr = reinterpret_cast<float2*>(a.scratch) + static_cast<size_t>(bh) * (ks + 1) * E;

    // the thread's element pairs: pair kk[i], column pp[i] (kk = -1: none); ec[i] the pair,
    // clamped to the last, for loads that every thread issues
    int kk[EPT], pp[EPT], ec[EPT];
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
        const int e = tid + NT * i;
        kk[i] = e < E ? e / P : -1;
        pp[i] = e < E ? e - kk[i] * P : 0;
        ec[i] = e < E ? e : E - 1;
    }
    constexpr int KH = EPT <= 2 ? 8 : EPT <= 4 ? 4 : 2;   // states loaded together
    auto soff = [&](int64_t t) { return (tb + t) * H + h; };

    // Tokens t0 .. t0+nt-1 (B and X also of token t0 - 1) into the slots; with_cdy also
    // their C and dy.
    auto stage = [&](int64_t t0, int nt, bool with_cdy) {
        __syncthreads();   // the previous block's readers are done
        const int nB = (nt + 1) * RN, nX = (nt + 1) * RP, nC = nt * RN, nD = nt * RP, nT = nt * KP;
        auto b_src = [&](int i, bool* zero) {   // B of unit i (token t0 - 1 + i / RN)
            const int j = i / RN, o = i - j * RN;
            const int64_t t = t0 - 1 + j;
            *zero = t < 0 && !carry;
            return t >= 0 ? Bm + ((tb + t) * G + g) * static_cast<int64_t>(RN) + o
                          : carry ? blp + (static_cast<int64_t>(b) * G + g) * RN + o
                                  : Bm + ((tb + t0) * G + g) * static_cast<int64_t>(RN) + o;
        };
        auto x_src = [&](int i, bool* zero) {
            const int j = i / RP, o = i - j * RP;
            const int64_t t = t0 - 1 + j;
            *zero = t < 0 && !carry;
            return t >= 0 ? x + ((tb + t) * H + h) * static_cast<int64_t>(RP) + o
                          : carry ? xlp + (static_cast<int64_t>(b) * H + h) * RP + o
                                  : x + ((tb + t0) * H + h) * static_cast<int64_t>(RP) + o;
        };
        auto c_src = [&](int i) {
            const int j = i / RN, o = i - j * RN;
            return Cm + ((tb + t0 + j) * G + g) * static_cast<int64_t>(RN) + o;
        };
        auto d_src = [&](int i) {
            const int j = i / RP, o = i - j * RP;
            return dy + ((tb + t0 + j) * H + h) * static_cast<int64_t>(RP) + o;
        };
        auto th_src = [&](int i) {
            const int j = i / KP, k = i - j * KP;
            return a.theta + ((tb + t0 + j) * G + g) * KP + k;
        };
        // Each thread's first two units of every array: the loads are issued together
        // (unconditionally, at clamped indices), then converted and stored, so that their
        // latencies overlap; the units past those (larger shapes) follow one by one.
        constexpr int K = 2;
        float vb[K], vx[K], vc[K], vd[K], vt[K], vs[3];
#pragma unroll
        for (int m = 0; m < K; ++m) {
            const int i = tid + m * NT;
            bool zb, zx;
            const T* pb = b_src(i < nB ? i : nB - 1, &zb);
            const T* px = x_src(i < nX ? i : nX - 1, &zx);
            const float lb = io<T>::load(pb), lx = io<T>::load(px);
            vb[m] = zb ? 0.f : lb;
            vx[m] = zx ? 0.f : lx;
            if (with_cdy) {
                vc[m] = io<T>::load(c_src(i < nC ? i : nC - 1));
                vd[m] = io<T>::load(d_src(i < nD ? i : nD - 1));
            }
            vt[m] = *th_src(i < nT ? i : nT - 1);
        }
        {
            const int j = tid < nt ? tid : nt - 1;
            vs[0] = a.dt[soff(t0 + j)];
            vs[1] = a.lam[soff(t0 + j)];
            vs[2] = a.At ? a.At[soff(t0 + j)] : Ah;
        }
#pragma unroll
        for (int m = 0; m < K; ++m) {
            const int i = tid + m * NT;
            if (i < nB) sB[i] = vb[m];
            if (i < nX) sX[i] = vx[m];
            if (with_cdy) {
                if (i < nC) sC[i] = vc[m];
                if (i < nD) sDY[i] = vd[m];
            }
            if (i < nT) {
                float sv, cv;
                sincos_acc(vt[m], &sv, &cv);
                sCs[i] = cv;
                sSn[i] = sv;
            }
        }
        if (tid < nt) {   // nt <= 16 < NT
            sSc[4 * tid] = vs[0];
            sSc[4 * tid + 1] = vs[1];
            sSc[4 * tid + 2] = vs[2];
        }
        for (int i = tid + K * NT; i < nB; i += NT) {
            bool z;
            const T* p = b_src(i, &z);
            sB[i] = z ? 0.f : io<T>::load(p);
        }
        for (int i = tid + K * NT; i < nX; i += NT) {
            bool z;
            const T* p = x_src(i, &z);
            sX[i] = z ? 0.f : io<T>::load(p);
        }
        if (with_cdy) {
            for (int i = tid + K * NT; i < nC; i += NT) sC[i] = io<T>::load(c_src(i));
            for (int i = tid + K * NT; i < nD; i += NT) sDY[i] = io<T>::load(d_src(i));
        }
        for (int i = tid + K * NT; i < nT; i += NT) {
            float sv, cv;
            sincos_acc(*th_src(i), &sv, &cv);
            sCs[i] = cv;
            sSn[i] = sv;
        }
        __syncthreads();
    };
    // U of rows (2k, 2k+1) at column p from B, X rows in LDS.  The forward step is inlined
    // at two places (the sweep that stores checkpoints and the recompute of a segment); its
    // multiply-adds are written out as fused operations with contraction off, so that both
    // places compute the same bits and the gradients do not depend on where the
    // checkpoints fall.
    auto uval = [&](const float* Bs, const float* Xs, int k, int p, float* u0, float* u1) {
#pragma clang fp contract(off)
        float s0 = 0.f, s1 = 0.f;
        for (int r = 0; r < R; ++r) {
            const float xv = Xs[r * P + p];
            s0 = __builtin_fmaf(Bs[r * N + 2 * k], xv, s0);
            s1 = __builtin_fmaf(Bs[r * N + 2 * k + 1], xv, s1);
        }
        *u0 = s0;
        *u1 = s1;
    };
    auto coeffs = [&](int j, float* al, float* be, float* ga) {
#pragma clang fp contract(off)
        const float dtv = sSc[4 * j], lv = sSc[4 * j + 1];
        *al = __expf(dtv * sSc[4 * j + 2]);
        *be = (1.f - lv) * dtv * *al;
        *ga = lv * dtv;
    };
    // one forward step of the token in slot j on the thread's pairs
    auto fwd_step = [&](int j, float2 (&hs)[EPT]) {
#pragma clang fp contract(off)
        float al, be, ga;
        coeffs(j, &al, &be, &ga);
        const float* Bp = sB + j * RN;
        const float* Xp = sX + j * RP;
#pragma unroll
        for (int i = 0; i < EPT; ++i) {
            if (kk[i] >= 0) {
                const int k = kk[i], p = pp[i];
                float up0, up1, u0, u1;
                uval(Bp, Xp, k, p, &up0, &up1);
                uval(Bp + RN, Xp + RP, k, p, &u0, &u1);
                const float v0 = __builtin_fmaf(al, hs[i].x, be * up0);
                const float v1 = __builtin_fmaf(al, hs[i].y, be * up1);
                const float c = sCs[j * KP + k], s = sSn[j * KP + k];
                hs[i].x = __builtin_fmaf(c, v0, __builtin_fmaf(-s, v1, ga * u0));
                hs[i].y = __builtin_fmaf(s, v0, __builtin_fmaf(c, v1, ga * u1));
            }
        }
    };
    auto store = [&](float2* dst, const float2 (&hs)[EPT]) {
#pragma unroll
        for (int i = 0; i < EPT; ++i) {
            const int e = tid + NT * i;
            if (kk[i] >= 0) dst[e] = hs[i];
        }
    };
    auto load = [&](const float2* src, float2 (&hs)[EPT]) {
#pragma unroll
        for (int i = 0; i < EPT; ++i) {
            const int e = tid + NT * i;
            if (kk[i] >= 0) hs[i] = src[e];
        }
    };

    // ---- forward sweep: the state before every segment
    float2 hs[EPT];
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
        const int e = tid + NT * i;
        hs[i] = float2{0.f, 0.f};
        if (kk[i] >= 0 && a.h0) {
            const int k = kk[i], p = pp[i];
            const size_t base = static_cast<size_t>(bh) * N * P;
            hs[i].x = state_load(a.h0, base + static_cast<size_t>(2 * k) * P + p, a.state_bf16);
            hs[i].y = state_load(a.h0, base + static_cast<size_t>(2 * k + 1) * P + p, a.state_bf16);
        }
    }
    // With one segment for the longest sequence (ks >= a.L) the scratch holds every state of
    // the sequence: the sweep stores them there and the reverse sweep recomputes nothing.
    const bool keep_all = ks >= a.L;
    if (keep_all) store(scr, hs);
    for (int64_t t0 = 0; t0 < L; t0 += TB) {
        const int nt = static_cast<int>(L - t0 < TB ? L - t0 : TB);
        stage(t0, nt, false);
        for (int j = 0; j < nt; ++j) {
            if (!keep_all && (t0 + j) % ks == 0) store(ck + ((t0 + j) / ks) * E, hs);
            fwd_step(j, hs);
            if (keep_all) store(scr + (t0 + j + 1) * E, hs);
        }
    }

    // ---- reverse sweep.  q_{t+1}, alpha_{t+1}, beta_{t+1} belong to the token after; the
    // final-state cotangent enters as a token after the last with alpha = 1, beta = 0.
    float2 qn[EPT];
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
        const int e = tid + NT * i;
        qn[i] = float2{0.f, 0.f};
        if (kk[i] >= 0 && a.dh_out) {
            const int k = kk[i], p = pp[i];
            const size_t base = static_cast<size_t>(bh) * N * P;
            qn[i].x = a.dh_out[base + static_cast<size_t>(2 * k) * P + p];
            qn[i].y = a.dh_out[base + static_cast<size_t>(2 * k + 1) * P + p];
        }
    }
    float an = 1.f, bn = 0.f;
    float dA_acc = 0.f, dD_acc = 0.f;   // thread sw * 64

    for (int64_t s = nseg - 1; s >= 0; --s) {
        const int64_t t0 = s * ks;
        const int len = static_cast<int>(L - t0 < ks ? L - t0 : ks);
        if (!keep_all) {   // h_{t0-1} .. h_{t0+len-1} into the scratch
            float2 hr[EPT];
            load(ck + s * E, hr);
            store(scr, hr);
            for (int bt = 0; bt < len; bt += TB) {
                const int nt = len - bt < TB ? len - bt : TB;
                stage(t0 + bt, nt, false);
                for (int j = 0; j < nt; ++j) {
                    fwd_step(j, hr);
                    store(scr + (bt + j + 1) * E, hr);
                }
            }
        }
        // h_t and h_{t-1} of the token being reversed, in registers; h_{t-2} is loaded a
        // token ahead, so the scratch's latency is off the chain of the sums
        for (int bt = ((len - 1) / TB) * TB; bt >= 0; bt -= TB) {
            const int nt = len - bt < TB ? len - bt : TB;
            stage(t0 + bt, nt, true);
            // Tokens nt-1 .. 0 in batches of TS: each thread steps its own pairs through the
            // batch's tokens (the adjoint is elementwise), leaving h_t, dU_t, the angle terms
            // and per-wave partial sums of each token in LDS; after one barrier the batch's
            // sums over columns, rows and the whole state run side by side.
            for (int jb = nt - 1; jb >= 0; jb -= TS) {
                const int nb = jb + 1 < TS ? jb + 1 : TS;
                // The batch's states into LDS, each thread its own pairs (no barrier): slot u
                // holds h_t of token jb - u, slot nb h_{t-1} of the last.  Their loads are
                // issued KH at a time, unconditionally (clamped indices), so that their
                // latencies overlap.
                for (int u0 = 0; u0 <= nb; u0 += KH) {
                    float2 hb[KH][EPT];
#pragma unroll
                    for (int d = 0; d < KH; ++d) {
                        const int u = u0 + d < nb ? u0 + d : nb;
                        const float2* src = scr + static_cast<int64_t>(bt + jb - u + 1) * E;
#pragma unroll
                        for (int i = 0; i < EPT; ++i) hb[d][i] = src[ec[i]];
                    }
#pragma unroll
                    for (int d = 0; d < KH; ++d) {
                        if (u0 + d <= nb) {
                            float* dst = sHL + (u0 + d) * N * P;
#pragma unroll
                            for (int i = 0; i < EPT; ++i) {
                                if (kk[i] >= 0) {
                                    const int n0 = (2 * kk[i]) * P + pp[i];
                                    dst[n0] = hb[d][i].x;
                                    dst[n0 + P] = hb[d][i].y;
                                }
                            }
                        }
                    }
                }
                // U_t of the token being reversed: computed for the batch's first token, then
                // taken from the U_{t-1} of the token before (the same slot, the same bits)
                float2 uc[EPT];
#pragma unroll
                for (int i = 0; i < EPT; ++i) {
                    uc[i] = float2{0.f, 0.f};
                    if (kk[i] >= 0) uval(sB + (jb + 1) * RN, sX + (jb + 1) * RP, kk[i], pp[i], &uc[i].x, &uc[i].y);
                }
                for (int u = 0; u < nb; ++u) {
                    const int j = jb - u;
                    float al, be, ga;
                    coeffs(j, &al, &be, &ga);
                    const float* Bp = sB + j * RN;
                    const float* Xp = sX + j * RP;
                    const float* Cc = sC + j * RN;
                    const float* Dc = sDY + j * RP;
                    const float* uHL = sHL + u * N * P;
                    const float* uHP = uHL + N * P;
                    float* uDU = sDU + u * N * P;
                    float* uTh = sTh + u * E;
                    float dal = 0.f, dbe = 0.f, dga = 0.f;
#pragma unroll
                    for (int i = 0; i < EPT; ++i) {
                        const int e = tid + NT * i;
                        if (kk[i] >= 0) {
                            const int k = kk[i], p = pp[i];
                            const int n0 = (2 * k) * P + p;
                            const float2 hp = float2{uHP[n0], uHP[n0 + P]};
                            float g0 = an * qn[i].x, g1 = an * qn[i].y;
                            for (int r = 0; r < R; ++r) {
                                const float dv = Dc[r * P + p];
                                g0 += Cc[r * N + 2 * k] * dv;
                                g1 += Cc[r * N + 2 * k + 1] * dv;
                            }
                            const float u0 = uc[i].x, u1 = uc[i].y;
                            float up0, up1;
                            uval(Bp, Xp, k, p, &up0, &up1);
                            uc[i] = float2{up0, up1};
                            dga += g0 * u0 + g1 * u1;
                            const float c = sCs[j * KP + k], sn = sSn[j * KP + k];
                            const float q0 = c * g0 + sn * g1, q1 = -sn * g0 + c * g1;
                            dal += q0 * hp.x + q1 * hp.y;
                            dbe += q0 * up0 + q1 * up1;
                            const float v0 = al * hp.x + be * up0, v1 = al * hp.y + be * up1;
                            uTh[e] = q1 * v0 - q0 * v1;
                            uDU[n0] = ga * g0 + bn * qn[i].x;
                            uDU[n0 + P] = ga * g1 + bn * qn[i].y;
                            qn[i] = float2{q0, q1};
                        }
                    }
                    // DPP, fixed order, all 64 lanes of every wave active
                    dal = wave_sum(dal);
                    dbe = wave_sum(dbe);
                    dga = wave_sum(dga);
                    if (lane == 0) {
                        float* rd = sRed + u * 3 * (NT / 64) + (tid >> 6);
                        rd[0] = dal;
                        rd[NT / 64] = dbe;
                        rd[2 * (NT / 64)] = dga;
                    }
                    an = al;
                    bn = be;
                }
                __syncthreads();
                // Each token's sums as one list of dot products, spread over the threads so
                // that they run side by side (one loop shape for all, no divergence inside):
                //   dC[r][n] = sum_p h_t[n][p] dy[r][p]      (RN tasks)
                //   dB[r][n] = sum_p dU[n][p] X[r][p]        (RN)
                //   dtheta[k] = sum_p (angle term)[k][p]     (KP; times a stride-0 one)
                //   dX[r][p] = sum_n B[r][n] dU[n][p]        (RP; plus D dy afterwards)
                // A wave runs one kind; the 4 lanes of a task take every 4th term and add
                // their parts by two DPP moves within the quad.
                // Four tokens at a time per task, their loads issued together.
                const int sub = tid & 3;
                for (int o = tid >> 2; o < tspan; o += NT / 4) {
                    const int kind = o < t1 ? 0 : o < t2 ? 1 : o < t3 ? 2 : 3;
                    const int q = o - (kind == 0 ? 0 : kind == 1 ? t1 : kind == 2 ? t2 : t3);
                    if (q >= (kind < 2 ? RN : kind == 2 ? KP : RP)) continue;   // whole quads
                    // operand a: slot-relative (h_t, dU or angle terms of the token's batch
                    // slot) or token-relative (B); operand b likewise (dy, X; dU; a constant)
                    int a_off, b_off, sb = 1, m = P;
                    const float* a_base;
                    const float* b_base;
                    int a_step, b_step, a_slot, b_slot;   // per token: slot stride or token stride
                    if (kind < 2) {
                        const int r = fdiv(q, invN), n = q - r * N;
                        a_base = kind == 0 ? sHL : sDU; a_off = n * P; a_slot = N * P; a_step = 0;
                        b_base = kind == 0 ? sDY : sX + RP; b_off = r * P; b_slot = 0; b_step = RP;
                    } else if (kind == 2) {
                        a_base = sTh; a_off = q * P; a_slot = E; a_step = 0;
                        b_base = &kOne; b_off = 0; b_slot = 0; b_step = 0; sb = 0;
                    } else {
                        const int r = fdiv(q, invP), p = q - r * P;
                        a_base = sB + RN; a_off = r * N; a_slot = 0; a_step = RN;
                        b_base = sDU; b_off = p; b_slot = N * P; b_step = 0; sb = P; m = N;
                    }
                    const int o_out = (kind == 0 ? 0 : kind == 1 ? RN : kind == 2 ? 2 * RN : 2 * RN + KP) + q;
                    for (int u0 = 0; u0 < nb; u0 += 4) {
                        float v[4];
#pragma unroll
                        for (int d = 0; d < 4; ++d) {
                            const int u = u0 + d < nb ? u0 + d : nb - 1;   // clamped: computed, not stored
                            const int j = jb - u;
                            const float* pa = a_base + a_off + u * a_slot + j * a_step;
                            const float* pb = b_base + b_off + u * b_slot + j * b_step;
                            float acc = 0.f;
#pragma unroll 4
                            for (int i = sub; i < m; i += 4) acc += pa[i] * pb[i * sb];
                            v[d] = acc;
                        }
#pragma unroll
                        for (int d = 0; d < 4; ++d) {
                            v[d] += dpp_move<0xB1>(v[d]);   // quad_perm [1, 0, 3, 2]
                            v[d] += dpp_move<0x4E>(v[d]);   // quad_perm [2, 3, 0, 1]
                        }
                        if (sub == 0) {
#pragma unroll
                            for (int d = 0; d < 4; ++d) {
                                if (u0 + d < nb) {
                                    const int j = jb - u0 - d;
                                    sOut[j * OW + o_out] = kind == 3 ? v[d] + Dh * sDY[j * RP + q] : v[d];
                                }
                            }
                        }
                    }
                }
                // whole-state sums of token u on wave u mod 4: the per-wave partials of
                // dalpha, dbeta, dgamma and the sum for dD; dA and dD are accumulated over the
                // tokens when the block is written out
                for (int u = tid >> 6; u < nb; u += NT / 64) {
                    const int j = jb - u;
                    const float* Xc = sX + (j + 1) * RP;
                    const float* Dc = sDY + j * RP;
                    const float* rd = sRed + u * 3 * (NT / 64);
                    float sd = 0.f;
                    for (int o = lane; o < RP; o += 64) sd += Dc[o] * Xc[o];
                    sd = wave_sum(sd);   // DPP, fixed order, all 64 lanes of this wave active
                    if (lane == 0) {
                        float sa = 0.f, sbt = 0.f, sg = 0.f;
                        for (int w = 0; w < NT / 64; ++w) {
                            sa += rd[w];
                            sbt += rd[NT / 64 + w];
                            sg += rd[2 * (NT / 64) + w];
                        }
                        float al, be, ga;
                        coeffs(j, &al, &be, &ga);
                        const float dtv = sSc[4 * j], lv = sSc[4 * j + 1], av = sSc[4 * j + 2];
                        float* so = sOut + j * OW + ntask;
                        so[0] = sa * av * al + sbt * (1.f - lv) * (al + dtv * av * al) + sg * lv;
                        so[1] = -sbt * dtv * al + sg * dtv;
                        so[2] = sa * dtv * al + sbt * (1.f - lv) * dtv * dtv * al;
                        so[3] = sd;
                    }
                }
                __syncthreads();   // the sums are read before the next batch overwrites them
            }
            // the block's outputs (visible after the last token's barrier), once per block
            const int64_t tf = tb + t0 + bt;   // first token of the block in the packed arrays
            for (int i = tid; i < nt * RN; i += NT) {
                const int j = i / RN, o = i - j * RN;
                (a.per_head ? a.dC_part : a.dC)[((tf + j) * GH + gh) * static_cast<int64_t>(RN) + o] = sOut[j * OW + o];
                (a.per_head ? a.dB_part : a.dB)[((tf + j) * GH + gh) * static_cast<int64_t>(RN) + o] = sOut[j * OW + RN + o];
            }
            for (int i = tid; i < nt * KP; i += NT) {
                const int j = i / KP, k = i - j * KP;
                (a.per_head ? a.dtheta_part : a.dtheta)[((tf + j) * GH + gh) * KP + k] = sOut[j * OW + 2 * RN + k];
            }
            for (int i = tid; i < nt * RP; i += NT) {
                const int j = i / RP, o = i - j * RP;
                a.dx[((tf + j) * H + h) * static_cast<int64_t>(RP) + o] = sOut[j * OW + 2 * RN + KP + o];
            }
            for (int j = tid; j < nt; j += NT) {
                const float* so = sOut + j * OW + 2 * RN + KP + RP;
                a.ddt[(tf + j) * H + h] = so[0];
                a.dlam[(tf + j) * H + h] = so[1];
                if (a.At) a.dA[(tf + j) * H + h] = so[2];
            }
            if (tid == sw * 64) {   // tokens last to first, as they were reversed
                for (int j = nt - 1; j >= 0; --j) {
                    const float* so = sOut + j * OW + 2 * RN + KP + RP;
                    if (!a.At) dA_acc += so[2];
                    dD_acc += so[3];
                }
            }
        }
    }

    // ---- h_0 and the carried previous input (its cotangent beta_1 q_1)
    if (a.dh0) {
#pragma unroll
        for (int i = 0; i < EPT; ++i) {
            const int e = tid + NT * i;
            if (kk[i] >= 0) {
                const int k = kk[i], p = pp[i];
                const size_t base = static_cast<size_t>(bh) * N * P;
                a.dh0[base + static_cast<size_t>(2 * k) * P + p] = an * qn[i].x;
                a.dh0[base + static_cast<size_t>(2 * k + 1) * P + p] = an * qn[i].y;
            }
        }
    }
    if (carry && (a.dbl || a.dxl)) {
        __syncthreads();
        for (int i = tid; i < RN; i += NT) sB[i] = ldv(blp, (static_cast<int64_t>(b) * G + g) * RN + i);
        for (int i = tid; i < RP; i += NT) sX[i] = ldv(xlp, (static_cast<int64_t>(b) * H + h) * RP + i);
#pragma unroll
        for (int i = 0; i < EPT; ++i) {
            const int e = tid + NT * i;
            if (kk[i] >= 0) {
                const int k = kk[i], p = pp[i];
                sDU[(2 * k) * P + p] = bn * qn[i].x;
                sDU[(2 * k + 1) * P + p] = bn * qn[i].y;
            }
        }
        __syncthreads();
        if (a.dbl) {
            float* dBo = a.per_head ? a.dbl_part : a.dbl;
            for (int o = tid; o < RN; o += NT) {
                const int r = o / N, n = o - r * N;
                float v = 0.f;
                for (int p = 0; p < P; ++p) v += sDU[n * P + p] * sX[r * P + p];
                dBo[(static_cast<int64_t>(b) * GH + gh) * RN + o] = v;
            }
        }
        if (a.dxl) {
            for (int o = tid; o < RP; o += NT) {
                const int r = o / P, p = o - r * P;
                float v = 0.f;
                for (int n = 0; n < N; ++n) v += sB[r * N + n] * sDU[n * P + p];
                a.dxl[static_cast<size_t>(bh) * RP + o] = v;
            }
        }
    } else if (a.dxl) {
        for (int o = tid; o < RP; o += NT) a.dxl[static_cast<size_t>(bh) * RP + o] = 0.f;
    }
    if (tid == sw * 64) {
        a.dA_part[bh] = dA_acc;
        a.dD_part[bh] = dD_acc;
    }
}

}  // namespace bg

bool backward_generic_supported(const BwdShape& s) {
    return s.N >= 2 && s.N % 2 == 0 && s.P >= 1 && s.N <= bg::kMaxDim && s.P <= bg::kMaxDim &&
           (s.N / 2) * s.P <= bg::NT * bg::kMaxEPT && s.R >= 1 && s.R <= bg::kMaxR;
}

// Tokens staged per block (TB, a power of two up to 16) and tokens per batch of sums (TS, a
// power of two up to TB): the pair with the fewest barriers per token (2 / TB + 2 / TS)
// whose LDS stays within 128 KB (a workgroup holds a CU alone: its registers allow no
// second), the larger TB on a tie.
static void backward_generic_blocks(const BwdShape& s, int* tb_out, int* ts_out) {
    int best_tb = 1, best_ts = 1;
    double best = 3.0;
    for (int tb = 16; tb >= 1; tb /= 2)
        for (int ts = tb; ts >= 1; ts /= 2) {
            const double cost = 1.0 / tb + 1.0 / ts;
            if (static_cast<size_t>(bg::Lds(s.N, s.P, s.R, tb, ts).total) * sizeof(float) <= 128 * 1024 &&
                cost < best - 1e-9) {
                best = cost;
                best_tb = tb;
                best_ts = ts;
            }
        }
    *tb_out = best_tb;
    *ts_out = best_ts;
}

size_t backward_generic_lds(const BwdShape& s) {
    int tb, ts;
    backward_generic_blocks(s, &tb, &ts);
    return static_cast<size_t>(bg::Lds(s.N, s.P, s.R, tb, ts).total) * sizeof(float);
}

// Tokens per recompute segment at each checkpoint level: level 0 the whole sequence (every
// state kept, no recompute pass), level 1 16 tokens (a state before every segment), level 2
// ceil(sqrt(L)) (about minimising checkpoints plus the segment scratch); each rounded up to a
// multiple of 16, so that staged blocks never straddle a segment.  The segment length changes
// where states are kept, not how they are computed.
static int64_t backward_generic_ks(const BwdShape& s, int level) {
    const int64_t L = s.L > 0 ? s.L : 1;
    const int64_t ks = 16;
    if (level == 1) return ks;
    const int64_t r = level == 0 ? L : static_cast<int64_t>(std::ceil(std::sqrt(static_cast<double>(L))));
    return ((r + ks - 1) / ks) * ks;
}

BwdLayout backward_generic_layout(const BwdShape& s, int level) {
    BwdLayout l{};
    auto al = [](size_t v) { return (v + 255) & ~static_cast<size_t>(255); };
    l.generic = true;
    l.parts = 1;
    l.ks = backward_generic_ks(s, level);
    l.seg_per_part = (s.L + l.ks - 1) / l.ks;
    l.grp = 1;
    const size_t bh = static_cast<size_t>(s.batch) * s.H;
    const size_t state = static_cast<size_t>(s.N) * s.P * 4;
    size_t off = 0;
    l.ckpt = off;
    off += al(bh * static_cast<size_t>(l.seg_per_part > 0 ? l.seg_per_part : 1) * state);
    l.scratch = off;
    off += al(bh * static_cast<size_t>(l.ks + 1) * state);
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
    off += al(bh * 4);
    l.dD_part = off;
    off += al(bh * 4);
    l.bytes = off;
    return l;
}

template <typename T, int EPT>
static hipError_t launch_generic_e(const BwdArgs& a, const BwdLayout& l, int tb, int ts, size_t lds, dim3 grid,
                                   hipStream_t st) {
    const hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(&bg::bwd_generic<T, EPT>), lds);
    if (e != hipSuccess) return e;
    bg::bwd_generic<T, EPT><<<grid, bg::NT, lds, st>>>(a, l.ks, tb, ts);
    return hipGetLastError();
}

template <typename T>
static hipError_t launch_generic_t(const BwdArgs& a, const BwdLayout& l, int ept, int tb, int ts, size_t lds,
                                   dim3 grid, hipStream_t st) {
    switch (ept) {
        case 1: return launch_generic_e<T, 1>(a, l, tb, ts, lds, grid, st);
        case 2: return launch_generic_e<T, 2>(a, l, tb, ts, lds, grid, st);
        case 4: return launch_generic_e<T, 4>(a, l, tb, ts, lds, grid, st);
        case 8: return launch_generic_e<T, 8>(a, l, tb, ts, lds, grid, st);
        default: return launch_generic_e<T, 16>(a, l, tb, ts, lds, grid, st);
    }
}

hipError_t launch_backward_generic(BwdArgs a, const BwdLayout& l, hipStream_t st) {
    uint8_t* ws = static_cast<uint8_t*>(a.workspace);
    a.ckpt = reinterpret_cast<float*>(ws + l.ckpt);
    a.scratch = reinterpret_cast<float*>(ws + l.scratch);
    a.per_head = l.per_head;
    if (l.per_head) {
        a.dB_part = reinterpret_cast<float*>(ws + l.dB_part);
        a.dC_part = reinterpret_cast<float*>(ws + l.dC_part);
        a.dtheta_part = reinterpret_cast<float*>(ws + l.dtheta_part);
        a.dbl_part = reinterpret_cast<float*>(ws + l.dbl_part);
    }
    a.dA_part = reinterpret_cast<float*>(ws + l.dA_part);
    a.dD_part = reinterpret_cast<float*>(ws + l.dD_part);
    a.parts = 1;
    a.seg_per_part = l.seg_per_part;
    const BwdShape s{a.batch, a.L, a.H, a.G, a.N, a.P, a.R};
    int tb, ts;
    backward_generic_blocks(s, &tb, &ts);
    const size_t lds = backward_generic_lds(s);
    const dim3 grid(static_cast<unsigned>(a.batch * a.H));
    hipError_t e;
    const int pairs = (a.N / 2) * a.P;
    const int ept = pairs <= bg::NT ? 1 : pairs <= 2 * bg::NT ? 2 : pairs <= 4 * bg::NT ? 4 : pairs <= 8 * bg::NT ? 8 : 16;
    if ((e = a.bf16 ? launch_generic_t<bf16_t>(a, l, ept, tb, ts, lds, grid, st)
                    : launch_generic_t<float>(a, l, ept, tb, ts, lds, grid, st)) != hipSuccess)
        return e;
    return launch_backward_sums(a, l, st);
}

}  // namespace m3
