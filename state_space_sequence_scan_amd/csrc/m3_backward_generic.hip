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
// registers, for the whole sequence.  A forward sweep keeps the state before every
// segment of `ks` tokens in the workspace; the reverse sweep takes the segments last to
// first, recomputes a segment's states into a per-(b, h) scratch (each thread its own
// pairs, so no synchronisation is needed for them), and walks its tokens backwards.
// Per token, the sums over columns (dB, dC, dtheta), over state rows (dX) and over the
// whole state (dalpha, dbeta, dgamma, dD) are taken from LDS copies of h_t, dU_t and the
// per-pair angle terms in a fixed order, so results do not depend on scheduling.  Group-
// shared gradients are written per head when H > G and summed afterwards, as in the fast
// kernel.  Staging each token's inputs costs two barriers per token: this path is for the
// small and unusual shapes; N = 128, P = 64 run the fast kernel.
#include <cmath>
#include <cstdlib>

#include "m3_common.h"
#include "m3_internal.h"

namespace m3 {
namespace bg {

constexpr int NT = 256;
constexpr int kMaxR = 8;
constexpr int kMaxEPT = 16;      // element pairs per thread: (N / 2) * P <= NT * kMaxEPT
constexpr int kMaxDim = 256;

// Dynamic LDS layout (floats), sized for this launch's N, P, R.
struct Lds {
    int bp, xp, b, x, c, dy, cs, sn, hL, dUL, thc, red, total;
    __host__ __device__ Lds(int N, int P, int R) {
        int o = 0;
        bp = o; o += R * N;        // B of the previous token (or the carry, or zeros)
        xp = o; o += R * P;        // X of the previous token
        b = o;  o += R * N;        // B of this token
        x = o;  o += R * P;
        c = o;  o += R * N;
        dy = o; o += R * P;
        cs = o; o += N / 2;        // cos, sin of this token's pair angles
        sn = o; o += N / 2;
        hL = o; o += N * P;        // h_t, (n, p) row-major
        dUL = o; o += N * P;       // dU_t
        thc = o; o += (N / 2) * P; // per (pair, column) terms of dtheta
        red = o; o += 3 * NT;      // per-thread partial sums of dalpha, dbeta, dgamma
        total = o;
    }
};

template <typename T>
__device__ __forceinline__ float ldv(const T* p, int64_t i) { return io<T>::load(p + i); }

// Sum over the 64 lanes of a wave in a fixed butterfly order; every lane gets it.
__device__ __forceinline__ float wave_sum_fixed(float v) {
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) v += __shfl_xor(v, o);
    return v;
}

template <typename T>
__global__ __launch_bounds__(NT) void bwd_generic(BwdArgs a, int64_t ks) {
    extern __shared__ __align__(16) float lds[];
    const int N = a.N, P = a.P, R = a.R, KP = N / 2, E = KP * P;
    const Lds lay(N, P, R);
    float* sBp = lds + lay.bp;
    float* sXp = lds + lay.xp;
    float* sB = lds + lay.b;
    float* sX = lds + lay.x;
    float* sC = lds + lay.c;
    float* sDY = lds + lay.dy;
    float* sCs = lds + lay.cs;
    float* sSn = lds + lay.sn;
    float* sHL = lds + lay.hL;
    float* sDU = lds + lay.dUL;
    float* sTh = lds + lay.thc;
    float* sRed = lds + lay.red;
    __shared__ float sScal[8];   // dt, lambda, decay rate of this token; reduced dalpha, dbeta, dgamma, dD

    const int bh = blockIdx.x;
    const int b = bh / a.H, h = bh - b * a.H, g = h / (a.H / a.G);
    const int tid = threadIdx.x, lane = tid & 63;
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

    const int EPT = (E + NT - 1) / NT;
    auto soff = [&](int64_t t) { return (tb + t) * H + h; };

    // Inputs of token t (and B, X of token t - 1) into LDS; with_cdy also C_t, dy_t.
    auto stage = [&](int64_t t, bool with_cdy) {
        __syncthreads();   // the previous step's readers are done
        for (int i = tid; i < R * N; i += NT) {
            sB[i] = ldv(Bm, ((tb + t) * G + g) * static_cast<int64_t>(R * N) + i);
            sBp[i] = t > 0 ? ldv(Bm, ((tb + t - 1) * G + g) * static_cast<int64_t>(R * N) + i)
                           : (carry ? ldv(blp, (static_cast<int64_t>(b) * G + g) * (R * N) + i) : 0.f);
            if (with_cdy) sC[i] = ldv(Cm, ((tb + t) * G + g) * static_cast<int64_t>(R * N) + i);
        }
        for (int i = tid; i < R * P; i += NT) {
            sX[i] = ldv(x, ((tb + t) * H + h) * static_cast<int64_t>(R * P) + i);
            sXp[i] = t > 0 ? ldv(x, ((tb + t - 1) * H + h) * static_cast<int64_t>(R * P) + i)
                           : (carry ? ldv(xlp, (static_cast<int64_t>(b) * H + h) * (R * P) + i) : 0.f);
            if (with_cdy) sDY[i] = ldv(dy, ((tb + t) * H + h) * static_cast<int64_t>(R * P) + i);
        }
        for (int k = tid; k < KP; k += NT) {
            float s, c;
            sincos_acc(a.theta[((tb + t) * G + g) * KP + k], &s, &c);
            sCs[k] = c;
            sSn[k] = s;
        }
        if (tid == 0) {
            sScal[0] = a.dt[soff(t)];
            sScal[1] = a.lam[soff(t)];
            sScal[2] = a.At ? a.At[soff(t)] : Ah;
        }
        __syncthreads();
    };
    // U of rows (2k, 2k+1) at column p from the B, X rows in LDS.  The forward step is
    // inlined at two places (the sweep that stores checkpoints and the recompute of a
    // segment); its multiply-adds are written out as fused operations with contraction
    // off, so that both places compute the same bits and the gradients do not depend on
    // where the checkpoints fall.
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
    auto coeffs = [&](float* al, float* be, float* ga) {
#pragma clang fp contract(off)
        const float dtv = sScal[0], lv = sScal[1];
        *al = __expf(dtv * sScal[2]);
        *be = (1.f - lv) * dtv * *al;
        *ga = lv * dtv;
    };
    // one forward step of the staged token on the thread's pairs
    auto fwd_step = [&](float2 (&hs)[kMaxEPT]) {
#pragma clang fp contract(off)
        float al, be, ga;
        coeffs(&al, &be, &ga);
#pragma unroll
        for (int i = 0; i < kMaxEPT; ++i) {
            const int e = tid + NT * i;
            if (i < EPT && e < E) {
                const int k = e / P, p = e - k * P;
                float up0, up1, u0, u1;
                uval(sBp, sXp, k, p, &up0, &up1);
                uval(sB, sX, k, p, &u0, &u1);
                const float v0 = __builtin_fmaf(al, hs[i].x, be * up0);
                const float v1 = __builtin_fmaf(al, hs[i].y, be * up1);
                const float c = sCs[k], s = sSn[k];
                hs[i].x = __builtin_fmaf(c, v0, __builtin_fmaf(-s, v1, ga * u0));
                hs[i].y = __builtin_fmaf(s, v0, __builtin_fmaf(c, v1, ga * u1));
            }
        }
    };
    auto store = [&](float2* dst, const float2 (&hs)[kMaxEPT]) {
#pragma unroll
        for (int i = 0; i < kMaxEPT; ++i) {
            const int e = tid + NT * i;
            if (i < EPT && e < E) {
                dst[e] = hs[i];
            }
        }
    };
    auto load = [&](const float2* src, float2 (&hs)[kMaxEPT]) {
#pragma unroll
        for (int i = 0; i < kMaxEPT; ++i) {
            const int e = tid + NT * i;
            if (i < EPT && e < E) {
                hs[i] = src[e];
            }
        }
    };

    // ---- forward sweep: the state before every segment
    float2 hs[kMaxEPT];
#pragma unroll
    for (int i = 0; i < kMaxEPT; ++i) {
        const int e = tid + NT * i;
        hs[i] = float2{0.f, 0.f};
        if (i < EPT && e < E && a.h0) {
            const int k = e / P, p = e - k * P;
            const size_t base = static_cast<size_t>(bh) * N * P;
            hs[i].x = state_load(a.h0, base + static_cast<size_t>(2 * k) * P + p, a.state_bf16);
            hs[i].y = state_load(a.h0, base + static_cast<size_t>(2 * k + 1) * P + p, a.state_bf16);
        }
    }
    for (int64_t t = 0; t < L; ++t) {
        if (t % ks == 0) store(ck + (t / ks) * E, hs);
        stage(t, false);
        fwd_step(hs);
    }

    // ---- reverse sweep.  q_{t+1}, alpha_{t+1}, beta_{t+1} belong to the token after; the
    // final-state cotangent enters as a token after the last with alpha = 1, beta = 0.
    float2 qn[kMaxEPT];
#pragma unroll
    for (int i = 0; i < kMaxEPT; ++i) {
        const int e = tid + NT * i;
        qn[i] = float2{0.f, 0.f};
        if (i < EPT && e < E && a.dh_out) {
            const int k = e / P, p = e - k * P;
            const size_t base = static_cast<size_t>(bh) * N * P;
            qn[i].x = a.dh_out[base + static_cast<size_t>(2 * k) * P + p];
            qn[i].y = a.dh_out[base + static_cast<size_t>(2 * k + 1) * P + p];
        }
    }
    float an = 1.f, bn = 0.f;
    float dA_acc = 0.f, dD_acc = 0.f;   // thread 0

    for (int64_t s = nseg - 1; s >= 0; --s) {
        const int64_t t0 = s * ks;
        const int len = static_cast<int>(L - t0 < ks ? L - t0 : ks);
        {   // h_{t0-1} .. h_{t0+len-1} into the scratch
            float2 hr[kMaxEPT];
            load(ck + s * E, hr);
            store(scr, hr);
            for (int j = 0; j < len; ++j) {
                stage(t0 + j, false);
                fwd_step(hr);
                store(scr + (j + 1) * E, hr);
            }
        }
        for (int j = len - 1; j >= 0; --j) {
            const int64_t t = t0 + j;
            stage(t, true);
            float al, be, ga;
            coeffs(&al, &be, &ga);
            float dal = 0.f, dbe = 0.f, dga = 0.f;
#pragma unroll
            for (int i = 0; i < kMaxEPT; ++i) {
                const int e = tid + NT * i;
                if (i < EPT && e < E) {
                    const int k = e / P, p = e - k * P;
                    const float2 ht = scr[(j + 1) * E + e], hp = scr[j * E + e];
                    float g0 = an * qn[i].x, g1 = an * qn[i].y;
                    for (int r = 0; r < R; ++r) {
                        const float dv = sDY[r * P + p];
                        g0 += sC[r * N + 2 * k] * dv;
                        g1 += sC[r * N + 2 * k + 1] * dv;
                    }
                    float u0, u1, up0, up1;
                    uval(sB, sX, k, p, &u0, &u1);
                    uval(sBp, sXp, k, p, &up0, &up1);
                    dga += g0 * u0 + g1 * u1;
                    const float c = sCs[k], sn = sSn[k];
                    const float q0 = c * g0 + sn * g1, q1 = -sn * g0 + c * g1;
                    dal += q0 * hp.x + q1 * hp.y;
                    dbe += q0 * up0 + q1 * up1;
                    const float v0 = al * hp.x + be * up0, v1 = al * hp.y + be * up1;
                    sTh[e] = q1 * v0 - q0 * v1;
                    const int n0 = (2 * k) * P + p;
                    sHL[n0] = ht.x;
                    sHL[n0 + P] = ht.y;
                    sDU[n0] = ga * g0 + bn * qn[i].x;
                    sDU[n0 + P] = ga * g1 + bn * qn[i].y;
                    qn[i] = float2{q0, q1};
                }
            }
            sRed[tid] = dal;
            sRed[NT + tid] = dbe;
            sRed[2 * NT + tid] = dga;
            __syncthreads();
            // column sums: dC = h_t dy^T, dB = dU X^T (per head when the group is shared)
            const int64_t go = ((tb + t) * GH + gh) * static_cast<int64_t>(R * N);
            float* dCo = a.per_head ? a.dC_part : a.dC;
            float* dBo = a.per_head ? a.dB_part : a.dB;
            for (int o = tid; o < R * N; o += NT) {
                const int r = o / N, n = o - r * N;
                float dc = 0.f, db = 0.f;
                for (int p = 0; p < P; ++p) {
                    dc += sHL[n * P + p] * sDY[r * P + p];
                    db += sDU[n * P + p] * sX[r * P + p];
                }
                dCo[go + o] = dc;
                dBo[go + o] = db;
            }
            float* dTo = a.per_head ? a.dtheta_part : a.dtheta;
            for (int k = tid; k < KP; k += NT) {
                float v = 0.f;
                for (int p = 0; p < P; ++p) v += sTh[k * P + p];
                dTo[((tb + t) * GH + gh) * KP + k] = v;
            }
            // row sums: dX = B^T dU + D dy
            for (int o = tid; o < R * P; o += NT) {
                const int r = o / P, p = o - r * P;
                float v = 0.f;
                for (int n = 0; n < N; ++n) v += sB[r * N + n] * sDU[n * P + p];
                a.dx[((tb + t) * H + h) * static_cast<int64_t>(R * P) + o] = v + Dh * sDY[o];
            }
            // whole-state sums, in a fixed order by wave 0
            if (tid < 64) {
                float sa = 0.f, sb = 0.f, sg = 0.f, sd = 0.f;
                for (int w = 0; w < NT / 64; ++w) {
                    sa += sRed[w * 64 + lane];
                    sb += sRed[NT + w * 64 + lane];
                    sg += sRed[2 * NT + w * 64 + lane];
                }
                for (int o = lane; o < R * P; o += 64) sd += sDY[o] * sX[o];
                sa = wave_sum_fixed(sa);
                sb = wave_sum_fixed(sb);
                sg = wave_sum_fixed(sg);
                sd = wave_sum_fixed(sd);
                if (tid == 0) {
                    const float dtv = sScal[0], lv = sScal[1], av = sScal[2];
                    a.ddt[soff(t)] = sa * av * al + sb * (1.f - lv) * (al + dtv * av * al) + sg * lv;
                    a.dlam[soff(t)] = -sb * dtv * al + sg * dtv;
                    const float dav = sa * dtv * al + sb * (1.f - lv) * dtv * dtv * al;
                    if (a.At) a.dA[soff(t)] = dav;
                    else dA_acc += dav;
                    dD_acc += sd;
                }
            }
            an = al;
            bn = be;
        }
    }

    // ---- h_0 and the carried previous input (its cotangent beta_1 q_1)
    if (a.dh0) {
#pragma unroll
        for (int i = 0; i < kMaxEPT; ++i) {
            const int e = tid + NT * i;
            if (i < EPT && e < E) {
                const int k = e / P, p = e - k * P;
                const size_t base = static_cast<size_t>(bh) * N * P;
                a.dh0[base + static_cast<size_t>(2 * k) * P + p] = an * qn[i].x;
                a.dh0[base + static_cast<size_t>(2 * k + 1) * P + p] = an * qn[i].y;
            }
        }
    }
    if (carry && (a.dbl || a.dxl)) {
        __syncthreads();
        for (int i = tid; i < R * N; i += NT) sBp[i] = ldv(blp, (static_cast<int64_t>(b) * G + g) * (R * N) + i);
        for (int i = tid; i < R * P; i += NT) sXp[i] = ldv(xlp, (static_cast<int64_t>(b) * H + h) * (R * P) + i);
#pragma unroll
        for (int i = 0; i < kMaxEPT; ++i) {
            const int e = tid + NT * i;
            if (i < EPT && e < E) {
                const int k = e / P, p = e - k * P;
                sDU[(2 * k) * P + p] = bn * qn[i].x;
                sDU[(2 * k + 1) * P + p] = bn * qn[i].y;
            }
        }
        __syncthreads();
        if (a.dbl) {
            float* dBo = a.per_head ? a.dbl_part : a.dbl;
            for (int o = tid; o < R * N; o += NT) {
                const int r = o / N, n = o - r * N;
                float v = 0.f;
                for (int p = 0; p < P; ++p) v += sDU[n * P + p] * sXp[r * P + p];
                dBo[(static_cast<int64_t>(b) * GH + gh) * (R * N) + o] = v;
            }
        }
        if (a.dxl) {
            for (int o = tid; o < R * P; o += NT) {
                const int r = o / P, p = o - r * P;
                float v = 0.f;
                for (int n = 0; n < N; ++n) v += sBp[r * N + n] * sDU[n * P + p];
                a.dxl[static_cast<size_t>(bh) * R * P + o] = v;
            }
        }
    } else if (a.dxl) {
        for (int o = tid; o < R * P; o += NT) a.dxl[static_cast<size_t>(bh) * R * P + o] = 0.f;
    }
    if (tid == 0) {
        a.dA_part[bh] = dA_acc;
        a.dD_part[bh] = dD_acc;
    }
}

}  // namespace bg

bool backward_generic_supported(const BwdShape& s) {
    return s.N >= 2 && s.N % 2 == 0 && s.P >= 1 && s.N <= bg::kMaxDim && s.P <= bg::kMaxDim &&
           (s.N / 2) * s.P <= bg::NT * bg::kMaxEPT && s.R >= 1 && s.R <= bg::kMaxR;
}

size_t backward_generic_lds(const BwdShape& s) {
    return static_cast<size_t>(bg::Lds(s.N, s.P, s.R).total) * sizeof(float);
}

// Tokens per recompute segment: 16 while a state before every segment fits the
// checkpoint budget (as for the fast kernel: 4 GiB, or M3_BACKWARD_CHECKPOINT_BYTES),
// else about sqrt(L), which minimises checkpoints plus the segment scratch.  The
// segment length changes where states are kept, not how they are computed.
int64_t backward_generic_ks(const BwdShape& s) {
    double budget = 4.0 * (1ull << 30);
    if (const char* e = std::getenv("M3_BACKWARD_CHECKPOINT_BYTES")) budget = std::strtod(e, nullptr);
    const int64_t L = s.L > 0 ? s.L : 1;
    const double per_state = static_cast<double>(s.batch) * s.H * s.N * s.P * 4;
    const int64_t ks = 16;
    if (per_state * static_cast<double>((L + ks - 1) / ks + ks + 1) <= budget) return ks;
    const int64_t r = static_cast<int64_t>(std::ceil(std::sqrt(static_cast<double>(L))));
    return r > ks ? r : ks;
}

BwdLayout backward_generic_layout(const BwdShape& s) {
    BwdLayout l{};
    auto al = [](size_t v) { return (v + 255) & ~static_cast<size_t>(255); };
    l.generic = true;
    l.parts = 1;
    l.ks = backward_generic_ks(s);
    l.seg_per_part = (s.L + l.ks - 1) / l.ks;
    l.grp = 1;
    const size_t bh = static_cast<size_t>(s.batch) * s.H;
    const size_t state = static_cast<size_t>(s.N) * s.P * 4;
    size_t off = 0;
    l.ckpt = off;
    off += al(bh * static_cast<size_t>(l.seg_per_part > 0 ? l.seg_per_part : 1) * state);
    l.scratch = off;
    off += al(bh * static_cast<size_t>(l.ks + 1) * state);
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
    const size_t lds = backward_generic_lds(s);
    const dim3 grid(static_cast<unsigned>(a.batch * a.H));
    hipError_t e;
    if (a.bf16) {
        if ((e = ensure_dynamic_lds(reinterpret_cast<const void*>(&bg::bwd_generic<bf16_t>), lds)) != hipSuccess) return e;
        bg::bwd_generic<bf16_t><<<grid, bg::NT, lds, st>>>(a, l.ks);
    } else {
        if ((e = ensure_dynamic_lds(reinterpret_cast<const void*>(&bg::bwd_generic<float>), lds)) != hipSuccess) return e;
        bg::bwd_generic<float><<<grid, bg::NT, lds, st>>>(a, l.ks);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return launch_backward_sums(a, l, st);
}

}  // namespace m3
