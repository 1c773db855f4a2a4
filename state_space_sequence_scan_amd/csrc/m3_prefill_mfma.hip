// m3_prefill_mfma.hip -- chunked prefill of the Mamba-3 scan on gfx950 matrix
// cores (bf16 operands, fp32 accumulation), state N = 128, head dim P = 64,
// rank R in {1, 2, 4}, chunk Q in {32, 64}.
//
// The chunked form is the one of m3_prefill_generic.hip (exponential-trapezoidal
// recurrence, Mamba-3 paper note "Solution 1"; rotation absorbed into B and C as
// a data-dependent RoPE, "Solution 2"; rank-R input, "Solution 3"; chunks
// computed in parallel with states passed between them, IBM "What is a Mamba
// model?", hardware-aware parallel scan).  Kernels:
//
//  rope_prep   one workgroup per (b, g, chunk): chunk-local angle prefix sums,
//              the rotated operands Bt = R(-phi) B and Ct = R(-phi) C in bf16,
//              token-major ([Q*R][N]) and, for Bt, also n-major ([N][Q*R]), plus
//              cos/sin of the chunk's total angle.  B, C and theta are shared by
//              the H/G heads of a group, so this work is done once per group, not
//              once per head.
//  scan_mfma   one workgroup (4 waves) per (b, h, segment of chunks).  The N x P
//              state lives in MFMA accumulators (wave w owns state rows
//              32w .. 32w+31).  Per chunk:
//                Y      = diag(e^cum) Ct S  +  (M o Ct Bt^T) X  +  D X
//                S     <- R(phi_end) [ e^{cum_end} S + Bt^T diag(s) X ]
//              with M the decay/trapezoid mask and s_j = e^{cum_end - cum_j} w_j.
//              The mask is applied to G^T = Bt Ct^T tiles in registers: the 16x16
//              accumulator layout of a 16x16x32 MFMA (4 consecutive rows per lane)
//              is exactly the A-operand layout of a 16x16x16 MFMA, so the masked
//              tile feeds the next contraction without leaving the registers.
//              In state-only mode (segment summaries) only the S update runs.
//  seg_pass    one workgroup per (b, h): combines the segment summaries into the
//              state entering each segment (sequential over segments).
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

__device__ __forceinline__ f32x4 mfma_k32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_k16(s16x4 a, s16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ __bf16 to_bf(float f) { return static_cast<__bf16>(f); }
__device__ __forceinline__ float from_bf(__bf16 b) { return static_cast<float>(b); }
__device__ __forceinline__ float bits_to_f(uint16_t u) { return __uint_as_float(static_cast<uint32_t>(u) << 16); }

// Workspace layout of the prepared operands for one (b, g, chunk).
struct PrepLayout {
    int QR;
    __host__ __device__ size_t bt() const { return 0; }                                    // [QR][N] bf16
    __host__ __device__ size_t ct() const { return static_cast<size_t>(QR) * N * 2; }      // [QR][N] bf16
    __host__ __device__ size_t btT() const { return static_cast<size_t>(QR) * N * 4; }     // [N][QR] bf16
    __host__ __device__ size_t cs() const { return static_cast<size_t>(QR) * N * 6; }      // [KP][2] fp32
    __host__ __device__ size_t bytes() const { return cs() + KP * 2 * sizeof(float); }
};

// ------------------------------------------------------------------------------------
// rope_prep
// ------------------------------------------------------------------------------------
template <int R, int Q>
__global__ __launch_bounds__(NT) void rope_prep(const uint16_t* __restrict__ B,
                                                const uint16_t* __restrict__ C,
                                                const float* __restrict__ theta, int64_t L, int G,
                                                int nchunks, uint8_t* __restrict__ prep) {
    constexpr int QR = Q * R;
    __shared__ float sCos[Q][KP], sSin[Q][KP];
    __shared__ __align__(16) uint16_t sB[QR][N + 8];
    const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int tid = threadIdx.x;
    const int64_t t0 = static_cast<int64_t>(c) * Q;
    const int nq = static_cast<int>(L - t0 < Q ? L - t0 : Q);
    const PrepLayout lay{QR};
    uint8_t* base = prep + ((static_cast<size_t>(b) * G + g) * nchunks + c) * lay.bytes();
    uint16_t* Bt = reinterpret_cast<uint16_t*>(base + lay.bt());
    uint16_t* Ct = reinterpret_cast<uint16_t*>(base + lay.ct());
    uint16_t* BtT = reinterpret_cast<uint16_t*>(base + lay.btT());
    float* cs = reinterpret_cast<float*>(base + lay.cs());

    // Chunk-local inclusive angle sums: 4 threads per pair, Q/4 tokens each.
    {
        constexpr int QP = Q / 4;
        const int k = tid % KP, part = tid / KP;
        float th[QP];
        float run = 0.f;
#pragma unroll
        for (int e = 0; e < QP; ++e) {
            const int i = part * QP + e;
            th[e] = (i < nq) ? theta[((b * L + t0 + i) * G + g) * KP + k] : 0.f;
            run += th[e];
            th[e] = run;
        }
        __shared__ float sPart[4][KP];
        sPart[part][k] = run;
        __syncthreads();
        float off = 0.f;
        for (int q = 0; q < part; ++q) off += sPart[q][k];
#pragma unroll
        for (int e = 0; e < QP; ++e) {
            float sn, cn;
            sincos_acc(th[e] + off, &sn, &cn);
            sCos[part * QP + e][k] = cn;
            sSin[part * QP + e][k] = sn;
        }
        if (part == 3) {
            // total angle of the chunk (tokens past the end add nothing)
            float sn, cn;
            sincos_acc(th[QP - 1] + off, &sn, &cn);
            cs[2 * k] = cn;
            cs[2 * k + 1] = sn;
        }
    }
    __syncthreads();
    // Rotate pairs: R(-phi) (x0, x1) = (c x0 + s x1, -s x0 + c x1).
    for (int idx = tid; idx < QR * KP; idx += NT) {
        const int row = idx / KP, k = idx - row * KP;
        const int i = row / R, r = row - i * R;
        float b0 = 0.f, b1 = 0.f, c0 = 0.f, c1 = 0.f;
        if (i < nq) {
            const size_t o = (((b * L + t0 + i) * G + g) * R + r) * static_cast<size_t>(N) + 2 * k;
            const uint32_t bb = *reinterpret_cast<const uint32_t*>(B + o);
            const uint32_t cc = *reinterpret_cast<const uint32_t*>(C + o);
            const float cn = sCos[i][k], sn = sSin[i][k];
            const float x0 = bits_to_f(bb & 0xffff), x1 = bits_to_f(bb >> 16);
            const float y0 = bits_to_f(cc & 0xffff), y1 = bits_to_f(cc >> 16);
            b0 = cn * x0 + sn * x1;
            b1 = -sn * x0 + cn * x1;
            c0 = cn * y0 + sn * y1;
            c1 = -sn * y0 + cn * y1;
        }
        const uint32_t pb = f32_to_bf16(b0) | (static_cast<uint32_t>(f32_to_bf16(b1)) << 16);
        const uint32_t pc = f32_to_bf16(c0) | (static_cast<uint32_t>(f32_to_bf16(c1)) << 16);
        *reinterpret_cast<uint32_t*>(Bt + static_cast<size_t>(row) * N + 2 * k) = pb;
        *reinterpret_cast<uint32_t*>(Ct + static_cast<size_t>(row) * N + 2 * k) = pc;
        *reinterpret_cast<uint32_t*>(&sB[row][2 * k]) = pb;
    }
    __syncthreads();
    // n-major copy: BtT[n][row], 8 rows per 16-byte store.
    for (int idx = tid; idx < N * (QR / 8); idx += NT) {
        const int n = idx / (QR / 8), r8 = idx - n * (QR / 8);
        uint16_t v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = sB[8 * r8 + e][n];
        uint4 w;
        w.x = v[0] | (static_cast<uint32_t>(v[1]) << 16);
        w.y = v[2] | (static_cast<uint32_t>(v[3]) << 16);
        w.z = v[4] | (static_cast<uint32_t>(v[5]) << 16);
        w.w = v[6] | (static_cast<uint32_t>(v[7]) << 16);
        *reinterpret_cast<uint4*>(BtT + static_cast<size_t>(n) * QR + 8 * r8) = w;
    }
}

// ------------------------------------------------------------------------------------
// scan_mfma
// ------------------------------------------------------------------------------------
struct ScanParams {
    const uint16_t* x;      // (b, L, H, R, P) bf16
    const float* dt;        // (b, L, H)
    const float* A;         // (H)
    const float* lam;       // (b, L, H)
    const float* D;         // (H)
    const uint8_t* prep;    // prepared operands, per (b, g, chunk)
    uint16_t* y;            // (b, L, H, R, P) bf16
    const float* s_init;    // state entering segment s: (b, H, nseg, N, P) fp32, or null
    const float* h_in;      // used when s_init is null (nseg == 1): (b, H, N, P), may be null
    const uint16_t* bl_in;  // carry in (b, G, R, N), may be null
    const uint16_t* xl_in;  // carry in (b, H, R, P), may be null
    float* h_out;           // final state (b, H, N, P), may be null
    float* seg_state;       // state-only mode: (b, H, nseg-1, N, P)
    float* seg_decay;       // state-only mode: (b, H, nseg-1)
    float* seg_rot;         // state-only mode: (b, H, nseg-1, KP, 2)
    int64_t L;
    int H, G, nchunks, nseg, chunks_per_seg;
};

// Initial state of segment 0 when no segment pass ran: h_in plus the beta term
// the first token gives the carried previous input.
template <int R>
__device__ float initial_state(const ScanParams& p, int b, int h, int g, int n, int col, float c1) {
    float s = p.h_in ? p.h_in[(static_cast<size_t>(b) * p.H + h) * N * P + n * P + col] : 0.f;
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

template <int R, int Q, bool FULL>
__global__ __launch_bounds__(NT) void scan_mfma(ScanParams p) {
    constexpr int QR = Q * R;
    constexpr int NB = QR / 16;          // 16-row blocks of the chunk
    constexpr int XS = QR + 8;           // row stride (elements) of sXT
    constexpr int BS = N + 8;            // row stride of sBt and sST
    static_assert(QR % 32 == 0 && Q <= 64, "tiling");

    __shared__ __align__(16) uint16_t sXT[P * XS];                 // X^T: [p][token*R + r]
    __shared__ __align__(16) uint16_t sBt[FULL ? QR * BS : 8];     // Bt token-major
    __shared__ __align__(16) uint16_t sST[FULL ? P * BS : 8];      // S^T (bf16): [p][n]
    __shared__ float sCum[Q], sEc[Q], sSc[Q], sW[Q], sGam[Q];
    __shared__ float sCs[KP * 2];
    __shared__ float sDec[1];

    const int seg = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int g = h / (p.H / p.G);
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int l16 = lane & 15, lg = lane >> 4;
    const PrepLayout lay{QR};
    const float Ah = p.A[h], Dh = p.D[h];
    const int c_begin = seg * p.chunks_per_seg;
    const int c_end = min(p.nchunks, c_begin + p.chunks_per_seg);
    const bool last_seg = (seg == p.nseg - 1);

    // ---- state accumulators: wave w, row tiles rt (n = 32w + 16rt + 4lg + i), col tiles ct (p = 16ct + l16)
    f32x4 sacc[2][4];
    if (FULL) {
        const float c1 = (p.L > 0 && p.bl_in && p.xl_in)
                             ? (1.f - p.lam[(static_cast<int64_t>(b) * p.L) * p.H + h]) *
                                   p.dt[(static_cast<int64_t>(b) * p.L) * p.H + h]
                             : 0.f;
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int ct = 0; ct < 4; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int n = 32 * w + 16 * rt + 4 * lg + i, col = 16 * ct + l16;
                    float v;
                    if (p.s_init)
                        v = p.s_init[((static_cast<size_t>(b) * p.H + h) * p.nseg + seg) * N * P + n * P + col];
                    else
                        v = initial_state<R>(p, b, h, g, n, col, c1);
                    sacc[rt][ct][i] = v;
                }
    } else {
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) sacc[rt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    if (FULL) {
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) {
                bf16x4 v = {to_bf(sacc[rt][ct][0]), to_bf(sacc[rt][ct][1]), to_bf(sacc[rt][ct][2]),
                            to_bf(sacc[rt][ct][3])};
                *reinterpret_cast<bf16x4*>(&sST[(16 * ct + l16) * BS + 32 * w + 16 * rt + 4 * lg]) = v;
            }
    }
    float dec_total = 0.f;                 // state-only: sum of chunk log-decays
    float rot_c = 1.f, rot_s = 0.f;        // state-only: total rotation of pair tid (tid < KP)

    for (int c = c_begin; c < c_end; ++c) {
        const int64_t t0 = static_cast<int64_t>(c) * Q;
        const int nq = static_cast<int>(p.L - t0 < Q ? p.L - t0 : Q);
        const uint8_t* pbase = p.prep + ((static_cast<size_t>(b) * p.G + g) * p.nchunks + c) * lay.bytes();
        const uint16_t* gBt = reinterpret_cast<const uint16_t*>(pbase + lay.bt());
        const uint16_t* gCt = reinterpret_cast<const uint16_t*>(pbase + lay.ct());
        const uint16_t* gBtT = reinterpret_cast<const uint16_t*>(pbase + lay.btT());
        const float* gCs = reinterpret_cast<const float*>(pbase + lay.cs());

        // (1) per-token scalars, one wave, lane = token
        if (w == 0) {
            const int i = lane;
            float a = 0.f, gm = 0.f, wv = 0.f;
            if (i < nq) {
                const int64_t t = t0 + i;
                const float dtv = p.dt[(b * p.L + t) * p.H + h], lv = p.lam[(b * p.L + t) * p.H + h];
                a = dtv * Ah;
                gm = lv * dtv;
                wv = gm;
                if (t + 1 < p.L)
                    wv += (1.f - p.lam[(b * p.L + t + 1) * p.H + h]) * p.dt[(b * p.L + t + 1) * p.H + h];
            }
            float cum = a;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const float o = __shfl_up(cum, off);
                if (lane >= off) cum += o;
            }
            const float cend = __shfl(cum, Q - 1);
            if (i < Q) {
                sCum[i] = cum;
                sEc[i] = __expf(cum);
                sSc[i] = __expf(cend - cum) * wv;
                sW[i] = wv;
                sGam[i] = gm;
            }
            if (lane == 0) sDec[0] = cend;
        }
        if (tid < 2 * KP) sCs[tid] = gCs[tid];

        // (2) X^T into LDS: 8x8 blocks (8 token-rank rows x 8 columns), transposed in registers
        for (int blk = tid; blk < QR; blk += NT) {
            const int rb = blk >> 3, po = blk & 7;
            uint16_t v[8][8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int row = 8 * rb + e;
                const int i = row / R, r = row - i * R;
                uint4 q = {0u, 0u, 0u, 0u};
                if (i < nq)
                    q = *reinterpret_cast<const uint4*>(
                        p.x + (((b * p.L + t0 + i) * p.H + h) * R + r) * static_cast<size_t>(P) + 8 * po);
                v[e][0] = q.x & 0xffff; v[e][1] = q.x >> 16;
                v[e][2] = q.y & 0xffff; v[e][3] = q.y >> 16;
                v[e][4] = q.z & 0xffff; v[e][5] = q.z >> 16;
                v[e][6] = q.w & 0xffff; v[e][7] = q.w >> 16;
            }
#pragma unroll
            for (int pp = 0; pp < 8; ++pp) {
                uint4 o;
                o.x = v[0][pp] | (static_cast<uint32_t>(v[1][pp]) << 16);
                o.y = v[2][pp] | (static_cast<uint32_t>(v[3][pp]) << 16);
                o.z = v[4][pp] | (static_cast<uint32_t>(v[5][pp]) << 16);
                o.w = v[6][pp] | (static_cast<uint32_t>(v[7][pp]) << 16);
                *reinterpret_cast<uint4*>(&sXT[(8 * po + pp) * XS + 8 * rb]) = o;
            }
        }
        // (3) Bt token-major into LDS
        if (FULL) {
            for (int idx = tid; idx < QR * (N / 8); idx += NT) {
                const int row = idx / (N / 8), c8 = idx - row * (N / 8);
                *reinterpret_cast<uint4*>(&sBt[row * BS + 8 * c8]) =
                    *reinterpret_cast<const uint4*>(gBt + static_cast<size_t>(row) * N + 8 * c8);
            }
        }
        __syncthreads();

        // (4) outputs
        if (FULL) {
            for (int a = w; a < NB; a += 4) {
                bf16x8 cf[4];
#pragma unroll
                for (int ks = 0; ks < 4; ++ks)
                    cf[ks] = *reinterpret_cast<const bf16x8*>(gCt + static_cast<size_t>(16 * a + l16) * N + 32 * ks + 8 * lg);
                f32x4 yacc[4];
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) {
                    yacc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks)
                        yacc[ct] = mfma_k32(cf[ks], *reinterpret_cast<const bf16x8*>(&sST[(16 * ct + l16) * BS + 32 * ks + 8 * lg]),
                                            yacc[ct]);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float ec = sEc[(16 * a + 4 * lg + i) / R];
#pragma unroll
                    for (int ct = 0; ct < 4; ++ct) yacc[ct][i] *= ec;
                }
                const int ti = (16 * a + l16) / R;
                const float cum_i = sCum[ti], gam_i = sGam[ti];
                for (int bb = 0; bb <= a; ++bb) {
                    f32x4 gt = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks)
                        gt = mfma_k32(*reinterpret_cast<const bf16x8*>(&sBt[(16 * bb + l16) * BS + 32 * ks + 8 * lg]), cf[ks], gt);
                    // gt[e] = (Ct Bt^T)[i = 16a + l16][j = 16bb + 4lg + e]
                    s16x4 mf;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int tj = (16 * bb + 4 * lg + e) / R;
                        const float m = (tj < ti) ? __expf(cum_i - sCum[tj]) * sW[tj] : ((tj == ti) ? gam_i : 0.f);
                        mf[e] = static_cast<short>(f32_to_bf16(m * gt[e]));
                    }
#pragma unroll
                    for (int ct = 0; ct < 4; ++ct)
                        yacc[ct] = mfma_k16(mf, *reinterpret_cast<const s16x4*>(&sXT[(16 * ct + l16) * XS + 16 * bb + 4 * lg]),
                                            yacc[ct]);
                }
                // skip term and store (rows 16a + 4lg + i, column 16ct + l16)
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) {
                    const s16x4 xv = *reinterpret_cast<const s16x4*>(&sXT[(16 * ct + l16) * XS + 16 * a + 4 * lg]);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int row = 16 * a + 4 * lg + i;
                        const int ti2 = row / R, r = row - ti2 * R;
                        if (ti2 < nq) {
                            const float yv = yacc[ct][i] + Dh * bits_to_f(static_cast<uint16_t>(xv[i]));
                            p.y[(((b * p.L + t0 + ti2) * p.H + h) * R + r) * static_cast<size_t>(P) + 16 * ct + l16] =
                                f32_to_bf16(yv);
                        }
                    }
                }
            }
            __syncthreads();   // every wave is done reading sST (S_{c-1})
        }

        // (5) state update: S <- R(phi_end) [e^{cum_end} S + Bt^T diag(s) X]
        {
            const float cend = sDec[0];
            const float decay = __expf(cend);
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) sacc[rt][ct] *= decay;
#pragma unroll
            for (int ks = 0; ks < QR / 32; ++ks) {
                bf16x8 af[2];
#pragma unroll
                for (int rt = 0; rt < 2; ++rt) {
                    const bf16x8 raw = *reinterpret_cast<const bf16x8*>(
                        gBtT + static_cast<size_t>(32 * w + 16 * rt + l16) * QR + 32 * ks + 8 * lg);
#pragma unroll
                    for (int e = 0; e < 8; ++e) af[rt][e] = to_bf(from_bf(raw[e]) * sSc[(32 * ks + 8 * lg + e) / R]);
                }
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) {
                    const bf16x8 bx = *reinterpret_cast<const bf16x8*>(&sXT[(16 * ct + l16) * XS + 32 * ks + 8 * lg]);
#pragma unroll
                    for (int rt = 0; rt < 2; ++rt) sacc[rt][ct] = mfma_k32(af[rt], bx, sacc[rt][ct]);
                }
            }
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int i = 0; i < 4; i += 2) {
                    const int k = (32 * w + 16 * rt + 4 * lg + i) >> 1;
                    const float cn = sCs[2 * k], sn = sCs[2 * k + 1];
#pragma unroll
                    for (int ct = 0; ct < 4; ++ct) {
                        const float s0 = sacc[rt][ct][i], s1 = sacc[rt][ct][i + 1];
                        sacc[rt][ct][i] = cn * s0 - sn * s1;
                        sacc[rt][ct][i + 1] = sn * s0 + cn * s1;
                    }
                }
            if (FULL) {
#pragma unroll
                for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                    for (int ct = 0; ct < 4; ++ct) {
                        bf16x4 v = {to_bf(sacc[rt][ct][0]), to_bf(sacc[rt][ct][1]), to_bf(sacc[rt][ct][2]),
                                    to_bf(sacc[rt][ct][3])};
                        *reinterpret_cast<bf16x4*>(&sST[(16 * ct + l16) * BS + 32 * w + 16 * rt + 4 * lg]) = v;
                    }
            } else {
                dec_total += cend;
                if (tid < KP) {
                    const float cn = sCs[2 * tid], sn = sCs[2 * tid + 1];
                    const float nc = cn * rot_c - sn * rot_s, ns = sn * rot_c + cn * rot_s;
                    rot_c = nc;
                    rot_s = ns;
                }
            }
        }
        __syncthreads();   // sXT / sST / scalars free for the next chunk
    }

    // epilogue
    if (FULL) {
        if (last_seg && p.h_out) {
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int ct = 0; ct < 4; ++ct)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int n = 32 * w + 16 * rt + 4 * lg + i, col = 16 * ct + l16;
                        p.h_out[(static_cast<size_t>(b) * p.H + h) * N * P + n * P + col] = sacc[rt][ct][i];
                    }
        }
    } else {
        const size_t sidx = (static_cast<size_t>(b) * p.H + h) * (p.nseg - 1) + seg;
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int ct = 0; ct < 4; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int n = 32 * w + 16 * rt + 4 * lg + i, col = 16 * ct + l16;
                    p.seg_state[sidx * N * P + n * P + col] = sacc[rt][ct][i];
                }
        if (tid == 0) p.seg_decay[sidx] = dec_total;
        if (tid < KP) {
            p.seg_rot[sidx * KP * 2 + 2 * tid] = rot_c;
            p.seg_rot[sidx * KP * 2 + 2 * tid + 1] = rot_s;
        }
    }
}

// ------------------------------------------------------------------------------------
// seg_pass: state entering each segment
// ------------------------------------------------------------------------------------
template <int R>
__global__ __launch_bounds__(NT) void seg_pass(ScanParams p, float* __restrict__ s_init) {
    const int bh = blockIdx.x;
    const int b = bh / p.H, h = bh - b * p.H, g = h / (p.H / p.G);
    const float c1 = (p.L > 0 && p.bl_in && p.xl_in)
                         ? (1.f - p.lam[(static_cast<int64_t>(b) * p.L) * p.H + h]) *
                               p.dt[(static_cast<int64_t>(b) * p.L) * p.H + h]
                         : 0.f;
    for (int idx = threadIdx.x; idx < KP * P; idx += NT) {
        const int k = idx / P, col = idx - k * P;
        float s0 = initial_state<R>(p, b, h, g, 2 * k, col, c1);
        float s1 = initial_state<R>(p, b, h, g, 2 * k + 1, col, c1);
        for (int s = 0; s < p.nseg; ++s) {
            float* out = s_init + ((static_cast<size_t>(bh) * p.nseg + s) * N) * P;
            out[(2 * k) * P + col] = s0;
            out[(2 * k + 1) * P + col] = s1;
            if (s == p.nseg - 1) break;
            const size_t sidx = static_cast<size_t>(bh) * (p.nseg - 1) + s;
            const float dec = __expf(p.seg_decay[sidx]);
            const float cn = p.seg_rot[sidx * KP * 2 + 2 * k], sn = p.seg_rot[sidx * KP * 2 + 2 * k + 1];
            const float* ds = p.seg_state + sidx * N * P;
            const float n0 = dec * (cn * s0 - sn * s1) + ds[(2 * k) * P + col];
            const float n1 = dec * (sn * s0 + cn * s1) + ds[(2 * k + 1) * P + col];
            s0 = n0;
            s1 = n1;
        }
    }
}

}  // namespace mf

// ------------------------------------------------------------------------------------
// host side
// ------------------------------------------------------------------------------------
bool mfma_supported(const PrefillArgs& a) {
    return a.bf16 && a.N == mf::N && a.P == mf::P && (a.R == 1 || a.R == 2 || a.R == 4) &&
           (a.Q == 32 || a.Q == 64);
}

static int choose_nseg(const PrefillArgs& a, int nchunks) {
    const int64_t slices = a.batch * a.H;
    const int64_t target = 512;                       // two workgroups per CU
    int64_t nseg = (target + slices - 1) / slices;
    const int64_t max_seg = nchunks / 4 > 0 ? nchunks / 4 : 1;   // at least ~4 chunks per segment
    if (nseg > max_seg) nseg = max_seg;
    if (nseg < 1) nseg = 1;
    return static_cast<int>(nseg);
}

struct MfmaWs {
    size_t prep, seg_state, seg_decay, seg_rot, s_init, total;
};

static MfmaWs mfma_ws(const PrefillArgs& a, int nchunks, int nseg) {
    MfmaWs w{};
    const mf::PrepLayout lay{a.Q * a.R};
    auto al = [](size_t v) { return (v + 255) & ~static_cast<size_t>(255); };
    size_t off = 0;
    w.prep = off;
    off += al(static_cast<size_t>(a.batch) * a.G * nchunks * lay.bytes());
    const size_t bh = static_cast<size_t>(a.batch) * a.H;
    if (nseg > 1) {
        w.seg_state = off;
        off += al(bh * (nseg - 1) * mf::N * mf::P * sizeof(float));
        w.seg_decay = off;
        off += al(bh * (nseg - 1) * sizeof(float));
        w.seg_rot = off;
        off += al(bh * (nseg - 1) * mf::KP * 2 * sizeof(float));
        w.s_init = off;
        off += al(bh * nseg * mf::N * mf::P * sizeof(float));
    }
    w.total = off;
    return w;
}

void plan_mfma(const PrefillArgs& a, PrefillPlan* plan) {
    const int nchunks = static_cast<int>((a.L + a.Q - 1) / a.Q);
    int nseg = nchunks > 0 ? choose_nseg(a, nchunks) : 1;
    if (nchunks > 0) {                       // no empty trailing segment
        const int cps = (nchunks + nseg - 1) / nseg;
        nseg = (nchunks + cps - 1) / cps;
    }
    plan->path = PrefillPath::Mfma;
    plan->nseg = nseg;
    plan->workspace = mfma_ws(a, nchunks, nseg).total;
    plan->lds = 0;
}

template <int R, int Q>
static hipError_t launch_mfma_rq(const PrefillArgs& a, const PrefillPlan& plan, hipStream_t st) {
    const int nchunks = static_cast<int>((a.L + a.Q - 1) / a.Q);
    if (nchunks == 0) return hipSuccess;
    const int nseg = plan.nseg;
    const int cps = (nchunks + nseg - 1) / nseg;
    const MfmaWs ws = mfma_ws(a, nchunks, nseg);
    uint8_t* base = static_cast<uint8_t*>(a.workspace);

    hipLaunchKernelGGL((mf::rope_prep<R, Q>), dim3(nchunks, a.G, static_cast<unsigned>(a.batch)), dim3(mf::NT), 0,
                       st, static_cast<const uint16_t*>(a.B), static_cast<const uint16_t*>(a.C), a.theta, a.L,
                       a.G, nchunks, base + ws.prep);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;

    mf::ScanParams p{};
    p.x = static_cast<const uint16_t*>(a.x);
    p.dt = a.dt;
    p.A = a.A;
    p.lam = a.lam;
    p.D = a.D;
    p.prep = base + ws.prep;
    p.y = static_cast<uint16_t*>(a.y);
    p.h_in = a.h_in;
    p.bl_in = static_cast<const uint16_t*>(a.bl_in);
    p.xl_in = static_cast<const uint16_t*>(a.xl_in);
    p.h_out = a.h_out;
    p.L = a.L;
    p.H = a.H;
    p.G = a.G;
    p.nchunks = nchunks;
    p.nseg = nseg;
    p.chunks_per_seg = cps;
    if (nseg > 1) {
        p.seg_state = reinterpret_cast<float*>(base + ws.seg_state);
        p.seg_decay = reinterpret_cast<float*>(base + ws.seg_decay);
        p.seg_rot = reinterpret_cast<float*>(base + ws.seg_rot);
        hipLaunchKernelGGL((mf::scan_mfma<R, Q, false>), dim3(nseg - 1, a.H, static_cast<unsigned>(a.batch)),
                           dim3(mf::NT), 0, st, p);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        float* s_init = reinterpret_cast<float*>(base + ws.s_init);
        hipLaunchKernelGGL((mf::seg_pass<R>), dim3(static_cast<unsigned>(a.batch * a.H)), dim3(mf::NT), 0, st, p,
                           s_init);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        p.s_init = s_init;
    }
    hipLaunchKernelGGL((mf::scan_mfma<R, Q, true>), dim3(nseg, a.H, static_cast<unsigned>(a.batch)), dim3(mf::NT),
                       0, st, p);
    return hipGetLastError();
}

hipError_t launch_prefill_mfma(const PrefillArgs& a, const PrefillPlan& plan, hipStream_t st) {
    switch (a.R * 100 + a.Q) {
        case 132: return launch_mfma_rq<1, 32>(a, plan, st);
        case 164: return launch_mfma_rq<1, 64>(a, plan, st);
        case 232: return launch_mfma_rq<2, 32>(a, plan, st);
        case 264: return launch_mfma_rq<2, 64>(a, plan, st);
        case 432: return launch_mfma_rq<4, 32>(a, plan, st);
        case 464: return launch_mfma_rq<4, 64>(a, plan, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace m3
