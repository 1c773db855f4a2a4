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
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 v = {to_bf(a), to_bf(b)};
    return __builtin_bit_cast(uint32_t, v);
}

template <int R, int Q>
__global__ __launch_bounds__(NT) void rope_prep(const uint16_t* __restrict__ B,
                                                const uint16_t* __restrict__ C,
                                                const float* __restrict__ theta, int64_t L, int G,
                                                int nchunks, uint8_t* __restrict__ prep) {
    constexpr int QR = Q * R;
    __shared__ float sCos[Q][KP], sSin[Q][KP];
    __shared__ float sPart[4][KP];
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
            run += (i < nq) ? theta[((b * L + t0 + i) * G + g) * KP + k] : 0.f;
            th[e] = run;
        }
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
        if (part == 3) {   // total angle of the chunk (tokens past the end add nothing)
            float sn, cn;
            sincos_acc(th[QP - 1] + off, &sn, &cn);
            cs[2 * k] = cn;
            cs[2 * k + 1] = sn;
        }
    }
    __syncthreads();
    // One unit = 8 consecutive rows (token, rank) x one rotation pair k:
    // R(-phi) (x0, x1) = (c x0 + s x1, -s x0 + c x1).  Token-major stores are
    // 4 bytes per row; the n-major copy is two 16-byte stores (rows 2k, 2k+1).
    for (int u = tid; u < (QR / 8) * KP; u += NT) {
        const int r8 = u / KP, k = u - r8 * KP;
        uint32_t lo[4] = {0u, 0u, 0u, 0u}, hi[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int row = 8 * r8 + e;
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
            const uint32_t pb = pack_bf16x2(b0, b1);
            *reinterpret_cast<uint32_t*>(Bt + static_cast<size_t>(row) * N + 2 * k) = pb;
            *reinterpret_cast<uint32_t*>(Ct + static_cast<size_t>(row) * N + 2 * k) = pack_bf16x2(c0, c1);
            if (e & 1) {
                lo[e >> 1] |= (pb & 0xffffu) << 16;
                hi[e >> 1] |= pb & 0xffff0000u;
            } else {
                lo[e >> 1] = pb & 0xffffu;
                hi[e >> 1] = pb >> 16;
            }
        }
        *reinterpret_cast<uint4*>(BtT + static_cast<size_t>(2 * k) * QR + 8 * r8) = uint4{lo[0], lo[1], lo[2], lo[3]};
        *reinterpret_cast<uint4*>(BtT + static_cast<size_t>(2 * k + 1) * QR + 8 * r8) = uint4{hi[0], hi[1], hi[2], hi[3]};
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

// Swap a value with the neighbouring lane (lane ^ 1) through a DPP quad permutation.
__device__ __forceinline__ float swap_adjacent(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));
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

template <int R, int Q, int NW, bool FULL>
__global__ __launch_bounds__(64 * NW) void scan_mfma(ScanParams p) {
    constexpr int NTH = 64 * NW;
    constexpr int QR = Q * R;
    constexpr int NB = QR / 16;          // 16-row blocks of the chunk
    constexpr int XS = QR + 8;           // row stride (elements) of sXT / sXsT
    constexpr int BS = N + 8;            // row stride of sBt and sST
    constexpr int RT = N / (16 * NW);    // 16-row state tiles per wave
    constexpr int KS = QR / 32;          // k-steps of the state contraction
    constexpr int BPT = (QR * (N / 8)) / NTH;              // 16-byte units of Bt per thread
    constexpr int RB = (QR * 8 / NTH) < 1 ? 1 : (QR * 8 / NTH);   // X staging unit: RB rows x 8 columns
    constexpr int XU = (QR / RB) * 8;    // X staging units per chunk (<= NTH)
    constexpr int MB = (NB + NW - 1) / NW;                 // row blocks per wave
    constexpr bool AF_EARLY = (QR <= 128);                 // prefetch Bt^T fragments a chunk ahead
    static_assert(RT >= 1 && QR % 32 == 0 && Q <= 64 && XU <= NTH && (QR * (N / 8)) % NTH == 0 && BPT >= 1 &&
                      (RB == 1 || RB == 2 || RB == 4),
                  "tiling");

    __shared__ __align__(16) uint16_t sXsT[P * XS];                // (s_j X_j)^T: [p][token*R + r]
    __shared__ __align__(16) uint16_t sXT[FULL ? P * XS : 8];      // X^T
    __shared__ __align__(16) uint16_t sBt[FULL ? QR * BS : 8];     // Bt token-major
    __shared__ __align__(16) uint16_t sST[FULL ? P * BS : 8];      // S^T (bf16): [p][n]
    __shared__ float sCum[2][Q], sEc[2][Q], sSc[2][Q], sW[2][Q], sGam[2][Q];   // by chunk parity
    __shared__ float sCs[2][KP * 2];
    __shared__ float sDec[2];

    int seg, h, b;
    xcd_decode(blockIdx.x, gridDim.x, p.H, FULL ? p.nseg : p.nseg - 1, &b, &h, &seg);
    const int g = h / (p.H / p.G);
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int l16 = lane & 15, lg = lane >> 4;
    const int n0 = 16 * RT * w;                  // first state row owned by this wave
    const PrepLayout lay{QR};
    const float Ah = p.A[h], Dh = p.D[h];
    const int c_begin = seg * p.chunks_per_seg;
    const int c_end = min(p.nchunks, c_begin + p.chunks_per_seg);
    const bool last_seg = (seg == p.nseg - 1);
    const size_t gbase = (static_cast<size_t>(b) * p.G + g) * p.nchunks;
    const int xrb = tid % (QR / RB), xpo = tid / (QR / RB);   // X unit: rows RB*xrb.., columns 8*xpo..

    // ---- state accumulators: rows n = n0 + 16rt + 4lg + i, columns p = 16ct + l16
    f32x4 sacc[RT][4];
    if (FULL) {
        const float c1 = (p.L > 0 && p.bl_in && p.xl_in)
                             ? (1.f - p.lam[(static_cast<int64_t>(b) * p.L) * p.H + h]) *
                                   p.dt[(static_cast<int64_t>(b) * p.L) * p.H + h]
                             : 0.f;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int ct = 0; ct < 4; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int n = n0 + 16 * rt + 4 * lg + i, col = 16 * ct + l16;
                    sacc[rt][ct][i] =
                        p.s_init ? p.s_init[((static_cast<size_t>(b) * p.H + h) * p.nseg + seg) * N * P + n * P + col]
                                 : initial_state<R>(p, b, h, g, n, col, c1);
                }
    } else {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) sacc[rt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // ---- registers holding the next chunk's inputs (raw loads; validity applied by the consumer)
    u32v<4 * RB> xr;            // X rows RB*xrb + e, columns 8*xpo .. +7
    u32v<4 * BPT> br;           // Bt units tid + NTH*e
    float pd0 = 0.f, pl0 = 0.f, pd1 = 0.f, pl1 = 0.f, pcs = 0.f;
    int pnq = 0;                // valid tokens of the prefetched chunk
    bfv<32> cf;                 // Ct fragments (4 k-steps) of the wave's current row block
    bfv<8 * KS * RT> af;        // Bt^T fragments of this wave's state rows

#define M3_FETCH(c_)                                                                                          \
    do {                                                                                                      \
        const int64_t t0f = static_cast<int64_t>(c_) * Q;                                                     \
        const int nqf = static_cast<int>(p.L - t0f < Q ? p.L - t0f : Q);                                      \
        pnq = nqf;                                                                                            \
        if (XU == NTH || tid < XU) {                                                                          \
            _Pragma("unroll") for (int e = 0; e < RB; ++e) {                                                  \
                const int row = RB * xrb + e;                                                                 \
                const int i = row / R, r = row - i * R;                                                       \
                const int ic = i < nqf ? i : nqf - 1;                                                         \
                set_quad(xr, e,                                                                               \
                         *reinterpret_cast<const uint4*>(p.x + (((b * p.L + t0f + ic) * p.H + h) * R + r) *   \
                                                                   static_cast<size_t>(P) + 8 * xpo));        \
            }                                                                                                 \
        }                                                                                                     \
        if (FULL) {                                                                                           \
            const uint16_t* gBt = reinterpret_cast<const uint16_t*>(p.prep + (gbase + (c_)) * lay.bytes() +   \
                                                                    lay.bt());                                \
            _Pragma("unroll") for (int e = 0; e < BPT; ++e)                                                   \
                set_quad(br, e, *reinterpret_cast<const uint4*>(gBt + static_cast<size_t>(tid + NTH * e) * 8)); \
        }                                                                                                     \
        if (w == 0) {                                                                                         \
            const int64_t tf = t0f + (lane < nqf ? lane : nqf - 1);                                           \
            const int64_t tf1 = (tf + 1 < p.L) ? tf + 1 : tf;                                                 \
            pd0 = p.dt[(b * p.L + tf) * p.H + h];                                                             \
            pl0 = p.lam[(b * p.L + tf) * p.H + h];                                                            \
            pd1 = p.dt[(b * p.L + tf1) * p.H + h];                                                            \
            pl1 = p.lam[(b * p.L + tf1) * p.H + h];                                                           \
        }                                                                                                     \
        if (tid < 2 * KP) pcs = reinterpret_cast<const float*>(p.prep + (gbase + (c_)) * lay.bytes() + lay.cs())[tid]; \
    } while (0)

#define M3_LOAD_CF(c_, a_)                                                                                    \
    do {                                                                                                      \
        const uint16_t* gCt = reinterpret_cast<const uint16_t*>(p.prep + (gbase + (c_)) * lay.bytes() + lay.ct()); \
        _Pragma("unroll") for (int ks = 0; ks < 4; ++ks)                                                      \
            set_oct(cf, ks, *reinterpret_cast<const bf16x8*>(gCt + static_cast<size_t>(16 * (a_) + l16) * N + 32 * ks + 8 * lg)); \
    } while (0)

#define M3_LOAD_AF(c_)                                                                                        \
    do {                                                                                                      \
        const uint16_t* gBtT = reinterpret_cast<const uint16_t*>(p.prep + (gbase + (c_)) * lay.bytes() + lay.btT()); \
        _Pragma("unroll") for (int ks = 0; ks < KS; ++ks)                                                     \
            _Pragma("unroll") for (int rt = 0; rt < RT; ++rt)                                                 \
                set_oct(af, ks * RT + rt,                                                                     \
                        *reinterpret_cast<const bf16x8*>(gBtT + static_cast<size_t>(n0 + 16 * rt + l16) * QR + 32 * ks + 8 * lg)); \
    } while (0)

    // Per-token scalars (wave 0, lane = token) of the prefetched chunk into parity slot q_.
#define M3_STAGE_SCALARS(q_)                                                                                  \
    do {                                                                                                      \
        if (w == 0) {                                                                                         \
            const bool valid = lane < pnq;                                                                    \
            const int64_t tl = static_cast<int64_t>(0);                                                       \
            (void)tl;                                                                                         \
            const float dtv = valid ? pd0 : 0.f, lv = valid ? pl0 : 0.f;                                      \
            const bool has1 = valid && (nextpos + lane + 1 < p.L);                                            \
            const float a = dtv * Ah;                                                                         \
            const float gm = lv * dtv;                                                                        \
            const float wv = gm + (has1 ? (1.f - pl1) * pd1 : 0.f);                                           \
            float cum = a;                                                                                    \
            _Pragma("unroll") for (int off = 1; off < 64; off <<= 1) {                                        \
                const float o = __shfl_up(cum, off);                                                          \
                if (lane >= off) cum += o;                                                                    \
            }                                                                                                 \
            const float cend = __shfl(cum, Q - 1);                                                            \
            if (lane < Q) {                                                                                   \
                sCum[q_][lane] = cum;                                                                         \
                sEc[q_][lane] = __expf(cum);                                                                  \
                sSc[q_][lane] = __expf(cend - cum) * wv;                                                      \
                sW[q_][lane] = wv;                                                                            \
                sGam[q_][lane] = gm;                                                                          \
            }                                                                                                 \
            if (lane == 0) sDec[q_] = cend;                                                                   \
        }                                                                                                     \
        if (tid < 2 * KP) sCs[q_][tid] = pcs;                                                                 \
    } while (0)

    // X^T and (s X)^T (small transposes in registers) and Bt into LDS.
#define M3_STAGE_TILES(q_)                                                                                    \
    do {                                                                                                      \
        if (XU == NTH || tid < XU) {                                                                          \
            float sc[RB];                                                                                     \
            uint4 xq[RB];                                                                                     \
            _Pragma("unroll") for (int e = 0; e < RB; ++e) {                                                  \
                const int tok = (RB * xrb + e) / R;                                                           \
                sc[e] = sSc[q_][tok];                                                                         \
                xq[e] = (tok < pnq) ? quad(xr, e) : uint4{0u, 0u, 0u, 0u};                                    \
            }                                                                                                 \
            _Pragma("unroll") for (int pp = 0; pp < 8; ++pp) {                                                \
                uint16_t v[RB];                                                                               \
                _Pragma("unroll") for (int e = 0; e < RB; ++e) {                                              \
                    const uint32_t wv = (pp < 2) ? xq[e].x : (pp < 4) ? xq[e].y : (pp < 6) ? xq[e].z : xq[e].w; \
                    v[e] = (pp & 1) ? static_cast<uint16_t>(wv >> 16) : static_cast<uint16_t>(wv & 0xffff);   \
                }                                                                                             \
                const int off = (8 * xpo + pp) * XS + RB * xrb;                                               \
                if constexpr (RB == 1) {                                                                      \
                    if (FULL) sXT[off] = v[0];                                                                \
                    sXsT[off] = static_cast<uint16_t>(pack_bf16x2(bits_to_f(v[0]) * sc[0], 0.f) & 0xffff);    \
                } else {                                                                                      \
                    uint32_t raw[RB / 2], scl[RB / 2];                                                        \
                    _Pragma("unroll") for (int e = 0; e < RB / 2; ++e) {                                      \
                        raw[e] = v[2 * e] | (static_cast<uint32_t>(v[2 * e + 1]) << 16);                      \
                        scl[e] = pack_bf16x2(bits_to_f(v[2 * e]) * sc[2 * e], bits_to_f(v[2 * e + 1]) * sc[2 * e + 1]); \
                    }                                                                                         \
                    if constexpr (RB == 2) {                                                                  \
                        if (FULL) *reinterpret_cast<uint32_t*>(&sXT[off]) = raw[0];                           \
                        *reinterpret_cast<uint32_t*>(&sXsT[off]) = scl[0];                                    \
                    } else {                                                                                  \
                        if (FULL) *reinterpret_cast<uint2*>(&sXT[off]) = uint2{raw[0], raw[1]};               \
                        *reinterpret_cast<uint2*>(&sXsT[off]) = uint2{scl[0], scl[1]};                        \
                    }                                                                                         \
                }                                                                                             \
            }                                                                                                 \
        }                                                                                                     \
        if (FULL) {                                                                                           \
            _Pragma("unroll") for (int e = 0; e < BPT; ++e) {                                                 \
                const int u = tid + NTH * e;                                                                  \
                *reinterpret_cast<uint4*>(&sBt[(u >> 4) * BS + 8 * (u & 15)]) = quad(br, e);                  \
            }                                                                                                 \
        }                                                                                                     \
    } while (0)

#define M3_WRITE_SST()                                                                                        \
    do {                                                                                                      \
        _Pragma("unroll") for (int rt = 0; rt < RT; ++rt)                                                     \
            _Pragma("unroll") for (int ct = 0; ct < 4; ++ct) {                                                \
                const uint2 v = {pack_bf16x2(sacc[rt][ct][0], sacc[rt][ct][1]),                               \
                                 pack_bf16x2(sacc[rt][ct][2], sacc[rt][ct][3])};                              \
                *reinterpret_cast<uint2*>(&sST[(16 * ct + l16) * BS + n0 + 16 * rt + 4 * lg]) = v;            \
            }                                                                                                 \
    } while (0)

    auto row_block = [&](int m) { return (m & 1) ? ((m + 1) * NW - 1 - w) : (m * NW + w); };  // snake order
    int64_t nextpos = 0;          // first token of the prefetched chunk

    // ---- prologue: chunk c_begin into LDS, chunk c_begin+1 into registers
    if (c_begin < c_end) {
        M3_FETCH(c_begin);
        nextpos = static_cast<int64_t>(c_begin) * Q;
        M3_STAGE_SCALARS(c_begin & 1);
        __syncthreads();
        M3_STAGE_TILES(c_begin & 1);
        if (FULL && row_block(0) < NB) M3_LOAD_CF(c_begin, row_block(0));
        if (!FULL || AF_EARLY) M3_LOAD_AF(c_begin);
        if (c_begin + 1 < c_end) {
            M3_FETCH(c_begin + 1);
            nextpos = static_cast<int64_t>(c_begin + 1) * Q;
        }
    }
    if (FULL) M3_WRITE_SST();
    __syncthreads();

    float dec_total = 0.f;                 // state-only: sum of chunk log-decays
    float rot_c = 1.f, rot_s = 0.f;        // state-only: total rotation of pair tid (tid < KP)

    for (int c = c_begin; c < c_end; ++c) {
        const int q = c & 1;
        const int64_t t0 = static_cast<int64_t>(c) * Q;
        const int nq = static_cast<int>(p.L - t0 < Q ? p.L - t0 : Q);
        const bool has_next = c + 1 < c_end;

        if (FULL) {
            // (4) outputs, row blocks in snake order across the waves (balances the causal work)
#pragma unroll
            for (int m = 0; m < MB; ++m) {
                const int a = row_block(m);
                if (a >= NB) continue;
                if (m > 0) M3_LOAD_CF(c, a);
                f32x4 yacc[4];
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) {
                    yacc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks)
                        yacc[ct] = mfma_k32(oct(cf, ks), *reinterpret_cast<const bf16x8*>(&sST[(16 * ct + l16) * BS + 32 * ks + 8 * lg]),
                                            yacc[ct]);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float ec = sEc[q][(16 * a + 4 * lg + i) / R];
#pragma unroll
                    for (int ct = 0; ct < 4; ++ct) yacc[ct][i] *= ec;
                }
                const int ti = (16 * a + l16) / R;
                const float cum_i = sCum[q][ti], gam_i = sGam[q][ti];
                auto mask = [&](int tj) {        // branch-free: every lane evaluates the exp
                    const float ex = __expf(fminf(cum_i - sCum[q][tj], 0.f)) * sW[q][tj];
                    return (tj < ti) ? ex : ((tj == ti) ? gam_i : 0.f);
                };
                for (int bb = 0; bb <= a; ++bb) {
                    f32x4 gt = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks)
                        gt = mfma_k32(*reinterpret_cast<const bf16x8*>(&sBt[(16 * bb + l16) * BS + 32 * ks + 8 * lg]), oct(cf, ks), gt);
                    // gt[e] = (Ct Bt^T)[i = 16a + l16][j = 16bb + 4lg + e]
                    float mv[4];
                    if (R == 4) {
                        const float m0 = mask(4 * bb + lg);
                        mv[0] = mv[1] = mv[2] = mv[3] = m0;
                    } else if (R == 2) {
                        const float m0 = mask(8 * bb + 2 * lg), m1 = mask(8 * bb + 2 * lg + 1);
                        mv[0] = mv[1] = m0;
                        mv[2] = mv[3] = m1;
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e) mv[e] = mask((16 * bb + 4 * lg + e) / R);
                    }
                    const uint2 mp = {pack_bf16x2(mv[0] * gt[0], mv[1] * gt[1]), pack_bf16x2(mv[2] * gt[2], mv[3] * gt[3])};
                    const s16x4 mf = __builtin_bit_cast(s16x4, mp);
#pragma unroll
                    for (int ct = 0; ct < 4; ++ct)
                        yacc[ct] = mfma_k16(mf, *reinterpret_cast<const s16x4*>(&sXT[(16 * ct + l16) * XS + 16 * bb + 4 * lg]),
                                            yacc[ct]);
                }
                // next chunk's Ct for the first row block: cf is dead once the last block is done
                if (m == MB - 1 || row_block(m + 1) >= NB) {
                    if (has_next && row_block(0) < NB) M3_LOAD_CF(c + 1, row_block(0));
                }
                // skip term, then store column pairs: lanes 2j and 2j+1 swap halves so
                // each writes two rows of two adjacent columns as 4-byte words
                const bool odd = l16 & 1;
                const int rbase = 16 * a + 4 * lg + (odd ? 2 : 0);
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) {
                    const s16x4 xv = *reinterpret_cast<const s16x4*>(&sXT[(16 * ct + l16) * XS + 16 * a + 4 * lg]);
                    float v[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) v[i] = yacc[ct][i] + Dh * bits_to_f(static_cast<uint16_t>(xv[i]));
                    const float r0 = swap_adjacent(odd ? v[0] : v[2]);
                    const float r1 = swap_adjacent(odd ? v[1] : v[3]);
                    const uint32_t w0 = odd ? pack_bf16x2(r0, v[2]) : pack_bf16x2(v[0], r0);
                    const uint32_t w1 = odd ? pack_bf16x2(r1, v[3]) : pack_bf16x2(v[1], r1);
                    const int col = 16 * ct + (l16 & ~1);
#pragma unroll
                    for (int qq = 0; qq < 2; ++qq) {
                        const int row = rbase + qq;
                        const int tk = row / R, r = row - tk * R;
                        if (tk < nq)
                            *reinterpret_cast<uint32_t*>(
                                p.y + (((b * p.L + t0 + tk) * p.H + h) * R + r) * static_cast<size_t>(P) + col) = qq ? w1 : w0;
                    }
                }
            }
            if (!AF_EARLY) M3_LOAD_AF(c);
        }
        if (has_next) M3_STAGE_SCALARS(q ^ 1);   // the other parity slot: nobody reads it now
        __syncthreads();   // S_{c-1} no longer read; next chunk's scalars visible

        // (5) state update: S <- R(phi_end) [e^{cum_end} S + Bt^T (s X)]
        {
            const float cend = sDec[q];
            const float decay = __expf(cend);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) sacc[rt][ct] *= decay;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) {
                    const bf16x8 bx = *reinterpret_cast<const bf16x8*>(&sXsT[(16 * ct + l16) * XS + 32 * ks + 8 * lg]);
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt) sacc[rt][ct] = mfma_k32(oct(af, ks * RT + rt), bx, sacc[rt][ct]);
                }
            if ((!FULL || AF_EARLY) && has_next) M3_LOAD_AF(c + 1);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int i = 0; i < 4; i += 2) {
                    const int k = (n0 + 16 * rt + 4 * lg + i) >> 1;
                    const float cn = sCs[q][2 * k], sn = sCs[q][2 * k + 1];
#pragma unroll
                    for (int ct = 0; ct < 4; ++ct) {
                        const float s0 = sacc[rt][ct][i], s1 = sacc[rt][ct][i + 1];
                        sacc[rt][ct][i] = cn * s0 - sn * s1;
                        sacc[rt][ct][i + 1] = sn * s0 + cn * s1;
                    }
                }
            if (FULL) {
                M3_WRITE_SST();
            } else {
                dec_total += cend;
                if (tid < KP) {
                    const float cn = sCs[q][2 * tid], sn = sCs[q][2 * tid + 1];
                    const float nc = cn * rot_c - sn * rot_s, ns = sn * rot_c + cn * rot_s;
                    rot_c = nc;
                    rot_s = ns;
                }
            }
        }
        if (has_next) {
            __syncthreads();   // the chunk's X / Bt tiles are no longer read
            M3_STAGE_TILES(q ^ 1);
            if (c + 2 < c_end) {
                M3_FETCH(c + 2);
                nextpos = static_cast<int64_t>(c + 2) * Q;
            }
        }
        __syncthreads();
    }
#undef M3_FETCH
#undef M3_LOAD_CF
#undef M3_LOAD_AF
#undef M3_STAGE_SCALARS
#undef M3_STAGE_TILES
#undef M3_WRITE_SST

    // epilogue
    if (FULL) {
        if (last_seg && p.h_out) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int ct = 0; ct < 4; ++ct)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int n = n0 + 16 * rt + 4 * lg + i, col = 16 * ct + l16;
                        p.h_out[(static_cast<size_t>(b) * p.H + h) * N * P + n * P + col] = sacc[rt][ct][i];
                    }
        }
    } else {
        const size_t sidx = (static_cast<size_t>(b) * p.H + h) * (p.nseg - 1) + seg;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int ct = 0; ct < 4; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int n = n0 + 16 * rt + 4 * lg + i, col = 16 * ct + l16;
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
    constexpr int NW = (Q * R >= 128) ? 8 : 4;   // waves per workgroup
    const int nchunks = static_cast<int>((a.L + a.Q - 1) / a.Q);
    if (nchunks == 0) return hipSuccess;
    const int nseg = plan.nseg;
    const int cps = (nchunks + nseg - 1) / nseg;
    if (static_cast<int64_t>(nseg) * a.H * a.batch > 0x7fffffffLL) return hipErrorInvalidValue;
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
        hipLaunchKernelGGL((mf::scan_mfma<R, Q, NW, false>), dim3(static_cast<unsigned>((nseg - 1) * a.H * a.batch)),
                           dim3(64 * NW), 0, st, p);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        float* s_init = reinterpret_cast<float*>(base + ws.s_init);
        hipLaunchKernelGGL((mf::seg_pass<R>), dim3(static_cast<unsigned>(a.batch * a.H)), dim3(mf::NT), 0, st, p,
                           s_init);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        p.s_init = s_init;
    }
    hipLaunchKernelGGL((mf::scan_mfma<R, Q, NW, true>), dim3(static_cast<unsigned>(nseg * a.H * a.batch)),
                       dim3(64 * NW), 0, st, p);
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
