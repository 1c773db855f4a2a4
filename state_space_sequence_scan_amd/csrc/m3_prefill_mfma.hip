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
//              token-major ([Q*R][N]), and cos/sin of the chunk's total angle
//              phi_end.  B, C and theta are shared by the H/G heads of a group, so
//              this work is done once per group, not once per head.
//  scan_mfma   one workgroup per (b, h, segment of chunks), 4 waves up to 64 rows
//              per chunk (Q * R), one or two 16-row blocks of the chunk per wave
//              (8 waves at 256 rows).  The N x P state lives in MFMA
//              accumulators, split over the waves in 16 x 16 tiles.  Per chunk:
//                Y      = diag(e^cum) Ct S  +  (M o Ct Bt^T) X  +  D X
//                S     <- R(phi_end) [ e^{cum_end} S  +  Bt^T diag(s) X ]
//              with M the decay/trapezoid mask and s_j = e^{cum_end - cum_j} w_j.
//              Y is computed transposed (Y^T = S^T Ct^T + X^T (M o G)^T), so a
//              lane ends up holding four consecutive columns of one output row.
//              The mask is applied to G^T = Bt Ct^T tiles in registers: the 16x16
//              accumulator layout of a 16x16x32 MFMA (4 consecutive rows per lane)
//              is exactly the B-operand layout of a 16x16x16 MFMA, so the masked
//              tile feeds the next contraction without leaving the registers.
//              Off the diagonal the decay factors into a row part and a column
//              part, each at most 1 (see scan_mfma), so those tiles need no
//              exponentials; D X is two more small contractions (D split into a
//              bf16 high and low part) so that it is not rounded to bf16.  The
//              state contraction reads Bt^T straight from the token-major Bt tile
//              in LDS with the transposing 64-bit LDS read of gfx950.
//              In state-only mode (segment summaries) only the S update runs.
//  seg_pass    one thread per (b, h, rotation pair, column): carries the pair
//              through the segment summaries, giving the state entering each
//              segment (sequential over segments).
#include "m3_mfma_common.h"

namespace m3 {
namespace mf {

// Workspace layout of the prepared operands for one (b, g, chunk).
struct PrepLayout {
    int QR;
    __host__ __device__ size_t bt() const { return 0; }                                    // [QR][N] bf16
    __host__ __device__ size_t ct() const { return static_cast<size_t>(QR) * N * 2; }      // [QR][N] bf16
    __host__ __device__ size_t cs() const { return static_cast<size_t>(QR) * N * 4; }      // [KP][2] fp32
    __host__ __device__ size_t bytes() const { return cs() + KP * 2 * sizeof(float); }
};

// ------------------------------------------------------------------------------------
// rope_prep
// ------------------------------------------------------------------------------------

template <int R, int Q>
__global__ __launch_bounds__(NT) void rope_prep(const uint16_t* __restrict__ B,
                                                const uint16_t* __restrict__ C,
                                                const float* __restrict__ theta, int64_t L, int G,
                                                int nchunks, uint8_t* __restrict__ prep,
                                                const int64_t* __restrict__ cu, int64_t T, Fusion fu) {
    constexpr int QR = Q * R;
    __shared__ float sCos[Q][KP], sSin[Q][KP];
    __shared__ float sPart[4][KP];
    // One workgroup per (b, angle group j, chunk).  The angle groups are those of the
    // B/C groups unless the fusion asks for finer ones (angles per head over shared B, C):
    // group j then reads B and C of group j / (Gt / G).
    const int Gt = fu.tgroups(G);
    const int c = blockIdx.x, j = blockIdx.y, b = blockIdx.z;
    const int g = j / (Gt / G);
    const int tid = threadIdx.x;
    const SeqSpan sp = seq_span(cu, b, L, T);
    const int64_t t0 = static_cast<int64_t>(c) * Q;
    if (t0 >= sp.len) return;                 // no such chunk in this sequence: nothing reads it
    const int nq = static_cast<int>(sp.len - t0 < Q ? sp.len - t0 : Q);
    const int64_t tg = sp.start + t0;         // first token of the chunk in the packed arrays
    const PrepLayout lay{QR};
    uint8_t* base = prep + ((static_cast<size_t>(b) * Gt + j) * nchunks + c) * lay.bytes();
    uint16_t* Bt = reinterpret_cast<uint16_t*>(base + lay.bt());
    uint16_t* Ct = reinterpret_cast<uint16_t*>(base + lay.ct());
    float* cs = reinterpret_cast<float*>(base + lay.cs());

    // One unit = one row (token, rank) x 4 consecutive rotation pairs k0 .. k0 + 3: 16 bytes
    // of B and of C per lane, a row on 16 lanes (so a row's RMSNorm before the rotation is
    // a sum over 16 lanes).  Rows past the sequence end read the last token's operands and
    // store zeros, so every lane of a row takes the same path.  The first units' operands
    // are loaded before the angle sums, so that their latency overlaps that phase.
    static_assert(KP == 64 && N == 128 && (QR * 16) % NT == 0, "16 lanes per row");
    constexpr int UPT = QR * 16 / NT;        // units per thread
    constexpr int PF = UPT < 4 ? UPT : 4;    // of which loaded ahead
    auto unit_src = [&](int e) __attribute__((always_inline)) -> size_t {
        const int u = tid + NT * e, row = u >> 4;
        const int i = row / R, r = row - i * R;
        const int ic = i < nq ? i : nq - 1;
        return (((tg + ic) * G + g) * R + r) * static_cast<size_t>(N) + 8 * (u & 15);
    };
    uint4 pb[PF], pc[PF];
#pragma unroll
    for (int e = 0; e < PF; ++e) {
        const size_t o = unit_src(e);
        pb[e] = *reinterpret_cast<const uint4*>(B + o);
        pc[e] = *reinterpret_cast<const uint4*>(C + o);
    }

    // Chunk-local inclusive angle sums: 4 threads per pair, Q/4 tokens each.
    {
        constexpr int QP = Q / 4;
        const int k = tid % KP, part = tid / KP;
        float th[QP];
        float run = 0.f;
#pragma unroll
        for (int e = 0; e < QP; ++e) {
            const int i = part * QP + e;
            run += (i < nq) ? theta[((tg + i) * Gt + j) * KP + k] : 0.f;
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
    // The rotation, R(-phi) (x0, x1) = (c x0 + s x1, -s x0 + c x1), unit by unit.
    const bool bc = fu.bc();
#pragma unroll
    for (int e8 = 0; e8 < UPT; ++e8) {
        const int u = tid + NT * e8;
        const int row = u >> 4, q4 = u & 15, k0 = 4 * q4;
        const int i = row / R, r = row - i * R;
        const int ic = i < nq ? i : nq - 1;
        uint4 bb, cc;
        if (e8 < PF) {
            bb = pb[e8];
            cc = pc[e8];
        } else {
            const size_t o = unit_src(e8);
            bb = *reinterpret_cast<const uint4*>(B + o);
            cc = *reinterpret_cast<const uint4*>(C + o);
        }
        const float4 cn4 = *reinterpret_cast<const float4*>(&sCos[ic][k0]);
        const float4 sn4 = *reinterpret_cast<const float4*>(&sSin[ic][k0]);
        const uint32_t bw[4] = {bb.x, bb.y, bb.z, bb.w}, cw[4] = {cc.x, cc.y, cc.z, cc.w};
        float x[8], y[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            x[2 * e] = bits_to_f(bw[e] & 0xffff);
            x[2 * e + 1] = bits_to_f(bw[e] >> 16);
            y[2 * e] = bits_to_f(cw[e] & 0xffff);
            y[2 * e + 1] = bits_to_f(cw[e] >> 16);
        }
        if (bc) {   // uniform
            const int wi = r * N + 8 * q4;
            if (fu.bnw) {
                float ss = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) ss += x[e] * x[e];
                const float sc = rsqrtf(row16_sum(ss) / N + fu.eps);
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] *= sc * fu.bnw[wi + e];
            }
            if (fu.cnw) {
                float ss = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) ss += y[e] * y[e];
                const float sc = rsqrtf(row16_sum(ss) / N + fu.eps);
#pragma unroll
                for (int e = 0; e < 8; ++e) y[e] *= sc * fu.cnw[wi + e];
            }
            if (fu.bbias) {
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] += fu.bbias[wi + e];
            }
            if (fu.cbias) {
#pragma unroll
                for (int e = 0; e < 8; ++e) y[e] += fu.cbias[wi + e];
            }
        }
        const float cn[4] = {cn4.x, cn4.y, cn4.z, cn4.w}, sn[4] = {sn4.x, sn4.y, sn4.z, sn4.w};
        uint32_t bo[4], co[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float x0 = x[2 * e], x1 = x[2 * e + 1], y0 = y[2 * e], y1 = y[2 * e + 1];
            bo[e] = pack_bf16x2(cn[e] * x0 + sn[e] * x1, -sn[e] * x0 + cn[e] * x1);
            co[e] = pack_bf16x2(cn[e] * y0 + sn[e] * y1, -sn[e] * y0 + cn[e] * y1);
        }
        const bool live = i < nq;
        *reinterpret_cast<uint4*>(Bt + static_cast<size_t>(row) * N + 8 * q4) =
            live ? uint4{bo[0], bo[1], bo[2], bo[3]} : uint4{0u, 0u, 0u, 0u};
        *reinterpret_cast<uint4*>(Ct + static_cast<size_t>(row) * N + 8 * q4) =
            live ? uint4{co[0], co[1], co[2], co[3]} : uint4{0u, 0u, 0u, 0u};
    }
}

// ------------------------------------------------------------------------------------
// scan_mfma
// ------------------------------------------------------------------------------------
// GATE: the output gate is applied (its input rows are loaded well before the store).
// ONORM: the output RMSNorm follows (after the gate), each output row over its P values.
//
// A chunk of 128 rows (R = 4 at Q = 32, R = 2 at Q = 64) runs on 4 waves, two row blocks
// each, and keeps no s X tile: the state contraction scales the Bt^T fragments by s
// instead.  That brings the output pass to 72 KB of LDS, and with at most 256 registers
// per lane two workgroups share a CU, so one workgroup's loads, barriers and state
// update overlap the other's matrix work (measured 14% faster than one 8-wave
// workgroup per CU).
template <int R, int Q>
constexpr bool kTwoPerCu = (Q * R == 128);
template <int R, int Q, bool FULL>
constexpr int kWavesPerSimd = (FULL && kTwoPerCu<R, Q>) ? 2 : 1;

template <int R, int Q, int NW, bool FULL, bool GATE, bool ONORM, bool MULTI = false>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(kWavesPerSimd<R, Q, FULL>)))
void scan_mfma(ScanParams p) {
    constexpr int NTH = 64 * NW;
    constexpr int QR = Q * R;
    constexpr bool NOXS = FULL && kTwoPerCu<R, Q>;   // state contraction scales Bt^T, reads X
    constexpr int NB = QR / 16;          // 16-row blocks of the chunk
    constexpr int BS = N + 8;            // row stride of sBt and sST
    constexpr int MB = NB > NW ? 2 : 1;  // output row blocks per wave
    constexpr int CT = NW > 8 ? 2 : 4;   // 16-column state tiles per wave
    constexpr int RT = 32 / (NW * CT);   // 16-row state tiles per wave
    constexpr int RW = 8 / RT;           // waves covering the N rows of one column range
    constexpr int KS = QR / 32;          // k-steps of the state contraction
    constexpr int BPT = (QR * (N / 8)) / NTH;              // 16-byte units of Bt per thread
    constexpr int XPT = (QR * (P / 8)) / NTH;              // 16-byte units of X per thread
    constexpr int VN = (NB * Q + NTH - 1) / NTH;           // column-factor entries per thread
    static_assert(RT >= 1 && RT * CT * NW == 32 && QR % 32 == 0 && Q <= 64 && (QR * (N / 8)) % NTH == 0 &&
                      BPT >= 1 && (QR * (P / 8)) % NTH == 0 && XPT >= 1 && (NB <= NW || NB == 2 * NW) &&
                      NW % 4 == 0,
                  "tiling");

    __shared__ __align__(16) uint16_t sXs[NOXS ? 8 : QR * P];      // s_j X_j, row-major, swizzled
    __shared__ __align__(16) uint16_t sX[FULL ? QR * P : 8];       // X, row-major, swizzled
    __shared__ __align__(16) uint16_t sBt[QR * BS];                // Bt token-major
    __shared__ __align__(16) uint16_t sST[FULL ? P * BS : 8];      // S^T (bf16): [p][n]
    __shared__ __align__(16) float sV[FULL ? NB * Q : 4];          // column factors [row block][token]
    __shared__ __align__(16) float sCum[2][Q], sSc[2][Q], sW[2][Q], sGam[2][Q];  // by chunk parity
    __shared__ float sCs[2][KP * 2];
    __shared__ float sDec[2];
    __shared__ __align__(16) float sOW[ONORM ? P : 4];              // output-norm weight of this head

    int seg, h, b;
    xcd_decode(blockIdx.x, gridDim.x, p.H, FULL ? p.nseg : p.nseg - 1, &b, &h, &seg);
    // MULTI: several short sequences per workgroup.  Sequences b .. b + nseq - 1 of head h
    // are swept as one run of chunks (they are adjacent in the token axis and each holds a
    // whole number of chunks), so each one's first chunk is fetched while the previous one
    // computes.  Where a sequence ends its look-ahead weight stops, its state is written out
    // and the state is reset to the next sequence's initial one.
    if (MULTI) b *= p.seqs;
    const int nseq = MULTI ? min(p.seqs, p.batch - b) : 1;
    const int g = h / (p.H / p.G);
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, uniform
    const int l16 = lane & 15, lg = lane >> 4;
    const int n0 = 16 * RT * (w % RW);           // first state row owned by this wave
    const int p0 = 16 * CT * (w / RW);           // first state column owned by this wave
    const PrepLayout lay{QR};
    const float Ah = p.A[h];
    const SeqSpan sp = seq_span(p.cu, b, p.L, p.T);
    const int64_t tb = sp.start, Lb = sp.len * nseq;   // first token and length of the sweep
    const int nchunks_b = static_cast<int>((Lb + Q - 1) / Q);
    const int c_begin = seg * p.chunks_per_seg;
    const int c_end = min(nchunks_b, c_begin + p.chunks_per_seg);
    const bool last_seg = (seg == p.nseg - 1);
    const size_t gbase = (static_cast<size_t>(b) * p.Gt + h / (p.H / p.Gt)) * p.nchunks;   // angle group's operands
    if (ONORM && tid < P) sOW[tid] = p.onw[h * P + tid];   // visible after the prologue's barrier
    const uint32_t HRP = static_cast<uint32_t>(p.H) * R * P;   // elements between tokens of x and y
    // Output row block(s) of this wave (uniform).  Waves w, w+4, .. share a SIMD.  With
    // one block per wave the order 0..3, 7..4, 8..11, 15..12 gives every SIMD the same
    // number of causal tiles (block a has a+1); with two, wave w takes blocks w and
    // 2NW-1-w (a_lo < a_hi), and the B tiles they share are read from LDS once.
    const int a_lo = (MB == 2) ? w : 4 * (w >> 2) + (((w >> 2) & 1) ? 3 - (w & 3) : (w & 3));
    const int a_hi = (MB == 2) ? 2 * NW - 1 - w : a_lo;
    const bool has_rows = NB >= NW || a_lo < NB;   // every wave has rows unless the chunk has fewer blocks
    // per-lane LDS bases (byte addresses); tile accesses add compile-time offsets
    const uint32_t aBtRow = lds_addr(&sBt[l16 * BS + 8 * lg]);                          // Bt tiles, A operand
    const uint32_t aBtTr = lds_addr(&sBt[(4 * lg + (l16 >> 2)) * BS + n0 + 4 * (l16 & 3)]);   // Bt^T, transposed
    const uint32_t aBtW = lds_addr(&sBt[(tid >> 4) * BS + 8 * (tid & 15)]);             // Bt staging
    uint32_t aXTr[4], aXsTr[CT];   // X^T and (s X)^T (X^T when NOXS), transposed: one base per 16-column tile
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
        aXTr[ct] = FULL ? lds_addr(&sX[xoff(4 * lg + (l16 >> 2), 16 * ct + 4 * (l16 & 3))]) : 0u;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
        aXsTr[ct] = lds_addr(&(NOXS ? sX : sXs)[xoff(4 * lg + (l16 >> 2), p0 + 16 * ct + 4 * (l16 & 3))]);
    const uint32_t aXW = FULL ? lds_addr(&sX[xoff(tid >> 3, 8 * (tid & 7))]) : 0u;      // X staging
    const uint32_t aXsW = lds_addr(&sXs[xoff(tid >> 3, 8 * (tid & 7))]);               // sX staging
    const uint32_t aST = FULL ? lds_addr(&sST[l16 * BS + 8 * lg]) : 0u;                 // S^T, A operand
    const uint32_t aSTW = FULL ? lds_addr(&sST[(p0 + l16) * BS + n0 + 4 * lg]) : 0u;    // S^T writes

    // D X as two exact bf16 contractions with diagonal operands D_hi I and D_lo I
    // (B operand of a 16x16x16 MFMA: lane holds rows k = 4lg + e of column l16).
    s16x4 dI_hi, dI_lo;
    {
        const float Dh = p.D[h];
        const __bf16 dh = to_bf(Dh);
        const __bf16 dl = to_bf(Dh - from_bf(dh));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            dI_hi[e] = (4 * lg + e == l16) ? __builtin_bit_cast(short, dh) : short(0);
            dI_lo[e] = (4 * lg + e == l16) ? __builtin_bit_cast(short, dl) : short(0);
        }
    }

    // ---- state accumulators: rows n = n0 + 16rt + 4lg + i, columns p = p0 + 16ct + l16
    f32x4 sacc[RT][CT];
    // initial state of sequence bs (first token tok0) when no segment pass ran
    auto init_state = [&](int bs, int64_t tok0) __attribute__((always_inline)) {
        const float c1 = (Lb > 0 && p.bl_in && p.xl_in)
                             ? (1.f - p.lam[tok0 * p.H + h]) * p.dt[tok0 * p.H + h]
                             : 0.f;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    sacc[rt][ct][i] = initial_state<R>(p, bs, h, g, n0 + 16 * rt + 4 * lg + i, p0 + 16 * ct + l16, c1);
    };
    // final state of sequence bs
    auto store_state = [&](int bs) __attribute__((always_inline)) {
        const size_t ho = (static_cast<size_t>(bs) * p.H + h) * N * P;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int n = n0 + 16 * rt + 4 * lg + i, col = p0 + 16 * ct + l16;
                    state_store(p.h_out, ho + n * P + col, sacc[rt][ct][i], p.state_bf16);
                }
    };
    if (FULL) {
        if (p.s_init) {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int n = n0 + 16 * rt + 4 * lg + i, col = p0 + 16 * ct + l16;
                        sacc[rt][ct][i] = p.s_init[((static_cast<size_t>(b) * p.H + h) * p.sinit_stride +
                                                    static_cast<size_t>(p.sinit_step) * seg) * N * P + n * P + col];
                    }
        } else {
            init_state(b, tb);
        }
    } else {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) sacc[rt][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // ---- registers holding the next chunk's inputs (raw loads; validity applied by the consumer)
    u32v<4 * XPT> xr;           // X units tid + NTH*e: row u / 8, columns 8 (u % 8) .. +7
    u32v<4 * BPT> br;           // Bt units tid + NTH*e
    float pd0 = 0.f, pl0 = 0.f, pd1 = 0.f, pl1 = 0.f, pa0 = 0.f, pcs = 0.f;
    int pnq = 0;                // valid tokens of the prefetched chunk
    bool pend = false;          // the prefetched chunk closes a sequence of a multi-sequence sweep
    bfv<32> cf0, cf1;           // Ct fragments (4 k-steps) of the wave's output row blocks a_lo, a_hi

    // Per-workgroup base pointers are uniform (scalar registers); per-lane offsets
    // within one chunk are 32-bit.
    //
    // Every path through the chunk loop issues the same sequence of global loads
    // and stores (chunk indices of prefetches are clamped, rows past the sequence
    // end are stored to a sink).  The vector-memory counter retires in issue order
    // and the compiler places its waits for the fewest operations any path issues
    // after a load; with equal sequences the wait for this chunk's operands never
    // drains the prefetch of the chunk after next.
    // prepared operands of chunk c of the sweep (with MULTI: chunk c % nchunks of sequence b + c / nchunks)
    const int gq = h / (p.H / p.Gt);
    auto prep_index = [&](int c) __attribute__((always_inline)) -> size_t {
        if constexpr (MULTI)
            return (static_cast<size_t>(b + c / p.nchunks) * p.Gt + gq) * p.nchunks + c % p.nchunks;
        else
            return gbase + c;
    };
#define M3_PREP(c_) (p.prep + prep_index(c_) * lay.bytes())

#define M3_FETCH_X(c_)                                                                                        \
    do {                                                                                                      \
        const int64_t t0f = static_cast<int64_t>(c_) * Q;                                                     \
        const int nqf = static_cast<int>(Lb - t0f < Q ? Lb - t0f : Q);                                        \
        pnq = nqf;                                                                                            \
        pend = MULTI && ((c_) + 1) % p.nchunks == 0;                                                          \
        {                                                                                                     \
            const uint16_t* xch = p.x + ((tb + t0f) * p.H + h) * static_cast<int64_t>(R * P);                 \
            _Pragma("unroll") for (int e = 0; e < XPT; ++e) {                                                 \
                const int u = tid + NTH * e, row = u >> 3;                                                    \
                const int i = row / R, r = row - i * R;                                                       \
                const int ic = i < nqf ? i : nqf - 1;                                                         \
                set_quad(xr, e, *reinterpret_cast<const uint4*>(                                              \
                                    xch + (static_cast<uint32_t>(ic) * HRP + static_cast<uint32_t>(r * P + 8 * (u & 7))))); \
            }                                                                                                 \
        }                                                                                                     \
        {   /* wave 0 uses these; the other waves read one broadcast address */                               \
            const float* dtc = p.dt + (tb + t0f) * p.H + h;                                                   \
            const float* lmc = p.lam + (tb + t0f) * p.H + h;                                                  \
            const int i0 = (w == 0 && lane < nqf) ? lane : 0;                                                 \
            const int i1 = (w == 0 && t0f + i0 + 1 < Lb) ? i0 + 1 : i0;                                       \
            pd0 = dtc[static_cast<uint32_t>(i0 * p.H)];                                                       \
            pl0 = lmc[static_cast<uint32_t>(i0 * p.H)];                                                       \
            pd1 = dtc[static_cast<uint32_t>(i1 * p.H)];                                                       \
            pl1 = lmc[static_cast<uint32_t>(i1 * p.H)];                                                       \
            pa0 = global_view(p.At ? p.At : p.dt)[(tb + t0f) * p.H + h + static_cast<uint32_t>(i0 * p.H)];  \
        }                                                                                                     \
    } while (0)

#define M3_FETCH_B(c_)                                                                                        \
    do {                                                                                                      \
        const uint16_t* gBt = reinterpret_cast<const uint16_t*>(M3_PREP(c_) + lay.bt());                      \
        _Pragma("unroll") for (int e = 0; e < BPT; ++e)                                                       \
            set_quad(br, e, *reinterpret_cast<const uint4*>(gBt + static_cast<uint32_t>(tid + NTH * e) * 8u)); \
        pcs = reinterpret_cast<const float*>(M3_PREP(c_) + lay.cs())[tid & (2 * KP - 1)];                     \
    } while (0)

#define M3_FETCH(c_)                                                                                          \
    do {                                                                                                      \
        M3_FETCH_X(c_);                                                                                       \
        M3_FETCH_B(c_);                                                                                       \
    } while (0)

#define M3_LOAD_CF(dst_, c_, a_)                                                                              \
    do {                                                                                                      \
        const uint16_t* gCt = reinterpret_cast<const uint16_t*>(M3_PREP(c_) + lay.ct());                      \
        _Pragma("unroll") for (int ks = 0; ks < 4; ++ks)                                                      \
            set_oct(dst_, ks, *reinterpret_cast<const bf16x8*>(                                               \
                                  gCt + static_cast<uint32_t>((16 * (a_) + l16) * N + 32 * ks + 8 * lg)));    \
    } while (0)

    // Per-token scalars (wave 0, lane = token) of the prefetched chunk into parity slot q_.
#define M3_STAGE_SCALARS(q_)                                                                                  \
    do {                                                                                                      \
        if (w == 0) {                                                                                         \
            const bool valid = lane < pnq;                                                                    \
            const float dtv = valid ? pd0 : 0.f, lv = valid ? pl0 : 0.f;                                      \
            const bool has1 = valid && (nextpos + lane + 1 < Lb) && !(pend && lane == Q - 1);                 \
            const float gm = lv * dtv;                                                                        \
            const float wv = gm + (has1 ? (1.f - pl1) * pd1 : 0.f);                                           \
            float cum = dtv * (p.At ? pa0 : Ah);                                                              \
            _Pragma("unroll") for (int off = 1; off < 64; off <<= 1) {                                        \
                const float o = __shfl_up(cum, off);                                                          \
                if (lane >= off) cum += o;                                                                    \
            }                                                                                                 \
            const float cend = __shfl(cum, Q - 1);                                                            \
            if (lane < Q) {                                                                                   \
                sCum[q_][lane] = cum;                                                                         \
                sSc[q_][lane] = __expf(cend - cum) * wv;                                                      \
                sW[q_][lane] = wv;                                                                            \
                sGam[q_][lane] = gm;                                                                          \
            }                                                                                                 \
            if (lane == 0) sDec[q_] = cend;                                                                   \
        }                                                                                                     \
        if (tid < 2 * KP) sCs[q_][tid] = pcs;                                                                 \
    } while (0)

    // X and s X (row-major, 16-byte chunks swizzled by row), Bt, and the column
    // factors of the off-diagonal mask tiles, into LDS.
#define M3_STAGE_TILES(q_)                                                                                    \
    do {                                                                                                      \
        _Pragma("unroll") for (int e = 0; e < XPT; ++e) {                                                     \
            const int u = tid + NTH * e, row = u >> 3;                                                        \
            const int tok = row / R;                                                                          \
            const uint4 xq = (tok < pnq) ? quad(xr, e) : uint4{0u, 0u, 0u, 0u};                               \
            if (FULL) lds_st(aXW + e * (NTH / 8) * P * 2, xq);                                         \
            if (!NOXS) {                                                                                      \
                const float sc = sSc[q_][tok];                                                                \
                const uint32_t wq[4] = {xq.x, xq.y, xq.z, xq.w};                                              \
                uint32_t sq[4];                                                                               \
                _Pragma("unroll") for (int k = 0; k < 4; ++k)                                                 \
                    sq[k] = pack_bf16x2(bits_to_f(wq[k] & 0xffff) * sc, bits_to_f(wq[k] >> 16) * sc);         \
                lds_st(aXsW + e * (NTH / 8) * P * 2, uint4{sq[0], sq[1], sq[2], sq[3]});               \
            }                                                                                                 \
        }                                                                                                     \
        _Pragma("unroll") for (int e = 0; e < BPT; ++e) lds_st(aBtW + e * (NTH / 16) * BS * 2, quad(br, e)); \
        if (FULL) {                                                                                           \
            _Pragma("unroll") for (int e = 0; e < VN; ++e) {                                                  \
                const int idx = tid + NTH * e;                                                                \
                const int ab = idx / Q, j = idx - ab * Q, ta = (16 * ab) / R;                                 \
                if (idx < NB * Q && j < ta)                                                                   \
                    sV[idx] = __expf(sCum[q_][ta - 1] - sCum[q_][j]) * sW[q_][j];                             \
            }                                                                                                 \
        }                                                                                                     \
    } while (0)

#define M3_WRITE_SST()                                                                                        \
    do {                                                                                                      \
        _Pragma("unroll") for (int rt = 0; rt < RT; ++rt)                                                     \
            _Pragma("unroll") for (int ct = 0; ct < CT; ++ct) {                                               \
                const uint2 v = {pack_bf16x2(sacc[rt][ct][0], sacc[rt][ct][1]),                               \
                                 pack_bf16x2(sacc[rt][ct][2], sacc[rt][ct][3])};                              \
                lds_st(aSTW + (16 * ct * BS + 16 * rt) * 2, v);                                        \
            }                                                                                                 \
    } while (0)

    // ---- output tiles.  yv[ct] (lane (l16, lg), element e) holds Y^T[p][i] for
    // p = 16ct + 4lg + e and output row i = 16a + l16.
    //
    // Decay of token j < i seen from token i is e^{cum_i - cum_j}.  For a column
    // block before row block a it factors through ref_a = cum at the token just
    // before the block: e^{cum_i - ref_a} (row part E_i) times e^{ref_a - cum_j}
    // (column part, stored with w_j in sV[a][j]).  Both parts are at most 1, so
    // neither overflows, and either one underflows only where the exact product
    // is at least as small.  The row part and e^{ref_a} of the inter-chunk term
    // are applied to the accumulators; only the diagonal tile evaluates the full
    // mask per element.

    // Operands of column block bb_ into register set S_ (A or B): the Bt tile (A operand
    // of G^T), the X^T tile (A operand of the 16x16x16 steps), and the column factors of
    // row block(s) a_lo / a_hi (v0 / v1).  The tile loops load set B for the next column
    // block before working on set A, so the LDS latency is covered by the work on A.
#define M3_LOAD_COLS(S_, bb_)                                                                                 \
    do {                                                                                                      \
        _Pragma("unroll") for (int ks = 0; ks < 4; ++ks)                                                      \
            btf##S_[ks] = lds_ld<bf16x8>(aBtRow + (16 * (bb_) * BS + 32 * ks) * 2);                           \
        _Pragma("unroll") for (int ct = 0; ct < 4; ++ct)                                                      \
            xf##S_[ct] = lds_tr4(aXTr[ct] + 16 * (bb_) * P * 2);                                              \
    } while (0)

    // Keeps the prefetches above the work on the other register set (the scheduler would
    // otherwise sink them next to their uses).
#define M3_FENCE() __builtin_amdgcn_sched_barrier(0)

#define M3_LOAD_V(vv_, a_, bb_)                                                                               \
    do {                                                                                                      \
        const float* vrow = &sV[(a_) * Q];                                                                    \
        if constexpr (R == 1) {                                                                               \
            vv_ = *reinterpret_cast<const float4*>(vrow + 16 * (bb_) + 4 * lg);                               \
        } else if constexpr (R == 2) {                                                                        \
            const float2 v2 = *reinterpret_cast<const float2*>(vrow + 8 * (bb_) + 2 * lg);                    \
            vv_ = float4{v2.x, v2.x, v2.y, v2.y};                                                             \
        } else {                                                                                              \
            const float v1 = vrow[4 * (bb_) + lg];                                                            \
            vv_ = float4{v1, v1, v1, v1};                                                                     \
        }                                                                                                     \
    } while (0)

    // gt_[e] = G[i = 16a + l16][j = 16bb + 4lg + e],  G = Ct Bt^T, from the Bt tile of set S_
#define M3_GTILE(gt_, cfv_, S_)                                                                               \
    do {                                                                                                      \
        gt_ = f32x4{0.f, 0.f, 0.f, 0.f};                                                                      \
        _Pragma("unroll") for (int ks = 0; ks < 4; ++ks) gt_ = mfma_k32(btf##S_[ks], oct(cfv_, ks), gt_);     \
    } while (0)

    // Off-diagonal tile with column factors vv_ (loaded by M3_LOAD_V).
#define M3_OFFDIAG(yv_, cfv_, S_, vv_)                                                                        \
    do {                                                                                                      \
        f32x4 gt;                                                                                             \
        M3_GTILE(gt, cfv_, S_);                                                                               \
        const uint2 mp = {pack_bf16x2(gt[0] * vv_.x, gt[1] * vv_.y), pack_bf16x2(gt[2] * vv_.z, gt[3] * vv_.w)}; \
        const s16x4 mf = __builtin_bit_cast(s16x4, mp);                                                       \
        _Pragma("unroll") for (int ct = 0; ct < 4; ++ct) yv_[ct] = mfma_k16(xf##S_[ct], mf, yv_[ct]);         \
    } while (0)

    // Diagonal tile: row part of the off-diagonal sum, the full mask, and D X.
#define M3_DIAG(yv_, cfv_, a_, S_)                                                                            \
    do {                                                                                                      \
        f32x4 gt;                                                                                             \
        M3_GTILE(gt, cfv_, S_);                                                                               \
        /* every value is loaded unconditionally (vector loads where R < 4) and selected after */            \
        const int ta = (16 * (a_)) / R;                                                                       \
        const float ref_raw = sCum[q][ta > 0 ? ta - 1 : 0];                                                   \
        const float ref = ta > 0 ? ref_raw : 0.f;                                                             \
        const int ti = (16 * (a_) + l16) / R;                                                                 \
        const float cum_i = sCum[q][ti], gam_i = sGam[q][ti];                                                 \
        const int j0 = (16 * (a_) + 4 * lg) / R;                                                              \
        float cj[4], wj[4];                                                                                   \
        if constexpr (R == 1) {                                                                               \
            const float4 c4 = *reinterpret_cast<const float4*>(&sCum[q][j0]);                                 \
            const float4 w4 = *reinterpret_cast<const float4*>(&sW[q][j0]);                                   \
            cj[0] = c4.x; cj[1] = c4.y; cj[2] = c4.z; cj[3] = c4.w;                                           \
            wj[0] = w4.x; wj[1] = w4.y; wj[2] = w4.z; wj[3] = w4.w;                                           \
        } else if constexpr (R == 2) {                                                                        \
            const float2 c2 = *reinterpret_cast<const float2*>(&sCum[q][j0]);                                 \
            const float2 w2 = *reinterpret_cast<const float2*>(&sW[q][j0]);                                   \
            cj[0] = cj[1] = c2.x; cj[2] = cj[3] = c2.y;                                                       \
            wj[0] = wj[1] = w2.x; wj[2] = wj[3] = w2.y;                                                       \
        } else {                                                                                              \
            cj[0] = cj[1] = cj[2] = cj[3] = sCum[q][j0];                                                      \
            wj[0] = wj[1] = wj[2] = wj[3] = sW[q][j0];                                                        \
        }                                                                                                     \
        const float ei = __expf(cum_i - ref);                                                                 \
        _Pragma("unroll") for (int ct = 0; ct < 4; ++ct) yv_[ct] *= ei;                                       \
        float mv[4];                                                                                          \
        _Pragma("unroll") for (int e = 0; e < 4; ++e) {                                                       \
            const int tj = (16 * (a_) + 4 * lg + e) / R;                                                      \
            const float ex = __expf(cum_i - cj[e]) * wj[e];                                                   \
            mv[e] = (tj < ti) ? ex : ((tj == ti) ? gam_i : 0.f);                                              \
        }                                                                                                     \
        const uint2 mp = {pack_bf16x2(gt[0] * mv[0], gt[1] * mv[1]), pack_bf16x2(gt[2] * mv[2], gt[3] * mv[3])}; \
        const s16x4 mf = __builtin_bit_cast(s16x4, mp);                                                       \
        _Pragma("unroll") for (int ct = 0; ct < 4; ++ct) {                                                    \
            yv_[ct] = mfma_k16(xf##S_[ct], mf, yv_[ct]);                                                      \
            yv_[ct] = mfma_k16(xf##S_[ct], dI_hi, yv_[ct]);                                                   \
            yv_[ct] = mfma_k16(xf##S_[ct], dI_lo, yv_[ct]);                                                   \
        }                                                                                                     \
    } while (0)

    // Lane (l16, lg) writes columns 16ct + 4lg .. +3 of output row 16a + l16: 8 bytes per tile.
    // With a gate the row's z values (same place as y; rows past the end read the last
    // token's) multiply y by silu(z) first.
    // Gate input of output row 16a_ + l16 into zr_ (rows past the end read the last token's),
    // loaded a phase ahead of the store that uses it.
#define M3_LOAD_Z(zr_, a_)                                                                                    \
    do {                                                                                                      \
        const int i = 16 * (a_) + l16;                                                                        \
        const int tk = i / R, r = i - tk * R;                                                                 \
        const uint16_t* zrow = p.z + ((tb + t0) * p.H + h) * static_cast<int64_t>(R * P) +                    \
                               (static_cast<uint32_t>(tk < nq ? tk : nq - 1) * HRP +                          \
                                static_cast<uint32_t>(r * P + 4 * lg));                                       \
        _Pragma("unroll") for (int ct = 0; ct < 4; ++ct) zr_[ct] = *reinterpret_cast<const uint2*>(zrow + 16 * ct); \
    } while (0)

    // Lane (l16, lg) writes columns 16ct + 4lg .. +3 of output row 16a + l16: 8 bytes per tile.
    // With the gate, the row's z values (zr_, from M3_LOAD_Z) multiply y by silu(z) first.
#define M3_STORE_Y(yv_, a_, zr_)                                                                              \
    do {                                                                                                      \
        const int i = 16 * (a_) + l16;                                                                        \
        const int tk = i / R, r = i - tk * R;                                                                 \
        if constexpr (GATE) {                                                                                 \
            _Pragma("unroll") for (int ct = 0; ct < 4; ++ct) {                                                \
                const uint2 zz = zr_[ct];                                                                     \
                yv_[ct][0] *= silu(bits_to_f(zz.x & 0xffff));                                                 \
                yv_[ct][1] *= silu(bits_to_f(zz.x >> 16));                                                    \
                yv_[ct][2] *= silu(bits_to_f(zz.y & 0xffff));                                                 \
                yv_[ct][3] *= silu(bits_to_f(zz.y >> 16));                                                    \
            }                                                                                                 \
        }                                                                                                     \
        if constexpr (ONORM) {   /* row i's 64 values sit in lanes l16, l16 + 16, + 32, + 48 */              \
            float ss = 0.f;                                                                                   \
            _Pragma("unroll") for (int ct = 0; ct < 4; ++ct)                                                  \
                _Pragma("unroll") for (int e = 0; e < 4; ++e) ss += yv_[ct][e] * yv_[ct][e];                  \
            ss += __shfl_xor(ss, 16);                                                                         \
            ss += __shfl_xor(ss, 32);                                                                         \
            const float sc = rsqrtf(ss * (1.f / P) + p.eps);                                                  \
            _Pragma("unroll") for (int ct = 0; ct < 4; ++ct) {                                                \
                const float4 wv = *reinterpret_cast<const float4*>(&sOW[16 * ct + 4 * lg]);                  \
                yv_[ct][0] *= sc * wv.x;                                                                      \
                yv_[ct][1] *= sc * wv.y;                                                                      \
                yv_[ct][2] *= sc * wv.z;                                                                      \
                yv_[ct][3] *= sc * wv.w;                                                                      \
            }                                                                                                 \
        }                                                                                                     \
        uint16_t* yrow = (tk < nq) ? ych + (static_cast<uint32_t>(tk) * HRP + static_cast<uint32_t>(r * P + 4 * lg)) \
                                   : p.y_sink + lane * 64;                                                    \
        _Pragma("unroll") for (int ct = 0; ct < 4; ++ct)                                                      \
            *reinterpret_cast<uint2*>(yrow + 16 * ct) =                                                       \
                uint2{pack_bf16x2(yv_[ct][0], yv_[ct][1]), pack_bf16x2(yv_[ct][2], yv_[ct][3])};              \
    } while (0)

    // Inter-chunk term for row block(s), scaled by e^{ref_a}: yv[ct] = e^{ref_a} S^T Ct^T.
#define M3_INTER_SCALE(yv_, a_)                                                                               \
    do {                                                                                                      \
        const int ta = (16 * (a_)) / R;                                                                       \
        const float er = ta > 0 ? __expf(sCum[q][ta - 1]) : 1.f;                                              \
        _Pragma("unroll") for (int ct = 0; ct < 4; ++ct) yv_[ct] *= er;                                       \
    } while (0)

    int64_t nextpos = 0;          // first token of the prefetched chunk

    // ---- prologue: chunk c_begin into LDS, chunk c_begin+1 into registers
    if (c_begin < c_end) {
        M3_FETCH(c_begin);
        nextpos = static_cast<int64_t>(c_begin) * Q;
        M3_STAGE_SCALARS(c_begin & 1);
        __syncthreads();
        const int q = c_begin & 1;
        M3_STAGE_TILES(q);
        if (FULL) {
            M3_LOAD_CF(cf0, c_begin, has_rows ? a_lo : 0);
            if (MB == 2) M3_LOAD_CF(cf1, c_begin, a_hi);
        } else {
            const int cf = c_begin + 1 < c_end ? c_begin + 1 : c_begin;
            M3_FETCH(cf);
            nextpos = static_cast<int64_t>(cf) * Q;
        }
    }
    if (FULL) M3_WRITE_SST();
    __syncthreads();

    // the state entering the current chunk is exactly zero (uniform): no incoming state
    const bool zero_init = !p.s_init && !p.h_in && !(p.bl_in && p.xl_in);
    bool zero_in = MULTI && zero_init;
    float dec_total = 0.f;                 // state-only: sum of chunk log-decays
    float rot_c = 1.f, rot_s = 0.f;        // state-only: total rotation of pair tid (tid < KP)

    for (int c = c_begin; c < c_end; ++c) {
        const int q = c & 1;
        const int64_t t0 = static_cast<int64_t>(c) * Q;
        const int nq = static_cast<int>(Lb - t0 < Q ? Lb - t0 : Q);
        const bool has_next = c + 1 < c_end;
        const int cn = has_next ? c + 1 : c;    // chunk of the register prefetches (clamped)
        if (FULL) {
            // next chunk's X and scalars, issued before this chunk's output contractions
            // so that the loads are in flight while the matrix cores work
            M3_FETCH_X(cn);
            nextpos = static_cast<int64_t>(cn) * Q;
        }

        if (FULL && has_rows) {
            uint16_t* ych = p.y + ((tb + t0) * p.H + h) * static_cast<int64_t>(R * P);
            bf16x8 btfA[4], btfB[4];
            s16x4 xfA[4], xfB[4];
            float4 v0A, v1A, v0B, v1B;
            f32x4 y0[4], y1[4];
            uint2 zr[4];   // gate input of the row block being finished (GATE only)
            if constexpr (GATE) M3_LOAD_Z(zr, a_lo);
            // (4a) inter-chunk term; with two row blocks the S^T fragments serve both.  The
            // fragments of column tile ct + 1 are read while tile ct is multiplied.  In a
            // multi-sequence sweep a state known to be zero (a sequence's first chunk without
            // an incoming state) adds nothing, and the products are skipped (not in the
            // one-sequence kernels: there it would save one chunk's term per sequence, and
            // the branch costs the waits of every other chunk).
            if (MULTI && zero_in) {
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) {
                    y0[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
                    y1[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
            } else {
                bf16x8 sf[2][4];
#pragma unroll
                for (int ks = 0; ks < 4; ++ks) sf[0][ks] = lds_ld<bf16x8>(aST + (32 * ks) * 2);
#pragma unroll
                for (int ct = 0; ct < 4; ++ct) {
                    if (ct + 1 < 4) {
#pragma unroll
                        for (int ks = 0; ks < 4; ++ks)
                            sf[(ct + 1) & 1][ks] = lds_ld<bf16x8>(aST + (16 * (ct + 1) * BS + 32 * ks) * 2);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    y0[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
                    y1[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks) {
                        y0[ct] = mfma_k32(sf[ct & 1][ks], oct(cf0, ks), y0[ct]);
                        if (MB == 2) y1[ct] = mfma_k32(sf[ct & 1][ks], oct(cf1, ks), y1[ct]);
                    }
                }
                M3_INTER_SCALE(y0, a_lo);
                if (MB == 2) M3_INTER_SCALE(y1, a_hi);
            }
            // (4b) intra-chunk tiles, column blocks in order; the diagonal tile closes a row block.
            // Two register sets: the operands of the next column block are read from LDS
            // while the current block is multiplied.
            M3_LOAD_COLS(A, 0);
            M3_LOAD_V(v0A, a_lo, 0);
            if (MB == 2) M3_LOAD_V(v1A, a_hi, 0);
            int bb = 0;
            for (; bb + 1 < a_lo; bb += 2) {   // column blocks bb (set A) and bb + 1 (set B)
                M3_LOAD_COLS(B, bb + 1);
                M3_LOAD_V(v0B, a_lo, bb + 1);
                if (MB == 2) M3_LOAD_V(v1B, a_hi, bb + 1);
                M3_FENCE();
                M3_OFFDIAG(y0, cf0, A, v0A);
                if (MB == 2) M3_OFFDIAG(y1, cf1, A, v1A);
                M3_LOAD_COLS(A, bb + 2);
                M3_LOAD_V(v0A, a_lo, bb + 2);
                if (MB == 2) M3_LOAD_V(v1A, a_hi, bb + 2);
                M3_FENCE();
                M3_OFFDIAG(y0, cf0, B, v0B);
                if (MB == 2) M3_OFFDIAG(y1, cf1, B, v1B);
            }
            if (bb < a_lo) {                   // one block left (bb = a_lo - 1): set A, then set A <- block a_lo
                M3_LOAD_COLS(B, a_lo);
                if (MB == 2) M3_LOAD_V(v1B, a_hi, a_lo);
                M3_FENCE();
                M3_OFFDIAG(y0, cf0, A, v0A);
                if (MB == 2) M3_OFFDIAG(y1, cf1, A, v1A);
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    btfA[k] = btfB[k];
                    xfA[k] = xfB[k];
                }
                v1A = v1B;
            }
            // set A holds block a_lo
            if constexpr (MB == 2) {
                if (a_lo + 1 < a_hi) {
                    M3_LOAD_COLS(B, a_lo + 1);
                    M3_LOAD_V(v1B, a_hi, a_lo + 1);
                } else {
                    M3_LOAD_COLS(B, a_hi);
                }
                M3_FENCE();
            }
            M3_DIAG(y0, cf0, a_lo, A);
            if (MB == 2) M3_OFFDIAG(y1, cf1, A, v1A);
            M3_STORE_Y(y0, a_lo, zr);
            M3_LOAD_CF(cf0, cn, a_lo);
            if constexpr (MB == 2) {
                if constexpr (GATE) M3_LOAD_Z(zr, a_hi);
                // set B holds block a_lo + 1 (or a_hi when that is the next one)
                bb = a_lo + 1;
                for (; bb + 1 < a_hi; bb += 2) {   // blocks bb (set B) and bb + 1 (set A)
                    M3_LOAD_COLS(A, bb + 1);
                    M3_LOAD_V(v1A, a_hi, bb + 1);
                    M3_FENCE();
                    M3_OFFDIAG(y1, cf1, B, v1B);
                    M3_LOAD_COLS(B, bb + 2);
                    if (bb + 2 < a_hi) M3_LOAD_V(v1B, a_hi, bb + 2);
                    M3_FENCE();
                    M3_OFFDIAG(y1, cf1, A, v1A);
                }
                if (bb < a_hi) {                   // bb = a_hi - 1 in set B; then set B <- block a_hi
                    M3_LOAD_COLS(A, a_hi);
                    M3_FENCE();
                    M3_OFFDIAG(y1, cf1, B, v1B);
                    M3_DIAG(y1, cf1, a_hi, A);
                } else {                           // set B holds block a_hi
                    M3_DIAG(y1, cf1, a_hi, B);
                }
                M3_STORE_Y(y1, a_hi, zr);
                M3_LOAD_CF(cf1, cn, a_hi);
            }
        } else if (FULL) {
            // A wave without output rows still issues the stores and loads of one.  (An
            // else branch: a separate if after the output work would merge this path's
            // fresh Ct load into the output path's view of the counters, and the output
            // path would then wait for every load in flight before its first product.)
            uint16_t* yrow = p.y_sink + lane * 64;
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) *reinterpret_cast<uint2*>(yrow + 16 * ct) = uint2{0u, 0u};
            M3_LOAD_CF(cf0, cn, 0);
        }
        if (FULL) M3_FETCH_B(cn);   // next chunk's Bt: registers held only across the state update
        // (5) state update: S <- R(phi_end) [e^{cum_end} S + Bt^T (s X)].  It reads only this
        // chunk's tiles and its own accumulators, so a wave starts it as soon as its outputs
        // are done, overlapping the output work of the other waves.
        {
            const float cend = sDec[q];
            const float decay = __expf(cend);
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) sacc[rt][ct] *= decay;
            // Operands of k-step ks into slot ks & 1: the reads of step ks + 1 are issued
            // before the products of step ks (the fence keeps them there), so each step's
            // LDS latency is covered by the previous step's matrix work.  Lane (l16, lg)
            // supplies contraction rows 32ks + 4lg + (0..3) and 32ks + 16 + 4lg + (0..3)
            // (the same assignment in both operands; 16 rows apart keeps the X tile reads
            // on the bank-conflict-free permutation).
            //   A operand: Bt^T rows n0 + 16rt + l16, read transposed
            //   B operand: (s X)^T column p = p0 + 16ct + l16, read transposed
            // Without the s X tile (NOXS) the B operand is X^T and the A operand is scaled by
            // s_j of its contraction rows in registers just before the products.
            bf16x8 bta[2][RT], bxs[2][CT];
            float4 ssv[2][2];   // NOXS: s of contraction rows 32ks + 4lg + (0..3) and 32ks + 16 + 4lg + (0..3)
            auto load_step = [&](int ks, int slot) __attribute__((always_inline)) {
                if constexpr (NOXS) {
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        const int r0 = 32 * ks + 16 * hh + 4 * lg;   // rows r0 .. r0 + 3 of token r0 / R ..
                        if constexpr (R == 4) {
                            const float v = sSc[q][r0 / 4];
                            ssv[slot][hh] = float4{v, v, v, v};
                        } else if constexpr (R == 2) {
                            const float2 v = *reinterpret_cast<const float2*>(&sSc[q][r0 / 2]);
                            ssv[slot][hh] = float4{v.x, v.x, v.y, v.y};
                        } else {
                            ssv[slot][hh] = *reinterpret_cast<const float4*>(&sSc[q][r0]);
                        }
                    }
                }
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) {
                    const uint32_t src = aBtTr + (32 * ks * BS + 16 * rt) * 2;
                    const s16x4 lo = lds_tr4(src), hi = lds_tr4(src + 16 * BS * 2);
                    bta[slot][rt] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                }
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    const uint32_t xa = aXsTr[ct] + 32 * ks * P * 2;
                    const s16x4 xlo = lds_tr4(xa), xhi = lds_tr4(xa + 16 * P * 2);
                    bxs[slot][ct] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(xlo, xhi, 0, 1, 2, 3, 4, 5, 6, 7));
                }
            };
            load_step(0, 0);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                if (ks + 1 < KS) load_step(ks + 1, (ks + 1) & 1);
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (NOXS) {
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt) {
                        bf16x8 v = bta[ks & 1][rt];
                        const float4 s0 = ssv[ks & 1][0], s1 = ssv[ks & 1][1];
                        const float sc[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
                        for (int e = 0; e < 8; ++e) v[e] = to_bf(from_bf(v[e]) * sc[e]);
                        bta[ks & 1][rt] = v;
                    }
                }
#pragma unroll
                for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt) sacc[rt][ct] = mfma_k32(bta[ks & 1][rt], bxs[ks & 1][ct], sacc[rt][ct]);
            }
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int i = 0; i < 4; i += 2) {
                    const int k = (n0 + 16 * rt + 4 * lg + i) >> 1;
                    const float cn = sCs[q][2 * k], sn = sCs[q][2 * k + 1];
#pragma unroll
                    for (int ct = 0; ct < CT; ++ct) {
                        const float s0 = sacc[rt][ct][i], s1 = sacc[rt][ct][i + 1];
                        sacc[rt][ct][i] = cn * s0 - sn * s1;
                        sacc[rt][ct][i + 1] = sn * s0 + cn * s1;
                    }
                }
            if (!FULL) {
                dec_total += cend;
                if (tid < KP) {
                    const float cn = sCs[q][2 * tid], sn = sCs[q][2 * tid + 1];
                    const float nc = cn * rot_c - sn * rot_s, ns = sn * rot_c + cn * rot_s;
                    rot_c = nc;
                    rot_s = ns;
                }
            }
        }
        if (has_next) M3_STAGE_SCALARS(q ^ 1);   // the other parity slot: nobody reads it now
        __syncthreads();   // this chunk's tiles, S_{c-1} and the column factors no longer read;
                           // next chunk's scalars visible
        const bool seq_end = MULTI && has_next && (c + 1) % p.nchunks == 0;   // uniform
        if (FULL && !seq_end) M3_WRITE_SST();
        if (has_next) M3_STAGE_TILES(q ^ 1);
        zero_in = MULTI && seq_end && zero_init;
        if (MULTI && seq_end) {   // after the staging, when the prefetch registers are free
            const int bs = b + c / p.nchunks;
            if (p.h_out) store_state(bs);
            init_state(bs + 1, tb + static_cast<int64_t>(c + 1) * Q);
            M3_WRITE_SST();
        }
        if (!FULL) {   // state-only mode has no output phase to hide the loads behind: a chunk further ahead
            const int cf = c + 2 < c_end ? c + 2 : c_end - 1;
            M3_FETCH(cf);
            nextpos = static_cast<int64_t>(cf) * Q;
        }
        __syncthreads();
    }
#undef M3_PREP
#undef M3_FETCH
#undef M3_FETCH_X
#undef M3_FETCH_B
#undef M3_LOAD_CF
#undef M3_STAGE_SCALARS
#undef M3_STAGE_TILES
#undef M3_WRITE_SST
#undef M3_LOAD_COLS
#undef M3_LOAD_V
#undef M3_FENCE
#undef M3_GTILE
#undef M3_OFFDIAG
#undef M3_DIAG
#undef M3_STORE_Y
#undef M3_LOAD_Z
#undef M3_INTER_SCALE

    // epilogue
    if (FULL) {
        if (last_seg && p.h_out) store_state(b + nseq - 1);
    } else {
        const size_t sidx = (static_cast<size_t>(b) * p.H + h) * (p.nseg - 1) + seg;
        float* so = p.seg_state + sidx * N * P;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int n = n0 + 16 * rt + 4 * lg + i, col = p0 + 16 * ct + l16;
                    so[n * P + col] = sacc[rt][ct][i];
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
    // One thread per (rotation pair k, column): blockIdx.y picks NT of the KP * P of them, so
    // each thread carries one pair through the segments.  The next segment's summary is
    // loaded before the current one is applied, keeping a load in flight across the chain.
    const int bh = blockIdx.x;
    const int b = bh / p.H, h = bh - b * p.H, g = h / (p.H / p.G);
    const int idx = blockIdx.y * NT + threadIdx.x;   // < KP * P: the grid's y extent is KP * P / NT
    const int k = idx / P, col = idx - k * P;
    const SeqSpan sp = seq_span(p.cu, b, p.L, p.T);
    const float c1 = (sp.len > 0 && p.bl_in && p.xl_in)
                         ? (1.f - p.lam[sp.start * p.H + h]) * p.dt[sp.start * p.H + h]
                         : 0.f;
    const float* __restrict__ seg_state = p.seg_state;
    const float* __restrict__ seg_rot = p.seg_rot;
    const float* __restrict__ seg_decay = p.seg_decay;
    const size_t sbase = static_cast<size_t>(bh) * (p.nseg - 1);
    auto summary = [&](int s, float* d, float* cn, float* sn, float* ds0, float* ds1) {
        const size_t sidx = sbase + s;
        *d = seg_decay[sidx];
        *cn = seg_rot[sidx * KP * 2 + 2 * k];
        *sn = seg_rot[sidx * KP * 2 + 2 * k + 1];
        const float* ds = seg_state + sidx * N * P;
        *ds0 = ds[(2 * k) * P + col];
        *ds1 = ds[(2 * k + 1) * P + col];
    };
    float s0 = initial_state<R>(p, b, h, g, 2 * k, col, c1);
    float s1 = initial_state<R>(p, b, h, g, 2 * k + 1, col, c1);
    float d = 0.f, cn = 1.f, sn = 0.f, ds0 = 0.f, ds1 = 0.f;
    if (p.nseg > 1) summary(0, &d, &cn, &sn, &ds0, &ds1);
    for (int s = 0; s < p.nseg; ++s) {
        float* out = s_init + ((static_cast<size_t>(bh) * p.nseg + s) * N) * P;
        out[(2 * k) * P + col] = s0;
        out[(2 * k + 1) * P + col] = s1;
        if (s == p.nseg - 1) break;
        const float dec = __expf(d), c = cn, si = sn, a0 = ds0, a1 = ds1;
        if (s + 1 < p.nseg - 1) summary(s + 1, &d, &cn, &sn, &ds0, &ds1);
        const float n0 = dec * (c * s0 - si * s1) + a0;
        const float n1 = dec * (si * s0 + c * s1) + a1;
        s0 = n0;
        s1 = n1;
    }
}

}  // namespace mf

// ------------------------------------------------------------------------------------
// host side
// ------------------------------------------------------------------------------------
bool mfma_supported(const PrefillArgs& a) {
    // per-lane offsets within one chunk of x and y are 32-bit
    const bool offsets_fit = static_cast<int64_t>(a.H) * a.R * a.P * a.Q < (int64_t{1} << 31);
    // Every launch stays under 2^32 work-items and rope_prep's grid is (chunks, G, batch);
    // larger shapes take the generic path.  The scan launches at most max(batch * H, 1023)
    // workgroups of at most 512 threads (segments are added only while batch * H < 512).
    const int64_t nchunks = (a.L + a.Q - 1) / a.Q;
    const int64_t Gt = a.fu.tgroups(a.G);
    const bool grid_fits = a.batch <= 65535 && Gt <= 65535 &&
                           nchunks * Gt * a.batch * mf::NT < (int64_t{1} << 32) &&
                           a.batch * a.H < (int64_t{1} << 23);
    return a.bf16 && a.N == mf::N && a.P == mf::P && (a.R == 1 || a.R == 2 || a.R == 4) &&
           (a.Q == 32 || a.Q == 64) && offsets_fit && grid_fits;
}

// Workgroups of the output pass that one CU holds at once: two for chunks of up to 128 rows
// (4 waves; registers, and LDS at 128 rows), one for 256 rows (LDS).  The CU count is MI355X's.
static int64_t scan_slots(const PrefillArgs& a) {
    constexpr int64_t kCUs = 256;
    return kCUs * (a.Q * a.R <= 128 ? 2 : 1);
}

// Segments per sequence: as many as fill the CUs in one round of workgroups.  Rounding
// down keeps the output pass to a single round (rounding up left a second round nearly
// empty).
static int choose_nseg(const PrefillArgs& a, int nchunks) {
    const int64_t slices = a.batch * a.H;
    int64_t nseg = scan_slots(a) / slices;
    const int64_t max_seg = nchunks / 4 > 0 ? nchunks / 4 : 1;   // at least ~4 chunks per segment
    if (nseg > max_seg) nseg = max_seg;
    if (nseg < 1) nseg = 1;
    return static_cast<int>(nseg);
}

// The state-only pass runs one workgroup per (b, h, summarised segment).  When those leave
// CUs idle (few (b, h) and few segments), each summarised segment is cut into `split`
// pieces that are summarised side by side; the segment pass then chains the pieces, and
// the output pass starts segment s from the state entering piece split * s.  Each piece
// keeps at least 4 chunks.
static int choose_state_split(const PrefillArgs& a, int nseg, int cps) {
    if (nseg < 2) return 1;
    int64_t f = scan_slots(a) / ((nseg - 1) * a.batch * a.H);
    if (f > cps / 4) f = cps / 4;
    return f < 1 ? 1 : static_cast<int>(f);
}

struct MfmaWs {
    size_t prep, sink, seg_state, seg_decay, seg_rot, s_init, total;
};

static size_t prep_bytes(const PrefillArgs& a) { return mf::PrepLayout{a.Q * a.R}.bytes(); }

static MfmaWs mfma_ws(const PrefillArgs& a, int nchunks, int nseg, int split) {
    MfmaWs w{};
    auto al = [](size_t v) { return (v + 255) & ~static_cast<size_t>(255); };
    size_t off = 0;
    w.prep = off;   // prepared operands per (b, angle group, chunk)
    off += al(static_cast<size_t>(a.batch) * a.fu.tgroups(a.G) * nchunks * prep_bytes(a));
    w.sink = off;
    off += al(64 * 64 * sizeof(uint16_t));
    const size_t bh = static_cast<size_t>(a.batch) * a.H;
    if (nseg > 1) {
        const size_t pieces = static_cast<size_t>(split) * (nseg - 1);   // summarised pieces per (b, h)
        w.seg_state = off;
        off += al(bh * pieces * mf::N * mf::P * sizeof(float));
        w.seg_decay = off;
        off += al(bh * pieces * sizeof(float));
        w.seg_rot = off;
        off += al(bh * pieces * mf::KP * 2 * sizeof(float));
        w.s_init = off;
        off += al(bh * (pieces + 1) * mf::N * mf::P * sizeof(float));
    }
    w.total = off;
    return w;
}

// Sequences per workgroup of the output pass.  A workgroup that sweeps one short sequence
// pays its whole load latency up front: nothing of the next chunk is in flight while the
// first one computes.  Equal-length batches whose sequences hold a few whole chunks each
// and whose (b, h) pairs fill at least four rounds of workgroups therefore give each
// workgroup several sequences of one head (about 16 chunks in all), swept one after another
// (plain calls only: no gate, no output norm).  Not at 128 rows per chunk: there two
// workgroups already share a CU and cover one another's loads, and the variant spills
// registers (measured 20-25% slower than one sequence per workgroup).
static bool multi_rows(int QR) { return QR != 128; }

static int choose_seqs(const PrefillArgs& a, int nchunks, int nseg) {
    if (a.cu || nseg != 1 || nchunks < 1 || nchunks > 4 || a.L % a.Q != 0 || a.fu.z || a.fu.onw ||
        !multi_rows(a.Q * a.R))
        return 1;
    int64_t s = (16 + nchunks - 1) / nchunks;
    const int64_t cap = a.batch * a.H / (4 * scan_slots(a));
    if (s > cap) s = cap;
    if (s > a.batch) s = a.batch;
    return s < 2 ? 1 : static_cast<int>(s);
}

void plan_mfma(const PrefillArgs& a, PrefillPlan* plan) {
    const int nchunks = static_cast<int>((a.L + a.Q - 1) / a.Q);
    // packed variable-length batches run each sequence in one sweep
    int nseg = (nchunks > 0 && !a.cu) ? choose_nseg(a, nchunks) : 1;
    int cps = nchunks > 0 ? (nchunks + nseg - 1) / nseg : 0;
    int split = choose_state_split(a, nseg, cps);
    if (split > 1) cps = split * ((cps + split - 1) / split);   // pieces of equal length
    if (nchunks > 0) nseg = (nchunks + cps - 1) / cps;           // no empty trailing segment
    if (nseg < 2) split = 1;
    const int seqs = choose_seqs(a, nchunks, nseg);
    if (seqs > 1) cps = seqs * nchunks;                          // one sweep over all of them
    plan->path = PrefillPath::Mfma;
    plan->nseg = nseg;
    plan->chunks_per_seg = cps;
    plan->state_split = split;
    plan->seqs = seqs;
    plan->workspace = mfma_ws(a, nchunks, nseg, split).total;
    plan->lds = 0;
}

template <int R, int Q>
static hipError_t launch_mfma_rq(const PrefillArgs& a, const PrefillPlan& plan, hipStream_t st) {
    // waves per workgroup: one per 16-row block of the chunk, at least 4; 16 blocks go two
    // to a wave (8 waves), which shares their Bt and X tile reads, and so do 8 blocks (4
    // waves, two workgroups per CU)
    constexpr int NB = Q * R / 16;
    constexpr int NW = NB > 4 ? NB / 2 : 4;
    const int nchunks = static_cast<int>((a.L + a.Q - 1) / a.Q);
    if (nchunks == 0) return hipSuccess;
    const int nseg = plan.nseg, cps = plan.chunks_per_seg, split = plan.state_split;
    const int pieces = split * (nseg - 1);   // summarised pieces per (b, h)
    if (static_cast<int64_t>(nseg > pieces ? nseg : pieces) * a.H * a.batch > 0x7fffffffLL) return hipErrorInvalidValue;
    const MfmaWs ws = mfma_ws(a, nchunks, nseg, split);
    uint8_t* base = static_cast<uint8_t*>(a.workspace);

    hipLaunchKernelGGL((mf::rope_prep<R, Q>), dim3(nchunks, a.fu.tgroups(a.G), static_cast<unsigned>(a.batch)),
                       dim3(mf::NT), 0, st, static_cast<const uint16_t*>(a.B), static_cast<const uint16_t*>(a.C),
                       a.theta, a.L, a.G, nchunks, base + ws.prep, a.cu, a.T, a.fu);
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
    p.y_sink = reinterpret_cast<uint16_t*>(base + ws.sink);
    p.h_in = a.h_in;
    p.state_bf16 = a.state_bf16 ? 1 : 0;
    p.bl_in = static_cast<const uint16_t*>(a.bl_in);
    p.xl_in = static_cast<const uint16_t*>(a.xl_in);
    p.h_out = a.h_out;
    p.L = a.L;
    p.cu = a.cu;
    p.T = a.T;
    p.At = a.fu.At;
    p.z = static_cast<const uint16_t*>(a.fu.z);
    p.onw = a.fu.onw;
    p.eps = a.fu.eps;
    p.Gt = a.fu.tgroups(a.G);
    p.H = a.H;
    p.G = a.G;
    p.nchunks = nchunks;
    p.nseg = nseg;
    p.chunks_per_seg = cps;
    p.seqs = plan.seqs;
    p.batch = static_cast<int>(a.batch);
    if (nseg > 1) {
        // state-only pass and segment pass over the pieces (split per summarised segment)
        mf::ScanParams ps = p;
        ps.nseg = pieces + 1;
        ps.chunks_per_seg = cps / split;
        ps.seg_state = reinterpret_cast<float*>(base + ws.seg_state);
        ps.seg_decay = reinterpret_cast<float*>(base + ws.seg_decay);
        ps.seg_rot = reinterpret_cast<float*>(base + ws.seg_rot);
        hipLaunchKernelGGL((mf::scan_mfma<R, Q, NW, false, false, false>),
                           dim3(static_cast<unsigned>(pieces * a.H * a.batch)), dim3(64 * NW), 0, st, ps);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        float* s_init = reinterpret_cast<float*>(base + ws.s_init);
        static_assert((mf::KP * mf::P) % mf::NT == 0, "seg_pass grid");
        hipLaunchKernelGGL((mf::seg_pass<R>), dim3(static_cast<unsigned>(a.batch * a.H), (mf::KP * mf::P) / mf::NT),
                           dim3(mf::NT), 0, st, ps,
                           s_init);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        p.s_init = s_init;
        p.sinit_stride = pieces + 1;
        p.sinit_step = split;
    }
    if constexpr (Q * R != 128) {   // multi_rows
        if (plan.seqs > 1) {   // plain calls only (choose_seqs)
            const int64_t groups = (a.batch + plan.seqs - 1) / plan.seqs;
            hipLaunchKernelGGL((mf::scan_mfma<R, Q, NW, true, false, false, true>),
                               dim3(static_cast<unsigned>(groups * a.H)), dim3(64 * NW), 0, st, p);
            return hipGetLastError();
        }
    }
    auto scan = p.onw ? (p.z ? mf::scan_mfma<R, Q, NW, true, true, true> : mf::scan_mfma<R, Q, NW, true, false, true>)
                      : (p.z ? mf::scan_mfma<R, Q, NW, true, true, false> : mf::scan_mfma<R, Q, NW, true, false, false>);
    hipLaunchKernelGGL(scan, dim3(static_cast<unsigned>(nseg * a.H * a.batch)),
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
