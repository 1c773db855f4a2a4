// m3_prefill_generic.hip -- chunked prefill of the Mamba-3 scan in fp32 vector
// arithmetic, for any shape whose chunk fits in LDS (gfx950).
//
// The chunked form (per (b, h), chunk of Q tokens, all sums chunk-local):
//   cum_i = sum_{j<=i} dt_j A                     (decay exponent)
//   phi_i = sum_{j<=i} theta_j                    (angle per pair k)
//   Bt_i  = R(-phi_i) B_i,   Ct_i = R(-phi_i) C_i (data-dependent RoPE: the
//           cumulative rotation absorbed into B and C, Mamba-3 paper note,
//           "Solution 2: a complex state that rotates")
//   w_j   = lambda_j dt_j + (1 - lambda_{j+1}) dt_{j+1}   (gamma_j plus the beta
//           weight the next step gives the same input: the implicit width-2
//           convolution of the exponential-trapezoidal rule, "Solution 1";
//           w = gamma at the last token of the sequence)
//   Y_i   = D X_i + e^{cum_i} Ct_i^T S  +  sum_{j<=i} m_ij (Ct_i^T Bt_j) X_j
//           m_ij = e^{cum_i - cum_j} w_j (j < i),   gamma_i (j = i)
//   S    <- R(phi_end) [ e^{cum_end} S + sum_j e^{cum_end - cum_j} w_j Bt_j X_j ]
// S is the state entering the chunk in the true frame, with the beta term of
// the chunk's first token already folded in (h + (1 - lambda) dt U_prev); after
// the last chunk it is exactly h_L.  The chunks are walked in order by one
// workgroup per (b, h) (the state passing of the chunked scan, IBM "What is a
// Mamba model?", hardware-aware parallel scan).
#include "m3_common.h"
#include "m3_internal.h"

namespace m3 {

// One workgroup of kThreads threads per (b, h): four waves per SIMD, so that the LDS
// latency of one wave's loop is covered by the others.
constexpr int kThreads = 1024;

template <typename T>
__global__ __launch_bounds__(kThreads) void prefill_generic(
    const T* __restrict__ x, const float* __restrict__ dt, const float* __restrict__ A,
    const float* __restrict__ lam, const float* __restrict__ theta, const T* __restrict__ B,
    const T* __restrict__ C, const float* __restrict__ Dv, const void* __restrict__ h_in,
    const T* __restrict__ bl_in, const T* __restrict__ xl_in, T* __restrict__ y,
    void* __restrict__ h_out, int64_t Lmax, int H, int G, int N, int P, int R, int Q, int state_bf16,
    const int64_t* __restrict__ cu, int64_t Tt, Fusion fu, int resident) {
    extern __shared__ float smem[];
    const int KP = N / 2, QR = Q * R;
    float* S = smem;                       // N*P
    float* Ct = S + N * P;                 // QR*N
    float* Bt = Ct + QR * N;               // QR*N
    float* X = Bt + QR * N;                // QR*P
    float* Gm = X + QR * P;                // QR*QR
    float* phi = Gm + QR * QR;             // Q*KP
    float* cum = phi + Q * KP;             // Q
    float* wv = cum + Q;                   // Q
    float* gam = wv + Q;                   // Q
    float* sv = gam + Q;                   // Q
    float* bsc = sv + Q;                   // Q*R: RMSNorm scale of each B row of the chunk (and,
                                           // later in the chunk, the output-norm scale of each row)
    float* csc = bsc + QR;                 // Q*R: same for C
    float* Yb = csc + QR;                  // QR*P: outputs before the output norm (with it only)
    const T* zg = static_cast<const T*>(fu.z);

    const int bh = blockIdx.x;
    const int b = bh / H, h = bh - b * H;
    const int g = h / (H / G);
    const int Gt = fu.tgroups(G), gt = h / (H / Gt);   // angle group
    // this sequence: tokens tb .. tb + L - 1 of the (possibly packed) token axis
    const SeqSpan sp = seq_span(cu, b, Lmax, Tt);
    const int64_t tb = sp.start, L = sp.len;
    const int tid = threadIdx.x, NT = blockDim.x;
    const float Ah = A[h], Dh = Dv[h];

    // Resident mode (short sequences, decided by the host): every input of this (b, h)
    // sequence is copied into LDS once, in one sweep of loads, and the chunks read their
    // operands from there instead of paying a round trip to memory per chunk and phase.
    float* rX = (fu.onw ? Yb + QR * P : Yb);   // [Lmax][R*P]
    float* rB = rX + Lmax * R * P;             // [Lmax][R*N]
    float* rC = rB + Lmax * R * N;             // [Lmax][R*N]
    float* rTh = rC + Lmax * R * N;            // [Lmax][KP]
    float* rDt = rTh + Lmax * KP;              // [Lmax]
    float* rLam = rDt + Lmax;                  // [Lmax]
    float* rAt = rLam + Lmax;                  // [Lmax]
    float* rZ = rAt + Lmax;                    // [Lmax][R*P] (gate only)
    if (resident) {
        for (int64_t u = tid; u < L * R * P; u += NT) {
            const int64_t t = u / (R * P), e = u - t * (R * P);
            rX[u] = io<T>::load(x + ((tb + t) * H + h) * static_cast<size_t>(R * P) + e);
            if (zg) rZ[u] = io<T>::load(zg + ((tb + t) * H + h) * static_cast<size_t>(R * P) + e);
        }
        for (int64_t u = tid; u < L * R * N; u += NT) {
            const int64_t t = u / (R * N), e = u - t * (R * N);
            rB[u] = io<T>::load(B + ((tb + t) * G + g) * static_cast<size_t>(R * N) + e);
            rC[u] = io<T>::load(C + ((tb + t) * G + g) * static_cast<size_t>(R * N) + e);
        }
        for (int64_t u = tid; u < L * KP; u += NT) {
            const int64_t t = u / KP, k = u - t * KP;
            rTh[u] = theta[((tb + t) * Gt + gt) * KP + k];
        }
        for (int64_t t = tid; t < L; t += NT) {
            rDt[t] = dt[(tb + t) * H + h];
            rLam[t] = lam[(tb + t) * H + h];
            rAt[t] = fu.At ? fu.At[(tb + t) * H + h] : Ah;
        }
    }
    // operand reads by token t of the sequence (0-based): LDS in resident mode, else memory
    auto DT = [&](int64_t t) { return resident ? rDt[t] : dt[(tb + t) * H + h]; };
    auto LAM = [&](int64_t t) { return resident ? rLam[t] : lam[(tb + t) * H + h]; };
    auto AT = [&](int64_t t) { return resident ? rAt[t] : (fu.At ? fu.At[(tb + t) * H + h] : Ah); };
    auto TH = [&](int64_t t, int k) { return resident ? rTh[t * KP + k] : theta[((tb + t) * Gt + gt) * KP + k]; };
    auto BV = [&](int64_t t, int r, int n) {
        return resident ? rB[(t * R + r) * N + n] : io<T>::load(B + (((tb + t) * G + g) * R + r) * static_cast<size_t>(N) + n);
    };
    auto CV = [&](int64_t t, int r, int n) {
        return resident ? rC[(t * R + r) * N + n] : io<T>::load(C + (((tb + t) * G + g) * R + r) * static_cast<size_t>(N) + n);
    };
    auto XV = [&](int64_t t, int e) {   // e < R * P
        return resident ? rX[t * R * P + e] : io<T>::load(x + ((tb + t) * H + h) * static_cast<size_t>(R * P) + e);
    };
    auto ZV = [&](int64_t t, int e) {
        return resident ? rZ[t * R * P + e] : io<T>::load(zg + ((tb + t) * H + h) * static_cast<size_t>(R * P) + e);
    };

    // Incoming state: h_in plus the beta term of the first token for the carry.
    const bool carry = (bl_in != nullptr) && (xl_in != nullptr) && L > 0;
    const float c1_first = carry ? (1.f - lam[tb * H + h]) * dt[tb * H + h] : 0.f;
    for (int idx = tid; idx < N * P; idx += NT) {
        const int n = idx / P, p = idx - n * P;
        float s = h_in ? state_load(h_in, static_cast<size_t>(bh) * N * P + idx, state_bf16) : 0.f;
        if (carry) {
            float u = 0.f;
            for (int r = 0; r < R; ++r)
                u += io<T>::load(bl_in + ((static_cast<size_t>(b) * G + g) * R + r) * N + n) *
                     io<T>::load(xl_in + (static_cast<size_t>(bh) * R + r) * P + p);
            s += c1_first * u;
        }
        S[idx] = s;
    }

    const int64_t nchunks = (L + Q - 1) / Q;
    for (int64_t c = 0; c < nchunks; ++c) {
        const int64_t t0 = c * Q;
        const int nq = static_cast<int>(L - t0 < Q ? L - t0 : Q);
        __syncthreads();   // previous chunk done with every LDS array

        // Per-token scalars; the decay exponents a_t = dt_t A are prefix-summed in
        // registers across the lanes of wave 0 when the chunk fits in one wave.
        for (int i = tid; i < (Q <= 64 ? 64 : Q); i += NT) {
            float a = 0.f, gm = 0.f, w = 0.f;
            if (i < nq) {
                const int64_t t = t0 + i;
                const float dtv = DT(t), lv = LAM(t);
                a = dtv * AT(t);
                gm = lv * dtv;
                w = gm;
                if (t + 1 < L) w += (1.f - LAM(t + 1)) * DT(t + 1);
            }
            if (Q <= 64) {   // i == lane of wave 0
                for (int off = 1; off < 64; off <<= 1) {
                    const float o = __shfl_up(a, off);
                    if (i >= off) a += o;
                }
            }
            if (i < Q) {
                cum[i] = a;
                gam[i] = gm;
                wv[i] = w;
            }
        }
        // Angles into LDS.  Up to 64 tokens per chunk, each pair's chunk-local prefix sum is
        // taken right here with lane shuffles over W lanes (W the power of two >= Q: tokens
        // i of pair k on lanes k W + i); longer chunks sum serially below.
        if (Q <= 64) {
            const int W = Q <= 1 ? 1 : 1 << (32 - __clz(Q - 1));
            for (int base = 0; base < KP * W; base += NT) {   // every lane of a wave takes the shuffles
                const int u = base + tid, k = u / W, i = u - k * W;
                float v = (u < KP * W && i < nq) ? TH(t0 + i, k) : 0.f;
                for (int off = 1; off < W; off <<= 1) {
                    const float o = __shfl_up(v, off, W);
                    if (i >= off) v += o;
                }
                if (u < KP * W && i < Q) phi[i * KP + k] = v;
            }
        } else {
            for (int idx = tid; idx < Q * KP; idx += NT) {
                const int i = idx / KP, k = idx - i * KP;
                phi[idx] = (i < nq) ? TH(t0 + i, k) : 0.f;
            }
        }
        // RMSNorm scales of the chunk's B and C rows (token, rank), when normalised.
        if (fu.bnw || fu.cnw) {
            for (int row = tid; row < QR; row += NT) {
                const int i = row / R, r = row - i * R;
                float sb = 0.f, sc = 0.f;
                if (i < nq) {
                    for (int n = 0; n < N; ++n) {
                        const float bv = BV(t0 + i, r, n), cv = CV(t0 + i, r, n);
                        sb += bv * bv;
                        sc += cv * cv;
                    }
                }
                bsc[row] = rsqrtf(sb / N + fu.eps);
                csc[row] = rsqrtf(sc / N + fu.eps);
            }
        }
        __syncthreads();
        // Chunk-local angle prefix sums of longer chunks, one pair per thread, within LDS.
        if (Q > 64) {
            for (int k = tid; k < KP; k += NT) {
                float acc = 0.f;
                for (int i = 0; i < Q; ++i) {
                    acc += phi[i * KP + k];
                    phi[i * KP + k] = acc;
                }
            }
        }
        if (Q > 64 && tid == 0) {
            float acc = 0.f;
            for (int i = 0; i < Q; ++i) {
                acc += cum[i];
                cum[i] = acc;
            }
        }
        __syncthreads();
        // Rotated B, C (R(-phi_i) on pairs) and X, as fp32 in LDS.
        for (int idx = tid; idx < Q * R * KP; idx += NT) {
            const int i = idx / (R * KP), rem = idx - i * R * KP, r = rem / KP, k = rem - r * KP;
            float b0 = 0.f, b1 = 0.f, c0 = 0.f, c1 = 0.f;
            if (i < nq) {
                float sn, cs;
                sincos_acc(phi[i * KP + k], &sn, &cs);
                float bb0 = BV(t0 + i, r, 2 * k), bb1 = BV(t0 + i, r, 2 * k + 1);
                float cc0 = CV(t0 + i, r, 2 * k), cc1 = CV(t0 + i, r, 2 * k + 1);
                const int wi = r * N + 2 * k;
                if (fu.bnw) {
                    bb0 *= bsc[i * R + r] * fu.bnw[wi];
                    bb1 *= bsc[i * R + r] * fu.bnw[wi + 1];
                }
                if (fu.cnw) {
                    cc0 *= csc[i * R + r] * fu.cnw[wi];
                    cc1 *= csc[i * R + r] * fu.cnw[wi + 1];
                }
                if (fu.bbias) {
                    bb0 += fu.bbias[wi];
                    bb1 += fu.bbias[wi + 1];
                }
                if (fu.cbias) {
                    cc0 += fu.cbias[wi];
                    cc1 += fu.cbias[wi + 1];
                }
                b0 = cs * bb0 + sn * bb1;
                b1 = -sn * bb0 + cs * bb1;
                c0 = cs * cc0 + sn * cc1;
                c1 = -sn * cc0 + cs * cc1;
            }
            Bt[(i * R + r) * N + 2 * k] = b0;
            Bt[(i * R + r) * N + 2 * k + 1] = b1;
            Ct[(i * R + r) * N + 2 * k] = c0;
            Ct[(i * R + r) * N + 2 * k + 1] = c1;
        }
        for (int idx = tid; idx < QR * P; idx += NT) {
            const int i = idx / (R * P);
            X[idx] = (i < nq) ? XV(t0 + i, idx - i * R * P) : 0.f;
        }
        __syncthreads();
        const float cend = cum[Q - 1];
        for (int j = tid; j < Q; j += NT) sv[j] = __expf(cend - cum[j]) * wv[j];
        // Masked intra-chunk block m_ij (Ct_i . Bt_j).
        for (int idx = tid; idx < QR * QR; idx += NT) {
            const int ir = idx / QR, js = idx - ir * QR;
            const int i = ir / R, j = js / R;
            float v = 0.f;
            if (j <= i) {
                float dot = 0.f;
#pragma unroll 4
                for (int n = 0; n < N; ++n) dot += Ct[ir * N + n] * Bt[js * N + n];
                const float m = (j < i) ? __expf(cum[i] - cum[j]) * wv[j] : gam[i];
                v = m * dot;
            }
            Gm[idx] = v;
        }
        __syncthreads();
        // Outputs.
        for (int idx = tid; idx < QR * P; idx += NT) {
            const int ir = idx / P, p = idx - ir * P;
            const int i = ir / R;
            if (i >= nq) continue;
            float st = 0.f;
#pragma unroll 4
            for (int n = 0; n < N; ++n) st += Ct[ir * N + n] * S[n * P + p];
            float acc = __expf(cum[i]) * st;
#pragma unroll 4
            for (int js = 0; js < (i + 1) * R; ++js) acc += Gm[ir * QR + js] * X[js * P + p];
            acc += Dh * X[ir * P + p];
            const size_t yi = ((tb + t0 + i) * H + h) * static_cast<size_t>(R * P) + (ir - i * R) * P + p;
            if (zg) acc *= silu(ZV(t0 + i, (ir - i * R) * P + p));
            if (fu.onw)
                Yb[idx] = acc;   // normalised below
            else
                io<T>::store(y + yi, acc);
        }
        __syncthreads();
        if (fu.onw) {   // output RMSNorm of each row (token, rank) over its P values: a wave per row
            const int lane = tid & 63, wave = tid >> 6;
            for (int ir = wave; ir < nq * R; ir += NT / 64) {
                float ss = 0.f;
                for (int p = lane; p < P; p += 64) ss += Yb[ir * P + p] * Yb[ir * P + p];
                ss = wave_sum(ss);
                if (lane == 0) bsc[ir] = rsqrtf(ss / P + fu.eps);
            }
            __syncthreads();
            for (int idx = tid; idx < nq * R * P; idx += NT) {
                const int ir = idx / P, p = idx - ir * P;
                const int i = ir / R;
                const size_t yi = ((tb + t0 + i) * H + h) * static_cast<size_t>(R * P) + (ir - i * R) * P + p;
                io<T>::store(y + yi, Yb[idx] * bsc[ir] * fu.onw[h * P + p]);
            }
        }
        // State update, one rotation pair x column per thread.
        const float decay = __expf(cend);
        for (int idx = tid; idx < KP * P; idx += NT) {
            const int k = idx / P, p = idx - k * P;
            float s0 = decay * S[(2 * k) * P + p], s1 = decay * S[(2 * k + 1) * P + p];
#pragma unroll 4
            for (int js = 0; js < QR; ++js) {
                const float xs = sv[js / R] * X[js * P + p];
                s0 += Bt[js * N + 2 * k] * xs;
                s1 += Bt[js * N + 2 * k + 1] * xs;
            }
            float sn, cs;
            sincos_acc(phi[(Q - 1) * KP + k], &sn, &cs);
            S[(2 * k) * P + p] = cs * s0 - sn * s1;
            S[(2 * k + 1) * P + p] = sn * s0 + cs * s1;
        }
    }
    __syncthreads();
    if (h_out)
        for (int idx = tid; idx < N * P; idx += NT)
            state_store(h_out, static_cast<size_t>(bh) * N * P + idx, S[idx], state_bf16);
}

// state_out carry: B and X of the last token (or the incoming carry when L == 0).  The grid's
// y index walks the sequences (the span is found once per workgroup), its x index the
// sequence's G R N carried B values followed by its H R P carried X values, in units of U
// (16 bytes when every row and pointer is 16-byte aligned, else one element).
template <typename T, typename U>
__global__ __launch_bounds__(256) void carry_out(const T* __restrict__ x, const T* __restrict__ B,
                                                 const T* __restrict__ bl_in, const T* __restrict__ xl_in,
                                                 T* __restrict__ bl_out, T* __restrict__ xl_out, int64_t batch,
                                                 int64_t Lmax, int H, int G, int N, int P, int R,
                                                 const int64_t* __restrict__ cu, int64_t Tt) {
    constexpr int E = static_cast<int>(sizeof(U) / sizeof(T));   // elements per unit
    const int64_t nb = static_cast<int64_t>(G) * R * N, nx = static_cast<int64_t>(H) * R * P;
    const int64_t ub = nb / E, ux = nx / E;
    for (int64_t b = blockIdx.y; b < batch; b += gridDim.y) {
        const SeqSpan sp = seq_span(cu, b, Lmax, Tt);
        const bool keep = bl_in && xl_in;   // an empty sequence passes the incoming carry on
        const U* sb = reinterpret_cast<const U*>(sp.len > 0 ? B + (sp.start + sp.len - 1) * nb
                                                            : (keep ? bl_in + b * nb : nullptr));
        const U* sx = reinterpret_cast<const U*>(sp.len > 0 ? x + (sp.start + sp.len - 1) * nx
                                                            : (keep ? xl_in + b * nx : nullptr));
        U* db = reinterpret_cast<U*>(bl_out ? bl_out + b * nb : nullptr);
        U* dx = reinterpret_cast<U*>(xl_out ? xl_out + b * nx : nullptr);
        for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < ub + ux; i += static_cast<int64_t>(gridDim.x) * 256) {
            if (i < ub) {
                if (db) db[i] = sb ? sb[i] : U{};
            } else if (dx) {
                dx[i - ub] = sx ? sx[i - ub] : U{};
            }
        }
    }
}

// The carried previous B through the same RMSNorm and bias as every B (one wave per
// row (b, g, r) of N values), into a copy the scan kernels read instead.
template <typename T>
__global__ __launch_bounds__(64) void carry_bc(const T* __restrict__ bl_in, T* __restrict__ out, int N, int R,
                                               Fusion fu) {
    const int64_t row = blockIdx.x;
    const int r = static_cast<int>(row % R);
    const int lane = threadIdx.x;
    const T* src = bl_in + row * N;
    float ss = 0.f;
    for (int n = lane; n < N; n += 64) {
        const float v = io<T>::load(src + n);
        ss += v * v;
    }
    const float sc = fu.bnw ? rsqrtf(wave_sum(ss) / N + fu.eps) : 1.f;
    for (int n = lane; n < N; n += 64) {
        float v = io<T>::load(src + n);
        if (fu.bnw) v *= sc * fu.bnw[r * N + n];
        if (fu.bbias) v += fu.bbias[r * N + n];
        io<T>::store(out + row * N + n, v);
    }
}

hipError_t launch_carry_bc(const PrefillArgs& a, void* out, hipStream_t st) {
    const unsigned rows = static_cast<unsigned>(a.batch * a.G * a.R);
    if (a.bf16)
        hipLaunchKernelGGL(carry_bc<bf16_t>, dim3(rows), dim3(64), 0, st, static_cast<const bf16_t*>(a.bl_in),
                           static_cast<bf16_t*>(out), a.N, a.R, a.fu);
    else
        hipLaunchKernelGGL(carry_bc<float>, dim3(rows), dim3(64), 0, st, static_cast<const float*>(a.bl_in),
                           static_cast<float*>(out), a.N, a.R, a.fu);
    return hipGetLastError();
}

size_t generic_lds_bytes(const PrefillArgs& a) {
    const size_t QR = static_cast<size_t>(a.Q) * a.R;
    return sizeof(float) * (static_cast<size_t>(a.N) * a.P + 2 * QR * a.N + QR * a.P + QR * QR +
                            static_cast<size_t>(a.Q) * (a.N / 2) + 4 * static_cast<size_t>(a.Q) + 2 * QR +
                            (a.fu.onw ? QR * a.P : 0));
}

// LDS of one whole sequence's inputs (resident mode): x (and the gate input), B, C, the
// angles, dt, lambda and the decay rate of every token, fp32.
static size_t resident_lds_bytes(const PrefillArgs& a) {
    const size_t per_token = static_cast<size_t>(a.R) * a.P * (a.fu.z ? 2 : 1) + 2 * static_cast<size_t>(a.R) * a.N +
                             a.N / 2 + 3;
    return sizeof(float) * per_token * static_cast<size_t>(a.L);
}

template <typename T>
static hipError_t launch_generic_t(const PrefillArgs& a, hipStream_t st) {
    // resident mode when the sequence's inputs fit in LDS beside the chunk arrays
    const bool resident = generic_lds_bytes(a) + resident_lds_bytes(a) <= 160 * 1024;
    const size_t shm = generic_lds_bytes(a) + (resident ? resident_lds_bytes(a) : 0);
    const hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(&prefill_generic<T>), shm);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(prefill_generic<T>, dim3(static_cast<unsigned>(a.batch * a.H)), dim3(kThreads), shm,
                       st, static_cast<const T*>(a.x), a.dt, a.A, a.lam, a.theta,
                       static_cast<const T*>(a.B), static_cast<const T*>(a.C), a.D, a.h_in,
                       static_cast<const T*>(a.bl_in), static_cast<const T*>(a.xl_in),
                       static_cast<T*>(a.y), a.h_out, a.L, a.H, a.G, a.N, a.P, a.R, a.Q,
                       a.state_bf16 ? 1 : 0, a.cu, a.T, a.fu, resident ? 1 : 0);
    return hipGetLastError();
}

hipError_t launch_prefill_generic(const PrefillArgs& a, hipStream_t st) {
    return a.bf16 ? launch_generic_t<bf16_t>(a, st) : launch_generic_t<float>(a, st);
}

template <typename T>
static hipError_t launch_carry_t(const PrefillArgs& a, hipStream_t st) {
    const int64_t nb = static_cast<int64_t>(a.G) * a.R * a.N, nx = static_cast<int64_t>(a.H) * a.R * a.P;
    auto al16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
    const bool vec = (nb * sizeof(T)) % 16 == 0 && (nx * sizeof(T)) % 16 == 0 && al16(a.x) && al16(a.B) &&
                     al16(a.bl_in) && al16(a.xl_in) && al16(a.bl_out) && al16(a.xl_out);
    const int64_t units = vec ? (nb + nx) * static_cast<int64_t>(sizeof(T)) / 16 : nb + nx;
    int64_t bx = (units + 255) / 256, by = a.batch;
    if (bx > 64) bx = 64;
    if (by > 65535) by = 65535;
    if (bx < 1) bx = 1;
    if (by < 1) by = 1;
    auto kern = vec ? carry_out<T, uint4> : carry_out<T, T>;
    hipLaunchKernelGGL(kern, dim3(static_cast<unsigned>(bx), static_cast<unsigned>(by)), dim3(256), 0, st,
                       static_cast<const T*>(a.x), static_cast<const T*>(a.B),
                       static_cast<const T*>(a.bl_in), static_cast<const T*>(a.xl_in),
                       static_cast<T*>(a.bl_out), static_cast<T*>(a.xl_out), a.batch, a.L, a.H,
                       a.G, a.N, a.P, a.R, a.cu, a.T);
    return hipGetLastError();
}

hipError_t launch_carry_out(const PrefillArgs& a, hipStream_t st) {
    return a.bf16 ? launch_carry_t<bf16_t>(a, st) : launch_carry_t<float>(a, st);
}

}  // namespace m3
