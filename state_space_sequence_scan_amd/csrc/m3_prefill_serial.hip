// m3_prefill_serial.hip -- token-serial prefill of the Mamba-3 scan for small states
// (gfx950, fp32 arithmetic, fp32 or bf16 io).
//
// The recurrence taken one token at a time (Mamba-3 paper note: the
// exponential-trapezoidal update of "Solution 1", the pair rotation of "Solution 2",
// the rank-R input and read-out of "Solution 3"; the output equation of IBM's "What is
// a Mamba model?"):
//   h_t = alpha_t M_t (h_{t-1} + (1 - lambda_t) dt_t U_{t-1}) + lambda_t dt_t U_t
//   y_t = C_t^T h_t + D X_t,        U_t = B_t X_t,  alpha_t = exp(dt_t A)
// (beta_t = (1 - lambda_t) dt_t alpha_t multiplies M_t U_{t-1}, as in the chunked
// kernels and the decode step).
//
// For a state of at most 256 (rotation pair, column) elements the chunked form spends
// most of a chunk in barriers and prefix scans over few elements; walking the tokens
// one by one has a dependent chain of three fused multiply-adds per token and element.
// One workgroup per (b, h) with one thread per pair k and column p (k fastest).  The
// operands of TB consecutive tokens are staged in LDS as fp32, alpha folded into the
// cos/sin table; the loads of the next block are issued before the current block is
// walked and stored to the other LDS buffer after it.  The read-out's sum over the
// state rows stays off the token chain: each thread leaves its two rows' share of
// C_t^T h_t in LDS, and after the block the threads sum those shares over the pairs
// for every (token, rank, column) at once and store y.
#include "m3_common.h"
#include "m3_internal.h"

namespace m3 {
namespace sr {

// Per-thread staging registers for one block: x, B and C elements, and (token, pair)
// entries of the angle table.  The host picks TB so that every thread's share fits.
constexpr int kEX = 8, kEB = 8, kEK = 4;
constexpr int kMaxThreads = 256;
constexpr int kMaxTB = 64;
constexpr int kMaxParts = 8192;   // floats of read-out shares per block: TB * R * KP * P
constexpr size_t kMaxLds = 128 * 1024;

// floor(u / d) for 0 <= u < 2^16 and d >= 1 through the float reciprocal inv = 1 / d:
// (u + 1/2) / d is at least 1/(2d) from an integer, a relative distance of at least
// 2^-17, far beyond the two roundings (each at most 2^-24) of the product.
__device__ __forceinline__ int fdiv(int u, float inv) {
    return static_cast<int>((static_cast<float>(u) + 0.5f) * inv);
}

struct Params {
    const void* x;
    const float* dt;
    const float* A;
    const float* At;
    const float* lam;
    const float* theta;
    const void* B;
    const void* C;
    const float* D;
    const void* h_in;
    const void* bl_in;
    const void* xl_in;
    void* y;
    void* h_out;
    const int64_t* cu;
    int64_t Lmax, T;
    int H, G, Gt, N, P, TB;
    int state_bf16;
};

// LDS of one block buffer, in floats: x, B, C, cos, sin, and (c1, c2) per token.
__host__ __device__ inline int block_floats(int TB, int R, int N, int P) {
    return TB * (R * P + 2 * R * N + N + 2);
}

template <typename T, int R>
__global__ __launch_bounds__(kMaxThreads) void prefill_serial(Params q) {
    extern __shared__ float smem[];
    const int N = q.N, P = q.P, KP = N / 2, TB = q.TB, H = q.H;
    const int NT = blockDim.x, tid = threadIdx.x;
    const int k = tid % KP, p = tid / KP;
    const int bh = blockIdx.x, b = bh / H, h = bh - b * H;
    const int g = h / (H / q.G), gt = h / (H / q.Gt);
    const SeqSpan sp = seq_span(q.cu, b, q.Lmax, q.T);
    const int64_t tb = sp.start, L = sp.len;
    const T* x = static_cast<const T*>(q.x);
    const T* B = static_cast<const T*>(q.B);
    const T* C = static_cast<const T*>(q.C);
    const float Ah = q.A[h], Dh = q.D[h];
    const int RP = R * P, RN = R * N, KPP = KP * P, lkp = __builtin_ctz(KP);
    const float invRP = 1.f / RP, invRN = 1.f / RN;
    const int fpb = block_floats(TB, R, N, P);
    float* parts = smem + 2 * fpb;   // [TB][R][P][KP]: read-out shares of the block

    // Block buffer layout (floats): X[TB][RP], B[TB][RN], C[TB][RN], cos[TB][KP],
    // sin[TB][KP], c1[TB], c2[TB].
    auto bufX = [&](int s) { return smem + s * fpb; };
    auto bufB = [&](int s) { return bufX(s) + TB * RP; };
    auto bufC = [&](int s) { return bufB(s) + TB * RN; };
    auto bufCs = [&](int s) { return bufC(s) + TB * RN; };
    auto bufSn = [&](int s) { return bufCs(s) + TB * KP; };
    auto bufW = [&](int s) { return bufSn(s) + TB * KP; };   // [TB][2]: c1, c2

    // Staging registers of one block: loads are unconditional (indices clamped to the
    // block's last element) so that no branch join makes the compiler wait for them.
    float rx[kEX], rb[kEB], rc[kEB], rth[kEK], rdt[kEK], ra[kEK];
    float rl1[1], rd1[1];   // lambda and dt of the thread's token (tid < nb)
    auto issue = [&](int64_t t0, int nb) {
        const int nx = nb * RP, nbn = nb * RN, nk = nb * KP;
#pragma unroll
        for (int e = 0; e < kEX; ++e) {
            const int u0 = tid + NT * e, u = u0 < nx ? u0 : nx - 1;
            const int t = fdiv(u, invRP), i = u - t * RP;
            rx[e] = io<T>::load(x + ((tb + t0 + t) * H + h) * static_cast<size_t>(RP) + i);
        }
#pragma unroll
        for (int e = 0; e < kEB; ++e) {
            const int u0 = tid + NT * e, u = u0 < nbn ? u0 : nbn - 1;
            const int t = fdiv(u, invRN), i = u - t * RN;
            const size_t o = ((tb + t0 + t) * q.G + g) * static_cast<size_t>(RN) + i;
            rb[e] = io<T>::load(B + o);
            rc[e] = io<T>::load(C + o);
        }
#pragma unroll
        for (int e = 0; e < kEK; ++e) {
            const int u0 = tid + NT * e, u = u0 < nk ? u0 : nk - 1;
            const int t = u >> lkp, kk = u & (KP - 1);
            const int64_t tok = tb + t0 + t;
            rth[e] = q.theta[(tok * q.Gt + gt) * KP + kk];
            rdt[e] = q.dt[tok * H + h];
            ra[e] = q.At ? q.At[tok * H + h] : Ah;
        }
        {
            const int t = tid < nb ? tid : nb - 1;
            const int64_t tok = tb + t0 + t;
            rd1[0] = q.dt[tok * H + h];
            rl1[0] = q.lam[tok * H + h];
        }
    };
    auto stage = [&](int s, int nb) {
        const int nx = nb * RP, nbn = nb * RN, nk = nb * KP;
        float* X = bufX(s);
        float* Bs = bufB(s);
        float* Cs = bufC(s);
        float* Co = bufCs(s);
        float* Si = bufSn(s);
        float* W = bufW(s);
#pragma unroll
        for (int e = 0; e < kEX; ++e) {
            const int u = tid + NT * e;
            if (u < nx) X[u] = rx[e];
        }
#pragma unroll
        for (int e = 0; e < kEB; ++e) {
            const int u = tid + NT * e;
            if (u < nbn) {
                Bs[u] = rb[e];
                Cs[u] = rc[e];
            }
        }
#pragma unroll
        for (int e = 0; e < kEK; ++e) {
            const int u = tid + NT * e;
            if (u < nk) {
                const float alpha = __expf(rdt[e] * ra[e]);
                float sn, cs;
                sincos_acc(rth[e], &sn, &cs);
                Co[u] = alpha * cs;
                Si[u] = alpha * sn;
            }
        }
        if (tid < nb) {
            W[2 * tid] = (1.f - rl1[0]) * rd1[0];   // c1: weight of the previous input, before the decay
            W[2 * tid + 1] = rl1[0] * rd1[0];       // c2 = gamma
        }
    };

    // Incoming state of this thread's two elements, and the previous input's U there.
    float h0 = 0.f, h1 = 0.f, up0 = 0.f, up1 = 0.f;
    const size_t so = static_cast<size_t>(bh) * N * P;
    if (p < P) {
        if (q.h_in) {
            h0 = state_load(q.h_in, so + static_cast<size_t>(2 * k) * P + p, q.state_bf16);
            h1 = state_load(q.h_in, so + static_cast<size_t>(2 * k + 1) * P + p, q.state_bf16);
        }
        if (q.bl_in && q.xl_in) {
            const T* bl = static_cast<const T*>(q.bl_in);
            const T* xl = static_cast<const T*>(q.xl_in);
            for (int r = 0; r < R; ++r) {
                const float xv = io<T>::load(xl + (static_cast<size_t>(bh) * R + r) * P + p);
                up0 += io<T>::load(bl + ((static_cast<size_t>(b) * q.G + g) * R + r) * N + 2 * k) * xv;
                up1 += io<T>::load(bl + ((static_cast<size_t>(b) * q.G + g) * R + r) * N + 2 * k + 1) * xv;
            }
        }
    }

    T* y = static_cast<T*>(q.y);
    const int64_t nblk = (L + TB - 1) / TB;
    if (nblk > 0) {
        issue(0, static_cast<int>(L < TB ? L : TB));
        stage(0, static_cast<int>(L < TB ? L : TB));
    }
    for (int64_t blk = 0; blk < nblk; ++blk) {
        const int s = static_cast<int>(blk & 1);
        const int64_t t0 = blk * TB;
        const int nb = static_cast<int>(L - t0 < TB ? L - t0 : TB);
        __syncthreads();   // block blk staged; the other buffer is free
        const bool more = blk + 1 < nblk;
        const int64_t t1 = t0 + TB;
        const int nb1 = more ? static_cast<int>(L - t1 < TB ? L - t1 : TB) : 0;
        if (more) issue(t1, nb1);

        const float* X = bufX(s);
        const float* Bs = bufB(s);
        const float* Cs = bufC(s);
        const float* Co = bufCs(s);
        const float* Si = bufSn(s);
        const float* W = bufW(s);
        if (p < P) {
#pragma unroll 2   // (4 measured slower)
            for (int i = 0; i < nb; ++i) {
                const float* xi = X + i * RP;
                const float* bi = Bs + i * RN;
                const float* ci = Cs + i * RN;
                float u0 = 0.f, u1 = 0.f;
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const float xv = xi[r * P + p];
                    u0 += bi[r * N + 2 * k] * xv;
                    u1 += bi[r * N + 2 * k + 1] * xv;
                }
                const float c1 = W[2 * i], c2 = W[2 * i + 1];
                const float cs = Co[i * KP + k], sn = Si[i * KP + k];   // alpha cos, alpha sin
                const float v0 = h0 + c1 * up0, v1 = h1 + c1 * up1;
                h0 = cs * v0 - sn * v1 + c2 * u0;
                h1 = sn * v0 + cs * v1 + c2 * u1;
                up0 = u0;
                up1 = u1;
#pragma unroll
                for (int r = 0; r < R; ++r)
                    parts[(i * R + r) * KPP + tid] = ci[r * N + 2 * k] * h0 + ci[r * N + 2 * k + 1] * h1;
            }
        }
        __syncthreads();   // every share of the block written
        // y of the block: (token, rank, column) o, its shares over the KP pairs (consecutive)
        for (int o = tid; o < nb * RP; o += NT) {
            const float* sh = parts + static_cast<size_t>(o) * KP;
            float acc = 0.f;
            for (int kk = 0; kk < KP; ++kk) acc += sh[kk];
            const int i = fdiv(o, invRP), e = o - i * RP;
            io<T>::store(y + ((tb + t0 + i) * H + h) * static_cast<size_t>(RP) + e, acc + Dh * X[o]);
        }
        if (more) stage(s ^ 1, nb1);
    }

    if (q.h_out && p < P) {
        state_store(q.h_out, so + static_cast<size_t>(2 * k) * P + p, h0, q.state_bf16);
        state_store(q.h_out, so + static_cast<size_t>(2 * k + 1) * P + p, h1, q.state_bf16);
    }
}

}  // namespace sr

// Threads per workgroup: KP * P rounded up to whole waves.
static int serial_threads(const PrefillArgs& a) {
    const int n = (a.N / 2) * a.P;
    return (n + 63) / 64 * 64;
}

static size_t serial_lds_at(const PrefillArgs& a, int tb) {
    return sizeof(float) * (2 * static_cast<size_t>(sr::block_floats(tb, a.R, a.N, a.P)) +
                            static_cast<size_t>(tb) * a.R * (a.N / 2) * a.P);
}

// Tokens per staged block: the largest power of two up to kMaxTB whose staging fits each
// thread's registers and whose two buffers and read-out shares fit 128 KiB of LDS.
static int serial_tb(const PrefillArgs& a) {
    const int nt = serial_threads(a);
    int tb = sr::kMaxTB;
    while (tb > 1 && (tb * a.R * a.P > nt * sr::kEX || tb * a.R * a.N > nt * sr::kEB ||
                      tb * (a.N / 2) > nt * sr::kEK || tb > nt ||
                      tb * a.R * (a.N / 2) * a.P > sr::kMaxParts || serial_lds_at(a, tb) > sr::kMaxLds))
        tb /= 2;
    return tb;
}

size_t serial_lds_bytes(const PrefillArgs& a) { return serial_lds_at(a, serial_tb(a)); }

bool serial_supported(const PrefillArgs& a) {
    const int KP = a.N / 2;
    const bool pow2 = KP >= 1 && KP <= 64 && (KP & (KP - 1)) == 0;
    return pow2 && KP * a.P <= sr::kMaxThreads && a.R >= 1 && a.R <= kMaxRankGeneric &&
           !a.fu.bc() && !a.fu.z && !a.fu.onw && a.batch * a.H < (int64_t{1} << 22) &&
           serial_lds_bytes(a) <= sr::kMaxLds;
}

template <typename T>
static hipError_t launch_serial_t(const PrefillArgs& a, hipStream_t st) {
    sr::Params q{};
    q.x = a.x;
    q.dt = a.dt;
    q.A = a.A;
    q.At = a.fu.At;
    q.lam = a.lam;
    q.theta = a.theta;
    q.B = a.B;
    q.C = a.C;
    q.D = a.D;
    q.h_in = a.h_in;
    q.bl_in = a.bl_in;
    q.xl_in = a.xl_in;
    q.y = a.y;
    q.h_out = a.h_out;
    q.cu = a.cu;
    q.Lmax = a.L;
    q.T = a.T;
    q.H = a.H;
    q.G = a.G;
    q.Gt = a.fu.tgroups(a.G);
    q.N = a.N;
    q.P = a.P;
    q.TB = serial_tb(a);
    q.state_bf16 = a.state_bf16 ? 1 : 0;
    void (*kernel)(sr::Params) = nullptr;
    switch (a.R) {
        case 1: kernel = sr::prefill_serial<T, 1>; break;
        case 2: kernel = sr::prefill_serial<T, 2>; break;
        case 3: kernel = sr::prefill_serial<T, 3>; break;
        case 4: kernel = sr::prefill_serial<T, 4>; break;
        case 5: kernel = sr::prefill_serial<T, 5>; break;
        case 6: kernel = sr::prefill_serial<T, 6>; break;
        case 7: kernel = sr::prefill_serial<T, 7>; break;
        case 8: kernel = sr::prefill_serial<T, 8>; break;
        default: return hipErrorInvalidValue;
    }
    const size_t shm = serial_lds_bytes(a);
    const hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void*>(kernel), shm);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>(a.batch * a.H)), dim3(serial_threads(a)), shm, st, q);
    return hipGetLastError();
}

hipError_t launch_prefill_serial(const PrefillArgs& a, hipStream_t st) {
    return a.bf16 ? launch_serial_t<bf16_t>(a, st) : launch_serial_t<float>(a, st);
}

}  // namespace m3
