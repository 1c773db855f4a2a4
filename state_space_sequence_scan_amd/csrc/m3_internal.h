// m3_internal.h -- launch descriptors shared by the C-ABI host code and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace m3 {

constexpr int kMaxRankGeneric = 8;

// Lets `kernel` launch with `bytes` of dynamic LDS on the current device: raises its limit
// with hipFuncSetAttribute the first time a size above 64 KB (or above what was set before)
// is asked for on a device, and does nothing on later calls, so that launches after the
// first enqueue nothing but the kernel (a caller may capture them in a graph).  In
// m3_api.cpp.
hipError_t ensure_dynamic_lds(const void* kernel, size_t bytes);

// Fused prologue/epilogue of a Mamba-3 layer around the scan (all optional):
// per-token decay rates, RMSNorm and bias of B and C before the rotation, and the
// output gate y * silu(z).
struct Fusion {
    const float* At = nullptr;      // per-token A: (b, L, H) prefill / (b, H) decode
    const float* bnw = nullptr;     // RMSNorm weight of B (R, N)
    const float* cnw = nullptr;     // RMSNorm weight of C (R, N)
    const float* bbias = nullptr;   // bias of B (R, N)
    const float* cbias = nullptr;   // bias of C (R, N)
    const void* z = nullptr;        // gate input, io dtype, laid out as y
    float eps = 1e-6f;
    const float* onw = nullptr;     // output RMSNorm weight (H, P), applied after the gate
    int Gt = 0;                     // angle groups (theta (.., Gt, N/2)); 0: the B/C groups
    __host__ __device__ bool bc() const { return bnw || cnw || bbias || cbias; }
    __host__ __device__ int tgroups(int G) const { return Gt > 0 ? Gt : G; }
};

struct DecodeArgs {
    void* h;                 // state, fp32 or bf16 (state_bf16)
    const void* b_last;
    const void* x_last;
    const void* x_t;
    const float* dt_t;
    const float* A;
    const float* lam_t;
    const float* theta_t;
    const void* B_t;
    const void* C_t;
    const float* D;
    void* y_t;
    int batch, H, G, N, P, R;
    int has_carry;
    bool bf16;               // io dtype
    bool state_bf16;         // state dtype
    Fusion fu;
};

bool decode_supported(const DecodeArgs& a);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t st);

struct PrefillArgs {
    const void* x;
    const float* dt;
    const float* A;
    const float* lam;
    const float* theta;
    const void* B;
    const void* C;
    const float* D;
    const void* h_in;        // may be null (zero state); fp32 or bf16 (state_bf16)
    const void* bl_in;       // carry in, may be null (with xl_in)
    const void* xl_in;
    void* y;
    void* h_out;             // may be null; fp32 or bf16 (state_bf16)
    void* bl_out;            // may be null
    void* xl_out;            // may be null
    void* workspace;
    size_t workspace_bytes;
    int64_t batch, L;        // sequences; their (maximum) length
    int H, G, N, P, R, Q;
    bool bf16;               // io dtype
    bool state_bf16;         // state dtype
    const int64_t* cu;       // packed variable-length batch: sequence starts (batch + 1), device; else null
    int64_t T;               // tokens in the packed batch (batch * L without cu)
    Fusion fu;
};

// Which kernel family runs a prefill, and the workspace it needs.
enum class PrefillPath { Generic, Mfma, Serial, Unsupported };
struct PrefillPlan {
    PrefillPath path;
    int nseg;                // segments per sequence (1 = one sweep per (b, h))
    int chunks_per_seg;      // chunks of each segment (the last may be shorter)
    int state_split;         // pieces each summarised segment is cut into for the state-only pass
    int seqs;                // matrix-core path: sequences swept one after another per workgroup
    size_t workspace;        // bytes
    size_t lds;              // dynamic LDS bytes of the main kernel
    size_t carry_off;        // workspace offset of the normalised carried-in B (fused calls)
    int q_block;             // generic path: the chunk is processed in blocks of this many
                             // tokens (the caller's chunk unless it does not fit in LDS)
};
PrefillPlan plan_prefill(const PrefillArgs& a);
hipError_t launch_prefill(const PrefillArgs& a, const PrefillPlan& plan, hipStream_t st);

// Generic family (any shape whose chunk fits in LDS), in m3_prefill_generic.hip.
size_t generic_lds_bytes(const PrefillArgs& a);
hipError_t launch_prefill_generic(const PrefillArgs& a, hipStream_t st);

// Token-serial kernel for small states (N/2 a power of two, N/2 * P <= 256, no fused
// norm, bias, gate or output norm), in m3_prefill_serial.hip.
bool serial_supported(const PrefillArgs& a);
size_t serial_lds_bytes(const PrefillArgs& a);
hipError_t launch_prefill_serial(const PrefillArgs& a, hipStream_t st);

// Matrix-core family (bf16, N = 128, P = 64, R in {1, 2, 4}, Q in {32, 64}),
// in m3_prefill_mfma.hip.
bool mfma_supported(const PrefillArgs& a);
void plan_mfma(const PrefillArgs& a, PrefillPlan* plan);
hipError_t launch_prefill_mfma(const PrefillArgs& a, const PrefillPlan& plan, hipStream_t st);

// Carry-out copy (B and X of the last token), in m3_prefill_generic.hip.
hipError_t launch_carry_out(const PrefillArgs& a, hipStream_t st);
// The carried-in B through the fusion's RMSNorm and bias, into `out` (b, G, R, N) io dtype.
hipError_t launch_carry_bc(const PrefillArgs& a, void* out, hipStream_t st);

// Backward pass (m3_backward.hip): N = 128, P = 64, R in {1, 2, 4}, fp32 or bf16 io.
struct BwdShape {
    int64_t batch, L;
    int H, G, N, P, R;
};
struct BwdLayout {            // byte offsets into the workspace
    size_t ckpt, scratch, dB_part, dC_part, dtheta_part, dbl_part, dA_part, dD_part, hloc, qloc, dec, ang, bytes;
    bool per_head;            // H > G: group-shared gradients are written per head, then summed
    int parts;                // S: the sequence of each (b, h) is split into S parts (1: no split)
    int64_t seg_per_part;     // recompute segments per part (the last part may hold fewer)
    int64_t grp;              // segments per checkpoint group (1: a checkpoint after every segment)
    bool generic;             // the generic kernel (any shape within its limits): parts 1, grp 1
    int64_t ks;               // generic kernel: tokens per recompute segment
    size_t kept_bytes;        // the checkpointed states and the recompute scratch together
};
// Number of parts the backward splits each sequence into, and the segments of
// each part: chosen from the shape alone so that results depend on nothing else.
void backward_parts(const BwdShape& s, int* parts, int64_t* seg_per_part);
struct BwdArgs {
    const void* x;
    const float* dt;
    const float* A;           // per head; unused when At is given
    const float* At;          // per-token decay rate (tokens, H), or null
    const float* lam;
    const float* theta;
    const void* B;
    const void* C;
    const float* D;
    const void* h0;           // may be null; fp32 or bf16 (state_bf16)
    const void* bl;           // carried previous input, may be null (with xl)
    const void* xl;
    const void* dy;           // io dtype
    const float* dh_out;      // may be null
    float* dx;
    float* ddt;
    float* dA;                // (H), or per token (tokens, H) when At is given
    float* dlam;
    float* dtheta;
    float* dB;
    float* dC;
    float* dD;
    float* dh0;               // may be null
    float* dbl;               // may be null
    float* dxl;               // may be null
    void* workspace;
    // filled by launch_backward from the layout
    float* ckpt;              // the state after each checkpoint group of each part
    float* scratch;           // (batch*H, S, grp, N, P): the states inside the group being reversed
    float* dB_part;
    float* dC_part;
    float* dtheta_part;
    float* dbl_part;
    float* dA_part;
    float* dD_part;
    float* hloc;              // (batch*H, S, N, P): local end state of each part, then its entering state
    float* qloc;              // (batch*H, S, N, P): local adjoint at each part's start, then the entering one
    double* dec;              // (batch*H, S): sum of dt*A over each part's tokens
    float* ang;               // (batch*H, S, N/2): sum of theta over each part's tokens, mod 2 pi
    int64_t seg_per_part;
    int64_t grp;              // segments per checkpoint group
    int64_t batch, L;         // L: the length, or with cu an upper bound on every sequence's length
    const int64_t* cu;        // packed sequence starts (batch + 1, device) or null
    int64_t T;                // tokens of the packed arrays (with cu)
    int H, G, N, P, R;
    int parts;
    bool per_head;
    bool bf16;
    bool state_bf16;
};
bool backward_supported(const BwdShape& s);
// Checkpoint levels, level 0 keeping the most states (and recomputing the fewest); every
// level gives the same gradient bits.
constexpr int kBackwardLevels = 2;
BwdLayout backward_layout(const BwdShape& s, int level);
hipError_t launch_backward(BwdArgs a, const BwdLayout& l, hipStream_t st);
// After the scan kernels: sums of the per-head partial gradients of group-shared inputs,
// the zero carry gradient when there is no carry, and dA, dD over batch (and parts).
hipError_t launch_backward_sums(const BwdArgs& a, const BwdLayout& l, hipStream_t st);
// Any other shape with N even, N and P at most 256, N / 2 * P at most 4096 and rank 1..8
// (m3_backward_generic.hip): one workgroup per (b, h), token-serial.
bool backward_generic_supported(const BwdShape& s);
constexpr int kBackwardGenericLevels = 3;
BwdLayout backward_generic_layout(const BwdShape& s, int level);
hipError_t launch_backward_generic(BwdArgs a, const BwdLayout& l, hipStream_t st);

}  // namespace m3
