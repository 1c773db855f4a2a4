// m3_api.cpp -- the C ABI declared in include/m3scan.h: argument checks,
// kernel selection, workspace sizing and launches on the caller's stream.
#include "m3scan.h"

#include <hip/hip_runtime.h>

#include <map>
#include <mutex>
#include <utility>

#include "m3_internal.h"

namespace {

constexpr int32_t kVersion = 200;  // 0.2.0: output norm, angles per head, allocation-free prefill
constexpr size_t kMaxLds = 160 * 1024;

bool dims_ok(const m3_dims* d, bool prefill) {
    if (!d) return false;
    if (d->batch < 1 || d->nheads < 1 || d->ngroups < 1 || d->headdim < 1 || d->dstate < 2 ||
        d->rank < 1)
        return false;
    if (prefill && (d->seqlen < 0 || d->chunk < 1)) return false;
    if (d->dstate % 2 != 0 || d->nheads % d->ngroups != 0) return false;
    if (d->io_dtype != M3_F32 && d->io_dtype != M3_BF16) return false;
    if (d->state_dtype != M3_F32 && d->state_dtype != M3_BF16) return false;
    // Index arithmetic inside the kernels is 32-bit for per-slice sizes.
    if (d->headdim > 4096 || d->dstate > 4096 || d->rank > 64 || d->nheads > (1 << 20)) return false;
    if (prefill && d->chunk > 4096) return false;
    return true;
}

m3::PrefillArgs make_prefill_args(const m3_dims* d) {
    m3::PrefillArgs a{};
    a.batch = d->batch;
    a.L = d->seqlen;
    a.H = static_cast<int>(d->nheads);
    a.G = static_cast<int>(d->ngroups);
    a.N = static_cast<int>(d->dstate);
    a.P = static_cast<int>(d->headdim);
    a.R = static_cast<int>(d->rank);
    a.Q = static_cast<int>(d->chunk);
    a.bf16 = d->io_dtype == M3_BF16;
    a.state_bf16 = d->state_dtype == M3_BF16;
    a.cu = nullptr;
    a.T = d->batch * d->seqlen;
    return a;
}

// The fused pieces into the kernels' descriptor; false for invalid ones (a norm weight
// without a positive eps, angle groups that are not a multiple of G dividing H).
bool copy_fusion(const m3_dims* d, const m3_fusion* f, m3::Fusion* out) {
    out->At = f->A_t;
    out->bnw = f->b_norm_w;
    out->cnw = f->c_norm_w;
    out->bbias = f->b_bias;
    out->cbias = f->c_bias;
    out->z = f->z;
    out->eps = f->norm_eps;
    out->onw = f->out_norm_w;
    out->Gt = f->theta_groups;
    if ((out->bnw || out->cnw || out->onw) && !(f->norm_eps > 0.f)) return false;
    if (f->theta_groups < 0) return false;
    if (f->theta_groups > 0 && (f->theta_groups % d->ngroups != 0 || d->nheads % f->theta_groups != 0)) return false;
    return true;
}

}  // namespace

namespace m3 {

hipError_t ensure_dynamic_lds(const void* kernel, size_t bytes) {
    if (bytes <= 64 * 1024) return hipSuccess;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    static std::mutex mu;
    static std::map<std::pair<int, const void*>, size_t> raised;   // (device, kernel) -> limit set
    std::lock_guard<std::mutex> lock(mu);
    size_t& cur = raised[{dev, kernel}];
    if (bytes <= cur) return hipSuccess;
    e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(bytes));
    if (e == hipSuccess) cur = bytes;
    return e;
}


// A fused call with a B/C norm or bias reserves, after the path's own workspace, room
// for a copy of the carried-in B (batch, G, R, N) in the io dtype: it normalises it there.
static void add_carry_room(const PrefillArgs& a, PrefillPlan* p) {
    if (!a.fu.bc()) return;   // only a fused norm or bias rewrites the carried B
    const size_t al = (p->workspace + 255) & ~static_cast<size_t>(255);
    p->carry_off = al;
    p->workspace = al + static_cast<size_t>(a.batch) * a.G * a.R * a.N * (a.bf16 ? 2 : 4);
}

PrefillPlan plan_prefill(const PrefillArgs& a) {
    PrefillPlan p{};
    p.path = PrefillPath::Unsupported;
    p.nseg = 1;
    p.state_split = 1;
    if (mfma_supported(a)) {
        plan_mfma(a, &p);
        add_carry_room(a, &p);
        return p;
    }
    if (serial_supported(a)) {   // small states: the tokens one by one
        p.path = PrefillPath::Serial;
        add_carry_room(a, &p);
        return p;
    }
    if (a.R > kMaxRankGeneric) return p;
    if (a.batch * a.H >= (int64_t{1} << 22)) return p;   // 1024-thread workgroups per (b, h): under 2^32 work-items
    // The chunked form gives the same result for any block size (up to rounding): a chunk
    // whose arrays do not fit in LDS is processed as consecutive blocks of half, a quarter, ..
    // of its tokens.
    PrefillArgs ab = a;
    while (generic_lds_bytes(ab) > kMaxLds && ab.Q > 1) ab.Q = (ab.Q + 1) / 2;
    const size_t lds = generic_lds_bytes(ab);
    if (lds <= kMaxLds) {
        p.path = PrefillPath::Generic;
        p.lds = lds;
        p.q_block = ab.Q;
        add_carry_room(a, &p);
    }
    return p;
}

hipError_t launch_prefill(const PrefillArgs& a0, const PrefillPlan& plan, hipStream_t st) {
    hipError_t e = hipSuccess;
    PrefillArgs a = a0;   // the scan kernels read the normalised carry; the carry copy-out the raw one
    if (a.fu.bc() && a.bl_in && a.xl_in) {
        void* buf = static_cast<uint8_t*>(a.workspace) + plan.carry_off;
        if ((e = launch_carry_bc(a0, buf, st)) != hipSuccess) return e;
        a.bl_in = buf;
    }
    if (plan.path == PrefillPath::Generic) {
        PrefillArgs ab = a;
        ab.Q = plan.q_block;
        e = launch_prefill_generic(ab, st);
    } else if (plan.path == PrefillPath::Serial) {
        e = launch_prefill_serial(a, st);
    } else if (plan.path == PrefillPath::Mfma) {
        if (a.L == 0) {
            e = launch_prefill_generic(a, st);   // no chunks: passes the state through
        } else {
            e = launch_prefill_mfma(a, plan, st);
        }
    } else {
        return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
    if (a0.bl_out || a0.xl_out) e = launch_carry_out(a0, st);
    return e;
}

}  // namespace m3

extern "C" {

const char* m3_status_string(m3_status s) {
    switch (s) {
        case M3_OK: return "ok";
        case M3_ERR_INVALID_ARG: return "invalid argument";
        case M3_ERR_UNSUPPORTED: return "unsupported shape or dtype";
        case M3_ERR_WORKSPACE: return "workspace too small";
        case M3_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

int32_t m3_version(void) { return kVersion; }

m3_status m3_prefill_workspace_size(const m3_dims* dims, size_t* bytes) {
    if (!bytes || !dims_ok(dims, true)) return M3_ERR_INVALID_ARG;
    const m3::PrefillArgs a = make_prefill_args(dims);
    const m3::PrefillPlan plan = m3::plan_prefill(a);
    if (plan.path == m3::PrefillPath::Unsupported) return M3_ERR_UNSUPPORTED;
    *bytes = plan.workspace;
    return M3_OK;
}

m3_status m3_prefill_sequences_per_workgroup(const m3_dims* dims, int32_t* seqs) {
    if (!seqs || !dims_ok(dims, true)) return M3_ERR_INVALID_ARG;
    const m3::PrefillArgs a = make_prefill_args(dims);
    const m3::PrefillPlan plan = m3::plan_prefill(a);
    if (plan.path == m3::PrefillPath::Unsupported) return M3_ERR_UNSUPPORTED;
    *seqs = (plan.path == m3::PrefillPath::Mfma && plan.seqs > 1) ? plan.seqs : 1;
    return M3_OK;
}

m3_status m3_prefill_fused_workspace_size(const m3_dims* dims, const m3_fusion* fusion, size_t* bytes) {
    if (!bytes || !fusion || !dims_ok(dims, true)) return M3_ERR_INVALID_ARG;
    m3::PrefillArgs a = make_prefill_args(dims);
    if (!copy_fusion(dims, fusion, &a.fu)) return M3_ERR_INVALID_ARG;
    const m3::PrefillPlan plan = m3::plan_prefill(a);
    if (plan.path == m3::PrefillPath::Unsupported) return M3_ERR_UNSUPPORTED;
    *bytes = plan.workspace;
    return M3_OK;
}

}  // extern "C"

namespace {

m3_status prefill_common(const m3_dims* dims, const int64_t* cu, int64_t total_tokens, const void* x,
                         const float* dt, const float* A, const float* lambda, const float* theta,
                         const void* B, const void* C, const float* D, const m3_fusion* fu,
                         const m3_state* state_in, m3_state* state_out, void* y, void* workspace,
                         size_t workspace_bytes, void* stream) {
    if (!dims_ok(dims, true)) return M3_ERR_INVALID_ARG;
    if (!A || !D) return M3_ERR_INVALID_ARG;
    const int64_t tokens = cu ? total_tokens : dims->batch * dims->seqlen;
    if (tokens > 0 && (!x || !dt || !lambda || !theta || !B || !C || !y)) return M3_ERR_INVALID_ARG;
    if (state_in) {
        if (!state_in->h) return M3_ERR_INVALID_ARG;
        if ((state_in->b_last == nullptr) != (state_in->x_last == nullptr)) return M3_ERR_INVALID_ARG;
    }
    m3::PrefillArgs a = make_prefill_args(dims);
    if (cu) {
        a.cu = cu;
        a.T = total_tokens;
    }
    a.x = x;
    a.dt = dt;
    a.A = A;
    a.lam = lambda;
    a.theta = theta;
    a.B = B;
    a.C = C;
    a.D = D;
    a.y = y;
    if (state_in) {
        a.h_in = state_in->h;
        a.bl_in = state_in->b_last;
        a.xl_in = state_in->x_last;
    }
    if (state_out) {
        a.h_out = state_out->h;
        a.bl_out = state_out->b_last;
        a.xl_out = state_out->x_last;
    }
    a.workspace = workspace;
    a.workspace_bytes = workspace_bytes;
    if (fu && !copy_fusion(dims, fu, &a.fu)) return M3_ERR_INVALID_ARG;
    const m3::PrefillPlan plan = m3::plan_prefill(a);
    if (plan.path == m3::PrefillPath::Unsupported) return M3_ERR_UNSUPPORTED;
    if (plan.workspace > 0 && (!workspace || workspace_bytes < plan.workspace)) return M3_ERR_WORKSPACE;
    const hipError_t e = m3::launch_prefill(a, plan, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? M3_OK : M3_ERR_HIP;
}

}  // namespace

extern "C" {

m3_status m3_prefill_chunked(const m3_dims* dims, const void* x, const float* dt,
                             const float* A, const float* lambda, const float* theta,
                             const void* B, const void* C, const float* D,
                             const m3_state* state_in, m3_state* state_out, void* y,
                             void* workspace, size_t workspace_bytes, void* stream) {
    return prefill_common(dims, nullptr, 0, x, dt, A, lambda, theta, B, C, D, nullptr, state_in, state_out,
                          y, workspace, workspace_bytes, stream);
}

m3_status m3_prefill_fused(const m3_dims* dims, const void* x, const float* dt, const float* A,
                           const float* lambda, const float* theta, const void* B, const void* C,
                           const float* D, const m3_fusion* fusion, const m3_state* state_in,
                           m3_state* state_out, void* y, void* workspace, size_t workspace_bytes,
                           void* stream) {
    if (!fusion) return M3_ERR_INVALID_ARG;
    return prefill_common(dims, nullptr, 0, x, dt, A, lambda, theta, B, C, D, fusion, state_in, state_out,
                          y, workspace, workspace_bytes, stream);
}

m3_status m3_prefill_varlen(const m3_dims* dims, const int64_t* cu_seqlens, int64_t total_tokens,
                            const void* x, const float* dt, const float* A, const float* lambda,
                            const float* theta, const void* B, const void* C, const float* D,
                            const m3_state* state_in, m3_state* state_out, void* y, void* workspace,
                            size_t workspace_bytes, void* stream) {
    if (!cu_seqlens || total_tokens < 0) return M3_ERR_INVALID_ARG;
    return prefill_common(dims, cu_seqlens, total_tokens, x, dt, A, lambda, theta, B, C, D, nullptr,
                          state_in, state_out, y, workspace, workspace_bytes, stream);
}

m3_status m3_prefill_varlen_fused(const m3_dims* dims, const int64_t* cu_seqlens, int64_t total_tokens,
                                  const void* x, const float* dt, const float* A, const float* lambda,
                                  const float* theta, const void* B, const void* C, const float* D,
                                  const m3_fusion* fusion, const m3_state* state_in, m3_state* state_out,
                                  void* y, void* workspace, size_t workspace_bytes, void* stream) {
    if (!cu_seqlens || total_tokens < 0 || !fusion) return M3_ERR_INVALID_ARG;
    return prefill_common(dims, cu_seqlens, total_tokens, x, dt, A, lambda, theta, B, C, D, fusion,
                          state_in, state_out, y, workspace, workspace_bytes, stream);
}

}  // extern "C"

// Workspace of m3_prefill_chunked_noalloc: one static array per GPU (the runtime gives
// every device its own copy of a __device__ variable).  Host code never uses the
// array's name as an address (on the host it names a host-side stand-in); it asks
// the runtime for each device's address once, with that device current, and keeps it.
namespace {

constexpr int kMaxDevices = 64;
__device__ __align__(256) unsigned char scratch[M3_NOALLOC_SCRATCH_BYTES];
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

m3_status scratch_of_current_device(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return M3_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return M3_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return M3_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return M3_OK;
}

}  // namespace

extern "C" {

m3_status m3_prefill_chunked_noalloc(const m3_dims* dims, const void* x, const float* dt,
                                     const float* A, const float* lambda, const float* theta,
                                     const void* B, const void* C, const float* D,
                                     const m3_state* state_in, m3_state* state_out, void* y,
                                     void* stream) {
    // the size check comes first: a shape beyond the array is refused before any HIP call
    size_t need = 0;
    const m3_status st = m3_prefill_workspace_size(dims, &need);
    if (st != M3_OK) return st;
    if (need > M3_NOALLOC_SCRATCH_BYTES) return M3_ERR_WORKSPACE;
    void* ws = nullptr;
    const m3_status sc = scratch_of_current_device(&ws);
    if (sc != M3_OK) return sc;
    return prefill_common(dims, nullptr, 0, x, dt, A, lambda, theta, B, C, D, nullptr, state_in, state_out,
                          y, ws, M3_NOALLOC_SCRATCH_BYTES, stream);
}

}  // extern "C"

namespace {

m3_status decode_common(const m3_dims* dims, void* h, const void* b_last, const void* x_last,
                        const void* x_t, const float* dt_t, const float* A, const float* lambda_t,
                        const float* theta_t, const void* B_t, const void* C_t, const float* D,
                        const m3_fusion* fu, void* y_t, void* stream) {
    if (!dims_ok(dims, false)) return M3_ERR_INVALID_ARG;
    if (!h || !x_t || !dt_t || !A || !lambda_t || !theta_t || !B_t || !C_t || !D || !y_t)
        return M3_ERR_INVALID_ARG;
    if ((b_last == nullptr) != (x_last == nullptr)) return M3_ERR_INVALID_ARG;
    m3::DecodeArgs a{};
    a.h = h;
    a.b_last = b_last;
    a.x_last = x_last;
    a.x_t = x_t;
    a.dt_t = dt_t;
    a.A = A;
    a.lam_t = lambda_t;
    a.theta_t = theta_t;
    a.B_t = B_t;
    a.C_t = C_t;
    a.D = D;
    a.y_t = y_t;
    a.batch = static_cast<int>(dims->batch);
    a.H = static_cast<int>(dims->nheads);
    a.G = static_cast<int>(dims->ngroups);
    a.N = static_cast<int>(dims->dstate);
    a.P = static_cast<int>(dims->headdim);
    a.R = static_cast<int>(dims->rank);
    a.has_carry = b_last != nullptr;
    a.bf16 = dims->io_dtype == M3_BF16;
    a.state_bf16 = dims->state_dtype == M3_BF16;
    if (fu && !copy_fusion(dims, fu, &a.fu)) return M3_ERR_INVALID_ARG;
    // one workgroup of at most 256 threads per (b, h): under 2^32 work-items per launch
    if (dims->batch * dims->nheads >= (int64_t{1} << 24)) return M3_ERR_UNSUPPORTED;
    if (!m3::decode_supported(a)) return M3_ERR_UNSUPPORTED;
    const hipError_t e = m3::launch_decode(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? M3_OK : M3_ERR_HIP;
}

}  // namespace

extern "C" {

m3_status m3_decode_step(const m3_dims* dims, void* h, const void* b_last, const void* x_last,
                         const void* x_t, const float* dt_t, const float* A,
                         const float* lambda_t, const float* theta_t, const void* B_t,
                         const void* C_t, const float* D, void* y_t, void* stream) {
    return decode_common(dims, h, b_last, x_last, x_t, dt_t, A, lambda_t, theta_t, B_t, C_t, D, nullptr, y_t,
                         stream);
}

m3_status m3_decode_step_fused(const m3_dims* dims, void* h, const void* b_last, const void* x_last,
                               const void* x_t, const float* dt_t, const float* A, const float* lambda_t,
                               const float* theta_t, const void* B_t, const void* C_t, const float* D,
                               const m3_fusion* fusion, void* y_t, void* stream) {
    if (!fusion) return M3_ERR_INVALID_ARG;
    return decode_common(dims, h, b_last, x_last, x_t, dt_t, A, lambda_t, theta_t, B_t, C_t, D, fusion, y_t,
                         stream);
}

}  // extern "C"

namespace {

m3::BwdShape bwd_shape(const m3_dims* d) {
    return m3::BwdShape{d->batch, d->seqlen, static_cast<int>(d->nheads), static_cast<int>(d->ngroups),
                        static_cast<int>(d->dstate), static_cast<int>(d->headdim), static_cast<int>(d->rank)};
}

// The fast kernel for its shape, else the generic one within its limits.
bool bwd_any_supported(const m3::BwdShape& s) {
    return m3::backward_supported(s) || m3::backward_generic_supported(s);
}
int bwd_levels(const m3::BwdShape& s) {
    return m3::backward_supported(s) ? m3::kBackwardLevels : m3::kBackwardGenericLevels;
}
m3::BwdLayout bwd_level(const m3::BwdShape& s, int level) {
    return m3::backward_supported(s) ? m3::backward_layout(s, level) : m3::backward_generic_layout(s, level);
}

// The layout a checkpoint budget asks for: the first level whose kept states fit it, else
// the level with the smallest workspace.
m3::BwdLayout bwd_layout_for_budget(const m3::BwdShape& s, size_t budget) {
    m3::BwdLayout best = bwd_level(s, 0);
    for (int lv = 0; lv < bwd_levels(s); ++lv) {
        const m3::BwdLayout l = bwd_level(s, lv);
        if (l.kept_bytes <= budget) return l;
        if (l.bytes < best.bytes) best = l;
    }
    return best;
}

// The layout a backward call runs with: the first level (the fewest recomputed states)
// whose workspace fits the one passed.  False when none does.
bool bwd_layout_for_workspace(const m3::BwdShape& s, size_t workspace_bytes, m3::BwdLayout* out) {
    for (int lv = 0; lv < bwd_levels(s); ++lv) {
        const m3::BwdLayout l = bwd_level(s, lv);
        if (l.bytes <= workspace_bytes) {
            *out = l;
            return true;
        }
    }
    return false;
}

constexpr size_t kDefaultCheckpointBudget = size_t{4} << 30;

}  // namespace

extern "C" {

m3_status m3_backward_workspace_size_budget(const m3_dims* dims, size_t checkpoint_bytes, size_t* bytes) {
    if (!bytes || !dims_ok(dims, true)) return M3_ERR_INVALID_ARG;
    const m3::BwdShape s = bwd_shape(dims);
    if (!bwd_any_supported(s)) return M3_ERR_UNSUPPORTED;
    *bytes = bwd_layout_for_budget(s, checkpoint_bytes).bytes;
    return M3_OK;
}

m3_status m3_backward_workspace_size(const m3_dims* dims, size_t* bytes) {
    return m3_backward_workspace_size_budget(dims, kDefaultCheckpointBudget, bytes);
}

m3_status m3_backward_parts(const m3_dims* dims, int32_t* parts, int64_t* tokens_per_part) {
    if (!parts || !tokens_per_part || !dims_ok(dims, true)) return M3_ERR_INVALID_ARG;
    const m3::BwdShape s = bwd_shape(dims);
    if (!bwd_any_supported(s)) return M3_ERR_UNSUPPORTED;
    int p = 1;
    int64_t spp = 0;
    if (m3::backward_supported(s)) m3::backward_parts(s, &p, &spp);   // the generic kernel never splits
    *parts = p;
    *tokens_per_part = p > 1 ? spp * 3 : s.L;
    return M3_OK;
}

}  // extern "C"

namespace {

m3_status backward_common(const m3_dims* dims, const int64_t* cu, int64_t total_tokens, const void* x,
                          const float* dt, const float* A, const float* At, const float* lambda, const float* theta,
                          const void* B, const void* C, const float* D, const m3_state* state_in,
                          const void* dy, const float* dh_out, const m3_grads* grads, void* workspace,
                          size_t workspace_bytes, void* stream) {
    if (!dims_ok(dims, true) || !grads) return M3_ERR_INVALID_ARG;
    if (!(A || At) || !D || !grads->dA || !grads->dD) return M3_ERR_INVALID_ARG;
    const bool any_tokens = (cu ? total_tokens : dims->batch * dims->seqlen) > 0;
    if (any_tokens && (!x || !dt || !lambda || !theta || !B || !C || !dy || !grads->dx || !grads->ddt ||
                       !grads->dlambda || !grads->dtheta || !grads->dB || !grads->dC))
        return M3_ERR_INVALID_ARG;
    if (state_in && !state_in->h) return M3_ERR_INVALID_ARG;
    const m3::BwdShape s = bwd_shape(dims);
    if (!bwd_any_supported(s)) return M3_ERR_UNSUPPORTED;
    // one workgroup of at most 512 threads per (b, h, part): under 2^32 work-items per launch
    // (the split into parts is the same at every level)
    if (s.batch * s.H * bwd_level(s, 0).parts >= (int64_t{1} << 23)) return M3_ERR_UNSUPPORTED;
    m3::BwdLayout lay{};
    if (!bwd_layout_for_workspace(s, workspace ? workspace_bytes : 0, &lay)) return M3_ERR_WORKSPACE;
    m3::BwdArgs a{};
    a.x = x;
    a.dt = dt;
    a.A = At ? nullptr : A;
    a.At = At;
    a.lam = lambda;
    a.theta = theta;
    a.B = B;
    a.C = C;
    a.D = D;
    a.h0 = state_in ? state_in->h : nullptr;
    a.bl = (state_in && state_in->b_last && state_in->x_last) ? state_in->b_last : nullptr;
    a.xl = (state_in && state_in->b_last && state_in->x_last) ? state_in->x_last : nullptr;
    a.dy = dy;
    a.dh_out = dh_out;
    a.dx = grads->dx;
    a.ddt = grads->ddt;
    a.dA = grads->dA;
    a.dlam = grads->dlambda;
    a.dtheta = grads->dtheta;
    a.dB = grads->dB;
    a.dC = grads->dC;
    a.dD = grads->dD;
    a.dh0 = grads->dh0;
    a.dbl = grads->db_last;
    a.dxl = grads->dx_last;
    a.workspace = workspace;
    a.batch = s.batch;
    a.L = s.L;
    a.H = s.H;
    a.G = s.G;
    a.N = s.N;
    a.P = s.P;
    a.R = s.R;
    a.bf16 = dims->io_dtype == M3_BF16;
    a.state_bf16 = dims->state_dtype == M3_BF16;
    a.cu = cu;
    a.T = cu ? total_tokens : s.batch * s.L;
    const hipError_t e = lay.generic ? m3::launch_backward_generic(a, lay, static_cast<hipStream_t>(stream))
                                     : m3::launch_backward(a, lay, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? M3_OK : M3_ERR_HIP;
}

}  // namespace

extern "C" {

m3_status m3_backward(const m3_dims* dims, const void* x, const float* dt, const float* A,
                      const float* lambda, const float* theta, const void* B, const void* C,
                      const float* D, const m3_state* state_in, const void* dy,
                      const float* dh_out, const m3_grads* grads, void* workspace,
                      size_t workspace_bytes, void* stream) {
    return backward_common(dims, nullptr, 0, x, dt, A, nullptr, lambda, theta, B, C, D, state_in, dy, dh_out,
                           grads, workspace, workspace_bytes, stream);
}

m3_status m3_backward_varlen(const m3_dims* dims, const int64_t* cu_seqlens, int64_t total_tokens,
                             const void* x, const float* dt, const float* A, const float* lambda,
                             const float* theta, const void* B, const void* C, const float* D,
                             const m3_state* state_in, const void* dy, const float* dh_out,
                             const m3_grads* grads, void* workspace, size_t workspace_bytes, void* stream) {
    if (!cu_seqlens || total_tokens < 0 || !dims) return M3_ERR_INVALID_ARG;
    // the workspace holds per-token partial gradients for batch * seqlen tokens
    if (dims->batch > 0 && dims->seqlen >= 0 && total_tokens > dims->batch * dims->seqlen) return M3_ERR_INVALID_ARG;
    return backward_common(dims, cu_seqlens, total_tokens, x, dt, A, nullptr, lambda, theta, B, C, D, state_in,
                           dy, dh_out, grads, workspace, workspace_bytes, stream);
}

m3_status m3_backward_per_token_A(const m3_dims* dims, const int64_t* cu_seqlens, int64_t total_tokens,
                                  const void* x, const float* dt, const float* A_t, const float* lambda,
                                  const float* theta, const void* B, const void* C, const float* D,
                                  const m3_state* state_in, const void* dy, const float* dh_out,
                                  const m3_grads* grads, void* workspace, size_t workspace_bytes,
                                  void* stream) {
    if (!dims || !A_t) return M3_ERR_INVALID_ARG;
    if (cu_seqlens) {
        if (total_tokens < 0) return M3_ERR_INVALID_ARG;
        if (dims->batch > 0 && dims->seqlen >= 0 && total_tokens > dims->batch * dims->seqlen)
            return M3_ERR_INVALID_ARG;
    }
    return backward_common(dims, cu_seqlens, cu_seqlens ? total_tokens : 0, x, dt, nullptr, A_t, lambda, theta, B,
                           C, D, state_in, dy, dh_out, grads, workspace, workspace_bytes, stream);
}

}  // extern "C"
