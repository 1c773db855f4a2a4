/*
 * m3scan.h -- C ABI of the Mamba-3 selective SSM scan for MI355X (gfx950).
 *
 * The operation (per batch b, head h with group g = h / (H/G), token t):
 *
 *   U_t     = B_t X_t                                  B_t: N x R, X_t: R x P
 *   h_t     = alpha_t M_t h_{t-1} + beta_t M_t U_{t-1} + gamma_t U_t
 *   Y_t     = C_t^T h_t + D_h X_t                       R x P outputs
 *   alpha_t = exp(dt_t A_h),  beta_t = (1 - lambda_t) dt_t alpha_t,
 *   gamma_t = lambda_t dt_t,  M_t = 2x2 rotations by theta_{t,k} on state rows (2k, 2k+1)
 *
 * Sources: the exponential-trapezoidal recurrence and its alpha/beta/gamma are
 * the "Mamba-3 paper note" (docsaid.org), section "Solution 1: a more expressive
 * discretisation"; the rotation (complex state == real state of twice the size
 * with a block-diagonal of 2x2 rotations; absorbed into B and C it is a
 * data-dependent RoPE) is section "Solution 2: a complex state that rotates";
 * the rank-R MIMO update with R read-outs is section "Solution 3: MIMO"; the
 * output equation y = C h + D x is IBM's "What is a Mamba model?" (state and
 * output equations).  The chunked prefill is the hardware-aware parallel scan
 * (same IBM page, selective scan section): chunks of `chunk` tokens computed in
 * parallel, states passed between them.
 *
 * Conventions fixed by this library where the pages leave a choice open:
 *   - rotation pairs are adjacent state rows (2k, 2k+1), counter-clockwise;
 *     pair k is (real, imaginary) of complex mode k;
 *   - the rotation multiplies the beta term as well (beta carries exp(dt A)
 *     of the complex A);
 *   - theta is the per-step angle already scaled by the caller;
 *   - B, C and theta are shared by the H/G heads of a group;
 *   - the previous input (B_0, X_0) at the start of a scan is zero unless a
 *     state is passed in.
 *
 * Layouts: contiguous, row-major, last index fastest.
 *   x, y   (batch, L, H, R, P)   io dtype       dt, lambda (batch, L, H) fp32
 *   A, D   (H)                   fp32           theta      (batch, L, G, N/2) fp32
 *   B, C   (batch, L, G, R, N)   io dtype       B[b,t,g,r,n] = (B_t)_{n,r}
 *   state h (batch, H, N, P) state dtype (fp32 by default; true frame)
 *   carry  b_last (batch, G, R, N), x_last (batch, H, R, P) io dtype
 *   Decode drops the L axis of every per-token tensor.
 *
 * Ownership and execution: every pointer is device memory owned by the caller.
 * The library never allocates, frees or synchronises; all work is enqueued on
 * `stream` (a hipStream_t; NULL = the null stream) and the call returns at once.
 * There is no global mutable state (except the static scratch array of
 * m3_prefill_chunked_noalloc, see there, and a mutex-guarded host-side record of
 * the kernels whose LDS limit has been raised on each device): calls on different
 * streams may run from different threads.  Outputs must not alias inputs unless
 * stated.  After a first call of a given shape on a device, a call enqueues kernel
 * launches only (no allocation, memset, synchronisation or attribute change), so it
 * can be captured in a HIP graph.
 *
 * Errors: argument and shape errors are returned before anything is launched.
 * Launch failures return M3_ERR_HIP.  Faults inside a kernel surface at the
 * caller's next synchronisation.  No C++ exception crosses this interface.
 * Value ranges (dt > 0, 0 <= lambda <= 1, A <= 0) are not checked: the
 * arithmetic is carried out on whatever is passed.
 */
#ifndef M3SCAN_H
#define M3SCAN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    M3_OK = 0,
    M3_ERR_INVALID_ARG = -1,   /* null pointer, non-positive size, N odd, H % G != 0 */
    M3_ERR_UNSUPPORTED = -2,   /* a shape/dtype combination no kernel here handles   */
    M3_ERR_WORKSPACE = -3,     /* workspace_bytes smaller than the size asked for     */
    M3_ERR_HIP = -4            /* a HIP launch or runtime call failed                 */
} m3_status;

typedef enum { M3_F32 = 0, M3_BF16 = 1 } m3_dtype;

typedef struct {
    int64_t batch;     /* b                                   >= 1 */
    int64_t seqlen;    /* L (prefill); ignored by decode      >= 0 */
    int64_t nheads;    /* H                                   >= 1 */
    int64_t ngroups;   /* G, divides H                        >= 1 */
    int64_t headdim;   /* P                                   >= 1 */
    int64_t dstate;    /* N, even                             >= 2 */
    int64_t rank;      /* R (1 = SISO)                        >= 1 */
    int64_t chunk;     /* Q, tokens per chunk; ignored by decode >= 1 */
    int32_t io_dtype;     /* m3_dtype of x, B, C, y and the carry                   */
    int32_t state_dtype;  /* m3_dtype of the state h; 0 = M3_F32.  With M3_BF16 the
                             state is stored in bf16 (rounded to nearest even) and
                             all arithmetic stays fp32: a decode step reads the bf16
                             state, updates it in fp32 and writes it back rounded
                             (half the state bytes of fp32); a prefill reads
                             state_in and writes state_out in bf16.              */
} m3_dims;

typedef struct {
    void* h;           /* (batch, H, N, P) in dims->state_dtype: the state after the
                          last token                                                  */
    void* b_last;      /* (batch, G, R, N) io dtype: B of the last token (the carry)    */
    void* x_last;      /* (batch, H, R, P) io dtype: X of the last token (the carry)    */
} m3_state;

/* Bytes of device workspace m3_prefill_chunked needs for these dims (may be 0).
 * Errors: M3_ERR_INVALID_ARG for bad dims or a NULL `bytes`. */
m3_status m3_prefill_workspace_size(const m3_dims* dims, size_t* bytes);

/* How many sequences of the batch one workgroup of the chunked prefill sweeps, one
 * after another, for these dims (m3_prefill_chunked without fusion).  A single
 * short sequence leaves its workgroup waiting on its own loads; batches of many
 * equal-length sequences of one to four whole chunks (the hardware-aware scan of
 * IBM's "What is a Mamba model?", parallel over sequences and heads) are therefore
 * swept several to a workgroup, the next sequence's first chunk fetched while the
 * current one computes, its state reset at the boundary (not at 128 rows per chunk,
 * chunk * rank, where two workgroups already share a compute unit).  1 means one sequence
 * per workgroup.  The choice depends on the dims only and does not change any
 * result bit.  Errors as m3_prefill_workspace_size, and M3_ERR_UNSUPPORTED for
 * dims no prefill kernel takes. */
m3_status m3_prefill_sequences_per_workgroup(const m3_dims* dims, int32_t* seqs);

/*
 * Chunked prefill: the whole sequence of `seqlen` tokens for every (b, h).
 * Computes y (batch, L, H, R, P) in the io dtype, rounded to nearest even from
 * fp32, and optionally the final state.
 *
 * state_in:  NULL, or the state to continue from; its h must be non-NULL and
 *            its carry (b_last, x_last) may be NULL (zero previous input).
 *            May alias state_out (read before written).
 * state_out: NULL, or where to write the final state; each of its fields may
 *            be NULL to skip it.  The carry written is a copy of B and X of
 *            the last token (the caller may equally keep those slices).
 * workspace: device memory of at least m3_prefill_workspace_size bytes
 *            (NULL allowed when that size is 0); contents on entry ignored.
 * Partial last chunks (L not a multiple of `chunk`) and L = 0 are allowed.
 * chunk:     the block size of the chunked form.  The result does not depend on it
 *            beyond rounding; the matrix-core kernels (bf16 io, N = 128, P = 64,
 *            R in {1, 2, 4}, chunk 32 or 64) use it as given, the fp32 vector
 *            kernels split a chunk whose arrays exceed LDS into halves (quarters, ..),
 *            and small states (N/2 a power of two, N/2 * P <= 256, no fused B/C
 *            norm, bias, gate or output norm) are scanned token by token, without
 *            chunks.
 */
m3_status m3_prefill_chunked(const m3_dims* dims, const void* x, const float* dt,
                             const float* A, const float* lambda, const float* theta,
                             const void* B, const void* C, const float* D,
                             const m3_state* state_in, m3_state* state_out, void* y,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * Chunked prefill of a packed batch of variable-length sequences.  Sequence s
 * is tokens cu_seqlens[s] .. cu_seqlens[s+1]-1 of one token axis of
 * total_tokens tokens; its scan starts afresh there (from state_in's slice s,
 * else from a zero state and a zero previous input), exactly as if it were run
 * alone through m3_prefill_chunked with batch 1.  The chunks of a sequence start
 * at its first token.
 *
 * dims:       batch = number of sequences; seqlen = an upper bound on every
 *             sequence's length (it sizes the launch and the workspace:
 *             m3_prefill_workspace_size(dims) covers this call too); the other
 *             fields as for m3_prefill_chunked.
 * cu_seqlens: device array of batch + 1 int64 offsets, non-decreasing, from 0
 *             to total_tokens.  It is read only by the kernels, so it is not
 *             checked here: offsets outside [0, total_tokens], decreasing ones
 *             or lengths above seqlen are clamped to those bounds (wrong results
 *             for such a sequence, never an access outside the arrays).
 * Layouts:    x, y (total_tokens, H, R, P); dt, lambda (total_tokens, H);
 *             theta (total_tokens, G, N/2); B, C (total_tokens, G, R, N);
 *             state_in / state_out per sequence, as for m3_prefill_chunked.
 * Errors:     as m3_prefill_chunked; also M3_ERR_INVALID_ARG for a NULL
 *             cu_seqlens or total_tokens < 0.
 */
m3_status m3_prefill_varlen(const m3_dims* dims, const int64_t* cu_seqlens, int64_t total_tokens,
                            const void* x, const float* dt, const float* A, const float* lambda,
                            const float* theta, const void* B, const void* C, const float* D,
                            const m3_state* state_in, m3_state* state_out, void* y,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * One decode step for every (b, h): reads the state h (dims->state_dtype) in
 * place, applies one token in fp32 and writes the new state back to h, and
 * writes y_t (batch, H, R, P).  y_t reads the new state before it is rounded to
 * a bf16 state.  This is the single-token recurrence step of the paper note's
 * "Problem definition" (its third problem: each generated token reads and writes
 * the whole state for little arithmetic, so the step is bound by memory
 * bandwidth) with the rank-R update of "Solution 3: MIMO", which raises the
 * arithmetic per state byte.  Its equations are those at the top of this file
 * at L = 1.
 *
 * b_last, x_last: B and X of the previous token (the trapezoid carry), in the
 *            io dtype; both NULL means a zero previous input.  They are only
 *            read, so the caller passes this call's B_t and x_t as the next
 *            call's b_last and x_last -- no copy, and no race between heads of
 *            a group that share b_last.
 * Per-token inputs: x_t (b,H,R,P), dt_t, lambda_t (b,H), theta_t (b,G,N/2),
 *            B_t, C_t (b,G,R,N).  dims->seqlen and dims->chunk are ignored.
 */
m3_status m3_decode_step(const m3_dims* dims, void* h, const void* b_last,
                         const void* x_last, const void* x_t, const float* dt_t,
                         const float* A, const float* lambda_t, const float* theta_t,
                         const void* B_t, const void* C_t, const float* D, void* y_t,
                         void* stream);

/*
 * Fused prologue and epilogue of a Mamba-3 layer around the scan (the pieces of
 * the layer next to it on the Mamba-3 blog, part 1, "Normalization" and
 * "Removing the short convolution", the per-token A of the paper note's
 * discretisation, the output norm of its "Architecture" section) and the layout
 * with angles per head.  Every pointer may be NULL (that piece is off); fp32
 * unless stated.
 *   A_t:       per-token decay rate replacing A: (batch, L, H) for a prefill,
 *              (batch, H) for a decode step (A must still be passed; it is not read).
 *   b_norm_w:  (R, N): B[b,t,g,r,:] is divided by its root mean square
 *              sqrt(mean(B^2) + norm_eps) and multiplied by b_norm_w[r,:] (BCNorm).
 *   c_norm_w:  (R, N): the same for C.
 *   b_bias, c_bias: (R, N) added to B and C after the norm.
 *              All four act before the rotation, on every B and C the scan reads,
 *              including a carried previous B: carries stay raw (as given).
 *   z:         gate, io dtype, laid out as y: y is returned as y * silu(z),
 *              silu(v) = v / (1 + exp(-v)).
 *   norm_eps:  > 0 when a norm weight is given.
 *   out_norm_w: (H, P): RMSNorm of the output before the out-projection (the paper
 *              note's "Architecture" section: kept in hybrid models): each row
 *              y[.., h, r, :] of P values is divided by sqrt(mean(y^2) + norm_eps) and
 *              multiplied by out_norm_w[h, :], after the gate when both are given.
 *   theta_groups: 0, or the number Gt of angle groups when the angles are grouped more
 *              finely than B and C (Gt = H: every head turns with its own angles over
 *              the B and C its group shares).  G divides Gt and Gt divides H; theta is
 *              then (batch, L, Gt, N/2) ((batch, Gt, N/2) for a decode step,
 *              (total_tokens, Gt, N/2) for a packed batch) and head h turns with angle
 *              group h / (H / Gt).  0 means Gt = G (the layout of the plain calls).
 */
typedef struct {
    const float* A_t;
    const float* b_norm_w;
    const float* c_norm_w;
    const float* b_bias;
    const float* c_bias;
    const void* z;
    float norm_eps;
    const float* out_norm_w;
    int32_t theta_groups;
} m3_fusion;

/* Bytes of device workspace m3_prefill_fused and m3_prefill_varlen_fused need for these
 * dims and this fusion (equal to m3_prefill_workspace_size when fusion->theta_groups is 0
 * or G; angles per head need room for operands prepared per angle group).
 * Errors: those of m3_prefill_workspace_size, and M3_ERR_INVALID_ARG for a NULL fusion or
 * bad theta_groups. */
m3_status m3_prefill_fused_workspace_size(const m3_dims* dims, const m3_fusion* fusion, size_t* bytes);

/* m3_prefill_chunked with the fused prologue/epilogue of `fusion` (non-NULL).
 * The workspace size depends on fusion->theta_groups: query it with
 * m3_prefill_fused_workspace_size.  The other arguments, layouts and errors as
 * m3_prefill_chunked, plus M3_ERR_INVALID_ARG for a NULL fusion, a norm weight with
 * norm_eps <= 0, or theta_groups not a multiple of G dividing H. */
m3_status m3_prefill_fused(const m3_dims* dims, const void* x, const float* dt, const float* A,
                           const float* lambda, const float* theta, const void* B, const void* C,
                           const float* D, const m3_fusion* fusion, const m3_state* state_in,
                           m3_state* state_out, void* y, void* workspace, size_t workspace_bytes,
                           void* stream);

/* m3_prefill_varlen with the fused prologue/epilogue of `fusion` (non-NULL; the pieces of
 * the layer next to the scan, Mamba-3 blog part 1, "Normalization" and "Removing the short
 * convolution", and the per-token A of the paper note's "Solution 1"), on a packed
 * batch: A_t is (total_tokens, H) and z is laid out as y, (total_tokens, H, R, P); a
 * carried b_last of state_in (per sequence) is normalised like B.  Workspace size:
 * m3_prefill_fused_workspace_size; the other arguments, layouts and errors as
 * m3_prefill_varlen, plus those of m3_prefill_fused. */
m3_status m3_prefill_varlen_fused(const m3_dims* dims, const int64_t* cu_seqlens, int64_t total_tokens,
                                  const void* x, const float* dt, const float* A, const float* lambda,
                                  const float* theta, const void* B, const void* C, const float* D,
                                  const m3_fusion* fusion, const m3_state* state_in, m3_state* state_out,
                                  void* y, void* workspace, size_t workspace_bytes, void* stream);

/* m3_decode_step with the fused prologue/epilogue of `fusion` (non-NULL; z and A_t
 * have the step's shapes (batch, H, R, P) and (batch, H)).  The carry b_last is the
 * raw previous B, normalised here like B_t. */
m3_status m3_decode_step_fused(const m3_dims* dims, void* h, const void* b_last, const void* x_last,
                               const void* x_t, const float* dt_t, const float* A, const float* lambda_t,
                               const float* theta_t, const void* B_t, const void* C_t, const float* D,
                               const m3_fusion* fusion, void* y_t, void* stream);

/* Gradients written by m3_backward; every array is fp32, in the layout of the
 * input it belongs to.  dh0, db_last and dx_last may be NULL (not wanted). */
typedef struct {
    float* dx;       /* (batch, L, H, R, P)                                        */
    float* ddt;      /* (batch, L, H)                                              */
    float* dA;       /* (H): summed over batch and tokens (per token: m3_backward_per_token_A) */
    float* dlambda;  /* (batch, L, H)                                              */
    float* dtheta;   /* (batch, L, G, N/2): summed over the heads of each group    */
    float* dB;       /* (batch, L, G, R, N): summed over the heads of each group   */
    float* dC;       /* (batch, L, G, R, N): summed over the heads of each group   */
    float* dD;       /* (H): summed over batch and tokens                         */
    float* dh0;      /* (batch, H, N, P): gradient of state_in->h                  */
    float* db_last;  /* (batch, G, R, N): of state_in->b_last (zero without a carry) */
    float* dx_last;  /* (batch, H, R, P): of state_in->x_last (zero without a carry) */
} m3_grads;

/* Bytes of device workspace m3_backward needs for these dims with a checkpoint
 * budget of 4 GiB (m3_backward_workspace_size_budget with checkpoint_bytes =
 * 2^32).  Errors: M3_ERR_INVALID_ARG for bad dims or a NULL `bytes`;
 * M3_ERR_UNSUPPORTED for shapes m3_backward does not handle. */
m3_status m3_backward_workspace_size(const m3_dims* dims, size_t* bytes);

/* Bytes of device workspace m3_backward needs for these dims when the states it
 * keeps for the reverse sweep may take at most `checkpoint_bytes` (a caller short
 * of memory passes less than the default 4 GiB, one with memory to spare more).
 * The states (N * P * 4 bytes each, per (b, h)) are kept at one of a few levels,
 * the first whose states fit the budget, else the level with the smallest
 * workspace: at dstate 128, headdim 64 (level 0) one after every third token,
 * (level 1) two levels of about sqrt(L / 3) states each (one after every group of
 * segments, and one group's states recomputed into a scratch) for one more
 * forward pass; at other shapes (level 0) every state, (level 1) one before every
 * 16-token segment plus one segment's 17 states, (level 2) segments of
 * ceil(sqrt(L)) tokens rounded up to a multiple of 16.  The workspace also holds,
 * when H > G, per-head copies of the group-shared gradients and, when the
 * sequences are split (m3_backward_parts), two N * P states per piece.  The
 * gradients are the same bits at every level.  Errors as
 * m3_backward_workspace_size. */
m3_status m3_backward_workspace_size_budget(const m3_dims* dims, size_t checkpoint_bytes, size_t* bytes);

/* How m3_backward divides the work for these dims: each (b, h) sequence is cut
 * into *parts pieces of *tokens_per_part tokens (the last may be shorter) that are
 * processed side by side, after a pass that gives each piece the state and the
 * adjoint it starts from; *parts is 1 (and *tokens_per_part the length) when the
 * (b, h) pairs alone fill the GPU, and always off the fast kernel's shape (N = 128,
 * P = 64).  The choice depends on the dims only, so the
 * rounding of the gradients does too.  Errors as m3_backward_workspace_size. */
m3_status m3_backward_parts(const m3_dims* dims, int32_t* parts, int64_t* tokens_per_part);

/*
 * Backward pass of the scan for training: the derivative of
 *     Loss = sum_t <dy_t, y_t> + <dh_out, h_L>
 * (y and h_L as m3_prefill_chunked computes them from the same inputs and
 * state_in) with respect to every input, by the adjoint method on the
 * recurrence of the Mamba-3 paper note ("Solution 1" update, "Solution 2"
 * rotation, "Solution 3" rank-R input/output).  The forward states are
 * recomputed from checkpoints in the workspace; nothing from a previous
 * prefill call is needed.
 *
 * Supported: dstate 128, headdim 64, rank 1, 2 or 4 (the fast kernel: sequences
 * split into pieces when the (b, h) pairs leave the GPU idle); any other even
 * dstate N and headdim P up to 256 with N / 2 * P at most 4096 and rank 1 to 8
 * (one workgroup per (b, h), token by token, never split); io dtype fp32 or bf16;
 * state_in->h in dims->state_dtype.  dims->chunk is ignored.  All arithmetic
 * is fp32, except the sums of dt*A and theta over the tokens of a piece of a
 * split sequence (fp64).  Results do not depend on scheduling (no atomics).
 * state_in:  NULL or as for m3_prefill_chunked (h non-NULL; carry optional).
 * dy:        (batch, L, H, R, P) in the io dtype.
 * dh_out:    NULL (zero) or (batch, H, N, P) fp32.
 * grads:     every pointer of m3_grads except dh0, db_last, dx_last non-NULL.
 * workspace: workspace_bytes of device memory, contents ignored: at least what
 *            m3_backward_workspace_size or m3_backward_workspace_size_budget
 *            returns for these dims; the call keeps states at the first level
 *            (the fewest recomputed) whose workspace fits workspace_bytes.
 * Errors:    M3_ERR_INVALID_ARG (NULL pointers, bad dims), M3_ERR_UNSUPPORTED,
 *            M3_ERR_WORKSPACE (no level fits workspace_bytes), M3_ERR_HIP -- all
 *            before any launch except the last.
 */
m3_status m3_backward(const m3_dims* dims, const void* x, const float* dt, const float* A,
                      const float* lambda, const float* theta, const void* B, const void* C,
                      const float* D, const m3_state* state_in, const void* dy,
                      const float* dh_out, const m3_grads* grads, void* workspace,
                      size_t workspace_bytes, void* stream);

/*
 * m3_backward for a packed batch of variable-length sequences (the gradients of
 * m3_prefill_varlen's outputs): sequence s is tokens cu_seqlens[s] ..
 * cu_seqlens[s+1]-1 and is differentiated as if run alone, from state_in's slice
 * s (else a zero state and previous input) to its own final state.
 *
 * dims:       batch = number of sequences; seqlen = an upper bound on every
 *             sequence's length; total_tokens <= batch * seqlen (the workspace,
 *             m3_backward_workspace_size(dims), holds per-token partial sums for
 *             that many tokens).
 * cu_seqlens: device array of batch + 1 int64 offsets, non-decreasing, from 0 to
 *             total_tokens; read only by the kernels and clamped there as in
 *             m3_prefill_varlen (wrong results for an inconsistent sequence, never
 *             an access outside the arrays).  Gradient rows of tokens that belong
 *             to no sequence are left undefined.
 * Layouts:    x, dy, dx (total_tokens, H, R, P); dt, lambda, ddt, dlambda
 *             (total_tokens, H); theta, dtheta (total_tokens, G, N/2); B, C, dB, dC
 *             (total_tokens, G, R, N); dh_out, state_in and the state gradients per
 *             sequence, as for m3_backward.
 * Errors:     as m3_backward; also M3_ERR_INVALID_ARG for a NULL cu_seqlens,
 *             total_tokens < 0 or total_tokens > batch * seqlen.
 */
m3_status m3_backward_varlen(const m3_dims* dims, const int64_t* cu_seqlens, int64_t total_tokens,
                             const void* x, const float* dt, const float* A, const float* lambda,
                             const float* theta, const void* B, const void* C, const float* D,
                             const m3_state* state_in, const void* dy, const float* dh_out,
                             const m3_grads* grads, void* workspace, size_t workspace_bytes, void* stream);

/*
 * m3_backward (cu_seqlens NULL) or m3_backward_varlen (cu_seqlens non-NULL) with a
 * per-token decay rate A_t in place of the per-head A: the discretisation of the
 * Mamba-3 paper note ("Solution 1") gives each token its own A_t, so the decay is
 * exp(dt_t A_t) (as m3_prefill_fused computes with fusion->A_t).
 *
 * A_t:       fp32, (batch, L, H), or (total_tokens, H) with cu_seqlens.
 * grads->dA: per token, in A_t's layout (not summed); with cu_seqlens, rows of
 *            tokens that belong to no sequence are left undefined.
 * total_tokens is read only with cu_seqlens.  Every other argument, the workspace
 * size and the errors as the call it stands for; also M3_ERR_INVALID_ARG for a
 * NULL A_t.
 */
m3_status m3_backward_per_token_A(const m3_dims* dims, const int64_t* cu_seqlens, int64_t total_tokens,
                                  const void* x, const float* dt, const float* A_t, const float* lambda,
                                  const float* theta, const void* B, const void* C, const float* D,
                                  const m3_state* state_in, const void* dy, const float* dh_out,
                                  const m3_grads* grads, void* workspace, size_t workspace_bytes,
                                  void* stream);

/*
 * For callers that cannot allocate device memory (work recorded under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): m3_prefill_chunked
 * without a workspace argument.  The workspace lives in a static device array of
 * M3_NOALLOC_SCRATCH_BYTES bytes inside this library; every GPU the call runs on
 * holds its own copy from the first such call until the process ends.  The call
 * allocates and frees nothing.
 *
 * Limit: dims whose m3_prefill_workspace_size exceeds M3_NOALLOC_SCRATCH_BYTES are
 * rejected with M3_ERR_WORKSPACE before anything is launched (call
 * m3_prefill_chunked with a workspace of your own for those).
 * Sharing: all calls on one GPU use that GPU's one array, so calls that can overlap
 * on one GPU (different streams, or threads without ordering between them) race
 * on it and must be serialised by the caller.  Nothing in the array needs to start
 * at zero; it keeps the last call's contents.
 * Arguments, layouts and the other errors: as m3_prefill_chunked; M3_ERR_HIP also
 * when the array's device address cannot be obtained.
 */
#define M3_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
m3_status m3_prefill_chunked_noalloc(const m3_dims* dims, const void* x, const float* dt,
                                     const float* A, const float* lambda, const float* theta,
                                     const void* B, const void* C, const float* D,
                                     const m3_state* state_in, m3_state* state_out, void* y,
                                     void* stream);

/* Static text for a status code. */
const char* m3_status_string(m3_status status);

/* Library version: major * 10000 + minor * 100 + patch. */
int32_t m3_version(void);

#ifdef __cplusplus
}
#endif

#endif /* M3SCAN_H */
