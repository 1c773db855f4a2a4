"""Two independent numpy formulations of the Mamba-3 scan -- TEST INFRASTRUCTURE ONLY.

They exist to pin the C oracle (``oracle.scan``); neither shares code with it
nor with the HIP library.  Shapes as in ``oracle.scan``.

scan_complex
    The state as N/2 complex modes per column p.  Mode k is the pair of real
    rows (2k, 2k+1) read as (real, imaginary).  The transition is the complex
    scalar exp(dt*A + i*theta) -- the "Mamba-3 paper note" (docsaid.org),
    section "Solution 2: a complex state that rotates": a complex SSM is a real
    SSM of twice the size whose transition is the decay times 2x2 rotations.
    The exponential-trapezoidal update (section "Solution 1") applies the
    complex alpha to both h_{t-1} and the beta term.

scan_dense
    The whole scan as one linear map: per (b, h) it builds each N x N
    transition T_t = alpha_t * blockdiag(rot(theta_t)) as a dense matrix,
    multiplies the products Phi(t, s) = T_t ... T_{s+1} out with matmul and
    assembles the (L*R) x (L*R) semiseparable matrix that maps X to Y.  The
    input X_s reaches h_t through gamma_s at step s and through
    beta_{s+1} M_{s+1} at step s+1 (the width-2 convolution that the
    trapezoid rule puts on the SSM input).  Use only for tiny shapes.
"""
from __future__ import annotations

import numpy as np


def _f64(*arrs):
    return [np.asarray(a, dtype=np.float64) for a in arrs]


def scan_complex(x, dt, A, lam, theta, B, C, D, state_in=None):
    x, dt, A, lam, theta, B, C, D = _f64(x, dt, A, lam, theta, B, C, D)
    b, L, H, R, P = x.shape
    G, N = B.shape[2], B.shape[4]
    K = N // 2
    grp = np.arange(H) // (H // G)                     # head -> group
    Bc = B[..., 0::2] + 1j * B[..., 1::2]              # (b,L,G,R,K)
    Cc = C[..., 0::2] + 1j * C[..., 1::2]
    z = np.zeros((b, H, K, P), dtype=np.complex128)
    u_prev = np.zeros((b, H, K, P), dtype=np.complex128)
    if state_in is not None:
        h0, bl, xl = state_in
        if h0 is not None:
            h0 = np.asarray(h0, dtype=np.float64)
            z = h0[:, :, 0::2, :] + 1j * h0[:, :, 1::2, :]
        if bl is not None and xl is not None:
            blc = np.asarray(bl, np.float64)[..., 0::2] + 1j * np.asarray(bl, np.float64)[..., 1::2]
            # u_prev[b,h,k,p] = sum_r blc[b,g(h),r,k] * xl[b,h,r,p]
            u_prev = np.einsum("bhrk,bhrp->bhkp", blc[:, grp], np.asarray(xl, np.float64))
    y = np.empty_like(x)
    for t in range(L):
        a = dt[:, t] * A[None, :]                                      # (b,H)
        th = theta[:, t][:, grp]                                       # (b,H,K)
        trans = np.exp(a[..., None] + 1j * th)                         # complex alpha
        u = np.einsum("bhrk,bhrp->bhkp", Bc[:, t][:, grp], x[:, t])
        beta = (1.0 - lam[:, t]) * dt[:, t]                            # times complex alpha
        gamma = lam[:, t] * dt[:, t]
        z = trans[..., None] * (z + beta[..., None, None] * u_prev) + gamma[..., None, None] * u
        # y[r,p] = sum_k Re(conj(c_k) z_k) = sum_k C[2k] Re z + C[2k+1] Im z
        y[:, t] = np.einsum("bhrk,bhkp->bhrp", np.conj(Cc[:, t][:, grp]), z).real \
            + D[None, :, None, None] * x[:, t]
        u_prev = u
    h_out = np.empty((b, H, N, P))
    h_out[:, :, 0::2] = z.real
    h_out[:, :, 1::2] = z.imag
    return y, h_out


def _transition(alpha, th, N):
    """Dense N x N matrix alpha * blockdiag([[cos, -sin], [sin, cos]])."""
    T = np.zeros((N, N))
    for k in range(N // 2):
        c, s = np.cos(th[k]), np.sin(th[k])
        T[2 * k, 2 * k], T[2 * k, 2 * k + 1] = c, -s
        T[2 * k + 1, 2 * k], T[2 * k + 1, 2 * k + 1] = s, c
    return alpha * T


def semiseparable_matrix(dt, A, lam, theta, B, C, D):
    """For one (b, h) slice: dt, lam (L,), A, D scalars, theta (L, N/2), B, C (L, R, N).

    Returns Mat of shape (L*R, L*R) with Y[(t,r), p] = sum Mat[(t,r),(s,r')] X[(s,r'), p].
    """
    L, R, N = B.shape
    T = [_transition(np.exp(dt[t] * A), theta[t], N) for t in range(L)]
    Mrot = [_transition(1.0, theta[t], N) for t in range(L)]
    beta = [(1.0 - lam[t]) * dt[t] * np.exp(dt[t] * A) for t in range(L)]
    gamma = [lam[t] * dt[t] for t in range(L)]
    I = np.eye(N)
    # Phi[t][s] = T_t ... T_{s+1}, Phi[t][t] = I
    Mat = np.zeros((L * R, L * R))
    for t in range(L):
        Phi = I.copy()                        # Phi(t, t)
        phis = {t: Phi}
        for s in range(t - 1, -1, -1):
            Phi = Phi @ T[s + 1]
            phis[s] = Phi
        for s in range(t + 1):
            # operator taking B_s[:, r'] into h_t
            op = phis[s] * gamma[s]
            if s < t:
                op = op + phis[s + 1] @ (beta[s + 1] * Mrot[s + 1])
            blk = C[t] @ op @ B[s].T          # (R, N) @ (N, N) @ (N, R)
            Mat[t * R:(t + 1) * R, s * R:(s + 1) * R] = blk
        Mat[t * R:(t + 1) * R, t * R:(t + 1) * R] += D * np.eye(R)
    return Mat


def scan_dense(x, dt, A, lam, theta, B, C, D):
    """Zero initial state; returns y only (b,L,H,R,P), via the semiseparable matrix."""
    x, dt, A, lam, theta, B, C, D = _f64(x, dt, A, lam, theta, B, C, D)
    b, L, H, R, P = x.shape
    G = B.shape[2]
    y = np.empty_like(x)
    for bi in range(b):
        for h in range(H):
            g = h // (H // G)
            Mat = semiseparable_matrix(dt[bi, :, h], A[h], lam[bi, :, h], theta[bi, :, g],
                                       B[bi, :, g], C[bi, :, g], D[h])
            y[bi, :, h] = (Mat @ x[bi, :, h].reshape(L * R, P)).reshape(L, R, P)
    return y
