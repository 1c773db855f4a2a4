"""The chunked form the HIP prefill computes, written in fp64 numpy, equals the
oracle.  This pins the algebra of the kernels before any kernel exists; it
shares no code with them.

Per (b, h), chunks of Q tokens, chunk-local inclusive sums
  cum_i = sum_{j<=i} dt_j A,  phi_{i,k} = sum_{j<=i} theta_{j,k},
rotated operands  Bt_i = R(-phi_i) B_i,  Ct_i = R(-phi_i) C_i,
look-ahead weight w_j = lambda_j dt_j + (1 - lambda_{j+1}) dt_{j+1}
(w = gamma at the last token of the sequence) and the carried state
S = h + (1 - lambda_next) dt_next U_last in the true frame:
  Y_i = D X_i + e^{cum_i} Ct_i^T S_in + sum_{j<=i} mask_ij (Ct_i^T Bt_j) X_j,
  mask_ij = e^{cum_i - cum_j} w_j (j < i),  gamma_i (j = i),
  S_out = R(phi_end) [ e^{cum_end} S_in + sum_j e^{cum_end - cum_j} w_j Bt_j X_j ].
Segments of chunks are summarised by (total decay, total angle, state) and
combined with the same S_out rule (the inter-segment pass)."""
import numpy as np
import pytest

import oracle
import pins


def _rot(v, ang):
    c, s = np.cos(ang), np.sin(ang)
    out = np.empty_like(v)
    out[..., 0::2] = c * v[..., 0::2] - s * v[..., 1::2]
    out[..., 1::2] = s * v[..., 0::2] + c * v[..., 1::2]
    return out


def chunked_scan(x, dt, A, lam, theta, B, C, D, Q, state_in=None, nseg=1):
    b, L, H, R, P = x.shape
    G, N = B.shape[2], B.shape[4]
    y = np.zeros_like(x)
    hout = np.zeros((b, H, N, P))
    nchunks = (L + Q - 1) // Q
    for bi in range(b):
        for h in range(H):
            g = h // (H // G)
            a = dt[bi, :, h] * A[h]
            lv, dv = lam[bi, :, h], dt[bi, :, h]
            w = lv * dv
            w[:-1] += (1 - lv[1:]) * dv[1:]
            S = np.zeros((N, P))
            if state_in is not None:
                h0, bl, xl = state_in
                S = h0[bi, h].copy()
                if L > 0:
                    S += (1 - lv[0]) * dv[0] * (bl[bi, g].T @ xl[bi, h])
            # chunk summaries (for the segment pass)
            seg_of = lambda c: min(c * nseg // max(nchunks, 1), nseg - 1)
            seg_first = [min(c for c in range(nchunks) if seg_of(c) == s) for s in range(nseg)]
            # pass 1: per-segment (decay, angle, state contribution)
            summ = []
            for s in range(nseg):
                cs = [c for c in range(nchunks) if seg_of(c) == s]
                dec, ang, St = 0.0, np.zeros(N // 2), np.zeros((N, P))
                for c in cs:
                    t0, t1 = c * Q, min((c + 1) * Q, L)
                    cum = np.cumsum(a[t0:t1])
                    phi = np.cumsum(theta[bi, t0:t1, g], axis=0)
                    Bt = _rot(B[bi, t0:t1, g], -phi[:, None, :])
                    sc = np.exp(cum[-1] - cum) * w[t0:t1]
                    dS = np.einsum("jrn,jrp->np", Bt * sc[:, None, None], x[bi, t0:t1, h])
                    St = _rot((np.exp(cum[-1]) * St + dS).T, phi[-1][None, :]).T
                    dec += cum[-1]
                    ang += phi[-1]
                summ.append((dec, ang, St))
            # pass 2: incoming state per segment
            S_in = [S]
            for s in range(nseg - 1):
                dec, ang, St = summ[s]
                S_in.append(_rot((np.exp(dec) * S_in[-1]).T, ang[None, :]).T + St)
            # pass 3: outputs, sweeping each segment from its incoming state
            for s in range(nseg):
                Sc = S_in[s]
                for c in [c for c in range(nchunks) if seg_of(c) == s]:
                    t0, t1 = c * Q, min((c + 1) * Q, L)
                    cum = np.cumsum(a[t0:t1])
                    phi = np.cumsum(theta[bi, t0:t1, g], axis=0)
                    Bt = _rot(B[bi, t0:t1, g], -phi[:, None, :])
                    Ct = _rot(C[bi, t0:t1, g], -phi[:, None, :])
                    n = t1 - t0
                    i, j = np.meshgrid(np.arange(n), np.arange(n), indexing="ij")
                    seg = cum[:, None] - cum[None, :]
                    mask = np.where(j < i, np.exp(np.where(j < i, seg, 0.0)) * w[t0:t1][None, :], 0.0)
                    mask[np.arange(n), np.arange(n)] = lv[t0:t1] * dv[t0:t1]
                    G_ = np.einsum("irn,jsn->irjs", Ct, Bt)
                    yin = np.einsum("ij,irjs,jsp->irp", mask, G_, x[bi, t0:t1, h])
                    yst = np.exp(cum)[:, None, None] * np.einsum("irn,np->irp", Ct, Sc)
                    y[bi, t0:t1, h] = yin + yst + D[h] * x[bi, t0:t1, h]
                    sc = np.exp(cum[-1] - cum) * w[t0:t1]
                    dS = np.einsum("jrn,jrp->np", Bt * sc[:, None, None], x[bi, t0:t1, h])
                    Sc = _rot((np.exp(cum[-1]) * Sc + dS).T, phi[-1][None, :]).T
            hout[bi, h] = Sc
    return y, hout


@pytest.mark.parametrize("Q,nseg,L", [(1, 1, 13), (4, 1, 13), (4, 3, 29), (7, 2, 23), (32, 1, 23),
                                      (5, 4, 40)])
def test_chunked_equals_oracle(Q, nseg, L):
    d = pins.rand_case(b=2, L=L, H=4, G=2, P=3, N=6, R=2, seed=21, theta_scale=4.0)
    st = pins.rand_state(d, seed=3)
    args = pins._args(d)
    y0, h0 = oracle.scan(*args, state_in=st)
    y1, h1 = chunked_scan(*args, Q=Q, state_in=st, nseg=nseg)
    assert pins._relerr(y1, y0) < 1e-12
    assert pins._relerr(h1, h0) < 1e-12
