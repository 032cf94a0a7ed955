"""fp64 numpy mirror of the chunkwise algorithm the HIP kernels implement (test-side only).

This is neither the oracle nor the GPU path: it restates, in plain numpy, the
chunk equations the kernels follow, so the algebra can be checked against the
token-by-token oracle at machine precision (the pages report that the chunk
form's gradients match a token-wise reference to machine precision in fp64:
anthology record LIT-802, takeaway 2, App. D.6). It also exposes per-chunk
intermediates for debugging kernels.

Chunk equations (normalising the state by the cumulative decay inside a chunk
folds the channel-wise decay into the two factors of each rank-one erase;
LIT-802 takeaway 2, wispaper "Efficient Parallel Training", chatpaper
abstract). For a chunk with start state S and chunk-local cumulative
log-decay gam_r = sum_{i<=r} g_i:

    A[r,i] = sum_c b_rc k_rc k_ic exp(gam_rc - gam_ic)     (i < r)
    M[r,i] = sum_c q_rc k_ic exp(gam_rc - gam_ic)          (i <= r)
    T  = (I + A)^-1            (one inverse for the erase and write sides)
    U  = T (W*V)               Wm = T (B*K*exp(gam))
    Delta = U - Wm S
    O  = (Q*exp(gam)) S + M Delta
    S' = diag(exp(gam_C)) S + Kd^T Delta,   Kd = K*exp(gam_C - gam)

A and M are formed per 16x16 block pair (R, I) with the exponent split at the
last row of block I, exp(gam_r - gam_i) = exp(gam_r - gam_R0) exp(gam_R0 -
gam_Iend) exp(gam_Iend - gam_i), so that for R > I every factor is <= 1.

Backward (derived by differentiating the equations above): the reverse state
chain is dS = diag(exp(gam_C)) dS' + P'^T dS' + Qt^T dO with P' = -Kd^T Wm and
Qt = Q*exp(gam) - M Wm; the intra-chunk gradients follow in chunk_bwd().
"""
import numpy as np

BLK = 16


def _pad(x, C):
    T = x.shape[0]
    NT = (T + C - 1) // C
    out = np.zeros((NT * C,) + x.shape[1:])
    out[:T] = x
    return out, NT


def chunk_factors(q, k, g, b, C):
    """Per-chunk factors from the chunk's rows (C x DK each)."""
    gam = np.cumsum(g, axis=0)
    blk = min(BLK, C)  # chunks shorter than a block are one block
    nb = C // blk
    A = np.zeros((C, C))
    M = np.zeros((C, C))
    for R in range(nb):
        r0 = R * blk
        rr = slice(r0, r0 + blk)
        E1 = np.exp(gam[rr] - gam[r0])               # <= 1
        for I in range(R + 1):
            ie = I * blk + blk - 1
            ii = slice(I * blk, I * blk + blk)
            s = np.exp(gam[r0] - gam[ie])             # <= 1 for I < R
            y = k[ii] * np.exp(gam[ie] - gam[ii])     # <= |k|
            A[rr, ii] = (b[rr] * k[rr] * E1 * s) @ y.T
            M[rr, ii] = (q[rr] * E1 * s) @ y.T
    A = np.tril(A, -1)
    M = np.tril(M, 0)
    return gam, A, M


def chunk_fwd(q, k, v, g, b, w, h0=None, C=64, keep=False):
    """One sequence: q, k, g, b [T, DK]; v, w [T, DV]. Returns o, S_T (and intermediates)."""
    T, DK = q.shape
    DV = v.shape[1]
    (q, NT), (k, _), (v, _), (g, _), (b, _), (w, _) = (_pad(x, C) for x in (q, k, v, g, b, w))
    S = np.zeros((DK, DV)) if h0 is None else h0.copy()
    o = np.zeros((NT * C, DV))
    inter = []
    for c in range(NT):
        sl = slice(c * C, (c + 1) * C)
        gam, A, M = chunk_factors(q[sl], k[sl], g[sl], b[sl], C)
        Tm = np.linalg.inv(np.eye(C) + A)
        Gam = np.exp(gam)
        GC = Gam[-1]
        X = w[sl] * v[sl]
        Kb = b[sl] * k[sl] * Gam
        Qg = q[sl] * Gam
        Kd = k[sl] * np.exp(gam[-1] - gam)
        U = Tm @ X
        Wm = Tm @ Kb
        Delta = U - Wm @ S
        o[sl] = Qg @ S + M @ Delta
        if keep:
            inter.append(dict(S=S.copy(), A=A, M=M, T=Tm, U=U, Wm=Wm, Delta=Delta, GC=GC, Kd=Kd, Qg=Qg,
                              Kb=Kb, gam=gam))
        S = GC[:, None] * S + Kd.T @ Delta
    if keep:
        return o[:T], S, inter
    return o[:T], S


def bilinear_bwd(x, y, gam, dF, lower_strict):
    """F[r,i] = sum_c x_rc y_ic exp(gam_rc - gam_ic) on the (strictly) lower triangle.
    Returns dx, dy and the contribution to dgam."""
    E = np.exp(gam[:, None, :] - gam[None, :, :])      # [r, i, c]
    mask = np.tril(np.ones(dF.shape), -1 if lower_strict else 0)
    dF = dF * mask
    xb = np.einsum("ri,ic,ric->rc", dF, y, E)
    yb = np.einsum("ri,rc,ric->ic", dF, x, E)
    dgam = x * xb - y * yb
    return xb, yb, dgam


def chunk_bwd(q, k, v, g, b, w, h0, do, dht=None, C=64):
    """Chunkwise backward for one sequence, returns dq, dk, dv, dg, db, dw, dh0."""
    T, DK = q.shape
    DV = v.shape[1]
    _, _, inter = chunk_fwd(q, k, v, g, b, w, h0, C, keep=True)
    (q, NT), (k, _), (v, _), (g, _), (b, _), (w, _), (do, _) = (_pad(x, C) for x in (q, k, v, g, b, w, do))
    dS_next = np.zeros((DK, DV)) if dht is None else dht.copy()
    grads = {n: np.zeros_like(x) for n, x in (("dq", q), ("dk", k), ("dv", v), ("dg", g), ("db", b),
                                              ("dw", w))}
    for c in range(NT - 1, -1, -1):
        sl = slice(c * C, (c + 1) * C)
        it = inter[c]
        S, M, Tm, U, Wm, Delta, GC, Kd, Qg, Kb, gam = (it[n] for n in
                                                         ("S", "M", "T", "U", "Wm", "Delta", "GC", "Kd",
                                                          "Qg", "Kb", "gam"))
        Gam = np.exp(gam)
        dO = do[sl]
        # reverse state chain in the P-form
        Pp = -Kd.T @ Wm
        Qt = Qg - M @ Wm
        dS_prev = GC[:, None] * dS_next + Pp.T @ dS_next + Qt.T @ dO
        # intra-chunk gradients
        dDelta = M.T @ dO + Kd @ dS_next
        dM = np.tril(dO @ Delta.T)
        dQg = dO @ S.T
        dY = Tm.T @ dDelta
        dA = -np.tril(dY @ Delta.T, -1)
        dKb = -dY @ S.T
        dKd = Delta @ dS_next.T
        dGC = np.sum(dS_next * S, axis=1)
        xbA, ybA, dgamA = bilinear_bwd(b[sl] * k[sl], k[sl], gam, dA, True)
        xbM, ybM, dgamM = bilinear_bwd(q[sl], k[sl], gam, dM, False)
        grads["dw"][sl] = dY * v[sl]
        grads["dv"][sl] = dY * w[sl]
        grads["dq"][sl] = dQg * Gam + xbM
        grads["db"][sl] = dKb * k[sl] * Gam + xbA * k[sl]
        grads["dk"][sl] = (dKb * b[sl] * Gam + dKd * np.exp(gam[-1] - gam) + xbA * b[sl] + ybA + ybM)
        dgam = dQg * Qg + dKb * Kb - dKd * Kd + dgamA + dgamM
        dgam[-1] += np.sum(dKd * Kd, axis=0) + GC * dGC
        grads["dg"][sl] = np.cumsum(dgam[::-1], axis=0)[::-1]
        dS_next = dS_prev
    out = {n: x[:T] for n, x in grads.items()}
    out["dh0"] = dS_next
    return out
