"""Chunkwise form of the KDA backward in fp64 (test infrastructure: the equations a chunked
backward kernel would evaluate, checked here against the token-by-token reverse-mode oracle).

Per head and 64-token chunk of n tokens, with incoming state S0 and the gradient Hn = dL/dS_n
of the state after the chunk (from later chunks, or dL/dht), "Autoresearch on Kimi Delta
Attention" (section "KDA in one minute") gives the step; unrolled over a chunk it reads
(G the in-chunk cumulative log-gate, rows are tokens):

    Kg = khat e^G,  Qg = qhat e^G,  Kd = khat e^(G_n - G)
    L  = strictly lower part of (Kg)(khat e^-G)^T,  A = diag(beta) L,  T = (I + A)^-1
    W  = T diag(beta) Kg,  U = T diag(beta) V,  Delta = U - W S0
    P  = lower part (with the diagonal) of (Qg)(khat e^-G)^T
    O  = scale (Qg S0 + P Delta),  S_n = diag(e^G_n) S0 + Kd^T Delta

and its reverse-mode derivative, term by term:

    dDelta = scale P^T dO + Kd Hn
    dS0    = scale Qg^T dO + diag(e^G_n) Hn - W^T dDelta          (the next chunk's Hn)
    dX     = T^T (-dDelta S0^T),  dY = T^T dDelta                  (X = diag(beta) Kg, Y = diag(beta) V)
    dA     = -(dX W^T + dY U^T) on the strictly lower part
    dbeta  = rowsum(dA * L) + rowsum(dX * Kg) + rowsum(dY * V),  dV = beta dY
    then the gated products L (khat, khat) and P (qhat, khat), the scalings of Kg, Qg, Kd and
    e^G_n, and dg as the reverse cumulative sum of dG over the chunk.

No blocking, no reference-row gating: exp(-G) is formed directly, so inputs must keep the
in-chunk decay moderate (the tests do).
"""
import numpy as np


def _gated_back(dM, a, b, G):
    """M_ij = sum_c a_ic b_jc e^(G_ic - G_jc) (any mask already applied to dM): returns
    (da, db, dG) of L = sum(dM * M)."""
    E, Ei = np.exp(G), np.exp(-G)
    ra = (dM @ (b * Ei)) * E      # sum_j dM_ij b_jc e^(G_ic - G_jc)
    rb = (dM.T @ (a * E)) * Ei    # sum_i dM_ij a_ic e^(G_ic - G_jc)
    return ra, rb, a * ra - b * rb


def chunk_backward(qh, kh, v, g, beta, S0, dO, Hn, scale):
    """One chunk of one head (qh, kh unit rows): (dqh, dkh, dv, dg, dbeta, dS0)."""
    n = qh.shape[0]
    G = np.cumsum(g, axis=0)
    Gn = G[-1]
    E, Ei = np.exp(G), np.exp(-G)
    Kg, Qg, Kd = kh * E, qh * E, kh * np.exp(Gn - G)
    L = np.tril(Kg @ (kh * Ei).T, -1)
    A = beta[:, None] * L
    T = np.linalg.inv(np.eye(n) + A)
    X, Y = beta[:, None] * Kg, beta[:, None] * v
    W, U = T @ X, T @ Y
    D = U - W @ S0
    P = np.tril(Qg @ (kh * Ei).T)
    # backward
    dD = scale * P.T @ dO + Kd @ Hn
    dP = np.tril(scale * dO @ D.T)
    dQg = scale * dO @ S0.T
    dS0 = scale * Qg.T @ dO + np.exp(Gn)[:, None] * Hn - W.T @ dD
    dKd = D @ Hn.T
    dGn = np.exp(Gn) * np.sum(Hn * S0, axis=1)
    dW = -dD @ S0.T
    dX, dY = T.T @ dW, T.T @ dD
    dA = np.tril(-(dX @ W.T + dY @ U.T), -1)
    dbeta = np.sum(dA * L, axis=1) + np.sum(dX * Kg, axis=1) + np.sum(dY * v, axis=1)
    dv = beta[:, None] * dY
    dKg = beta[:, None] * dX
    dL = beta[:, None] * dA
    da, db, dG = _gated_back(dL, kh, kh, G)
    dkh = da + db
    dq2, dk2, dG2 = _gated_back(dP, qh, kh, G)
    dqh = dq2
    dkh = dkh + dk2
    dG = dG + dG2
    dkh = dkh + dKg * E
    dG = dG + dKg * Kg
    dqh = dqh + dQg * E
    dG = dG + dQg * Qg
    dkh = dkh + dKd * np.exp(Gn - G)
    dG = dG - dKd * Kd
    dGn = dGn + np.sum(dKd * Kd, axis=0)
    dG[-1] += dGn
    dg = np.cumsum(dG[::-1], axis=0)[::-1]
    return dqh, dkh, dv, dg, dbeta, dS0


def chunked_backward(q, k, v, g, beta, do, h0=None, cu_seqlens=None, scale=None, dht=None, chunk=64):
    """The whole backward by chunks: forward states at chunk starts by the token recurrence
    (fp64), then the chunks in reverse with chunk_backward.  Returns (dq, dk, dv, dg, dbeta,
    dh0) like oracle_bwd."""
    q, k, v, g, beta, do = (np.asarray(a, dtype=np.float64) for a in (q, k, v, g, beta, do))
    B, T, H, dk = q.shape
    dvd = v.shape[-1]
    if scale is None:
        scale = dk ** -0.5
    flat = lambda a: a.reshape((B * T,) + a.shape[2:])
    qf, kf, vf, gf, bf, dof = (flat(a) for a in (q, k, v, g, beta, do))

    def unit(x):
        nrm = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
        return np.where(nrm > 0, x / np.where(nrm > 0, nrm, 1.0), 0.0), nrm

    qh, qn = unit(qf)
    kh, kn = unit(kf)
    if cu_seqlens is None:
        seqs = [(b * T, (b + 1) * T) for b in range(B)]
    else:
        cu = np.asarray(cu_seqlens, dtype=np.int64)
        seqs = [(int(cu[i]), int(cu[i + 1])) for i in range(len(cu) - 1)]
    dqh, dkh = np.zeros_like(qf), np.zeros_like(kf)
    dv, dg, dbeta = np.zeros_like(vf), np.zeros_like(gf), np.zeros_like(bf)
    dh0 = np.zeros((len(seqs), H, dk, dvd))
    for n, (t0, t1) in enumerate(seqs):
        for h in range(H):
            S = np.zeros((dk, dvd)) if h0 is None else np.array(h0[n, h], dtype=np.float64)
            starts = list(range(t0, t1, chunk))
            S0s = []
            for c0 in starts:
                S0s.append(S.copy())
                for t in range(c0, min(c0 + chunk, t1)):
                    a = np.exp(gf[t, h])[:, None] * S
                    delta = vf[t, h] - a.T @ kh[t, h]
                    S = a + bf[t, h] * np.outer(kh[t, h], delta)
            Hn = np.zeros((dk, dvd)) if dht is None else np.array(dht[n, h], dtype=np.float64)
            for c0, S0 in reversed(list(zip(starts, S0s))):
                c1 = min(c0 + chunk, t1)
                r = chunk_backward(qh[c0:c1, h], kh[c0:c1, h], vf[c0:c1, h], gf[c0:c1, h], bf[c0:c1, h],
                                   S0, dof[c0:c1, h], Hn, scale)
                dqh[c0:c1, h], dkh[c0:c1, h], dv[c0:c1, h], dg[c0:c1, h], dbeta[c0:c1, h] = r[:5]
                Hn = r[5]
            dh0[n, h] = Hn

    def unnorm(dxh, xh, xn):
        proj = dxh - xh * np.sum(xh * dxh, axis=-1, keepdims=True)
        return np.where(xn > 0, proj / np.where(xn > 0, xn, 1.0), 0.0)

    shp = lambda a, ref: a.reshape(ref.shape)
    return (shp(unnorm(dqh, qh, qn), q), shp(unnorm(dkh, kh, kn), k), shp(dv, v), shp(dg, g),
            shp(dbeta, beta), dh0)
