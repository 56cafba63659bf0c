"""Reverse-mode derivative of the fp64 token-by-token KDA recurrence.

TEST INFRASTRUCTURE ONLY (see the package docstring).

"Autoresearch on Kimi Delta Attention" fixes what a training path must supply:
its stage "Frozen outside the loop" asks for exact KDA with full gradients checked
against an independent reference, and its phase "Move the path into CUDA" runs
the reverse recurrence over value tiles.  The forward step is the one the same
page's section "KDA in one minute" describes (the oracle in kda_oracle.c):

    a      = Diag(exp(g_t)) S_{t-1}
    delta  = v_t - a^T khat_t
    S_t    = a + beta_t khat_t delta^T
    o_t    = scale * S_t^T qhat_t,        qhat = q / ||q||, khat = k / ||k|| (0 for 0)

Given dL/do_t for every token and dL/dS_T (the final state's gradient), this module
walks the tokens backwards with G = dL/dS_t, in fp64, by the chain rule written out
term by term (u = khat^T G, one value per column):

    G       += scale qhat do^T                          (o_t reads S_t)
    dqhat    = scale S_t do
    dv       = beta u
    dbeta    = u . delta
    dkhat    = beta (G delta - a u)
    da       = G - beta khat u^T
    dg       = rowsum(a * da)                          (a depends on g through exp)
    G        = Diag(exp(g_t)) da                       (dL/dS_{t-1})

then dq = (dqhat - qhat (qhat . dqhat)) / ||q|| (0 for a zero vector), the same for k,
and dL/dh0 = G after the first token.  The forward states are recomputed here in
fp64 with numpy (`forward_states`); tests pin that forward to kda_oracle.c and the
gradients to central finite differences of it.
"""
import numpy as np


def _seqs(B, T, cu_seqlens):
    if cu_seqlens is None:
        return [(b * T, (b + 1) * T) for b in range(B)]
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    assert B == 1 and cu[0] == 0 and cu[-1] == T and np.all(np.diff(cu) >= 0)
    return [(int(cu[i]), int(cu[i + 1])) for i in range(len(cu) - 1)]


def _unit(x):
    """x / ||x|| over the last axis and ||x|| (a zero vector stays zero)."""
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return np.where(n > 0, x / np.where(n > 0, n, 1.0), 0.0), n


def forward_states(q, k, v, g, beta, h0=None, cu_seqlens=None, scale=None):
    """fp64 forward that also returns, per sequence, the state before every token.

    Returns (out [B, T, H, dv], ht [N, H, dk, dv], prev) with prev[n] of shape
    [L_n, H, dk, dv] (the state each token of sequence n starts from)."""
    q, k, v, g, beta = (np.asarray(a, dtype=np.float64) for a in (q, k, v, g, beta))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    if scale is None:
        scale = dk ** -0.5
    qf, kf, vf, gf, bf = (a.reshape((B * T,) + a.shape[2:]) for a in (q, k, v, g, beta))
    qh, _ = _unit(qf)
    kh, _ = _unit(kf)
    seqs = _seqs(B, T, cu_seqlens)
    out = np.zeros((B * T, H, dv))
    ht = np.zeros((len(seqs), H, dk, dv))
    prev = []
    for n, (t0, t1) in enumerate(seqs):
        S = np.zeros((H, dk, dv)) if h0 is None else np.array(h0[n], dtype=np.float64)
        P = np.zeros((t1 - t0, H, dk, dv))
        for t in range(t0, t1):
            P[t - t0] = S
            a = np.exp(gf[t])[:, :, None] * S
            delta = vf[t] - np.einsum("hc,hcj->hj", kh[t], a)
            S = a + bf[t][:, None, None] * kh[t][:, :, None] * delta[:, None, :]
            out[t] = scale * np.einsum("hc,hcj->hj", qh[t], S)
        ht[n] = S
        prev.append(P)
    return out.reshape(B, T, H, dv), ht, prev


def oracle_bwd(q, k, v, g, beta, do, h0=None, cu_seqlens=None, scale=None, dht=None):
    """Gradients of L with dL/dout = do [B, T, H, dv] and dL/dht = dht [N, H, dk, dv]
    (None: 0).  Returns (dq, dk, dv, dg, dbeta, dh0) in fp64, shaped like the inputs
    (dh0 like h0, [N, H, dk, dv])."""
    q, k, v, g, beta, do = (np.asarray(a, dtype=np.float64) for a in (q, k, v, g, beta, do))
    B, T, H, dk = q.shape
    dvd = v.shape[-1]
    if scale is None:
        scale = dk ** -0.5
    _, _, prev = forward_states(q, k, v, g, beta, h0, cu_seqlens, scale)
    flat = lambda a: a.reshape((B * T,) + a.shape[2:])
    qf, kf, vf, gf, bf, dof = (flat(a) for a in (q, k, v, g, beta, do))
    qh, qn = _unit(qf)
    kh, kn = _unit(kf)
    dqh = np.zeros_like(qf)
    dkh = np.zeros_like(kf)
    dvv = np.zeros_like(vf)
    dgg = np.zeros_like(gf)
    dbb = np.zeros_like(bf)
    seqs = _seqs(B, T, cu_seqlens)
    dh0 = np.zeros((len(seqs), H, dk, dvd))
    for n, (t0, t1) in enumerate(seqs):
        G = np.zeros((H, dk, dvd)) if dht is None else np.array(dht[n], dtype=np.float64)
        for t in range(t1 - 1, t0 - 1, -1):
            e = np.exp(gf[t])[:, :, None]
            a = e * prev[n][t - t0]
            delta = vf[t] - np.einsum("hc,hcj->hj", kh[t], a)
            b = bf[t][:, None]
            S = a + b[:, :, None] * kh[t][:, :, None] * delta[:, None, :]
            G = G + scale * qh[t][:, :, None] * dof[t][:, None, :]
            dqh[t] = scale * np.einsum("hcj,hj->hc", S, dof[t])
            u = np.einsum("hc,hcj->hj", kh[t], G)
            dvv[t] = b * u
            dbb[t] = np.sum(u * delta, axis=-1)
            dkh[t] = b * (np.einsum("hcj,hj->hc", G, delta) - np.einsum("hcj,hj->hc", a, u))
            da = G - b[:, :, None] * kh[t][:, :, None] * u[:, None, :]
            dgg[t] = np.sum(a * da, axis=-1)
            G = e * da
        dh0[n] = G
    # through the L2 normalisation: d(x/|x|) = (I - xhat xhat^T) / |x|
    def unnorm(dxh, xh, xn):
        proj = dxh - xh * np.sum(xh * dxh, axis=-1, keepdims=True)
        return np.where(xn > 0, proj / np.where(xn > 0, xn, 1.0), 0.0)
    dq = unnorm(dqh, qh, qn)
    dkk = unnorm(dkh, kh, kn)
    shp = lambda a, ref: a.reshape(ref.shape)
    return shp(dq, q), shp(dkk, k), shp(dvv, v), shp(dgg, g), shp(dbb, beta), dh0
