"""A numerical model of the chunkwise forward with every matrix-core operand rounded to a
chosen 16-bit format (test infrastructure: it reproduces the study behind the choice of fp16
over bf16 operands).

The chunk step is the one "Autoresearch on Kimi Delta Attention", section "KDA in one
minute", points to (matrix products inside a 64-token chunk, the state carried between
chunks): per chunk, with G the in-chunk cumulative log-gate,

    L = strict lower part of (khat e^G)(khat e^-G)^T,   T = (I + diag(beta) L)^-1
    W = T diag(beta)(khat e^G),   U = T diag(beta) V,   Delta = U - W S0
    P = lower part of (qhat e^G)(khat e^-G)^T
    O = scale (qhat e^G S0 + P Delta),   S_n = diag(e^G_n) S0 + (khat e^(G_n - G))^T Delta

Every operand of a product that the kernels run on the matrix cores (the Gram factors, W, U,
qhat e^G, Tinv, the state copy, Delta, (khat e^(G_n-G))^T, P) is rounded to the format; sums
are fp32; the state itself is fp32; the output is rounded to bf16 as the kernels write it.
Gram factors of 16-row blocks a > b are split around the last row r of block b (both factors
e^(G_i - G_r), e^(G_r - G_j) at most 1, as in the kernels); the diagonal 16 x 16 blocks are
formed in fp32.  It is a model of the operand rounding, not of the kernels' blocking.
"""
import numpy as np

from workloads.kda_inputs import round_bf16


def round_to(x, fmt):
    x = np.asarray(x, dtype=np.float32)
    if fmt == "fp16":
        return x.astype(np.float16).astype(np.float32)
    if fmt == "bf16":
        return round_bf16(x)
    if fmt == "fp32":
        return x
    raise ValueError(fmt)


def _mm(a, b, fmt):
    return np.matmul(round_to(a, fmt), round_to(b, fmt), dtype=np.float32)


def _gated_gram(x, y, G, fmt, strict):
    """M_ij = sum_c x_ic y_jc e^(G_ic - G_jc) on (strictly) lower 16 x 16 blocks, factors <= 1."""
    n = x.shape[0]
    M = np.zeros((n, n), dtype=np.float32)
    for a0 in range(0, n, 16):
        a1 = min(a0 + 16, n)
        for b0 in range(0, a0 + 1, 16):
            b1 = min(b0 + 16, n)
            if b0 < a0:
                r = b1 - 1
                M[a0:a1, b0:b1] = _mm(x[a0:a1] * np.exp(G[a0:a1] - G[r]), (y[b0:b1] * np.exp(G[r] - G[b0:b1])).T, fmt)
            else:
                blk = (x[a0:a1].astype(np.float64) * np.exp(G[a0:a1]).astype(np.float64)) @ \
                      (y[b0:b1].astype(np.float64) * np.exp(-G[b0:b1]).astype(np.float64)).T
                M[a0:a1, b0:b1] = np.tril(blk, -1 if strict else 0).astype(np.float32)
    return M


def chunked_forward(q, k, v, g, beta, h0, scale, fmt, chunk=64):
    """q, k, v, g [T, H, d], beta [T, H], h0 [H, d, d] -> (out [T, H, d] bf16 values, ht [H, d, d])."""
    T, H, dk = q.shape
    dv = v.shape[-1]
    out = np.zeros((T, H, dv), dtype=np.float32)
    ht = np.zeros((H, dk, dv), dtype=np.float32)

    def unit(x):
        x = x.astype(np.float64)
        n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
        return (x / np.where(n > 0, n, 1.0)).astype(np.float32)

    for h in range(H):
        S = np.array(h0[h], dtype=np.float32)
        qh, kh = unit(q[:, h]), unit(k[:, h])
        for c0 in range(0, T, chunk):
            c1 = min(c0 + chunk, T)
            n = c1 - c0
            G = np.cumsum(g[c0:c1, h].astype(np.float32), axis=0)
            E, Gn = np.exp(G), G[-1]
            b = beta[c0:c1, h].astype(np.float32)
            Kg, Qg, Kd = kh[c0:c1] * E, qh[c0:c1] * E, kh[c0:c1] * np.exp(Gn - G)
            L = _gated_gram(kh[c0:c1], kh[c0:c1], G, fmt, strict=True)
            Tm = np.linalg.inv(np.eye(n, dtype=np.float32) + b[:, None] * L).astype(np.float32)
            W = _mm(Tm, b[:, None] * Kg, fmt)
            U = _mm(Tm, b[:, None] * v[c0:c1, h], fmt)
            D = U - _mm(W, S, fmt)
            P = _gated_gram(qh[c0:c1], kh[c0:c1], G, fmt, strict=False)
            O = scale * (_mm(Qg, S, fmt) + _mm(P, D, fmt))
            out[c0:c1, h] = round_bf16(O)
            S = np.exp(Gn)[:, None] * S + _mm(Kd.T, D, fmt)
        ht[h] = S
    return out, ht
