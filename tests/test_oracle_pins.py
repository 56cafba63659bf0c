"""Pins of the fp64 oracle against facts fixed by the pages and by mathematics.

Each test is chosen so that a plausible slip in the oracle (a dropped decay,
decay on the wrong axis or after the write, output read before the update, a
sign error in the correction, a missing normalisation, a misplaced scale, a
transposed state) fails at least one of them.  None of them calls the HIP
path.  The brute-force and mpmath references below build the dk x dk
transition matrices explicitly, a different code path from the oracle's
rank-one updates.
"""
import math
import os

import numpy as np
import pytest

from oracle import oracle_fwd
from workloads import make_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _unit(x):
    n = np.linalg.norm(x, axis=-1, keepdims=True)
    return np.where(n > 0, x / np.where(n > 0, n, 1), 0.0)


def _rand(rng, B, T, H, dk, dv, gscale=0.3):
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    v = rng.standard_normal((B, T, H, dv))
    g = -gscale * rng.random((B, T, H, dk))
    beta = rng.random((B, T, H))
    h0 = rng.standard_normal((B, H, dk, dv))
    return q, k, v, g, beta, h0


def brute_force(q, k, v, g, beta, h0, scale):
    """S_t = M_t S_{t-1} + beta_t khat_t v_t^T with M_t = (I - beta_t khat khat^T) Diag(exp g_t),
    built as explicit dk x dk matrices (one sequence per batch row)."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    out = np.zeros((B, T, H, dv))
    ht = np.zeros((B, H, dk, dv))
    I = np.eye(dk)
    for b in range(B):
        for h in range(H):
            S = np.zeros((dk, dv)) if h0 is None else h0[b, h].copy()
            for t in range(T):
                kh = _unit(k[b, t, h])
                qh = _unit(q[b, t, h])
                M = (I - beta[b, t, h] * np.outer(kh, kh)) @ np.diag(np.exp(g[b, t, h]))
                S = M @ S + beta[b, t, h] * np.outer(kh, v[b, t, h])
                out[b, t, h] = scale * S.T @ qh
            ht[b, h] = S
    return out, ht


def test_brute_force_small():
    rng = np.random.default_rng(11)
    for (B, T, H, dk, dv) in [(1, 1, 1, 4, 4), (2, 8, 2, 5, 3), (1, 7, 3, 8, 6)]:
        q, k, v, g, beta, h0 = _rand(rng, B, T, H, dk, dv)
        o, ht = oracle_fwd(q, k, v, g, beta, h0, scale=0.37)
        ob, hb = brute_force(q, k, v, g, beta, h0, 0.37)
        np.testing.assert_allclose(o, ob, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(ht, hb, rtol=1e-12, atol=1e-12)


def test_mpmath_50_digits():
    mp = pytest.importorskip("mpmath")
    mp.mp.dps = 50
    rng = np.random.default_rng(5)
    T, d = 4, 4
    q, k, v, g, beta, h0 = _rand(rng, 1, T, 1, d, d, gscale=2.0)
    o, ht = oracle_fwd(q, k, v, g, beta, h0, scale=0.5)
    S = mp.matrix([[mp.mpf(float(h0[0, 0, i, j])) for j in range(d)] for i in range(d)])
    for t in range(T):
        kv = [mp.mpf(float(x)) for x in k[0, t, 0]]
        qv = [mp.mpf(float(x)) for x in q[0, t, 0]]
        kn = mp.sqrt(sum(x * x for x in kv))
        qn = mp.sqrt(sum(x * x for x in qv))
        kh = [x / kn for x in kv]
        qh = [x / qn for x in qv]
        b = mp.mpf(float(beta[0, t, 0]))
        M = mp.matrix(d, d)
        for i in range(d):
            for j in range(d):
                M[i, j] = ((1 if i == j else 0) - b * kh[i] * kh[j]) * mp.e ** mp.mpf(float(g[0, t, 0, j]))
        W = mp.matrix(d, d)
        for i in range(d):
            for j in range(d):
                W[i, j] = b * kh[i] * mp.mpf(float(v[0, t, 0, j]))
        S = M * S + W
        for j in range(d):
            ref = mp.mpf("0.5") * sum(S[i, j] * qh[i] for i in range(d))
            assert abs(float(ref) - o[0, t, 0, j]) <= 1e-13 * max(1.0, abs(float(ref)))
    for i in range(d):
        for j in range(d):
            assert abs(float(S[i, j]) - ht[0, 0, i, j]) <= 1e-13 * max(1.0, abs(float(S[i, j])))


def test_beta_zero_is_pure_decay():
    """beta = 0: S_t = Diag(exp(sum_{s<=t} g_s)) h0 and o_t = scale S_t^T qhat_t."""
    rng = np.random.default_rng(1)
    B, T, H, dk, dv = 1, 40, 2, 6, 5  # dk != dv catches a transposed state
    q, k, v, g, beta, h0 = _rand(rng, B, T, H, dk, dv, gscale=0.5)
    beta[:] = 0.0
    o, ht = oracle_fwd(q, k, v, g, beta, h0, scale=1.3)
    G = np.cumsum(g, axis=1)
    for h in range(H):
        for t in range(T):
            S = np.exp(G[0, t, h])[:, None] * h0[0, h]
            np.testing.assert_allclose(o[0, t, h], 1.3 * S.T @ _unit(q[0, t, h]), rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(ht[0, h], np.exp(G[0, -1, h])[:, None] * h0[0, h], rtol=1e-12)


def test_beta_zero_alpha_one_keeps_h0_and_is_linear_in_qhat():
    rng = np.random.default_rng(2)
    q, k, v, g, beta, h0 = _rand(rng, 1, 16, 2, 8, 8)
    beta[:] = 0.0
    g[:] = 0.0
    o, ht = oracle_fwd(q, k, v, g, beta, h0, scale=0.25)
    np.testing.assert_array_equal(ht, h0)
    qh = _unit(q)
    ref = 0.25 * np.einsum("thc,hcj->thj", qh[0], h0[0])
    np.testing.assert_allclose(o[0], ref, rtol=1e-13, atol=1e-14)


def test_single_token_from_zero_state():
    """T = 1, h0 = 0: S = beta khat v^T and o = scale beta (khat . qhat) v."""
    rng = np.random.default_rng(3)
    q, k, v, g, beta, _ = _rand(rng, 1, 1, 3, 7, 4, gscale=3.0)
    o, ht = oracle_fwd(q, k, v, g, beta, None, scale=0.8)
    for h in range(3):
        kh, qh = _unit(k[0, 0, h]), _unit(q[0, 0, h])
        np.testing.assert_allclose(ht[0, h], beta[0, 0, h] * np.outer(kh, v[0, 0, h]), rtol=1e-13)
        np.testing.assert_allclose(o[0, 0, h], 0.8 * beta[0, 0, h] * (kh @ qh) * v[0, 0, h],
                                   rtol=1e-12, atol=1e-15)


def test_single_token_with_state():
    """T = 1: S = (I - beta khat khat^T) Diag(alpha) h0 + beta khat v^T."""
    rng = np.random.default_rng(4)
    q, k, v, g, beta, h0 = _rand(rng, 1, 1, 2, 5, 3, gscale=1.0)
    o, ht = oracle_fwd(q, k, v, g, beta, h0, scale=1.0)
    for h in range(2):
        kh = _unit(k[0, 0, h])
        b = beta[0, 0, h]
        S = (np.eye(5) - b * np.outer(kh, kh)) @ np.diag(np.exp(g[0, 0, h])) @ h0[0, h] + b * np.outer(kh, v[0, 0, h])
        np.testing.assert_allclose(ht[0, h], S, rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(o[0, 0, h], S.T @ _unit(q[0, 0, h]), rtol=1e-12, atol=1e-15)


def test_orthonormal_keys_overwrite_exactly():
    """alpha = 1, beta = 1, orthonormal keys: S_T^T khat_j = v_j for every written key and
    S_T^T x = h0^T x for x orthogonal to all keys (the delta rule replaces, it does not add)."""
    rng = np.random.default_rng(6)
    d, T, dv = 8, 5, 6
    Qm, _ = np.linalg.qr(rng.standard_normal((d, d)))
    keys = Qm[:, :T].T * rng.uniform(0.5, 3.0, size=(T, 1))  # any positive length
    k = keys[None, :, None, :]
    q = rng.standard_normal((1, T, 1, d))
    v = rng.standard_normal((1, T, 1, dv))
    g = np.zeros((1, T, 1, d))
    beta = np.ones((1, T, 1))
    h0 = rng.standard_normal((1, 1, d, dv))
    _, ht = oracle_fwd(q, k, v, g, beta, h0, scale=1.0)
    S = ht[0, 0]
    for j in range(T):
        np.testing.assert_allclose(S.T @ Qm[:, j], v[0, j, 0], rtol=1e-12, atol=1e-12)
    for j in range(T, d):
        np.testing.assert_allclose(S.T @ Qm[:, j], h0[0, 0].T @ Qm[:, j], rtol=1e-12, atol=1e-12)


def test_norm_scale_invariance_is_exact():
    """Per-token rescaling of q and k by powers of two leaves o and ht bitwise unchanged."""
    rng = np.random.default_rng(7)
    q, k, v, g, beta, h0 = _rand(rng, 1, 30, 2, 8, 8)
    o1, h1 = oracle_fwd(q, k, v, g, beta, h0)
    sq = 2.0 ** rng.integers(-20, 21, size=(1, 30, 2, 1))
    sk = 2.0 ** rng.integers(-20, 21, size=(1, 30, 2, 1))
    o2, h2 = oracle_fwd(q * sq, k * sk, v, g, beta, h0)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(h1, h2)


def test_linear_in_v_and_h0_jointly():
    rng = np.random.default_rng(8)
    q, k, v, g, beta, h0 = _rand(rng, 1, 25, 2, 6, 4)
    _, _, v2, _, _, h02 = _rand(rng, 1, 25, 2, 6, 4)
    o1, s1 = oracle_fwd(q, k, v, g, beta, h0)
    o2, s2 = oracle_fwd(q, k, v2, g, beta, h02)
    o3, s3 = oracle_fwd(q, k, 2.0 * v - 0.5 * v2, g, beta, 2.0 * h0 - 0.5 * h02)
    np.testing.assert_allclose(o3, 2.0 * o1 - 0.5 * o2, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(s3, 2.0 * s1 - 0.5 * s2, rtol=1e-11, atol=1e-12)
    o4, _ = oracle_fwd(q, k, v, g, beta, h0, scale=3.0)
    o5, _ = oracle_fwd(q, k, v, g, beta, h0, scale=1.5)
    np.testing.assert_allclose(o4, 2.0 * o5, rtol=1e-14)


def test_head_and_value_column_permutation():
    rng = np.random.default_rng(9)
    q, k, v, g, beta, h0 = _rand(rng, 1, 20, 4, 6, 5)
    o, s = oracle_fwd(q, k, v, g, beta, h0)
    ph = np.array([2, 0, 3, 1])
    pc = np.array([4, 1, 0, 3, 2])
    o2, s2 = oracle_fwd(q[:, :, ph], k[:, :, ph], v[:, :, ph][..., pc], g[:, :, ph], beta[:, :, ph],
                        h0[:, ph][..., pc])
    np.testing.assert_array_equal(o2, o[:, :, ph][..., pc])
    np.testing.assert_array_equal(s2, s[:, ph][..., pc])


def test_varlen_equals_separate_runs_and_empty_sequences():
    rng = np.random.default_rng(10)
    lens = [5, 0, 17, 1, 0, 9]
    T = sum(lens)
    q, k, v, g, beta, _ = _rand(rng, 1, T, 2, 6, 4)
    N = len(lens)
    h0 = rng.standard_normal((N, 2, 6, 4))
    cu = np.concatenate([[0], np.cumsum(lens)])
    o, s = oracle_fwd(q, k, v, g, beta, h0, cu_seqlens=cu)
    for n in range(N):
        a, b = cu[n], cu[n + 1]
        if b == a:
            np.testing.assert_array_equal(s[n], h0[n])
            continue
        on, sn = oracle_fwd(q[:, a:b], k[:, a:b], v[:, a:b], g[:, a:b], beta[:, a:b], h0[n:n + 1])
        np.testing.assert_array_equal(o[:, a:b], on)
        np.testing.assert_array_equal(s[n], sn[0])


def test_continuation_through_final_state():
    """Running [0, T1) and then [T1, T) from ht equals one run (the h0/ht pair resumes)."""
    rng = np.random.default_rng(12)
    q, k, v, g, beta, h0 = _rand(rng, 1, 50, 2, 6, 6)
    o, s = oracle_fwd(q, k, v, g, beta, h0)
    T1 = 23
    oa, sa = oracle_fwd(q[:, :T1], k[:, :T1], v[:, :T1], g[:, :T1], beta[:, :T1], h0)
    ob, sb = oracle_fwd(q[:, T1:], k[:, T1:], v[:, T1:], g[:, T1:], beta[:, T1:], sa)
    np.testing.assert_array_equal(np.concatenate([oa, ob], axis=1), o)
    np.testing.assert_array_equal(sb, s)


def test_needle_long_memory_closed_form():
    """h0 = 0; one write at t = 0; beta = 0 and g ~ -1e-4 after: the write survives the
    whole sequence, o_{T-1} = scale beta_0 sum_c qhat_c exp(sum_{t>=1} g_tc) khat_0c v_0."""
    rng = np.random.default_rng(13)
    T, d = 3000, 16
    q, k, v, g, beta, _ = _rand(rng, 1, T, 1, d, d)
    g[:] = -1e-4 * (1 + 0.01 * rng.standard_normal(g.shape))
    beta[:] = 0.0
    beta[0, 0, 0] = 0.7
    o, s = oracle_fwd(q, k, v, g, beta, None, scale=0.3)
    decay = np.exp(g[0, 1:, 0].sum(axis=0))
    ref = 0.3 * 0.7 * np.sum(_unit(q[0, -1, 0]) * decay * _unit(k[0, 0, 0])) * v[0, 0, 0]
    np.testing.assert_allclose(o[0, -1, 0], ref, rtol=1e-9)


def test_deep_gate_leaves_only_the_last_write():
    rng = np.random.default_rng(14)
    q, k, v, g, beta, h0 = _rand(rng, 1, 12, 2, 8, 8)
    g[:] = -20.0
    _, s = oracle_fwd(q, k, v, g, beta, h0)
    for h in range(2):
        last = beta[0, -1, h] * np.outer(_unit(k[0, -1, h]), v[0, -1, h])
        assert np.linalg.norm(s[0, h] - last) <= 1e-7 * np.linalg.norm(last)


def test_zero_vectors_normalise_to_zero():
    rng = np.random.default_rng(15)
    q, k, v, g, beta, h0 = _rand(rng, 1, 6, 1, 4, 4)
    k[0, 2, 0] = 0.0
    q[0, 4, 0] = 0.0
    o, s = oracle_fwd(q, k, v, g, beta, h0)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(s))
    np.testing.assert_array_equal(o[0, 4, 0], 0.0)
    # a zero key writes nothing: token 2 only decays the state
    o1, s1 = oracle_fwd(q[:, :2], k[:, :2], v[:, :2], g[:, :2], beta[:, :2], h0)
    _, s2 = oracle_fwd(q[:, :3], k[:, :3], v[:, :3], g[:, :3], beta[:, :3], h0)
    np.testing.assert_allclose(s2[0, 0], np.exp(g[0, 2, 0])[:, None] * s1[0, 0], rtol=1e-14)


def test_extreme_bf16_magnitudes_are_normalised():
    """Entries near the bf16 maximum: fp64 norms stay finite and the result is the same as for
    the vector scaled down by a power of two."""
    x = make_inputs(1, 20, 2, 16, 16, seed=3, dtype="bf16")
    q, k = x.q.astype(np.float64), x.k.astype(np.float64)
    q[0, 5, 1, 3] = 3.3e38
    k[0, 7, 0, 0] = -3.3e38
    o1, s1 = oracle_fwd(q, k, x.v, x.g, x.beta, x.h0)
    q2, k2 = q.copy(), k.copy()
    q2[0, 5, 1] *= 2.0 ** -120
    k2[0, 7, 0] *= 2.0 ** -120
    o2, s2 = oracle_fwd(q2, k2, x.v, x.g, x.beta, x.h0)
    assert np.all(np.isfinite(o1))
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(s1, s2)


def test_norm_constant_printed_on_the_page_pins_d128():
    vals = {}
    with open(os.path.join(GOLDEN, "norm_constant.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                key, val = line.split()
                vals[key] = float(val)
    sigma, page_value = vals["sigma"], vals["value"]

    def e_inv_norm(d):
        return math.exp(math.lgamma((d - 1) / 2) - math.lgamma(d / 2)) / (math.sqrt(2) * sigma)

    assert abs(e_inv_norm(int(vals["dim"])) - page_value) < 1e-10
    assert abs(e_inv_norm(64) - page_value) > 1e-2 and abs(e_inv_norm(256) - page_value) > 1e-2
    # Monte Carlo agrees with the closed form (independent check of the formula itself)
    rng = np.random.default_rng(0)
    xs = sigma * rng.standard_normal((200000, 128))
    mc = np.mean(1.0 / np.linalg.norm(xs, axis=1))
    assert abs(mc - page_value) < 2e-4
