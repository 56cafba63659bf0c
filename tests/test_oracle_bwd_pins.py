"""Pins of the backward oracle (oracle/kda_oracle_bwd.py), CPU only.

Its forward (numpy, fp64) is pinned to the C oracle, which test_oracle_pins.py pins
to closed forms; its gradients are pinned to central finite differences of that
forward, component by component, on small random problems, so that a dropped term,
a wrong sign, a transposed operand or a wrong index in any gradient fails here.
Special cases with a closed form pin it further: with beta = 0 the state only
decays, and a single token from a zero state gives o = scale beta (qhat.khat) v.
"""
import numpy as np
import pytest

from oracle import oracle_fwd
from oracle.kda_oracle_bwd import forward_states, oracle_bwd


def _problem(B, T, H, dk, dv, seed, cu=None, h0=True):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, H, dk)) * np.exp(0.5 * rng.standard_normal((B, T, H, 1)))
    k = rng.standard_normal((B, T, H, dk)) * np.exp(0.5 * rng.standard_normal((B, T, H, 1)))
    v = rng.standard_normal((B, T, H, dv))
    g = -np.exp(-1.0 + 0.5 * rng.standard_normal((B, T, H, dk)))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))
    N = B if cu is None else len(cu) - 1
    h0v = 0.3 * rng.standard_normal((N, H, dk, dv)) if h0 else None
    return q, k, v, g, beta, h0v


def test_numpy_forward_matches_the_c_oracle():
    q, k, v, g, beta, h0 = _problem(2, 37, 3, 8, 6, seed=1)
    o1, h1, _ = forward_states(q, k, v, g, beta, h0, None, 0.3)
    o2, h2 = oracle_fwd(q, k, v, g, beta, h0, None, 0.3)
    np.testing.assert_allclose(o1, o2, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(h1, h2, rtol=1e-10, atol=1e-12)
    cu = np.array([0, 5, 5, 19, 30])
    q, k, v, g, beta, h0 = _problem(1, 30, 2, 8, 4, seed=2, cu=cu)
    o1, h1, _ = forward_states(q, k, v, g, beta, h0, cu, 0.5)
    o2, h2 = oracle_fwd(q, k, v, g, beta, h0, cu, 0.5)
    np.testing.assert_allclose(o1, o2, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(h1, h2, rtol=1e-10, atol=1e-12)


def _loss(args, wo, wh, cu, scale):
    o, h, _ = forward_states(*args, cu, scale)
    return float(np.sum(o * wo) + np.sum(h * wh))


@pytest.mark.parametrize("packed", [False, True])
def test_gradients_match_finite_differences(packed):
    cu = np.array([0, 4, 4, 11]) if packed else None
    B, T = (1, 11) if packed else (2, 6)
    H, dk, dv, scale = 2, 5, 3, 0.4
    args = list(_problem(B, T, H, dk, dv, seed=3, cu=cu))
    rng = np.random.default_rng(4)
    N = B if cu is None else len(cu) - 1
    wo = rng.standard_normal((B, T, H, dv))
    wh = rng.standard_normal((N, H, dk, dv))
    grads = oracle_bwd(*args[:5], wo, args[5], cu, scale, wh)
    eps = 1e-6
    for i, name in enumerate(["q", "k", "v", "g", "beta", "h0"]):
        x = args[i]
        flat = x.reshape(-1)
        idx = rng.choice(flat.size, size=min(flat.size, 25), replace=False)
        num = []
        for j in idx:
            old = flat[j]
            flat[j] = old + eps
            lp = _loss(args, wo, wh, cu, scale)
            flat[j] = old - eps
            lm = _loss(args, wo, wh, cu, scale)
            flat[j] = old
            num.append((lp - lm) / (2 * eps))
        ana = grads[i].reshape(-1)[idx]
        np.testing.assert_allclose(ana, np.array(num), rtol=1e-5, atol=1e-7, err_msg=name)


def test_beta_zero_pure_decay_closed_form():
    """beta = 0: S_t = Diag(exp(G_t)) h0 and o_t = scale qhat_t^T Diag(exp(G_t)) h0, so
    dh0 = sum_t exp(G_t) qhat_t do_t^T scale + exp(G_T) dht, dv = 0, and dbeta = u.delta."""
    q, k, v, g, beta, h0 = _problem(1, 9, 2, 4, 3, seed=5)
    beta[:] = 0.0
    rng = np.random.default_rng(6)
    do = rng.standard_normal((1, 9, 2, 3))
    dht = rng.standard_normal((1, 2, 4, 3))
    dq, dk, dv, dg, dbeta, dh0 = oracle_bwd(q, k, v, g, beta, do, h0, None, 0.7, dht)
    G = np.cumsum(g[0], axis=0)                                   # [T, H, dk]
    qh = q[0] / np.linalg.norm(q[0], axis=-1, keepdims=True)
    ref = 0.7 * np.einsum("thc,thc,thj->hcj", np.exp(G), qh, do[0]) + np.exp(G[-1])[:, :, None] * dht[0]
    np.testing.assert_allclose(dh0[0], ref, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(dv, 0.0)


def test_single_token_from_zero_state():
    """One token, S0 = 0: o = scale beta (qhat.khat) v, ht = beta khat v^T."""
    q, k, v, g, beta, _ = _problem(1, 1, 1, 6, 4, seed=7)
    rng = np.random.default_rng(8)
    do = rng.standard_normal((1, 1, 1, 4))
    dq, dk, dv, dg, dbeta, dh0 = oracle_bwd(q, k, v, g, beta, do, None, None, 0.5, None)
    qh = q[0, 0, 0] / np.linalg.norm(q[0, 0, 0])
    kh = k[0, 0, 0] / np.linalg.norm(k[0, 0, 0])
    b = beta[0, 0, 0]
    np.testing.assert_allclose(dv[0, 0, 0], 0.5 * b * np.dot(qh, kh) * do[0, 0, 0], rtol=1e-12)
    np.testing.assert_allclose(dbeta[0, 0, 0], 0.5 * np.dot(qh, kh) * np.dot(v[0, 0, 0], do[0, 0, 0]), rtol=1e-12)
    np.testing.assert_allclose(dg, 0.0, atol=1e-15)  # the zero state has nothing to decay


def test_zero_vectors_get_zero_gradients():
    q, k, v, g, beta, h0 = _problem(1, 5, 1, 4, 3, seed=9)
    q[0, 2] = 0.0
    k[0, 3] = 0.0
    do = np.random.default_rng(10).standard_normal((1, 5, 1, 3))
    dq, dk, *_ = oracle_bwd(q, k, v, g, beta, do, h0, None, 0.5, None)
    np.testing.assert_array_equal(dq[0, 2], 0.0)
    np.testing.assert_array_equal(dk[0, 3], 0.0)
