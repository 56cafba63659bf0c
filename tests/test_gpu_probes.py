"""GPU probes for the shortcuts the pages describe as rejected, plus resume and salted
inputs, through the C ABI.

"Kernel Design Agents (KDA) optimize Kimi Delta Attention (KDA)", section
"03 - Reward hacking" lists the rejected candidates (a distribution constant in
place of the L2 norm, zeroed initial-state channels, hard-coded packed
boundaries, history truncated to a short window, decays that overflow past 126
bits, an fp16 decay table); section "04 - Hardening" adds fresh seeds, replay,
boundary lengths, saturated gates and repeated keys.  Each probe below has an
expected value that does not come from the GPU: a closed form of the
recurrence, or the fp64 oracle.
"""
import os

import numpy as np
import pytest

from kda_gpu_util import TOL, rel_rmse, run_gpu, run_oracle
from workloads.kda_inputs import KDAInputs, make_inputs, round_bf16

pytestmark = pytest.mark.gpu


def _inputs(q, k, v, g, beta, h0=None, cu=None, scale=0.125, name="probe"):
    f32 = lambda a: np.ascontiguousarray(a, dtype=np.float32)
    return KDAInputs(f32(round_bf16(q)), f32(round_bf16(k)), f32(round_bf16(v)), f32(g),
                     f32(round_bf16(beta)), None if h0 is None else f32(h0),
                     None if cu is None else np.ascontiguousarray(cu, dtype=np.int32),
                     float(scale), "bf16", name)


def _unit(x):
    n = np.linalg.norm(x.astype(np.float64), axis=-1, keepdims=True)
    return np.where(n > 0, x / np.where(n > 0, n, 1.0), 0.0)


def test_needle_survives_long_history():
    """A single write at t = 0 read back after ~3,000 slow-decay tokens with beta = 0 in
    between: o_{T-1} = scale beta_0 sum_c qhat_{T-1,c} exp(sum_{t>=1} g_{t,c}) khat_{0,c} v_0."""
    rng = np.random.default_rng(11)
    B, T, H, dk, dv = 1, 3001, 2, 128, 128
    q = rng.standard_normal((B, T, H, dk)).astype(np.float32)
    k = rng.standard_normal((B, T, H, dk)).astype(np.float32)
    v = rng.standard_normal((B, T, H, dv)).astype(np.float32)
    g = (-1e-4 * (1.0 + 0.01 * rng.standard_normal((B, T, H, dk)))).astype(np.float32)
    beta = np.zeros((B, T, H), np.float32)
    beta[:, 0] = 1.0
    x = _inputs(q, k, v, g, beta, scale=1.0 / np.sqrt(dk))
    o, h = run_gpu(x)
    qh, kh = _unit(x.q[0, -1].astype(np.float64)), _unit(x.k[0, 0].astype(np.float64))
    decay = np.exp(x.g[0, 1:].astype(np.float64).sum(axis=0))  # [H, dk]
    ref = x.scale * np.einsum("hc,hc,hc->h", qh, decay, kh)[:, None] * x.v[0, 0].astype(np.float64)
    err = rel_rmse(o[0, -1], ref)
    print("needle: rel error of the last output %.3e" % err, flush=True)
    assert err <= TOL


def test_beta_zero_reads_decayed_initial_state():
    """beta = 0: the state only decays, o_t = scale (Diag(exp(G_t)) h0)^T qhat_t, with the
    initial state's energy in a random subset of key channels."""
    rng = np.random.default_rng(12)
    B, T, H, dk, dv = 1, 200, 3, 128, 64
    h0 = np.zeros((1, H, dk, dv), np.float32)
    rows = rng.choice(dk, size=37, replace=False)
    h0[0, :, rows] = rng.standard_normal((len(rows), H, dv)).astype(np.float32)
    g = (-np.exp(-3.0 + rng.standard_normal((B, T, H, dk)))).astype(np.float32)
    x = _inputs(rng.standard_normal((B, T, H, dk)), rng.standard_normal((B, T, H, dk)),
                rng.standard_normal((B, T, H, dv)), g, np.zeros((B, T, H)), h0=h0)
    o, h = run_gpu(x)
    G = np.cumsum(x.g[0].astype(np.float64), axis=0)           # [T, H, dk]
    qh = _unit(x.q[0].astype(np.float64))                       # [T, H, dk]
    ref = x.scale * np.einsum("thc,thc,hcv->thv", qh, np.exp(G), h0[0].astype(np.float64))
    ref_h = np.exp(G[-1])[:, :, None] * h0[0]
    eo, eh = rel_rmse(o[0], ref), rel_rmse(h[0], ref_h)
    print("beta = 0: out %.3e state %.3e" % (eo, eh), flush=True)
    assert eo <= TOL and eh <= TOL


def test_repeated_keys_with_full_writes():
    """One key repeated over whole chunks with beta = 1 and no decay: (I + L) is all-ones
    lower triangular, the hardest case for the inverse."""
    rng = np.random.default_rng(13)
    B, T, H, dk, dv = 1, 192, 2, 128, 128
    k = np.repeat(rng.standard_normal((B, 1, H, dk)), T, axis=1)
    k[:, 128:] = rng.standard_normal((B, T - 128, H, dk))  # the third chunk: fresh keys
    x = _inputs(rng.standard_normal((B, T, H, dk)), k, rng.standard_normal((B, T, H, dv)),
                np.zeros((B, T, H, dk)), np.ones((B, T, H)),
                h0=0.1 * rng.standard_normal((1, H, dk, dv)))
    o, h = run_gpu(x)
    ro, rh = run_oracle(x)
    eo, eh = rel_rmse(o, ro), rel_rmse(h, rh)
    print("repeated keys: out %.3e state %.3e" % (eo, eh), flush=True)
    assert eo <= TOL and eh <= TOL


def test_slow_and_deep_channels_in_one_chunk():
    """Per-channel mix of g = -1e-4 and g = -20 inside every chunk (decays far past 126
    bits next to channels that barely forget)."""
    rng = np.random.default_rng(14)
    B, T, H, dk, dv = 1, 320, 2, 128, 128
    deep = rng.random((1, 1, H, dk)) < 0.5
    g = np.where(deep, -20.0, -1e-4) * (1.0 + 0.01 * rng.standard_normal((B, T, H, dk)))
    x = _inputs(rng.standard_normal((B, T, H, dk)), rng.standard_normal((B, T, H, dk)),
                rng.standard_normal((B, T, H, dv)), g, 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H)))),
                h0=0.1 * rng.standard_normal((1, H, dk, dv)))
    o, h = run_gpu(x)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(h))
    ro, rh = run_oracle(x)
    eo, eh = rel_rmse(o, ro), rel_rmse(h, rh)
    print("mixed gates: out %.3e state %.3e" % (eo, eh), flush=True)
    assert eo <= TOL and eh <= TOL


@pytest.mark.parametrize("split", [1000, 1024])
def test_resume_from_final_state(split):
    """Tokens [0, split) then [split, T) with h0 = the first call's final state match the
    one-call run (bitwise equality is not expected: the chunking shifts)."""
    x = make_inputs(1, 2500, 3, 128, 128, seed=15, dtype="bf16")
    o_full, h_full = run_gpu(x)
    a = make_inputs(1, split, 3, 128, 128, seed=15, dtype="bf16")
    for name in ("q", "k", "v", "g", "beta"):
        setattr(a, name, np.ascontiguousarray(getattr(x, name)[:, :split]))
    a.h0 = x.h0
    o1, h1 = run_gpu(a)
    b = make_inputs(1, 2500 - split, 3, 128, 128, seed=15, dtype="bf16")
    for name in ("q", "k", "v", "g", "beta"):
        setattr(b, name, np.ascontiguousarray(getattr(x, name)[:, split:]))
    b.h0 = h1.astype(np.float32)
    o2, h2 = run_gpu(b)
    eo = rel_rmse(np.concatenate([o1, o2], axis=1), o_full)
    eh = rel_rmse(h2, h_full)
    ro, rh = run_oracle(x)
    print("resume at %d: vs one call out %.3e state %.3e; vs oracle out %.3e state %.3e"
          % (split, eo, eh, rel_rmse(np.concatenate([o1, o2], axis=1), ro), rel_rmse(h2, rh)), flush=True)
    assert eo <= TOL and eh <= TOL
    assert rel_rmse(np.concatenate([o1, o2], axis=1), ro) <= TOL and rel_rmse(h2, rh) <= TOL


def test_long_boundary_lengths_packed():
    """Packed lengths around chunk boundaries up to one 8,191-token sequence, with empty
    sequences; each sequence also checked on its own."""
    lens = [8191, 0, 1, 2, 63, 64, 65, 127, 128, 129, 0]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    x = make_inputs(1, int(cu[-1]), 2, 128, 128, seed=16, dtype="bf16", cu_seqlens=cu)
    o, h = run_gpu(x)
    ro, rh = run_oracle(x)
    assert rel_rmse(o, ro) <= TOL and rel_rmse(h, rh) <= TOL
    for n, L in enumerate(lens):
        s, e = cu[n], cu[n + 1]
        if L == 0:
            np.testing.assert_array_equal(h[n], x.h0[n])
        else:
            assert rel_rmse(o[:, s:e], ro[:, s:e]) <= TOL, n
            assert rel_rmse(h[n], rh[n]) <= TOL, n


def test_salted_inputs():
    """A fresh seed on every run (printed, so a failure can be replayed)."""
    seed = int.from_bytes(os.urandom(4), "little")
    print("salt seed %d" % seed, flush=True)
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, 700, size=6)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    x = make_inputs(1, int(cu[-1]), 4, 128, 128, seed=seed, dtype="bf16", cu_seqlens=cu)
    o, h = run_gpu(x)
    ro, rh = run_oracle(x)
    eo, eh = rel_rmse(o, ro), rel_rmse(h, rh)
    print("salted: out %.3e state %.3e" % (eo, eh), flush=True)
    assert eo <= TOL and eh <= TOL
