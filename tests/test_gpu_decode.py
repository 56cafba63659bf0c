"""GPU parity of the token-by-token entry point (kda_decode) against the fp64 oracle,
through the C ABI.

kda_decode evaluates the recurrence one token at a time in fp32 (the step that
"Autoresearch on Kimi Delta Attention", section "KDA in one minute", describes),
so the final state matches the oracle to fp32 rounding; outputs in bf16 carry
the bf16 rounding of the result.  Gates: the state within STATE_TOL everywhere;
the output within 1e-5 (fp32 io) or TOL (bf16 io, about one bf16 rounding).
"""
import numpy as np
import pytest

from kda_gpu_util import TOL, rel_rmse, run_gpu, run_gpu_decode, run_oracle, to_device
from workloads import make_inputs
from workloads.kda_inputs import BF16_MAX, KDAInputs, round_bf16

pytestmark = pytest.mark.gpu

STATE_TOL = 1e-5
F32_OUT_TOL = 1e-5


def _check(x, label, d=None):
    o, h = run_gpu_decode(x, d)
    ro, rh = run_oracle(x)
    eo, eh = rel_rmse(o, ro), rel_rmse(h, rh)
    print("%s: rel-RMSE out %.3e state %.3e" % (label, eo, eh), flush=True)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(h))
    assert eo <= (F32_OUT_TOL if x.dtype == "f32" else TOL), (label, eo)
    assert eh <= STATE_TOL, (label, eh)
    return o, h, ro, rh


def test_decode_step_batch():
    """One token for each of 64 sequences, 8 heads, d = 128."""
    _check(make_inputs(64, 1, 8, 128, 128, seed=201, dtype="bf16"), "decode B=64 bf16")


@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128), (128, 64), (128, 128)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_head_sizes_and_dtypes(dk, dv, dtype):
    _check(make_inputs(5, 3, 3, dk, dv, seed=dk + 3 * dv, dtype=dtype), "decode T=3 dk=%d dv=%d %s" % (dk, dv, dtype))


def test_decode_null_initial_state():
    x = make_inputs(7, 2, 4, 128, 128, seed=202, dtype="f32", h0_std=None)
    _check(x, "decode h0 NULL")


def test_decode_packed_with_empty_sequences():
    lens = [0, 1, 2, 0, 5, 3, 1]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    x = make_inputs(1, int(cu[-1]), 4, 128, 128, seed=203, dtype="bf16", cu_seqlens=cu)
    o, h, ro, rh = _check(x, "decode packed")
    for n, L in enumerate(lens):
        if L == 0:
            np.testing.assert_array_equal(h[n], x.h0[n])  # an empty sequence returns h0 exactly


def test_decode_steps_in_place_match_one_sequence():
    """Sixteen calls with one token each, the state updated in place (ht = h0), against the
    oracle over the sixteen-token sequence."""
    import torch
    import gated_delta_rule_39_amd.kda as kda
    x = make_inputs(3, 16, 4, 128, 128, seed=204, dtype="bf16")
    d = to_device(x)
    state = d["h0"].clone()
    outs = []
    for t in range(16):
        sl = lambda a: a[:, t:t + 1].contiguous()
        o, h = kda.decode(sl(d["q"]), sl(d["k"]), sl(d["v"]), sl(d["g"]), sl(d["beta"]), state, None, x.scale,
                          ht=state)
        assert h.data_ptr() == state.data_ptr()
        outs.append(o)
    torch.cuda.synchronize()
    o = torch.cat(outs, dim=1).float().cpu().numpy()
    ro, rh = run_oracle(x)
    eo, eh = rel_rmse(o, ro), rel_rmse(state.cpu().numpy(), rh)
    print("16 in-place decode steps: out %.3e state %.3e" % (eo, eh), flush=True)
    assert eo <= TOL and eh <= STATE_TOL


def test_decode_extreme_inputs():
    """q/k entries near the bf16 maximum, zero q/k vectors, beta exactly 0 and 1, and the
    gate regimes from no decay to near-total forgetting, in one batch."""
    rng = np.random.default_rng(205)
    B, T, H, d = 6, 4, 4, 128
    q = rng.standard_normal((B, T, H, d)).astype(np.float32)
    k = rng.standard_normal((B, T, H, d)).astype(np.float32)
    q[0, :, 0, :3] = 0.9 * BF16_MAX
    k[1, :, 1, 5] = -0.7 * BF16_MAX
    q[2, 1] = 0.0
    k[3, 2] = 0.0
    g = np.empty((B, T, H, d), np.float32)
    g[..., 0, :] = 0.0
    g[..., 1, :] = -1e-4
    g[..., 2, :] = -20.0
    g[..., 3, :] = -np.exp(-2.0 + rng.standard_normal((B, T, d)))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))
    beta[::2, 0] = 0.0
    beta[1::2, 1] = 1.0
    x = KDAInputs(round_bf16(q), round_bf16(k), round_bf16(rng.standard_normal((B, T, H, d))),
                  np.ascontiguousarray(g), round_bf16(beta),
                  (0.1 * rng.standard_normal((B, H, d, d))).astype(np.float32), None, d ** -0.5, "bf16", "extreme")
    _check(x, "decode extreme inputs")


def test_decode_agrees_with_the_chunked_forward():
    """Both entry points against the oracle on a 150-token batch (several chunks)."""
    x = make_inputs(2, 150, 4, 128, 128, seed=206, dtype="bf16")
    d = to_device(x)
    o1, h1 = run_gpu(x, d)
    o2, h2 = run_gpu_decode(x, d)
    ro, rh = run_oracle(x)
    print("T=150: fwd out %.3e state %.3e; decode out %.3e state %.3e"
          % (rel_rmse(o1, ro), rel_rmse(h1, rh), rel_rmse(o2, ro), rel_rmse(h2, rh)), flush=True)
    assert rel_rmse(o1, ro) <= TOL and rel_rmse(h1, rh) <= TOL
    assert rel_rmse(o2, ro) <= TOL and rel_rmse(h2, rh) <= STATE_TOL


def test_decode_benchmark_shape():
    """The decode workload the benchmark times: 256 sequences x 1 token, H = 32, d = 128;
    every output and state element against the oracle."""
    _check(make_inputs(256, 1, 32, 128, 128, seed=5, dtype="bf16", name="decode-256x1"), "decode 256x1x32")
