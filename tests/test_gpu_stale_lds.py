"""Every kernel must read only LDS it wrote in the same launch.

LDS keeps what the previous kernel on a compute unit left there.  With KDA_TEST_LDS_FILL set,
the library fills the whole LDS of every compute unit with a NaN or Inf pattern before each
kernel it launches (kda_test_fill_lds); a read of a word the kernel did not write then shows
as a non-finite output or a parity failure.  Every path: the fused forward, the two-kernel
forward, packed batches on the persistent scan and on the one-workgroup-per-chain scan, the
decode step and the backward (fixed-length and packed).
"""
import numpy as np
import pytest

from kda_gpu_util import gate, run_gpu, run_gpu_decode, run_oracle, to_device
from workloads import make_inputs

pytestmark = pytest.mark.gpu

PATTERNS = {"nan": "0x7fc00000", "inf": "0x7f800000", "neg-inf": "0xff800000"}


def _packed(seed, H=4, d=128):
    lens = [300, 0, 1, 17, 64, 65, 130, 33]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return make_inputs(1, int(cu[-1]), H, d, d, seed=seed, dtype="bf16", cu_seqlens=cu)


@pytest.mark.parametrize("pattern", sorted(PATTERNS))
@pytest.mark.parametrize("path", ["fused", "two-kernel", "packed", "packed-chains"])
def test_forward_reads_no_stale_lds(path, pattern, monkeypatch):
    monkeypatch.setenv("KDA_TEST_LDS_FILL", PATTERNS[pattern])
    if path == "two-kernel":
        monkeypatch.setenv("KDA_FUSED", "0")
    if path == "packed-chains":
        monkeypatch.setenv("KDA_TASK_SCAN", "0")
    x = _packed(31) if path.startswith("packed") else make_inputs(1, 333, 4, 128, 128, seed=32, dtype="bf16")
    o, h = run_gpu(x)
    assert np.isfinite(o).all() and np.isfinite(h).all(), "non-finite output after a %s LDS fill" % pattern
    ro, rh = run_oracle(x)
    gate(x, o, h, ro, rh, "%s after a %s LDS fill" % (path, pattern))


@pytest.mark.parametrize("pattern", sorted(PATTERNS))
def test_decode_reads_no_stale_lds(pattern, monkeypatch):
    monkeypatch.setenv("KDA_TEST_LDS_FILL", PATTERNS[pattern])
    x = make_inputs(8, 1, 4, 128, 128, seed=33, dtype="bf16")
    o, h = run_gpu_decode(x)
    assert np.isfinite(o).all() and np.isfinite(h).all()
    ro, rh = run_oracle(x)
    gate(x, o, h, ro, rh, "decode after a %s LDS fill" % pattern)


@pytest.mark.parametrize("pattern", sorted(PATTERNS))
@pytest.mark.parametrize("packed", [False, True])
def test_backward_reads_no_stale_lds(packed, pattern, monkeypatch):
    import torch
    import gated_delta_rule_39_amd.kda as kda
    from oracle import oracle_bwd
    monkeypatch.setenv("KDA_TEST_LDS_FILL", PATTERNS[pattern])
    x = _packed(34, H=2) if packed else make_inputs(1, 200, 4, 128, 128, seed=35, dtype="bf16")
    d = to_device(x)
    do = np.random.default_rng(36).standard_normal(x.v.shape).astype(np.float32)
    do_d = torch.from_numpy(do).to("cuda").to(torch.bfloat16)
    got = kda.bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], do_d, d["h0"], d["cu_seqlens"], x.scale)
    torch.cuda.synchronize()
    ref = oracle_bwd(x.q, x.k, x.v, x.g, x.beta, do_d.float().cpu().numpy(), x.h0, x.cu_seqlens, x.scale, None)
    for name, a, r in zip(["dq", "dk", "dv", "dg", "dbeta", "dh0"], got, ref):
        a = a.float().cpu().numpy()
        assert np.isfinite(a).all(), "%s non-finite after a %s LDS fill" % (name, pattern)
        err = float(np.linalg.norm(a - r) / np.linalg.norm(r))
        tol = 1e-4 if name in ("dg", "dh0") else 5e-3  # the fp32 gradients, as in test_gpu_bwd.py
        assert err <= tol, "%s rel %.3e after a %s LDS fill" % (name, err, pattern)
