"""Parity at the benchmark sizes (B x 8192 tokens, H=32, dk=dv=128) against the
full fp64 oracle, in the launch configuration bench.py times.  Besides the global
relative RMSE, every sequence's own output and final-state error is reported and
must also pass (a per-sequence view catches errors confined to short sequences)."""
import time

import numpy as np
import pytest

from kda_gpu_util import TOL, rel_rmse, run_gpu, run_oracle
from workloads import make_config

pytestmark = pytest.mark.gpu


def _check_workload(idx, packed=False, two_kernel_too=False, monkeypatch=None):
    t0 = time.time()
    x = make_config(idx, packed=packed)
    print("workload %d (%s): generated in %.1fs" % (idx, x.name, time.time() - t0), flush=True)
    o, h = run_gpu(x)
    t1 = time.time()
    ro, rh = run_oracle(x)
    print("  oracle %.1fs" % (time.time() - t1), flush=True)
    if two_kernel_too:
        # the same inputs through the two-kernel path (the default path here is the fused kernel)
        monkeypatch.setenv("KDA_FUSED", "0")
        o2, h2 = run_gpu(x)
        monkeypatch.delenv("KDA_FUSED")
        e2o, e2h = rel_rmse(o2, ro), rel_rmse(h2, rh)
        print("  two-kernel path: rel-RMSE out %.3e state %.3e" % (e2o, e2h), flush=True)
        assert e2o <= TOL and e2h <= TOL
    eo, eh = rel_rmse(o, ro), rel_rmse(h, rh)
    print("  rel-RMSE out %.3e state %.3e; max|err| out %.3e" % (eo, eh, np.max(np.abs(o - ro))), flush=True)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(h))
    assert eo <= TOL and eh <= TOL
    worst = (0.0, 0.0)
    for n, (a, b) in enumerate(x.seq_bounds()):
        of, rf = o.reshape(-1, *o.shape[2:])[a:b], ro.reshape(-1, *ro.shape[2:])[a:b]
        if b > a:
            worst = (max(worst[0], rel_rmse(of, rf)), max(worst[1], rel_rmse(h[n], rh[n])))
    print("  worst per-sequence rel-RMSE out %.3e state %.3e" % worst, flush=True)
    assert worst[0] <= TOL and worst[1] <= TOL


def test_fixed_8192(monkeypatch):
    _check_workload(1, two_kernel_too=True, monkeypatch=monkeypatch)


def test_varlen_uniform_8192():
    _check_workload(2)


def test_varlen_skewed_8192():
    _check_workload(3)


def test_stress_4x8192():
    _check_workload(4)


def test_stress_4x8192_packed():
    """The stress batch as four packed sequences (cu_seqlens = [0, 8192, 16384, 24576, 32768])."""
    _check_workload(4, packed=True)
