"""Parity at the benchmark sizes (B x 8192 tokens, H=32, dk=dv=128) against the
full fp64 oracle, in the launch configuration bench.py times.  Every bound of
kda_gpu_util.gate applies: relative RMSE over the whole tensor and over every
(sequence, head) on its own, and the element-wise bound on every output and
final-state entry."""
import time

import pytest

from kda_gpu_util import gate, run_gpu, run_oracle
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
        gate(x, o2, h2, ro, rh, "  %s, two-kernel path" % x.name)
    gate(x, o, h, ro, rh, "  %s" % x.name)


def test_fixed_8192(monkeypatch):
    _check_workload(1, two_kernel_too=True, monkeypatch=monkeypatch)


def test_varlen_uniform_8192():
    _check_workload(2)


def test_varlen_skewed_8192():
    _check_workload(3)


def test_stress_4x8192(monkeypatch):
    _check_workload(4, two_kernel_too=True, monkeypatch=monkeypatch)


def test_stress_4x8192_packed():
    """The stress batch as four packed sequences (cu_seqlens = [0, 8192, 16384, 24576, 32768])."""
    _check_workload(4, packed=True)
