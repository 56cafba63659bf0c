"""GPU parity of the backward pass (kda_bwd) against the fp64 backward oracle
(oracle/kda_oracle_bwd.py, pinned to finite differences), through the C ABI.

Gate: relative RMSE against the oracle <= 5e-3 for the gradients written in the
inputs' dtype (dq, dk, dv, dbeta: bf16 rounding of the result itself) and <= 1e-4
for the fp32 ones (dg, dh0; every product of the chunkwise form is fp32 on the matrix
cores).
"""
import numpy as np
import pytest

from kda_gpu_util import TOL, rel_rmse, to_device
from oracle import oracle_bwd
from workloads import make_inputs
from workloads.kda_inputs import round_bf16

pytestmark = pytest.mark.gpu

F32_TOL = 1e-4


def _dout(x, seed, with_dht=True):
    rng = np.random.default_rng(seed)
    do = rng.standard_normal(x.v.shape).astype(np.float32)
    if x.dtype == "bf16":
        do = round_bf16(do)
    N = x.num_seqs
    dht = (0.5 * rng.standard_normal((N,) + x.v.shape[2:3] + (x.q.shape[-1], x.v.shape[-1]))).astype(np.float32) \
        if with_dht else None
    return do, dht


def _check(x, do, dht, label):
    import torch
    import gated_delta_rule_39_amd.kda as kda
    d = to_device(x)
    io = torch.bfloat16 if x.dtype == "bf16" else torch.float32
    t = lambda a, dt: None if a is None else torch.from_numpy(np.ascontiguousarray(a)).cuda().to(dt)
    outs = kda.bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], t(do, io), d["h0"], d["cu_seqlens"], x.scale,
                   t(dht, torch.float32))
    torch.cuda.synchronize()
    got = [o.float().cpu().numpy().astype(np.float64) for o in outs]
    ref = oracle_bwd(x.q, x.k, x.v, x.g, x.beta, do, x.h0, x.cu_seqlens, x.scale, dht)
    names = ["dq", "dk", "dv", "dg", "dbeta", "dh0"]
    errs = {n: rel_rmse(a, b) for n, a, b in zip(names, got, ref)}
    print("%s: %s" % (label, " ".join("%s %.2e" % kv for kv in errs.items())), flush=True)
    for n, a in zip(names, got):
        assert np.all(np.isfinite(a)), n
    io_tol = F32_TOL if x.dtype != "bf16" else TOL
    for n in ["dq", "dk", "dv", "dbeta"]:
        assert errs[n] <= io_tol, (label, n, errs[n])
    for n in ["dg", "dh0"]:
        assert errs[n] <= F32_TOL, (label, n, errs[n])
    return got, ref


def test_bwd_fixed_rows():
    x = make_inputs(2, 150, 3, 128, 128, seed=301, dtype="bf16")
    _check(x, *_dout(x, 302), "bwd fixed B=2 T=150 H=3")


@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128), (128, 64)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_bwd_head_sizes_and_dtypes(dk, dv, dtype):
    x = make_inputs(1, 70, 2, dk, dv, seed=dk + dv + (dtype == "f32"), dtype=dtype)
    _check(x, *_dout(x, 303), "bwd dk=%d dv=%d %s" % (dk, dv, dtype))


def test_bwd_packed_with_empty_sequences_and_no_dht():
    lens = [0, 1, 64, 65, 130, 0, 7]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    x = make_inputs(1, int(cu[-1]), 2, 128, 128, seed=304, dtype="bf16", cu_seqlens=cu)
    do, _ = _dout(x, 305, with_dht=False)
    got, ref = _check(x, do, None, "bwd packed, dht None")
    for n, L in enumerate(lens):
        if L == 0:
            np.testing.assert_array_equal(got[5][n], 0.0)  # ht = h0 and dht = 0: dh0 = 0


def test_bwd_null_h0_and_gate_regimes():
    for gate in ["slow", "deep", "zero"]:
        x = make_inputs(1, 100, 2, 128, 128, seed=306, dtype="f32", gate=gate, h0_std=None)
        _check(x, *_dout(x, 307), "bwd gate=%s h0 None" % gate)


def test_bwd_zero_vectors_and_large_entries():
    x = make_inputs(1, 90, 2, 128, 128, seed=308, dtype="bf16")
    x.q[0, 5] = 0.0
    x.k[0, 9] = 0.0
    x.q[0, 20, 0, :3] = float(round_bf16(np.array([1e30], np.float32))[0])
    x.k[0, 33, 1, 7] = float(round_bf16(np.array([-3e35], np.float32))[0])
    _check(x, *_dout(x, 309), "bwd zero vectors and large entries")


def test_bwd_packed_assorted_lengths_fp32():
    # lengths on both sides of the 8-token checkpoint segments and the 64-token chunks
    lens = [1, 7, 8, 9, 15, 16, 17, 63, 64, 65, 129, 3]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    x = make_inputs(1, int(cu[-1]), 2, 128, 128, seed=310, dtype="f32", cu_seqlens=cu)
    _check(x, *_dout(x, 311), "bwd packed assorted lengths f32")


def test_bwd_long_sequence_fp32():
    # 138 segments of 8 tokens (the last one partial), every value part of dv = 128
    x = make_inputs(1, 1100, 2, 128, 128, seed=312, dtype="f32")
    _check(x, *_dout(x, 313), "bwd T=1100 f32")


def test_bwd_rows_shorter_than_a_segment():
    x = make_inputs(3, 5, 2, 64, 128, seed=314, dtype="bf16")
    _check(x, *_dout(x, 315), "bwd B=3 T=5 dk=64 dv=128")


def test_bwd_deterministic():
    import torch
    import gated_delta_rule_39_amd.kda as kda
    x = make_inputs(1, 300, 4, 128, 128, seed=316, dtype="bf16")
    do, dht = _dout(x, 317)
    d = to_device(x)
    t = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).cuda().to(dt)
    args = (d["q"], d["k"], d["v"], d["g"], d["beta"], t(do, torch.bfloat16), d["h0"], None, x.scale,
            t(dht, torch.float32))
    first = [o.clone() for o in kda.bwd(*args)]
    second = kda.bwd(*args)
    torch.cuda.synchronize()
    for a, b in zip(first, second):
        assert torch.equal(a, b)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_bwd_many_short_rows(dtype):
    # 128 (sequence, head) pairs of one partial chunk each: 1,024 scan workgroups, a multiple
    # of 8 pairs (the slices of a pair on one compute die)
    x = make_inputs(64, 24, 2, 128, 128, seed=318, dtype=dtype)
    _check(x, *_dout(x, 319), "bwd B=64 T=24 H=2 %s" % dtype)


def test_bwd_many_packed_sequences():
    rng = np.random.default_rng(320)
    lens = rng.integers(0, 40, size=80)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    x = make_inputs(1, int(cu[-1]), 4, 128, 64, seed=321, dtype="bf16", cu_seqlens=cu)
    _check(x, *_dout(x, 322), "bwd packed 80 sequences H=4 dv=64")


@pytest.mark.parametrize("gmean", [-4.75, -5.25])
def test_bwd_diagonal_blocks_at_the_factor_limit(gmean):
    # The diagonal 16 x 16 blocks of the gated products run on the matrix cores with factors
    # e^(G - G_mid) when the gate falls by at most 40 nats over either half of the block, and
    # term by term past that.  g = -4.75 per token falls 38 nats over 8 tokens (factors near
    # e^38), g = -5.25 falls 42 (the term-by-term path); both in fp32 against the oracle.
    x = make_inputs(1, 140, 2, 128, 128, seed=324, dtype="f32")
    rng = np.random.default_rng(325)
    x.g[...] = (gmean * (1 + 0.002 * rng.standard_normal(x.g.shape))).astype(np.float32)
    _check(x, *_dout(x, 326), "bwd g=%.1f per token" % gmean)


def test_bwd_full_size_sampled_heads():
    # the fixed 8,192-token batch of 32 heads, in the launch configuration bench.py times;
    # two heads checked against the oracle (each head's backward is independent of the others)
    import torch
    import gated_delta_rule_39_amd.kda as kda
    from workloads import make_config
    x = make_config(1)
    B, T, H, dk, dv = x.shape
    do = round_bf16(np.random.default_rng(323).standard_normal(x.v.shape).astype(np.float32))
    d = to_device(x)
    t = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).cuda().to(dt)
    outs = kda.bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], t(do, torch.bfloat16), d["h0"], None, x.scale)
    torch.cuda.synchronize()
    got = [o.float().cpu().numpy().astype(np.float64) for o in outs]
    for h in (3, 30):
        sl = lambda a: np.ascontiguousarray(a[:, :, h:h + 1])
        ref = oracle_bwd(sl(x.q), sl(x.k), sl(x.v), sl(x.g), sl(x.beta), sl(do), x.h0[:, h:h + 1], None,
                         x.scale, None)
        names = ["dq", "dk", "dv", "dg", "dbeta", "dh0"]
        errs = {}
        for n, a, r in zip(names, got, ref):
            a_h = a[:, h:h + 1] if n == "dh0" else a[:, :, h:h + 1]
            errs[n] = rel_rmse(a_h, r)
        print("bwd full size, head %d: %s" % (h, " ".join("%s %.2e" % kv for kv in errs.items())), flush=True)
        for n in ["dq", "dk", "dv", "dbeta"]:
            assert errs[n] <= TOL, (h, n, errs[n])
        for n in ["dg", "dh0"]:
            assert errs[n] <= F32_TOL, (h, n, errs[n])


def test_bwd_in_a_captured_graph():
    # kda_bwd captured once, replayed with new inputs copied into the captured buffers;
    # every replay bitwise equal to an eager call on the same inputs
    import torch
    import gated_delta_rule_39_amd.kda as kda
    xs = [make_inputs(1, 300, 4, 128, 128, seed=330 + i, dtype="bf16") for i in range(2)]
    dos = [round_bf16(np.random.default_rng(340 + i).standard_normal(xs[0].v.shape).astype(np.float32))
           for i in range(2)]
    t = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).cuda().to(dt)
    bufs = to_device(xs[0])
    bufs["do"] = t(dos[0], torch.bfloat16)
    call = lambda: kda.bwd(bufs["q"], bufs["k"], bufs["v"], bufs["g"], bufs["beta"], bufs["do"], bufs["h0"],
                           None, xs[0].scale)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = call()
    for rep in range(4):
        x, do = xs[rep % 2], dos[rep % 2]
        d = to_device(x)
        for name in ("q", "k", "v", "g", "beta", "h0"):
            bufs[name].copy_(d[name])
        bufs["do"].copy_(t(do, torch.bfloat16))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [o.clone() for o in outs]
        ref = kda.bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], t(do, torch.bfloat16), d["h0"], None, x.scale)
        torch.cuda.synchronize()
        for a, b in zip(got, ref):
            assert torch.equal(a, b), rep
