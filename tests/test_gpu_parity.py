"""GPU parity of the HIP forward against the fp64 oracle (through the C ABI).

Gates (kda_gpu_util.gate): relative RMSE <= 5e-3 on the output and on the
final state, over the whole tensor and over every (sequence, head) on its own,
and an element-wise bound on every entry.  Sizes here run in seconds on the
oracle yet span several chunks and 16-row tiles, partial last chunks and
packed sequences; every legal dtype and head size goes through each of the
three kernel paths (the fused kernel, the two-kernel path, packed sequences);
the benchmark shapes are in test_gpu_workloads.py.
"""
import numpy as np
import pytest

from kda_gpu_util import TOL, gate, rel_rmse, run_gpu, run_oracle, to_device
from workloads import make_config, make_inputs

pytestmark = pytest.mark.gpu


def _check(x, label, tol=TOL):
    o, h = run_gpu(x)
    ro, rh = run_oracle(x)
    gate(x, o, h, ro, rh, label, tol)
    return o, h, ro, rh


def test_tiny_fixed_fp32_config():
    x = make_config(0)
    _check(x, "tiny fp32 explicit zero h0")
    x.h0 = None
    _check(x, "tiny fp32 NULL h0")


@pytest.mark.parametrize("T", [1, 63, 64, 65, 200])
def test_fixed_bf16_d128_lengths(T):
    x = make_inputs(1, T, 4, 128, 128, seed=100 + T, dtype="bf16")
    _check(x, "fixed bf16 T=%d" % T)


@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128), (128, 64)])
def test_head_sizes(dk, dv):
    x = make_inputs(2, 150, 3, dk, dv, seed=dk + dv, dtype="bf16")
    _check(x, "dk=%d dv=%d" % (dk, dv))


# Every legal (dtype, dk, dv) through each kernel path: fixed-length rows with few chains take
# the fused kernel, KDA_FUSED=0 the chunk kernel + state scan, cu_seqlens the chunk map +
# chunk kernel + state scan ("Kernel Design Agents (KDA) optimize Kimi Delta Attention (KDA)",
# section "04 - Hardening": correct on every legal input).
@pytest.mark.parametrize("path", ["fused", "two-kernel", "packed"])
@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128), (128, 64), (128, 128)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_every_dtype_and_head_size_on_every_path(dtype, dk, dv, path, monkeypatch):
    seed = 17 * dk + 3 * dv + (0 if dtype == "f32" else 1) + {"fused": 0, "two-kernel": 5, "packed": 9}[path]
    if path == "packed":
        lens = [130, 0, 1, 64, 257, 63]
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        x = make_inputs(1, int(cu[-1]), 3, dk, dv, seed=seed, dtype=dtype, cu_seqlens=cu)
    else:
        x = make_inputs(2, 333, 3, dk, dv, seed=seed, dtype=dtype)
    if path == "two-kernel":
        monkeypatch.setenv("KDA_FUSED", "0")
    _check(x, "%s dk=%d dv=%d %s" % (dtype, dk, dv, path))


@pytest.mark.parametrize("packed", [False, True])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_zero_query_and_key_vectors(dtype, packed):
    """Exact zero q or k rows (a zero vector normalises to zero: no read, no write), scattered
    and over a whole chunk of one head, against the oracle."""
    if packed:
        lens = [200, 3, 190]
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        x = make_inputs(1, int(cu[-1]), 4, 128, 128, seed=61, dtype=dtype, cu_seqlens=cu)
    else:
        x = make_inputs(2, 200, 4, 128, 128, seed=62, dtype=dtype)
    rng = np.random.default_rng(63)
    B, T = x.q.shape[:2]
    zq = rng.random((B, T, 4)) < 0.1
    zk = rng.random((B, T, 4)) < 0.1
    x.q[zq] = 0.0
    x.k[zk] = 0.0
    x.k[0, 64:128, 2] = 0.0   # a whole chunk of head 2 writes nothing
    x.q[0, 128:192, 1] = 0.0  # a whole chunk of head 1 reads nothing
    o, h, ro, rh = _check(x, "zero q/k rows, %s, packed=%s" % (dtype, packed))
    np.testing.assert_array_equal(o[0, 128:192, 1], 0.0)  # qhat = 0 gives o = 0 exactly
    assert np.all(ro[0, 128:192, 1] == 0.0)


# slow: every diagonal tile on fp16; mid (about 17 bits of decay per half tile): the
# fp32 diagonal tiles; deep (about 230 bits): the exact variant.
@pytest.mark.parametrize("gate", ["slow", "mid", "deep", "zero"])
def test_gate_regimes(gate):
    x = make_inputs(1, 300, 4, 128, 128, seed=7, dtype="bf16", gate=gate)
    _check(x, "gate=%s" % gate)


def test_packed_boundary_lengths():
    lens = [0, 1, 2, 63, 64, 65, 127, 128, 129, 7, 0]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    x = make_inputs(1, int(cu[-1]), 2, 128, 128, seed=3, dtype="bf16", cu_seqlens=cu)
    o, h, ro, rh = _check(x, "packed boundary lengths")
    for n, L in enumerate(lens):
        if L == 0:
            np.testing.assert_array_equal(h[n], x.h0[n])  # empty sequence: ht = h0


def test_deterministic_and_replay_with_new_contents():
    import torch
    x = make_inputs(1, 333, 4, 128, 128, seed=21, dtype="bf16")
    d = to_device(x)
    o1, h1 = run_gpu(x, d)
    o2, h2 = run_gpu(x, d)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(h1, h2)
    # new contents in the same device buffers, same launch: results follow the new inputs
    y = make_inputs(1, 333, 4, 128, 128, seed=22, dtype="bf16")
    dy = to_device(y)
    for key in ("q", "k", "v", "g", "beta", "h0"):
        d[key].copy_(dy[key])
    o3, h3 = run_gpu(y, d)
    ro, rh = run_oracle(y)
    gate(y, o3, h3, ro, rh, "replay with new contents")


def test_norm_rescale_invariance_is_exact():
    x = make_inputs(1, 130, 2, 128, 128, seed=5, dtype="bf16")
    o1, h1 = run_gpu(x)
    rng = np.random.default_rng(0)
    x.q = (x.q * 2.0 ** rng.integers(-20, 21, size=x.q.shape[:-1] + (1,))).astype(np.float32)
    x.k = (x.k * 2.0 ** rng.integers(-20, 21, size=x.k.shape[:-1] + (1,))).astype(np.float32)
    o2, h2 = run_gpu(x)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(h1, h2)


def test_in_place_state_update():
    import gated_delta_rule_39_amd.kda as kda
    import torch
    x = make_inputs(1, 100, 2, 128, 128, seed=9, dtype="bf16")
    d = to_device(x)
    ref_o, ref_h = run_gpu(x, d)
    st = d["h0"].clone()
    out, ht = kda.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], st, None, x.scale, ht=st)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(st.cpu().numpy(), ref_h)


# The persistent chunk kernel reads the first 64 items of each workgroup from a staged
# table and later ones from the chunk table: a small grid makes every workgroup walk
# hundreds of items, fixed-length and packed.
@pytest.mark.parametrize("packed", [False, True])
def test_long_walks_of_the_chunk_kernel(packed, monkeypatch):
    """Three chunk workgroups (KDA_CHUNK_WGS=3): long persistent walks; fixed-length rows
    take the fused kernel, whose scan workgroups then wait on most records."""
    monkeypatch.setenv("KDA_CHUNK_WGS", "3")
    if packed:
        lens = [700, 1, 64, 1333, 0, 999, 65, 1000]
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        x = make_inputs(1, int(cu[-1]), 6, 64, 64, seed=21, dtype="bf16", cu_seqlens=cu)
    else:
        x = make_inputs(2, 2100, 6, 64, 64, seed=22, dtype="bf16")
    _check(x, "chunk kernel on 3 workgroups, packed=%s" % packed)


@pytest.mark.parametrize("slice_", ["16", "32", "64"])
def test_scan_slice_widths(slice_, monkeypatch):
    monkeypatch.setenv("KDA_SCAN_SLICE", slice_)
    monkeypatch.setenv("KDA_FUSED", "0")  # the slice width belongs to the two-kernel path
    x = make_inputs(1, 333, 3, 128, 128, seed=5, dtype="bf16")
    _check(x, "scan slice %s" % slice_)


@pytest.mark.parametrize("B,T,H,dk,dv", [(1, 1000, 4, 128, 128), (2, 777, 3, 64, 128), (3, 130, 5, 128, 64),
                                         (1, 64, 32, 128, 128)])
def test_fused_and_two_kernel_paths(B, T, H, dk, dv, monkeypatch):
    """Fixed-length rows with few (row, head) chains take the fused kernel (chunk walk and
    scan side by side); KDA_FUSED=0 takes the two kernels.  Both against the oracle, and
    against each other."""
    x = make_inputs(B, T, H, dk, dv, seed=B * 1000 + T + H, dtype="bf16")
    d = to_device(x)
    o1, h1 = run_gpu(x, d)
    monkeypatch.setenv("KDA_FUSED", "0")
    o2, h2 = run_gpu(x, d)
    ro, rh = run_oracle(x)
    print("B=%d T=%d H=%d dk=%d dv=%d: fused out %.3e state %.3e; two-kernel out %.3e state %.3e; "
          "between them out %.3e state %.3e" % (B, T, H, dk, dv, rel_rmse(o1, ro), rel_rmse(h1, rh),
                                                rel_rmse(o2, ro), rel_rmse(h2, rh), rel_rmse(o1, o2),
                                                rel_rmse(h1, h2)), flush=True)
    gate(x, o1, h1, ro, rh, "fused")
    gate(x, o2, h2, ro, rh, "two-kernel")
    assert rel_rmse(o1, o2) <= 1e-3 and rel_rmse(h1, h2) <= 1e-3


def test_fused_back_to_back_calls_read_fresh_records():
    """The fused kernel hands records over through memory with per-call flags: twenty calls
    on one workspace, alternating two sets of input contents, must each reproduce that set's
    result bitwise (a record or flag left over from the previous call would change it)."""
    import torch
    import gated_delta_rule_39_amd.kda as kda
    xa = make_inputs(1, 1500, 8, 128, 128, seed=41, dtype="bf16")
    xb = make_inputs(1, 1500, 8, 128, 128, seed=42, dtype="bf16")
    da, db = to_device(xa), to_device(xb)
    ws = torch.empty(kda.workspace_size(1, 1500, 8, 128, 128), dtype=torch.uint8, device="cuda")
    run = lambda d, x: kda.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], None, x.scale, workspace=ws)
    ref = {}
    for i in range(20):
        x, d = (xa, da) if i % 2 == 0 else (xb, db)
        o, h = run(d, x)
        torch.cuda.synchronize()
        o, h = o.float().cpu().numpy(), h.cpu().numpy()
        if x.seed not in ref:
            ref[x.seed] = (o, h)
            ro, rh = run_oracle(x)
            gate(x, o.astype(np.float64), h.astype(np.float64), ro, rh, "back-to-back seed %d" % x.seed)
        else:
            np.testing.assert_array_equal(o, ref[x.seed][0])
            np.testing.assert_array_equal(h, ref[x.seed][1])


def test_fused_deferred_items_on_long_walks(monkeypatch):
    """Deep gates (every item takes the exact pass, published after the walk) with only three
    chunk workgroups: the chain workgroups wait on records published late."""
    monkeypatch.setenv("KDA_CHUNK_WGS", "3")
    x = make_inputs(1, 700, 4, 128, 128, seed=43, dtype="bf16", gate="deep")
    _check(x, "fused, deep gates, 3 chunk workgroups")


@pytest.mark.parametrize("gate_kind", ["base", "deep"])
def test_fused_scan_workgroups_take_chunk_items(gate_kind, monkeypatch):
    """The fused kernel's scan workgroups walk the first KDA_FUSE_ROUNDS rounds of chunk items
    (redoing their own deferred ones: deep gates) before their chains start.  Three chunk
    workgroups and eight chains: with five rounds the scan workgroups produce most records.
    Which workgroup computes an item must not change a bit of the result."""
    monkeypatch.setenv("KDA_CHUNK_WGS", "3")
    x = make_inputs(1, 1000, 4, 128, 128, seed=44, dtype="bf16", gate=gate_kind)
    d = to_device(x)
    ref = None
    for rounds in ("0", "1", "2", "5"):
        monkeypatch.setenv("KDA_FUSE_ROUNDS", rounds)
        o, h = run_gpu(x, d)
        if ref is None:
            ro, rh = run_oracle(x)
            gate(x, o, h, ro, rh, "fused, %s gates, no shared rounds" % gate_kind)
            ref = (o, h)
        else:
            np.testing.assert_array_equal(o, ref[0])
            np.testing.assert_array_equal(h, ref[1])


def test_fused_forward_in_a_captured_graph():
    # kda_fwd captured once and replayed with new inputs copied into the captured buffers:
    # every replay must match an eager call on the same inputs (a captured fused call derives
    # its flag value from a launch counter in the workspace, advanced before every replay, so
    # no replay can take a flag left by an earlier one)
    import torch
    import gated_delta_rule_39_amd.kda as kda
    xs = [make_inputs(1, 1000, 8, 128, 128, seed=500 + i, dtype="bf16") for i in range(3)]
    bufs = to_device(xs[0])
    ws = torch.empty(1 << 28, dtype=torch.uint8, device="cuda")
    out = torch.empty((1, 1000, 8, 128), dtype=torch.bfloat16, device="cuda")
    ht = torch.empty((1, 8, 128, 128), dtype=torch.float32, device="cuda")
    call = lambda: kda.fwd(bufs["q"], bufs["k"], bufs["v"], bufs["g"], bufs["beta"], bufs["h0"], None,
                           xs[0].scale, out=out, ht=ht, workspace=ws)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for rep in range(6):
        x = xs[rep % 3]
        d = to_device(x)
        for name in ("q", "k", "v", "g", "beta", "h0"):
            bufs[name].copy_(d[name])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got_o, got_h = out.clone(), ht.clone()
        assert kda.fwd_status(ws) == 0, rep
        ref_o, ref_h = kda.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], None, x.scale)
        torch.cuda.synchronize()
        assert torch.equal(got_o, ref_o) and torch.equal(got_h, ref_h), rep
        # an eager call on the captured workspace between replays (its flags carry another value)
        if rep == 2:
            kda.fwd(bufs["q"], bufs["k"], bufs["v"], bufs["g"], bufs["beta"], bufs["h0"], None, x.scale,
                    workspace=ws)
            torch.cuda.synchronize()


def test_fused_wait_that_gives_up_is_reported(monkeypatch):
    """KDA_SPIN_LIMIT=1 with one chunk workgroup: the scan workgroups' bounded waits give up
    long before the chunk factors appear (the failure is forced from the host; every kernel
    still runs to its end).  The outputs those workgroups could not finish are NaN and
    kda_fwd_status reports KDA_ERR_TIMEOUT; the next call on the same workspace, with the
    default limit, is correct and reports KDA_OK."""
    import torch
    import gated_delta_rule_39_amd.kda as kda
    x = make_inputs(1, 2000, 4, 128, 128, seed=71, dtype="bf16")
    d = to_device(x)
    ws = torch.empty(kda.workspace_size(1, 2000, 4, 128, 128), dtype=torch.uint8, device="cuda")
    call = lambda: kda.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], None, x.scale, workspace=ws)
    monkeypatch.setenv("KDA_SPIN_LIMIT", "1")
    monkeypatch.setenv("KDA_CHUNK_WGS", "1")
    out, ht = call()
    torch.cuda.synchronize()  # every workgroup exits
    st = kda.fwd_status(ws)
    print("forced give-up: status %d, NaN in out %d of %d, in ht %d of %d"
          % (st, int(torch.isnan(out.float()).sum()), out.numel(), int(torch.isnan(ht).sum()), ht.numel()),
          flush=True)
    assert st == 8  # KDA_ERR_TIMEOUT
    assert bool(torch.isnan(ht).any()) and bool(torch.isnan(out.float()).any())
    monkeypatch.delenv("KDA_SPIN_LIMIT")
    monkeypatch.delenv("KDA_CHUNK_WGS")
    out, ht = call()
    torch.cuda.synchronize()
    assert kda.fwd_status(ws) == 0
    ro, rh = run_oracle(x)
    gate(x, out.float().cpu().numpy().astype(np.float64), ht.cpu().numpy().astype(np.float64), ro, rh,
         "after a forced give-up, same workspace")


@pytest.mark.parametrize("bad", ["first", "decreasing", "last"])
def test_validate_cu_seqlens_rejects_bad_offsets(bad, monkeypatch):
    """KDA_VALIDATE_CU_SEQLENS=1: kda_fwd copies cu_seqlens to the host and rejects offsets that
    do not start at 0, decrease, or do not end at seqlen, with KDA_ERR_BAD_ARG and before any
    launch (the outputs keep their contents); valid offsets still run."""
    import torch
    import gated_delta_rule_39_amd.kda as kda
    monkeypatch.setenv("KDA_VALIDATE_CU_SEQLENS", "1")
    good = np.array([0, 100, 250, 400], dtype=np.int32)
    x = make_inputs(1, 400, 2, 64, 64, seed=81, dtype="bf16", cu_seqlens=good)
    d = to_device(x)
    wrong = {"first": [5, 100, 250, 400], "decreasing": [0, 300, 250, 400], "last": [0, 100, 250, 399]}[bad]
    cu_bad = torch.tensor(wrong, dtype=torch.int32, device="cuda")
    out = torch.full((1, 400, 2, 64), 7.0, dtype=torch.bfloat16, device="cuda")
    ht = torch.full((3, 2, 64, 64), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(kda.KDAError) as err:
        kda.fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["h0"], cu_bad, x.scale, out=out, ht=ht)
    assert err.value.code == 3  # KDA_ERR_BAD_ARG
    torch.cuda.synchronize()
    assert bool((out.float() == 7.0).all()) and bool((ht == 7.0).all())
    o, h = run_gpu(x, d)  # the valid offsets pass the same check
    ro, rh = run_oracle(x)
    gate(x, o, h, ro, rh, "validated cu_seqlens")


# Packed batches take the persistent state scan: sequences of at least KDA_LONG_CHUNKS
# chunks walk one at a time (on 32-column slices when they are few), shorter ones are
# pipelined (the next task's state, header maxima and first chunk fetched during the
# current one).  Every split of a batch with one long sequence, short ones and empty ones,
# the pipelined walk with one queue (3 workgroups) and with one workgroup per queue, and
# the one-workgroup-per-chain scan.
@pytest.mark.parametrize("env", [{}, {"KDA_LONG_CHUNKS": "1"}, {"KDA_LONG_CHUNKS": "0"},
                                 {"KDA_LONG_CHUNKS": "1024"}, {"KDA_TASK_SCAN": "3"},
                                 {"KDA_TASK_SCAN": "8"}, {"KDA_TASK_SCAN": "13", "KDA_LONG_CHUNKS": "2"},
                                 {"KDA_TASK_SCAN": "0"}, {"KDA_LONG_SLICE": "64"}, {"KDA_LONG_SLICE": "32", "KDA_LONG_CHUNKS": "2"}],
                         ids=["default", "all-long", "no-long", "all-short", "3wg", "8wg", "13wg-long2", "off", "long-wide",
                              "long-narrow"])
def test_persistent_scan_task_classes(env, monkeypatch):
    for k, v in env.items():
        monkeypatch.setenv(k, v)
    rng = np.random.default_rng(77)
    lens = [700, 0, 1, 64, 65, 129] + [int(v) for v in rng.integers(1, 100, size=40)] + [0, 3]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    x = make_inputs(1, int(cu[-1]), 8, 128, 128, seed=79, dtype="bf16", cu_seqlens=cu)
    o, h, ro, rh = _check(x, "persistent scan %s" % env)
    for n, L in enumerate(lens):
        if L == 0:
            np.testing.assert_array_equal(h[n], x.h0[n])  # empty sequence: ht = h0


@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 64), (64, 128)])
def test_persistent_scan_head_sizes(dk, dv):
    """The long class on 32-column slices next to 64-column short tasks, every head size."""
    lens = [900, 5, 70, 1, 33, 200, 0, 64]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    x = make_inputs(1, int(cu[-1]), 5, dk, dv, seed=dk * 3 + dv, dtype="bf16", cu_seqlens=cu)
    _check(x, "persistent scan dk=%d dv=%d" % (dk, dv))


# Chunks of at most 32 tokens (short sequences, short last chunks) share one 64-row pass of the
# chunk kernel two by two in chunk order, across sequence boundaries; with an odd count the
# last one runs alone.  Deep gates send every pass to the exact variant, which redoes each
# chunk of a pair on its own; three chunk workgroups walk many passes each.
@pytest.mark.parametrize("gate_kind", ["base", "mid", "deep"])
@pytest.mark.parametrize("dtype,dk,dv", [("bf16", 128, 128), ("f32", 128, 128), ("bf16", 64, 128),
                                         ("f32", 128, 64)])
def test_paired_short_chunks(dtype, dk, dv, gate_kind, monkeypatch):
    monkeypatch.setenv("KDA_CHUNK_WGS", "3")
    rng = np.random.default_rng(dk + 7 * dv)
    lens = [32, 1, 33, 96, 0, 31, 2, 200] + [int(v) for v in rng.integers(1, 33, size=20)] + [64, 17]
    tails = [L - 64 * ((L - 1) // 64) for L in lens if L > 0]
    n_short = sum(1 for t in tails if t <= 32)
    if n_short % 2 == 0:
        lens.append(5)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    x = make_inputs(1, int(cu[-1]), 3, dk, dv, seed=dk + dv, dtype=dtype, cu_seqlens=cu,
                    gate=gate_kind)
    o, h, ro, rh = _check(x, "paired short chunks %s dk=%d dv=%d gate=%s" % (dtype, dk, dv, gate_kind))
    for n, L in enumerate(lens):
        if L == 0:
            np.testing.assert_array_equal(h[n], x.h0[n])


# A record holds only what its chunk's tokens fill: the row blocks and token halves past a
# chunk's end are neither stored by the chunk kernel nor loaded by the scan (a load of them
# reads zeros).  A workspace whose every byte is 0xFF (NaN in fp16 and fp32) before the call
# shows that nothing reads a part that was never written: partial last chunks on the fused
# path, the two-kernel path and in packed batches, where pairs of short chunks share a pass.
@pytest.mark.parametrize("path", ["fused", "two-kernel", "packed"])
def test_unwritten_record_parts_are_never_read(path, monkeypatch):
    import torch
    import gated_delta_rule_39_amd.kda as kda
    if path == "packed":
        lens = [1, 17, 33, 48, 64, 100, 5, 130, 16, 32, 0, 2]
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        x = make_inputs(1, int(cu[-1]), 3, 128, 128, seed=97, dtype="bf16", cu_seqlens=cu)
    else:
        x = make_inputs(2, 177, 3, 128, 128, seed=98, dtype="bf16")  # last chunk: 49 tokens
    if path == "two-kernel":
        monkeypatch.setenv("KDA_FUSED", "0")
    B, T, H, dk, dv = x.shape
    n = 0 if x.cu_seqlens is None else x.num_seqs
    wsb = kda.workspace_size(B, T, H, dk, dv, kda.KDA_BF16, n)
    ws = torch.full((wsb,), 255, dtype=torch.uint8, device="cuda:0")
    o, h = run_gpu(x, workspace=ws)
    ro, rh = run_oracle(x)
    gate(x, o, h, ro, rh, "NaN-filled workspace, %s" % path)
