"""The chunkwise backward equations (tests/chunk_bwd_ref.py: the products a chunked backward
kernel would evaluate per 64-token chunk, with a reverse scan carrying dL/dS between chunks)
agree with the token-by-token reverse-mode oracle to fp64 rounding.  CPU only."""
import numpy as np
import pytest

from chunk_bwd_ref import chunked_backward
from oracle import oracle_bwd
from workloads import make_inputs

NAMES = ["dq", "dk", "dv", "dg", "dbeta", "dh0"]


def _rel(a, b):
    return float(np.linalg.norm(np.asarray(a) - np.asarray(b)) / max(np.linalg.norm(b), 1e-300))


def _grads(x, seed, chunk=64):
    rng = np.random.default_rng(seed)
    do = rng.standard_normal(x.v.shape)
    dht = 0.5 * rng.standard_normal((x.num_seqs, x.q.shape[2], x.q.shape[3], x.v.shape[3]))
    ref = oracle_bwd(x.q, x.k, x.v, x.g, x.beta, do, x.h0, x.cu_seqlens, x.scale, dht)
    got = chunked_backward(x.q, x.k, x.v, x.g, x.beta, do, x.h0, x.cu_seqlens, x.scale, dht, chunk=chunk)
    return got, ref


@pytest.mark.parametrize("gate", ["base", "mid", "zero"])
def test_chunked_backward_matches_token_recurrence(gate):
    x = make_inputs(1, 150, 2, 32, 16, seed=401, dtype="f32", gate=gate)
    got, ref = _grads(x, 402)
    for n, a, b in zip(NAMES, got, ref):
        assert _rel(a, b) < 1e-9, (gate, n, _rel(a, b))


def test_chunked_backward_packed_and_chunk_size():
    lens = [1, 63, 64, 65, 0, 130]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    x = make_inputs(1, int(cu[-1]), 2, 16, 16, seed=403, dtype="f32", cu_seqlens=cu)
    for chunk in (64, 16, 1):
        got, ref = _grads(x, 404, chunk=chunk)
        for n, a, b in zip(NAMES, got, ref):
            assert _rel(a, b) < 1e-9, (chunk, n, _rel(a, b))


def test_chunked_backward_catches_a_dropped_term():
    # the same comparison with one term of the derivation removed fails: the identity
    # above is not vacuous
    import chunk_bwd_ref as cb
    x = make_inputs(1, 70, 1, 16, 16, seed=405, dtype="f32")
    orig = cb._gated_back
    try:
        cb._gated_back = lambda dM, a, b, G: (lambda r: (r[0], r[1], 0.0 * r[2]))(orig(dM, a, b, G))
        got, ref = _grads(x, 406)
    finally:
        cb._gated_back = orig
    assert _rel(got[3], ref[3]) > 1e-3  # dg loses the gated products' terms
