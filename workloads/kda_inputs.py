"""Seeded input generators for the KDA forward workloads.

The pages measure the forward on fixed-length sequences and varlen batches of
8,192 tokens ("Kernel Design Agents (KDA) optimize Kimi Delta Attention
(KDA)", section "01 - Results") and on real Kimi-Linear prefills that are not
available here; these synthetic inputs stand in for them.  Stress inputs
follow the probes of section "04 - Hardening" (deep decays, saturated gates,
boundary lengths, repeated keys) and the gate depths of section
"03 - Reward hacking".

Every array is returned as numpy: bf16 tensors as float32 arrays whose values
are exactly representable in bf16 (round-to-nearest-even), so that the oracle
(fp64) and the GPU (bf16) receive the very same numbers.
"""
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

BF16_MAX = 3.3895313892515355e38


def round_bf16(x):
    """Round to the nearest bf16 value (ties to even); returns float32."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = x.view(np.uint32)
    r = (u >> 16) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u
    r &= np.uint32(0xFFFF0000)
    return r.view(np.float32)


@dataclass
class KDAInputs:
    q: np.ndarray            # [B, T, H, dk]
    k: np.ndarray            # [B, T, H, dk]
    v: np.ndarray            # [B, T, H, dv]
    g: np.ndarray            # [B, T, H, dk] float32, natural-log gate (<= 0)
    beta: np.ndarray         # [B, T, H]
    h0: Optional[np.ndarray]  # [N, H, dk, dv] float32 or None
    cu_seqlens: Optional[np.ndarray]  # [N + 1] int32 or None
    scale: float
    dtype: str               # "bf16" or "f32": dtype of q, k, v, beta and out
    name: str = ""
    seed: int = 0
    meta: dict = field(default_factory=dict)

    @property
    def shape(self):
        B, T, H, dk = self.q.shape
        return B, T, H, dk, self.v.shape[-1]

    @property
    def num_seqs(self):
        return self.q.shape[0] if self.cu_seqlens is None else len(self.cu_seqlens) - 1

    @property
    def tokens(self):
        return self.q.shape[0] * self.q.shape[1]

    def seq_bounds(self):
        """(start, end) token offsets of each sequence in the flattened [B*T] order."""
        B, T = self.q.shape[:2]
        if self.cu_seqlens is None:
            return [(b * T, (b + 1) * T) for b in range(B)]
        cu = self.cu_seqlens
        return [(int(cu[i]), int(cu[i + 1])) for i in range(len(cu) - 1)]


def _base_qk(rng, shape, heavy=None):
    """z * s with z ~ N(0,1) (or Student-t(3) where heavy) and s ~ LogNormal(0, 0.5) per token."""
    z = rng.standard_normal(shape, dtype=np.float32)
    if heavy is not None and heavy.any():
        t3 = rng.standard_t(3, size=shape).astype(np.float32)
        z = np.where(heavy, t3, z)
    s = np.exp(0.5 * rng.standard_normal(shape[:-1] + (1,), dtype=np.float32))
    return z * s


def _base_gate(rng, shape):
    return (-np.exp(-2.0 + rng.standard_normal(shape, dtype=np.float32))).astype(np.float32)


def _sigmoid(x):
    return (1.0 / (1.0 + np.exp(-x))).astype(np.float32)


def _finish(q, k, v, g, beta, h0, cu, scale, dtype, name, seed, meta=None):
    if dtype == "bf16":
        q, k, v, beta = round_bf16(q), round_bf16(k), round_bf16(v), round_bf16(beta)
    else:
        q, k, v, beta = (np.asarray(a, dtype=np.float32) for a in (q, k, v, beta))
    g = np.ascontiguousarray(g, dtype=np.float32)
    h0 = None if h0 is None else np.ascontiguousarray(h0, dtype=np.float32)
    cu = None if cu is None else np.ascontiguousarray(cu, dtype=np.int32)
    return KDAInputs(np.ascontiguousarray(q), np.ascontiguousarray(k), np.ascontiguousarray(v),
                     g, np.ascontiguousarray(beta), h0, cu, float(scale), dtype, name, seed,
                     meta or {})


def make_inputs(B=1, T=64, H=2, dk=64, dv=64, *, seed=0, dtype="bf16", h0_std=0.1,
                cu_seqlens=None, gate="base", name="custom"):
    """Base generator of the tiny/fixed configs with arbitrary sizes.

    q, k: N(0,1) times a per-token LogNormal(0, 0.5) scale; v ~ N(0,1);
    g = -exp(N(-2, 1)); beta = sigmoid(N(0,1)); h0 ~ N(0, h0_std) or None.
    ``gate`` may be "base", "slow" (-1e-4), "mid" (-1.5), "deep" (-20) or "zero".
    """
    rng = np.random.default_rng(seed)
    q = _base_qk(rng, (B, T, H, dk))
    k = _base_qk(rng, (B, T, H, dk))
    v = rng.standard_normal((B, T, H, dv), dtype=np.float32)
    if gate == "base":
        g = _base_gate(rng, (B, T, H, dk))
    elif gate == "slow":
        g = (-1e-4 * (1 + 0.01 * rng.standard_normal((B, T, H, dk)))).astype(np.float32)
    elif gate == "mid":
        g = (-1.5 * (1 + 0.01 * rng.standard_normal((B, T, H, dk)))).astype(np.float32)
    elif gate == "deep":
        g = (-20.0 * (1 + 0.01 * rng.standard_normal((B, T, H, dk)))).astype(np.float32)
    elif gate == "zero":
        g = np.zeros((B, T, H, dk), dtype=np.float32)
    else:
        raise ValueError(gate)
    beta = _sigmoid(rng.standard_normal((B, T, H), dtype=np.float32))
    N = B if cu_seqlens is None else len(cu_seqlens) - 1
    h0 = None if h0_std is None else (h0_std * rng.standard_normal((N, H, dk, dv))).astype(np.float32)
    return _finish(q, k, v, g, beta, h0, cu_seqlens, dk ** -0.5, dtype, name, seed)


# ---------------------------------------------------------------------------
# The five named workloads (sizes and distributions of the benchmark set)
# ---------------------------------------------------------------------------

def _config0(seed):
    # tiny fixed-length, fp32, h0 = 0 (passed as an explicit zero state)
    x = make_inputs(1, 256, 2, 64, 64, seed=seed, dtype="f32", h0_std=None, name="tiny-fixed")
    x.h0 = np.zeros((1, 2, 64, 64), dtype=np.float32)
    return x


def _config1(seed):
    return make_inputs(1, 8192, 32, 128, 128, seed=seed, dtype="bf16", h0_std=0.1,
                       name="fixed-8192")


def _varlen_uniform_lengths(rng, total=8192, lo=256, hi=2048):
    lens = []
    while True:
        L = int(rng.integers(lo, hi + 1))
        while L % 64 == 0:
            L = int(rng.integers(lo, hi + 1))
        if sum(lens) + L >= total:
            L = total - sum(lens)
            lens.append(L)
            break
        lens.append(L)
    if lens[-1] % 64 == 0:  # keep every length off the 64-token grid
        lens[-1] -= 1
        lens[-2] += 1
    return lens


def _config2(seed):
    rng = np.random.default_rng(seed)
    lens = _varlen_uniform_lengths(rng)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    H, d = 32, 128
    x = make_inputs(1, 8192, H, d, d, seed=seed + 1000, dtype="bf16", h0_std=0.1,
                    cu_seqlens=cu, name="varlen-uniform-8192")
    x.meta["lengths"] = lens
    return x


def _config3(seed):
    rng = np.random.default_rng(seed)
    H, d, total, long_len = 32, 128, 8192, 6000
    short_total = total - long_len
    shorts = []
    while sum(shorts) < short_total:
        L = int(np.clip(round(float(np.exp(np.log(20.0) + rng.standard_normal()))), 1, 100))
        if sum(shorts) + L > short_total:
            L = short_total - sum(shorts)
        shorts.append(L)
    pos = int(rng.integers(0, len(shorts) + 1))
    lens = shorts[:pos] + [long_len] + shorts[pos:]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    N = len(lens)
    heavy_seq = rng.random(N) < 0.5
    heavy_seq[pos] = True
    heavy_tok = np.repeat(heavy_seq, lens)[None, :, None, None]
    q = _base_qk(rng, (1, total, H, d), heavy_tok)
    k = _base_qk(rng, (1, total, H, d), heavy_tok)
    z = rng.standard_normal((1, total, H, d), dtype=np.float32)
    t3 = rng.standard_t(3, size=(1, total, H, d)).astype(np.float32)
    v = np.where(heavy_tok, t3, z)
    g = _base_gate(rng, (1, total, H, d))
    beta = _sigmoid(rng.standard_normal((1, total, H), dtype=np.float32))
    h0 = (0.1 * rng.standard_normal((N, H, d, d))).astype(np.float32)
    x = _finish(q, k, v, g, beta, h0, cu, d ** -0.5, "bf16", "varlen-skewed-8192", seed,
                {"lengths": lens, "long_index": pos})
    return x


def _config4(seed, packed=False):
    rng = np.random.default_rng(seed)
    B, T, H, d = 4, 8192, 32, 128
    q = _base_qk(rng, (B, T, H, d))
    k = _base_qk(rng, (B, T, H, d))
    v = rng.standard_normal((B, T, H, d), dtype=np.float32)
    g = _base_gate(rng, (B, T, H, d))
    jit = lambda: (1 + 0.01 * rng.standard_normal((B, T, 8, d))).astype(np.float32)
    g[:, :, 0:8] = -1e-4 * jit()                 # near-zero decay (long memory)
    g[:, :, 8:16] = -20.0 * jit()                # near-total forgetting
    mix = rng.random((B, 1, 8, d)) < 0.5         # per (sequence, head, channel) choice
    g[:, :, 16:24] = np.where(mix, -1e-4 * jit(), -20.0 * jit())
    beta = _sigmoid(rng.standard_normal((B, T, H), dtype=np.float32))
    u = rng.random((B, T, H))
    beta[u < 0.1] = 0.0
    beta[u > 0.9] = 1.0
    # 1% of tokens carry 1-4 q/k entries near the bf16 maximum magnitude
    for arr in (q, k):
        tok = np.argwhere(rng.random((B, T, H)) < 0.01)
        nent = rng.integers(1, 5, size=len(tok))
        for (b, t, h), m in zip(tok, nent):
            ch = rng.choice(d, size=m, replace=False)
            arr[b, t, h, ch] = (rng.choice([-1.0, 1.0], size=m)
                                * rng.uniform(0.5, 1.0, size=m) * BF16_MAX).astype(np.float32)
    # 2% of (64-token chunk, head) pairs repeat one key for the whole chunk
    nch = T // 64
    rep = np.argwhere(rng.random((B, nch, H)) < 0.02)
    for b, c, h in rep:
        k[b, c * 64:(c + 1) * 64, h] = k[b, c * 64, h]
    h0 = (0.1 * rng.standard_normal((B, H, d, d))).astype(np.float32)
    cu = None
    if packed:
        q, k, v, g, beta = (a.reshape((1, B * T) + a.shape[2:]) for a in (q, k, v, g, beta))
        cu = np.arange(B + 1, dtype=np.int32) * T
    return _finish(q, k, v, g, beta, h0, cu, d ** -0.5, "bf16",
                   "stress-4x8192" + ("-packed" if packed else ""), seed)


CONFIGS = {
    0: ("tiny fixed-length: B=1 T=256 H=2 d=64 fp32", _config0, 0),
    1: ("fixed-length prefill: B=1 T=8192 H=32 d=128 bf16", _config1, 1),
    2: ("varlen uniform lengths, 8192 tokens, H=32 d=128 bf16", _config2, 2),
    3: ("varlen skewed (one 6000-token sequence), 8192 tokens, H=32 d=128 bf16", _config3, 3),
    4: ("stress B=4 T=8192 H=32 d=128 bf16", _config4, 4),
}


def make_config(idx, seed=None, packed=False):
    """Inputs of workload ``idx`` (0-4) with its fixed seed, or with ``seed`` (a salt)."""
    desc, fn, s0 = CONFIGS[idx]
    s = s0 if seed is None else seed
    x = fn(s, packed=packed) if idx == 4 else fn(s)
    x.seed = s
    x.meta.setdefault("description", desc)
    return x
