"""ctypes front end of the fp64 token-by-token KDA oracle in ``kda_oracle.c``.

TEST INFRASTRUCTURE ONLY (see the package docstring).  The recurrence it wraps
is the gated delta rule with per-channel decay, one step per token, in fp64:
"Autoresearch on Kimi Delta Attention", section "KDA in one minute" (the
operator), and "Kernel Design Agents (KDA) optimize Kimi Delta Attention
(KDA)", section "01 - Results" (a token-by-token fp64 recurrence is the
accuracy reference).

Inputs are converted to fp64 exactly (bf16 and fp32 values are representable
in fp64), so the oracle sees the very numbers the GPU receives.
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
_LIB = os.path.join(_HERE, "libkda_oracle.so")
_lib = None


def build_oracle(force=False, out=None, extra_flags=()):
    """Compile kda_oracle.c with gcc (fp64, OpenMP) into libkda_oracle.so (or into `out`, with
    `extra_flags` added: the CPU sanitizer test builds an instrumented copy this way)."""
    target = out or _LIB
    if force or out or not os.path.exists(target) or os.path.getmtime(target) < os.path.getmtime(_SRC):
        tmp = target + ".tmp%d" % os.getpid()
        # -ffp-contract=off keeps each multiply and add separately rounded, as written.
        cmd = ["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC"] + list(extra_flags)
        cmd += ["-o", tmp, _SRC, "-lm"]
        subprocess.check_call(cmd)
        os.replace(tmp, target)
    return target


def _load():
    global _lib
    if _lib is None:
        path = os.environ.get("KDA_ORACLE_LIBRARY")  # another build of kda_oracle.c (sanitizer test)
        if not path:
            path = _LIB
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build_oracle()
        lib = ctypes.CDLL(path)
        p = ctypes.c_void_p
        lib.kda_oracle_fwd.argtypes = [ctypes.c_int64, p, ctypes.c_int64, ctypes.c_int64,
                                       ctypes.c_int64, p, p, p, p, p, p, ctypes.c_double, p, p,
                                       ctypes.c_int]
        lib.kda_oracle_fwd.restype = ctypes.c_int
        lib.kda_oracle_max_threads.argtypes = []
        lib.kda_oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def oracle_threads():
    return int(_load().kda_oracle_max_threads())


def _f64(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def oracle_fwd(q, k, v, g, beta, h0=None, cu_seqlens=None, scale=None, nthreads=0):
    """Run the fp64 recurrence.

    Shapes follow the library: q, k, g ``[B, T, H, dk]``; v ``[B, T, H, dv]``;
    beta ``[B, T, H]``; h0 ``[N, H, dk, dv]`` or None.  With ``cu_seqlens``
    (length N+1 token offsets) B must be 1 and the T tokens are N packed
    sequences; without it each of the B rows is a sequence.  ``scale`` defaults
    to dk**-0.5.  Returns ``(out [B, T, H, dv], ht [N, H, dk, dv])`` in fp64.
    """
    q, k, v, g, beta = _f64(q), _f64(k), _f64(v), _f64(g), _f64(beta)
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    assert k.shape == q.shape and g.shape == q.shape
    assert v.shape == (B, T, H, dv) and beta.shape == (B, T, H)
    if cu_seqlens is None:
        cu = np.arange(B + 1, dtype=np.int64) * T
    else:
        assert B == 1, "packed sequences need B == 1"
        cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int64))
        assert cu[0] == 0 and cu[-1] == T and np.all(np.diff(cu) >= 0)
    N = len(cu) - 1
    if scale is None:
        scale = dk ** -0.5
    h0a = None if h0 is None else _f64(h0)
    if h0a is not None:
        assert h0a.shape == (N, H, dk, dv)
    out = np.zeros((B, T, H, dv), dtype=np.float64)
    ht = np.zeros((N, H, dk, dv), dtype=np.float64)
    rc = _load().kda_oracle_fwd(N, _ptr(cu), H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                _ptr(beta), _ptr(h0a), float(scale), _ptr(out), _ptr(ht),
                                int(nthreads))
    if rc != 0:
        raise RuntimeError("kda_oracle_fwd failed (%d)" % rc)
    return out, ht
