"""Python binding of the KDA forward C ABI (include/kda.h).

Argument marshalling only: every step of the forward runs in the HIP library.
PyTorch provides device memory and the current stream.  There is no other
code path: if the library is missing, importing this module fails.
"""
import ctypes
import os
import re

import torch  # loaded first so the library binds to the HIP runtime torch uses

_PKG = os.path.dirname(os.path.abspath(__file__))
# KDA_LIBRARY=path loads another build of this same library (the CPU sanitizer test loads a
# build whose host code carries AddressSanitizer and UndefinedBehaviorSanitizer)
LIB_PATH = os.environ.get("KDA_LIBRARY") or os.path.join(_PKG, "libkda.so")
HEADER = os.path.join(os.path.dirname(_PKG), "include", "kda.h")

if not os.path.exists(LIB_PATH):
    raise ImportError("%s is not built: run __graft_entry__.build() (hipcc, gfx950) first" % LIB_PATH)
_lib = ctypes.CDLL(LIB_PATH)

KDA_BF16, KDA_F32 = 0, 1
STATUS = {0: "KDA_OK", 1: "KDA_ERR_NULL", 2: "KDA_ERR_UNSUPPORTED", 3: "KDA_ERR_BAD_ARG",
          4: "KDA_ERR_ALIGN", 5: "KDA_ERR_WORKSPACE", 6: "KDA_ERR_ALIAS", 7: "KDA_ERR_HIP",
          8: "KDA_ERR_TIMEOUT"}


class Problem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64), ("num_seqs", ctypes.c_int64),
                ("heads", ctypes.c_int32), ("dk", ctypes.c_int32), ("dv", ctypes.c_int32),
                ("dtype", ctypes.c_int32)]


_P = ctypes.c_void_p
_lib.kda_fwd_workspace_size.argtypes = [ctypes.POINTER(Problem)]
_lib.kda_fwd_workspace_size.restype = ctypes.c_size_t
_lib.kda_fwd_validate.argtypes = [ctypes.POINTER(Problem), _P, _P, _P, _P, _P, _P, _P, ctypes.c_float,
                                  _P, _P, _P, ctypes.c_size_t]
_lib.kda_fwd_validate.restype = ctypes.c_int
_lib.kda_fwd.argtypes = [ctypes.POINTER(Problem), _P, _P, _P, _P, _P, _P, _P, ctypes.c_float, _P, _P, _P,
                         ctypes.c_size_t, _P]
_lib.kda_fwd.restype = ctypes.c_int
_lib.kda_fwd_noalloc.argtypes = [ctypes.POINTER(Problem), _P, _P, _P, _P, _P, _P, _P, ctypes.c_float, _P, _P, _P]
_lib.kda_fwd_noalloc.restype = ctypes.c_int
_lib.kda_fwd_status.argtypes = [_P, ctypes.c_size_t, _P]
_lib.kda_fwd_status.restype = ctypes.c_int
_lib.kda_decode.argtypes = [ctypes.POINTER(Problem), _P, _P, _P, _P, _P, _P, _P, ctypes.c_float, _P, _P, _P]
_lib.kda_decode.restype = ctypes.c_int
_lib.kda_bwd_workspace_size.argtypes = [ctypes.POINTER(Problem)]
_lib.kda_bwd_workspace_size.restype = ctypes.c_size_t
_lib.kda_bwd.argtypes = [ctypes.POINTER(Problem)] + [_P] * 7 + [ctypes.c_float] + [_P] * 9 + [ctypes.c_size_t, _P]
_lib.kda_bwd.restype = ctypes.c_int
_lib.kda_status_string.argtypes = [ctypes.c_int]
_lib.kda_status_string.restype = ctypes.c_char_p
_lib.kda_test_fill_lds.argtypes = [ctypes.c_uint32, _P]
_lib.kda_test_fill_lds.restype = ctypes.c_int
_lib.kda_version.argtypes = []
_lib.kda_version.restype = ctypes.c_int


class KDAError(RuntimeError):
    def __init__(self, code):
        self.code = code
        super().__init__(_lib.kda_status_string(code).decode())


def declared_functions():
    """Names of the functions include/kda.h declares."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(kda_\w+)\s*\(", text, re.M)))


def library():
    return _lib


def version():
    return _lib.kda_version()


def test_fill_lds(bits, stream=None):
    """Test hook: fill every compute unit's LDS with the 32-bit pattern `bits` (kda_test_fill_lds)."""
    import torch
    st = stream if stream is not None else torch.cuda.current_stream()
    rc = _lib.kda_test_fill_lds(ctypes.c_uint32(bits & 0xFFFFFFFF), ctypes.c_void_p(st.cuda_stream))
    if rc != 0:
        raise RuntimeError("kda_test_fill_lds: %s" % _lib.kda_status_string(rc).decode())


def make_problem(B, T, H, dk, dv, dtype, num_seqs=0):
    return Problem(int(B), int(T), int(num_seqs), int(H), int(dk), int(dv), int(dtype))


def workspace_size(B, T, H, dk, dv, dtype=KDA_BF16, num_seqs=0):
    return int(_lib.kda_fwd_workspace_size(ctypes.byref(make_problem(B, T, H, dk, dv, dtype, num_seqs))))


def bwd_workspace_size(B, T, H, dk, dv, dtype=KDA_BF16, num_seqs=0):
    return int(_lib.kda_bwd_workspace_size(ctypes.byref(make_problem(B, T, H, dk, dv, dtype, num_seqs))))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dtype_code(dt):
    if dt == torch.bfloat16:
        return KDA_BF16
    if dt == torch.float32:
        return KDA_F32
    raise TypeError("q, k, v and beta must be bfloat16 or float32, got %s" % dt)


def _check(q, k, v, g, beta, h0, cu_seqlens, extra):
    """Shape, dtype and layout checks shared by fwd and decode; returns (B, T, H, dk, dv, N, code)."""
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    code = _dtype_code(q.dtype)
    for name, t_ in (("k", k), ("v", v), ("beta", beta)):
        if t_.dtype != q.dtype:
            raise TypeError("%s must have q's dtype" % name)
    if g.dtype != torch.float32:
        raise TypeError("g must be float32")
    tensors = [q, k, v, g, beta] + [x for x in (h0, cu_seqlens) + tuple(extra) if x is not None]
    for t_ in tensors:
        if not t_.is_cuda or not t_.is_contiguous():
            raise ValueError("all tensors must be contiguous device tensors")
    if k.shape != q.shape or g.shape != q.shape or v.shape != (B, T, H, dv) or beta.shape != (B, T, H):
        raise ValueError("inconsistent shapes")
    if cu_seqlens is not None:
        if cu_seqlens.dtype != torch.int32:
            raise TypeError("cu_seqlens must be int32")
        N = cu_seqlens.numel() - 1
    else:
        N = B
    if h0 is not None and (h0.dtype != torch.float32 or tuple(h0.shape) != (N, H, dk, dv)):
        raise ValueError("h0 must be float32 [N, H, dk, dv]")
    return B, T, H, dk, dv, N, code


def fwd(q, k, v, g, beta, h0=None, cu_seqlens=None, scale=None, *, out=None, ht=None, workspace=None,
        output_final_state=True, stream=None):
    """KDA forward.  Shapes: q, k, g [B, T, H, dk]; v [B, T, H, dv]; beta [B, T, H];
    h0 [N, H, dk, dv] fp32 or None; cu_seqlens int32 [N + 1] (B must be 1) or None.
    Returns (out [B, T, H, dv] in q's dtype, ht [N, H, dk, dv] fp32 or None)."""
    B, T, H, dk, dv, N, code = _check(q, k, v, g, beta, h0, cu_seqlens, (out, ht, workspace))
    if scale is None:
        scale = dk ** -0.5
    prob = make_problem(B, T, H, dk, dv, code, N if cu_seqlens is not None else 0)
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=q.dtype, device=q.device)
    if ht is None and output_final_state:
        ht = torch.empty((N, H, dk, dv), dtype=torch.float32, device=q.device)
    wsb = int(_lib.kda_fwd_workspace_size(ctypes.byref(prob)))
    if workspace is None:
        workspace = torch.empty(max(wsb, 256), dtype=torch.uint8, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    rc = _lib.kda_fwd(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0),
                      _ptr(cu_seqlens), float(scale), _ptr(out), _ptr(ht), _ptr(workspace),
                      workspace.numel() * workspace.element_size(), ctypes.c_void_p(stream))
    if rc != 0:
        raise KDAError(rc)
    return out, ht


def fwd_noalloc(q, k, v, g, beta, h0=None, cu_seqlens=None, scale=None, *, out, ht=None, stream=None):
    """kda_fwd_noalloc: the forward with the library's static device workspace (no allocation in
    the call; problems larger than KDA_NOALLOC_SCRATCH_BYTES raise KDA_ERR_WORKSPACE).  The caller
    passes `out` (and `ht`, or None for no final state)."""
    B, T, H, dk, dv, N, code = _check(q, k, v, g, beta, h0, cu_seqlens, (out, ht))
    if scale is None:
        scale = dk ** -0.5
    prob = make_problem(B, T, H, dk, dv, code, N if cu_seqlens is not None else 0)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    rc = _lib.kda_fwd_noalloc(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0),
                              _ptr(cu_seqlens), float(scale), _ptr(out), _ptr(ht), ctypes.c_void_p(stream))
    if rc != 0:
        raise KDAError(rc)
    return out, ht


def fwd_status(workspace, stream=None):
    """Outcome of the most recent fwd call on `workspace` (kda_fwd_status): returns the status
    code (0 = KDA_OK, 8 = KDA_ERR_TIMEOUT: a wait of the fused kernel gave up and its outputs
    hold NaN).  Synchronises the stream."""
    if stream is None:
        stream = torch.cuda.current_stream(workspace.device).cuda_stream
    return int(_lib.kda_fwd_status(_ptr(workspace), workspace.numel() * workspace.element_size(),
                                   ctypes.c_void_p(stream)))


def decode(q, k, v, g, beta, h0=None, cu_seqlens=None, scale=None, *, out=None, ht=None,
           output_final_state=True, stream=None):
    """The same forward, token by token (kda_decode): for decode steps (T = 1) and short
    continuations.  Arguments and results as for fwd; no workspace.  Pass ht=h0 to update
    the state in place."""
    B, T, H, dk, dv, N, code = _check(q, k, v, g, beta, h0, cu_seqlens, (out, ht))
    if scale is None:
        scale = dk ** -0.5
    prob = make_problem(B, T, H, dk, dv, code, N if cu_seqlens is not None else 0)
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=q.dtype, device=q.device)
    if ht is None and output_final_state:
        ht = torch.empty((N, H, dk, dv), dtype=torch.float32, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    rc = _lib.kda_decode(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0),
                         _ptr(cu_seqlens), float(scale), _ptr(out), _ptr(ht), ctypes.c_void_p(stream))
    if rc != 0:
        raise KDAError(rc)
    return out, ht


def bwd(q, k, v, g, beta, do, h0=None, cu_seqlens=None, scale=None, dht=None, *, workspace=None, stream=None):
    """Gradients of the forward (kda_bwd) for dL/dout = do and dL/dht = dht (None: 0).
    Returns (dq, dk, dv, dg, dbeta, dh0): dq, dk, dv, dbeta in q's dtype, dg and dh0 fp32
    (dh0 is the gradient with respect to the initial state, also when h0 is None)."""
    B, T, H, dk, dv, N, code = _check(q, k, v, g, beta, h0, cu_seqlens, (do, dht, workspace))
    if do.shape != v.shape or do.dtype != q.dtype:
        raise ValueError("do must have v's shape and q's dtype")
    if dht is not None and (dht.dtype != torch.float32 or tuple(dht.shape) != (N, H, dk, dv)):
        raise ValueError("dht must be float32 [N, H, dk, dv]")
    if scale is None:
        scale = dk ** -0.5
    prob = make_problem(B, T, H, dk, dv, code, N if cu_seqlens is not None else 0)
    dq, dkk, dvv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    dg, dbeta = torch.empty_like(g), torch.empty_like(beta)
    dh0 = torch.empty((N, H, dk, dv), dtype=torch.float32, device=q.device)
    wsb = int(_lib.kda_bwd_workspace_size(ctypes.byref(prob)))
    if workspace is None:
        workspace = torch.empty(max(wsb, 256), dtype=torch.uint8, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    rc = _lib.kda_bwd(ctypes.byref(prob), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0),
                      _ptr(cu_seqlens), float(scale), _ptr(do), _ptr(dht), _ptr(dq), _ptr(dkk), _ptr(dvv),
                      _ptr(dg), _ptr(dbeta), _ptr(dh0), _ptr(workspace),
                      workspace.numel() * workspace.element_size(), ctypes.c_void_p(stream))
    if rc != 0:
        raise KDAError(rc)
    return dq, dkk, dvv, dg, dbeta, dh0
