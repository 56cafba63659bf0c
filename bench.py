"""Benchmark of the MI355X KDA forward (one GPU).

A step is one kda_fwd over the 8,192-token fixed-length prefill
(B=1, T=8192, H=32, dk=dv=128, bf16 q/k/v/beta, fp32 gates and state, h0 given),
with its inputs resident in HBM before the timed region starts.  Prints ONE
JSON line on stdout; everything else goes to stderr.

The run fails closed: after timing, the output and final state of the timed
inputs are checked against the fp64 oracle, and then new input contents are
written into the same buffers and checked again; a failed check reports no
speed.  The oracle run on the whole batch is also the CPU baseline.

Per-kernel durations come from HIP events that kda_fwd_timed records between
the library's kernels on the stream they run on, in a second pass over the same
steps (the headline timing has no events between the kernels).

Beside the headline workload the line also carries the two 8,192-token varlen
batches (uniform and skewed lengths), timed the same way (W untimed calls, then K
timed calls) and checked against the oracle, and the geomean of the three.  Their inputs
are drawn and uploaded before any timing and their legs run right after the
headline one's, with their oracle checks afterwards: the GPU then runs all timed
legs without idling while the host draws inputs or runs the oracle (an idle GPU
drops its clock, and W = 5 calls do not bring it back).  The line further carries
the headline workload with cold caches, a decode step (kda_decode) over 256
sequences with its HBM roofline, the backward pass, and the serial bound of the
state pass (the chain-latency bound: the longest chain's chunks times the step
latency of a lone chain); --no-extra skips these, for profiling runs.

The roofline of the fused kernel counts the method minimum as its algorithmic
bytes (every input read once, the output written once, h0 and ht once); the
bytes the design itself moves (its per-chunk records written and read back) are
reported beside them as design_bytes.  traffic, mfma_util_pct and valu_busy_pct
come from the committed rocprofv3 counter summary (profiles/traffic.json) while
it matches the kernel sources.
"""
import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16/bf16 MFMA, published (no sparsity)
MFMA_F32_PEAK_TFLOPS = 157.3  # MI355X dense fp32 matrix (v_mfma_f32_*), published
TOL = 5e-3


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# algorithmic work of one forward (per chunk-head / per token-head figures)
# ---------------------------------------------------------------------------

def record_bytes(dk, dv):
    """Bytes of the per-(chunk, head) record the chunk walk hands to the scan: W, Qhat*exp(G),
    (Khat*exp(G_last-G))^T (fp16, 64 x dk each), the masked attention (fp16 64 x 64), U (fp16
    64 x dv), {exp(G_last), row exponent} per key channel and a 16-byte header."""
    return 64 * dk * 2 * 3 + 64 * 64 * 2 + 64 * dv * 2 + dk * 8 + 16


def algorithmic_work(x, n_chunks):
    """Bytes and MFMA flops each kernel must move / do, counting every tensor once
    (triangular products as triangles).  n_chunks = number of (sequence) chunks."""
    B, T, H, dk, dv = x.shape
    toks = B * T
    N = x.num_seqs
    es = 2 if x.dtype == "bf16" else 4
    C = 64
    ch = n_chunks * H
    rec = record_bytes(dk, dv)
    prep_bytes = toks * H * ((2 * dk + dv) * es + dk * 4 + es) + ch * rec
    state_io = N * H * dk * dv * 4 * (1 + (x.h0 is not None))
    scan_bytes = ch * (rec - 16) + toks * H * dv * es + state_io
    tri_incl = C * (C + 1) // 2
    tri_strict = C * (C - 1) // 2
    prep_flops = ch * 2 * (tri_strict * dk + tri_incl * dk + tri_incl * dk + tri_incl * dv)
    scan_flops = ch * 2 * (C * dk * dv * 3 + tri_incl * dv)
    return dict(prep_bytes=prep_bytes, scan_bytes=scan_bytes, prep_flops=prep_flops, scan_flops=scan_flops)


def method_min_bytes(x):
    """The fused minimum: every input read once, the output written once, the initial state read
    and the final state written once (1,538 bytes per token and head at dk = dv = 128 with bf16
    q, k, v, beta and out, fp32 g)."""
    B, T, H, dk, dv = x.shape
    es = 2 if x.dtype == "bf16" else 4
    per_tok_head = (2 * dk + dv) * es + dk * 4 + es + dv * es
    state = x.num_seqs * H * dk * dv * 4 * ((x.h0 is not None) + 1)
    return B * T * H * per_tok_head + state


def n_chunks_of(x):
    return sum((e - s + 63) // 64 for s, e in x.seq_bounds())


# ---------------------------------------------------------------------------
# HIP events through the runtime torch already loaded
# ---------------------------------------------------------------------------

def hip_runtime():
    path = None
    with open("/proc/self/maps") as f:
        for line in f:
            if "libamdhip64.so" in line:
                path = line.split()[-1]
                break
    if path is None:
        raise RuntimeError("libamdhip64 is not loaded")
    hip = ctypes.CDLL(path)
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    return hip


def counters_from_profiles(kernel):
    """The committed counter summary of `kernel` (HBM bytes per launch, MFMA and VALU busy), if
    it was taken on the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
    except ValueError:
        return None
    k = rec.get("kernels", {}).get(kernel)
    if k is None or k.get("source_sha256") != kernel_source_hash(kernel):
        return None
    return k


def traffic_from_profiles(kernel):
    k = counters_from_profiles(kernel)
    return None if k is None else k.get("hbm_bytes_per_launch")


KERNEL_SOURCES = {"chunk_prep_kernel": ["kda_device.h", "kda_prep.h"],
                  "state_scan_kernel": ["kda_device.h", "kda_scan.h"],
                  "fused_fwd_kernel": ["kda_device.h", "kda_prep.h", "kda_scan.h", "kda_fused.h"]}


def takes_fused_path(x, torch):
    """The library's choice (csrc/kda_api.cpp): fixed-length rows whose (row, head, 64-column
    slice) chains fit in a quarter of the compute units run as one fused kernel."""
    if x.cu_seqlens is not None or os.environ.get("KDA_FUSED", "1")[:1] == "0":
        return False
    B, T, H, dk, dv = x.shape
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    return T > 0 and B * H * (dv // 64) * 4 <= cus


def kernel_source_hash(kernel):
    """sha256 over the source files that define `kernel` (counters go stale when they change)."""
    h = hashlib.sha256()
    d = os.path.join(ROOT, "gated_delta_rule_39_amd", "csrc")
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(d, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def prepare_varlen_legs(lib, kda, make_config, upload, dev, torch):
    """Inputs, outputs and workspaces of the other two 8,192-token workloads (uniform and
    skewed varlen batches), made and uploaded before any timing, so that the GPU runs the
    timed legs back to back instead of idling while the host draws the next inputs."""
    legs = []
    for idx in (2, 3):
        y = make_config(idx)
        B, T, H, dk, dv = y.shape
        io = torch.bfloat16 if y.dtype == "bf16" else torch.float32
        d = upload(y)
        N = y.num_seqs
        o = torch.empty((B, T, H, dv), dtype=io, device=dev)
        h = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
        prob = kda.make_problem(B, T, H, dk, dv, kda.KDA_BF16 if io == torch.bfloat16 else kda.KDA_F32,
                                N if d["cu"] is not None else 0)
        wsb = int(lib.kda_fwd_workspace_size(ctypes.byref(prob)))
        ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
        P = lambda t_: None if t_ is None else ctypes.c_void_p(t_.data_ptr())
        argv = [ctypes.byref(prob), P(d["q"]), P(d["k"]), P(d["v"]), P(d["g"]), P(d["beta"]), P(d["h0"]),
                P(d["cu"]), ctypes.c_float(y.scale), P(o), P(h), P(ws), ctypes.c_size_t(wsb),
                ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)]
        legs.append({"y": y, "d": d, "o": o, "h": h, "ws": ws, "prob": prob, "argv": argv})
    return legs


def time_varlen_legs(legs, lib, W, K, torch):
    """Each varlen leg as the headline one: W untimed calls, then K timed calls."""
    for leg in legs:
        argv = leg["argv"]
        for _ in range(W):
            if lib.kda_fwd(*argv):
                raise RuntimeError("kda_fwd failed")
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(K):
            lib.kda_fwd(*argv)
        e1.record()
        torch.cuda.synchronize()
        leg["ms"] = e0.elapsed_time(e1) / K


def extra_measurements(args, lib, kda, legs, upload, dev, torch, argv1, out1, ht1, x1):
    """The varlen legs' parity against the oracle (their outputs are those of the last timed
    call), their geomean with the headline workload, and the headline workload with cold
    caches (a 512 MiB buffer written before every call, outside the timed call)."""
    from oracle import oracle_fwd
    rel = lambda a, b: float(np.linalg.norm(a.astype(np.float64) - b) / np.linalg.norm(b))
    res = {"ok": True}
    per = {}
    for leg in legs:
        y, o, h, ms = leg["y"], leg["o"], leg["h"], leg["ms"]
        B, T = y.shape[0], y.shape[1]
        ro, rh = oracle_fwd(y.q, y.k, y.v, y.g, y.beta, y.h0, y.cu_seqlens, y.scale)
        eo, eh = rel(o.float().cpu().numpy(), ro), rel(h.cpu().numpy(), rh)
        good = eo <= TOL and eh <= TOL
        res["ok"] = res["ok"] and good
        per[y.name] = {"tokens_per_s": round(B * T / (ms * 1e-3), 1) if good else None,
                       "ms_per_step": round(ms, 5), "sequences": int(y.num_seqs),
                       "out_rel_rmse": eo, "state_rel_rmse": eh}
        log("workload %s: %.4f ms/step, parity out %.2e state %.2e" % (y.name, ms, eo, eh))
    res["workloads"] = per
    legs.clear()  # their buffers are no longer needed

    # headline workload with cold caches
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    times = []
    for _ in range(10):
        flush.fill_(1)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        lib.kda_fwd(*argv1)
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    del flush
    B1, T1 = x1.shape[0], x1.shape[1]
    cold_ms = float(np.median(times))
    res["cold"] = {"ms_per_call": round(cold_ms, 5), "tokens_per_s": round(B1 * T1 / (cold_ms * 1e-3), 1),
                   "calls": len(times), "note": "512 MiB written before every call, outside its timing"}
    res["decode"] = decode_measurement(args, lib, kda, upload, dev, torch)
    res["ok"] = res["ok"] and res["decode"]["ok"]
    res["backward"] = backward_measurement(kda, dev, torch)
    res["ok"] = res["ok"] and res["backward"]["ok"]
    return res


def chain_latency(kda, dev, torch, x, kernel_ms, reps=20):
    """The serial bound of the state pass: the longest chain's chunks times the latency of one
    chunk step of a lone chain (one head of the same sequence length, 64-column slices, the
    two-kernel path, so that nothing else shares the GPU): the step the fused kernel's scan
    workgroups repeat, without the chunk walk running beside it."""
    import ctypes as ct
    B, T, H, dk, dv = x.shape
    y_q = torch.zeros((1, T, 1, dk), dtype=torch.bfloat16, device=dev).normal_()
    y_k = torch.zeros_like(y_q).normal_()
    y_v = torch.zeros((1, T, 1, dv), dtype=torch.bfloat16, device=dev).normal_()
    y_g = -torch.rand((1, T, 1, dk), dtype=torch.float32, device=dev) * 0.2
    y_b = torch.full((1, T, 1), 0.5, dtype=torch.bfloat16, device=dev)
    saved = {k_: os.environ.get(k_) for k_ in ("KDA_FUSED", "KDA_SCAN_SLICE")}
    os.environ["KDA_FUSED"], os.environ["KDA_SCAN_SLICE"] = "0", "64"
    try:
        hip = hip_runtime()
        lib = kda.library()
        prob = kda.make_problem(1, T, 1, dk, dv, kda.KDA_BF16, 0)
        wsb = int(lib.kda_fwd_workspace_size(ct.byref(prob)))
        ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
        out = torch.empty_like(y_v)
        P = lambda t_: ct.c_void_p(t_.data_ptr())
        argv = [ct.byref(prob), P(y_q), P(y_k), P(y_v), P(y_g), P(y_b), None, None, ct.c_float(dk ** -0.5),
                P(out), None, P(ws), ct.c_size_t(wsb), ct.c_void_p(torch.cuda.current_stream(dev).cuda_stream)]
        for _ in range(5):
            lib.kda_fwd(*argv)
        rows = []
        for _ in range(reps):
            row = (ct.c_void_p * 4)()
            for j in range(4):
                e = ct.c_void_p()
                hip.hipEventCreate(ct.byref(e))
                row[j] = e
            lib.kda_fwd_timed(*argv, ct.cast(row, ct.c_void_p))
            rows.append(row)
        torch.cuda.synchronize()

        def el(a, b):
            f = ct.c_float()
            hip.hipEventElapsedTime(ct.byref(f), a, b)
            return f.value
        scan_ms = float(np.median([el(r[2], r[3]) for r in rows]))
        for r in rows:
            for j in range(4):
                hip.hipEventDestroy(r[j])
    finally:
        for k_, v_ in saved.items():
            if v_ is None:
                os.environ.pop(k_, None)
            else:
                os.environ[k_] = v_
    steps = (T + 63) // 64
    step_us = 1e3 * scan_ms / steps
    return {"steps": steps, "step_us": round(step_us, 4), "bound_us": round(step_us * steps, 2),
            "kernel_us": round(1e3 * float(kernel_ms), 2), "frac": round(step_us * steps / (1e3 * float(kernel_ms)), 4),
            "note": "step latency of one 64-column chain measured alone (state scan of a 1-head problem, "
                    "the whole scan kernel divided by its chunks)"}


def bwd_chunk_flops(dk, dv):
    """Matrix-core flops (2 m n k per product) of the chunkwise backward per 64-token chunk and
    head, product by product; a lower-triangular 64 x 64 operand counts its 10 formed 16 x 16
    blocks (10/16 of the square).  Factors: the gated Grams L and P (64 x 64 over dk), the
    off-diagonal blocks of T = (I + diag(beta) L)^-1 (16 block products), W = T X and U = T Y.
    Forward scan: W S0 and Kd^T D.  Reverse scan: Kd Hn, W^T dD, Qg^T dO and P^T dO.
    Gradients: dQg = dO S0^T, dW = dD S0^T, dKd = D Hn^T, dP = dO D^T, dX = T^T dW,
    dY = T^T dD, dA = dX W^T + dY U^T, and the four products of the gated backward (two per
    Gram)."""
    tri = 10.0 / 16.0
    mm = lambda m, n, k: 2.0 * m * n * k
    factors = 2 * tri * mm(64, 64, dk) + 16 * mm(16, 16, 16) + tri * (mm(64, dk, 64) + mm(64, dv, 64))
    fwd = mm(64, dv, dk) + mm(dk, dv, 64)
    rev = 3 * mm(64, dv, dk) + tri * mm(64, dv, 64)
    grad_a = 3 * mm(64, dk, dv) + tri * (mm(64, 64, dv) + mm(64, dk, 64) + mm(64, dv, 64) + mm(64, 64, dk + dv))
    grad_b = 4 * tri * mm(64, dk, 64)
    return factors + fwd + rev + grad_a + grad_b


def backward_measurement(kda, dev, torch, calls=3):
    """kda_bwd on the headline workload (B=1, T=8192, H=32, d=128, bf16), timed over a few
    calls, with its parity checked on a small problem against the fp64 backward oracle (the
    oracle keeps every state, too large at full size)."""
    from oracle import oracle_bwd
    from workloads import make_config, make_inputs
    rel = lambda a, b: float(np.linalg.norm(a.astype(np.float64) - b) / np.linalg.norm(b))
    t = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(dt)
    # parity on a small problem
    y = make_inputs(1, 200, 4, 128, 128, seed=11, dtype="bf16")
    do = np.random.default_rng(12).standard_normal(y.v.shape).astype(np.float32)
    do_d = t(do, torch.bfloat16)
    do = do_d.float().cpu().numpy()
    got = kda.bwd(t(y.q, torch.bfloat16), t(y.k, torch.bfloat16), t(y.v, torch.bfloat16), t(y.g, torch.float32),
                  t(y.beta, torch.bfloat16), do_d, t(y.h0, torch.float32), None, y.scale)
    torch.cuda.synchronize()
    ref = oracle_bwd(y.q, y.k, y.v, y.g, y.beta, do, y.h0, None, y.scale, None)
    errs = {n: rel(a.float().cpu().numpy(), r) for n, a, r in zip(["dq", "dk", "dv", "dg", "dbeta", "dh0"], got, ref)}
    good = all(e <= TOL for e in errs.values())
    # timing on the headline workload
    x = make_config(1)
    B, T, H, dk, dv = x.shape
    args_ = [t(x.q, torch.bfloat16), t(x.k, torch.bfloat16), t(x.v, torch.bfloat16), t(x.g, torch.float32),
             t(x.beta, torch.bfloat16), t(np.random.default_rng(13).standard_normal(x.v.shape), torch.bfloat16),
             t(x.h0, torch.float32), None, x.scale]
    kda.bwd(*args_)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(calls):
        kda.bwd(*args_)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / calls
    # the two packed 8,192-token batches
    varlen = {}
    for i in (2, 3):
        y2 = make_config(i)
        cu = torch.from_numpy(np.ascontiguousarray(y2.cu_seqlens)).to(dev)
        a2 = [t(y2.q, torch.bfloat16), t(y2.k, torch.bfloat16), t(y2.v, torch.bfloat16), t(y2.g, torch.float32),
              t(y2.beta, torch.bfloat16), t(np.random.default_rng(14).standard_normal(y2.v.shape), torch.bfloat16),
              t(y2.h0, torch.float32), cu, y2.scale]
        kda.bwd(*a2)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(calls):
            kda.bwd(*a2)
        e1.record()
        torch.cuda.synchronize()
        ms2 = e0.elapsed_time(e1) / calls
        varlen[y2.name] = {"ms_per_call": round(ms2, 3), "tokens_per_s": round(y2.shape[1] / (ms2 * 1e-3), 1),
                           "sequences": int(y2.num_seqs), "longest": int(np.max(np.diff(y2.cu_seqlens)))}
    # bytes every call must move: inputs (q, k, v bf16, g fp32, beta, dout) and gradients once, h0 and dh0
    # reads q, k, v, dout (bf16), g (fp32), beta; writes dq, dk, dv (bf16), dg (fp32), dbeta
    nbytes = B * T * H * (16 * dk + 6 * dv + 4) + 2 * H * dk * dv * 4
    chunks = B * ((T + 63) // 64)
    flops = bwd_chunk_flops(dk, dv) * chunks * H
    tflops = flops / (ms * 1e-3) / 1e12
    ws = kda.bwd_workspace_size(B, T, H, dk, dv)
    log("backward %s: %.3f ms/call, parity (B=1 T=200 H=4) %s" % (x.name, ms, errs))
    return {"ok": good, "workload": "backward of %s (B=1 T=8192 H=32 d=128 bf16)" % x.name,
            "ms_per_call": round(ms, 3), "tokens_per_s": round(B * T / (ms * 1e-3), 1) if good else None,
            "workspace_bytes": int(ws),
            "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_F32_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tflops / MFMA_F32_PEAK_TFLOPS, 4),
                         "peak_note": "dense fp32 matrix cores (every product is v_mfma_f32_16x16x4f32)",
                         "flops_per_call": int(flops), "bytes_per_call": int(nbytes),
                         "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 5),
                         "note": "chunkwise (64-token chunks): factors, one kernel walking both state "
                                 "scans, two gradient kernels; flops are the products of the chunkwise "
                                 "form (%.1f M per chunk and head)" % (bwd_chunk_flops(dk, dv) / 1e6)},
            "parity_small": errs, "varlen": varlen}


def decode_measurement(args, lib, kda, upload, dev, torch, B=256, verify=True):
    """One decode step (kda_decode, one token per sequence) of B sequences at H=32, d=128:
    timed like the forward, checked against the oracle, with its HBM roofline (the fp32
    state is read once and written once per call)."""
    from oracle import oracle_fwd
    from workloads import make_inputs
    rel = lambda a, b: float(np.linalg.norm(a.astype(np.float64) - b) / np.linalg.norm(b))
    y = make_inputs(B, 1, 32, 128, 128, seed=5, dtype="bf16", name="decode-%dx1" % B)
    Bd, T, H, dk, dv = y.shape
    d = upload(y)
    o = torch.empty((Bd, T, H, dv), dtype=torch.bfloat16, device=dev)
    h = torch.empty((Bd, H, dk, dv), dtype=torch.float32, device=dev)
    prob = kda.make_problem(Bd, T, H, dk, dv, kda.KDA_BF16, 0)
    P = lambda t_: None if t_ is None else ctypes.c_void_p(t_.data_ptr())
    argv = [ctypes.byref(prob), P(d["q"]), P(d["k"]), P(d["v"]), P(d["g"]), P(d["beta"]), P(d["h0"]), None,
            ctypes.c_float(y.scale), P(o), P(h), ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)]
    for _ in range(args.warmup):
        rc = lib.kda_decode(*argv)
        if rc:
            raise kda.KDAError(rc)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        lib.kda_decode(*argv)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    eo = eh = None
    good = False
    if verify:
        ro, rh = oracle_fwd(y.q, y.k, y.v, y.g, y.beta, y.h0, None, y.scale)
        eo, eh = rel(o.float().cpu().numpy(), ro), rel(h.cpu().numpy(), rh)
        good = eo <= TOL and eh <= TOL
    nbytes = Bd * H * (2 * dk * dv * 4 + 2 * dk * 2 + dk * 4 + dv * 2 + 2 + dv * 2)
    gbs = nbytes / (ms * 1e-3) / 1e9
    log("decode %s: %.4f ms/call, %.0f GB/s, parity out %s state %s" % (y.name, ms, gbs, eo, eh))
    return {"ok": good, "workload": "decode step: %d sequences x 1 token, H=32, dk=dv=128, bf16 io, fp32 state "
                                    "in and out" % Bd,
            "ms_per_step": round(ms, 5), "tokens_per_s": round(Bd * T / (ms * 1e-3), 1) if good else None,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK_GBS, 4), "bytes_per_call": int(nbytes)},
            "out_rel_rmse": eo, "state_rel_rmse": eh}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # the GPU's clock settles within a few tens of milliseconds of sustained work: with 5
    # warm-up steps the timed steps ran about 9 % slower than with 50 or more
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", type=int, default=1, help="benchmark workload index (1 = fixed 8192)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-verify", action="store_true", help="skip parity (then no speed is reported)")
    ap.add_argument("--copy-calibration", type=int, default=0,
                    help="run only a plain device copy of this many MiB (counter calibration)")
    ap.add_argument("--backward", action="store_true",
                    help="time only the backward pass (kda_bwd) of the headline workload; prints its own line")
    ap.add_argument("--decode", action="store_true",
                    help="time only the decode step (kda_decode, 256 sequences x 1 token); prints its own line")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the varlen workloads and the cold-cache timing (profiling runs)")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (use --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        log("no GPU visible")
        sys.exit(1)
    dev = torch.device("cuda:0")

    if args.copy_calibration:
        n = args.copy_calibration << 20
        a = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        log("copy calibration: %d bytes read + %d bytes written per copy, 5 copies" % (n, n))
        return

    import gated_delta_rule_39_amd.kda as kda
    from workloads import make_config

    if args.backward:
        r = backward_measurement(kda, dev, torch, calls=max(1, min(args.steps, 5)))
        ok = r.pop("ok")
        line = {"metric": "KDA backward tokens/s (dq, dk, dv, dg, dbeta, dh0)",
                "value": r["tokens_per_s"] if ok else None, "unit": "tokens/s", "n_gpus": 1,
                "steps": max(1, min(args.steps, 5)), "warmup": 1, "ms_per_step": r["ms_per_call"],
                "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
                "data": "synthetic", "config": {"workload": r["workload"]}, "roofline": r["roofline"],
                "parity_small": r["parity_small"], "varlen": r["varlen"]}
        print(json.dumps(line), flush=True)
        if not ok:
            sys.exit(1)
        return

    if args.decode:
        def upload_bf16(y):
            t = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(dt)
            return dict(q=t(y.q, torch.bfloat16), k=t(y.k, torch.bfloat16), v=t(y.v, torch.bfloat16),
                        g=t(y.g, torch.float32), beta=t(y.beta, torch.bfloat16),
                        h0=None if y.h0 is None else t(y.h0, torch.float32), cu=None)
        r = decode_measurement(args, kda.library(), kda, upload_bf16, dev, torch, verify=not args.no_verify)
        ok = r.pop("ok")
        line = {"metric": "KDA decode step tokens/s (one token per sequence)",
                "value": r["tokens_per_s"] if ok else None, "unit": "tokens/s", "n_gpus": 1,
                "steps": args.steps, "warmup": args.warmup, "ms_per_step": r["ms_per_step"],
                "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
                "data": "synthetic", "config": {"workload": r["workload"]}, "roofline": r["roofline"],
                "parity": {"out_rel_rmse": r["out_rel_rmse"], "state_rel_rmse": r["state_rel_rmse"]}}
        print(json.dumps(line), flush=True)
        if not ok and not args.no_verify:
            sys.exit(1)
        return

    t0 = time.time()
    x = make_config(args.workload)
    log("workload %s (%s) generated in %.1fs" % (x.name, x.meta.get("description"), time.time() - t0))
    B, T, H, dk, dv = x.shape
    io = torch.bfloat16 if x.dtype == "bf16" else torch.float32

    def upload(y):
        t = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(dt)
        return dict(q=t(y.q, io), k=t(y.k, io), v=t(y.v, io), g=t(y.g, torch.float32), beta=t(y.beta, io),
                    h0=None if y.h0 is None else t(y.h0, torch.float32),
                    cu=None if y.cu_seqlens is None else t(y.cu_seqlens, torch.int32))

    d = upload(x)
    N = x.num_seqs
    out = torch.empty((B, T, H, dv), dtype=io, device=dev)
    ht = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    prob = kda.make_problem(B, T, H, dk, dv, kda.KDA_BF16 if io == torch.bfloat16 else kda.KDA_F32,
                            N if d["cu"] is not None else 0)
    lib = kda.library()
    wsb = int(lib.kda_fwd_workspace_size(ctypes.byref(prob)))
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    P = lambda t_: None if t_ is None else ctypes.c_void_p(t_.data_ptr())
    argv = [ctypes.byref(prob), P(d["q"]), P(d["k"]), P(d["v"]), P(d["g"]), P(d["beta"]), P(d["h0"]),
            P(d["cu"]), ctypes.c_float(x.scale), P(out), P(ht), P(ws), ctypes.c_size_t(wsb),
            ctypes.c_void_p(stream)]
    lib.kda_fwd_timed.argtypes = list(lib.kda_fwd.argtypes) + [ctypes.c_void_p]
    lib.kda_fwd_timed.restype = ctypes.c_int

    # the other workloads' inputs, ready before any timing (their legs run right after this one)
    legs = []
    if not args.no_extra and not args.no_verify:
        t0 = time.time()
        legs = prepare_varlen_legs(lib, kda, make_config, upload, dev, torch)
        log("varlen workloads generated and uploaded in %.1fs" % (time.time() - t0))

    hip = hip_runtime()
    K, W = args.steps, args.warmup
    marks = []
    for _ in range(K):
        row = (ctypes.c_void_p * 4)()
        for j in range(4):
            e = ctypes.c_void_p()
            if hip.hipEventCreate(ctypes.byref(e)) != 0:
                raise RuntimeError("hipEventCreate failed")
            row[j] = e
        marks.append(row)

    for _ in range(W):
        rc = lib.kda_fwd(*argv)
        if rc:
            raise kda.KDAError(rc)
    torch.cuda.synchronize()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t_start = time.perf_counter()
    ev0.record()
    for i in range(K):
        rc = lib.kda_fwd(*argv)
        if rc:
            raise kda.KDAError(rc)
    ev1.record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_start
    ms_total = ev0.elapsed_time(ev1)
    ms_per_step = ms_total / K
    # per-kernel durations: the same K steps again with events between the kernels (the
    # events themselves add a few microseconds per step, so they stay out of the timing above)
    for i in range(K):
        rc = lib.kda_fwd_timed(*argv, ctypes.cast(marks[i], ctypes.c_void_p))
        if rc:
            raise kda.KDAError(rc)
    torch.cuda.synchronize()
    # the varlen legs right after this one, with no host work in between (their parity is
    # checked afterwards, from the outputs of their last timed call)
    if legs:
        time_varlen_legs(legs, lib, W, K, torch)

    def elapsed(a, b):
        f = ctypes.c_float()
        hip.hipEventElapsedTime(ctypes.byref(f), a, b)
        return f.value

    per_call = np.array([elapsed(m[0], m[3]) for m in marks])
    k_map = np.mean([elapsed(m[0], m[1]) for m in marks])
    k_prep = np.mean([elapsed(m[1], m[2]) for m in marks])
    k_scan = np.mean([elapsed(m[2], m[3]) for m in marks])
    for m in marks:
        for j in range(4):
            hip.hipEventDestroy(m[j])
    fused = takes_fused_path(x, torch)
    if fused:
        log("timed %d steps: %.4f ms/step (wall %.4f ms/step); kernels: fused forward %.4f ms"
            % (K, ms_per_step, 1e3 * t_wall / K, k_prep))
    else:
        log("timed %d steps: %.4f ms/step (wall %.4f ms/step); kernels: chunk map %.4f ms, chunk %.4f ms, "
            "scan %.4f ms" % (K, ms_per_step, 1e3 * t_wall / K, k_map, k_prep, k_scan))

    tokens = B * T
    value = tokens / (ms_per_step * 1e-3)

    # ---- fail-closed parity: timed inputs, then new contents in the same buffers ----
    parity = {}
    cpu_baseline = None
    ok = True
    if not args.no_verify:
        from oracle import oracle_fwd, oracle_threads
        import oracle.kda_oracle as okm
        o_gpu = out.float().cpu().numpy()
        h_gpu = ht.cpu().numpy()
        t1 = time.perf_counter()
        ro, rh = oracle_fwd(x.q, x.k, x.v, x.g, x.beta, x.h0, x.cu_seqlens, x.scale)
        t_or = time.perf_counter() - t1
        rel = lambda a, b: float(np.linalg.norm(a.astype(np.float64) - b) / np.linalg.norm(b))
        parity["out_rel_rmse"] = rel(o_gpu, ro)
        parity["state_rel_rmse"] = rel(h_gpu, rh)
        reps, t_sum = 1, t_or
        while not args.no_cpu_baseline and t_sum < 10.0 and reps < 100:  # about 10 s of CPU work
            t1 = time.perf_counter()
            oracle_fwd(x.q, x.k, x.v, x.g, x.beta, x.h0, x.cu_seqlens, x.scale)
            t_sum += time.perf_counter() - t1
            reps += 1
        cpu_baseline = {"value": round(tokens * reps / t_sum, 1), "unit": "tokens/s",
                        "cores": okm.oracle_threads(), "kind": "oracle",
                        "sample": "the whole timed batch (%d tokens x %d heads), fp64 token-by-token, "
                                  "%d runs in %.1f s" % (tokens, H, reps, t_sum)}
        del ro, rh
        # replay: new contents in the same buffers, same call; check 4 heads against the oracle
        y = make_config(args.workload, seed=1000 + args.workload)
        # the same sequence boundaries (a varlen draw with another seed has other lengths)
        y.cu_seqlens = x.cu_seqlens
        if x.h0 is not None and (y.h0 is None or y.h0.shape != x.h0.shape):
            y.h0 = np.ascontiguousarray(-x.h0[::-1])
        dy = upload(y)
        for key in ("q", "k", "v", "g", "beta", "h0"):
            if d[key] is not None:
                d[key].copy_(dy[key])
        rc = lib.kda_fwd(*argv)
        torch.cuda.synchronize()
        hs = slice(0, 4)
        ys = lambda a: np.ascontiguousarray(a[:, :, hs]) if a.ndim >= 3 else a
        ro2, rh2 = oracle_fwd(ys(y.q), ys(y.k), ys(y.v), ys(y.g), np.ascontiguousarray(y.beta[:, :, hs]),
                              None if y.h0 is None else np.ascontiguousarray(y.h0[:, hs]),
                              y.cu_seqlens, y.scale)
        parity["replay_out_rel_rmse"] = rel(out.float().cpu().numpy()[:, :, hs], ro2)
        parity["replay_state_rel_rmse"] = rel(ht.cpu().numpy()[:, hs], rh2)
        ok = all(v_ <= TOL for v_ in parity.values()) and rc == 0
        log("parity: " + json.dumps(parity))
        if args.no_cpu_baseline:
            cpu_baseline = None

    extra = {}
    if not args.no_extra and not args.no_verify:
        extra = extra_measurements(args, lib, kda, legs, upload, dev, torch, argv, out, ht, x)
        ok = ok and extra.pop("ok")

    nch = n_chunks_of(x)
    wk = algorithmic_work(x, nch)
    mm_bytes = method_min_bytes(x)
    if fused:
        # one kernel does the whole forward: its algorithmic bytes are the method minimum
        # (inputs and output once, h0 and ht once); the record round trip is the design's own
        dom_bytes, dom_ms, kname = mm_bytes, k_prep, "fused_fwd_kernel"
        design_bytes = wk["prep_bytes"] + wk["scan_bytes"]
    else:
        # the split path: the dominant kernel's own reads and writes (its record traffic included)
        dominant = "chunk" if k_prep >= k_scan else "scan"
        dom_bytes = wk["prep_bytes"] if dominant == "chunk" else wk["scan_bytes"]
        dom_ms = k_prep if dominant == "chunk" else k_scan
        kname = "chunk_prep_kernel" if dominant == "chunk" else "state_scan_kernel"
        design_bytes = dom_bytes
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9
    counters = counters_from_profiles(kname) or {}
    traffic = counters.get("hbm_bytes_per_launch")
    total_flops = wk["prep_flops"] + wk["scan_flops"]
    chain = chain_latency(kda, dev, torch, x, dom_ms) if fused and not args.no_extra else None
    res = {
        "metric": "KDA fwd tokens/s @ H=32,d=128, 8192-token fixed+varlen; % bf16 MFMA peak",
        "value": round(value, 1) if ok and not args.no_verify else None,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16xf32",
        "data": "synthetic",
        "config": {"workload": x.name, "global_batch": B, "seq_len": T, "heads": H, "dk": dk, "dv": dv,
                   "io_dtype": x.dtype, "parallelism": "single-gpu",
                   "value_is": "tokens/s of this workload alone; the geomean over the three 8,192-token "
                               "workloads (fixed, varlen uniform, varlen skewed) is "
                               "geomean_fixed_varlen_tokens_per_s"},
        "roofline": {"bound": "hbm", "kernel": kname, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "algorithmic_bytes": int(dom_bytes),
                     "algorithmic_basis": ("method minimum: q, k, v, g, beta read once, out written once, "
                                           "h0 read and ht written once (1,538 B per token and head at "
                                           "d = 128, bf16)") if fused else
                                          "the kernel's own reads and writes, its chunk records included",
                     "kernel_ms": round(float(dom_ms), 5),
                     "design_bytes": int(design_bytes),
                     "design_frac": round(design_bytes / (dom_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "mfma_util_pct": counters.get("MfmaUtil"), "valu_busy_pct": counters.get("VALUBusy"),
                     "counters_note": "traffic, mfma_util_pct and valu_busy_pct from profiles/traffic.json "
                                      "(rocprofv3 counters of the same kernel sources), null when stale"},
        "chain_latency": chain,
        "kernels_ms": ({"chunk_map": round(float(k_map), 5), "fused_fwd": round(float(k_prep), 5)} if fused else
                       {"chunk_map": round(float(k_map), 5), "chunk_prep": round(float(k_prep), 5),
                        "state_scan": round(float(k_scan), 5)}),
        "mfma": {"flops_per_step": total_flops,
                 "frac_of_peak": round(total_flops / (ms_per_step * 1e-3) / (MFMA_F16_PEAK_TFLOPS * 1e12), 5),
                 "peak_tflops": MFMA_F16_PEAK_TFLOPS},
        "hbm_frac_whole_step": round((wk["prep_bytes"] + wk["scan_bytes"]) / (ms_per_step * 1e-3) / 1e9
                                     / HBM_PEAK_GBS, 4),
        "call_ms_percentiles": {"p10": round(float(np.percentile(per_call, 10)), 5),
                                "p50": round(float(np.percentile(per_call, 50)), 5),
                                "p90": round(float(np.percentile(per_call, 90)), 5),
                                "note": "per call, from the events of the second pass (first to last mark)"},
        "parity": parity,
        "cpu_baseline": cpu_baseline,
    }
    res.update(extra)
    if res.get("workloads") and res["value"] is not None:
        vals = [res["value"]] + [w["tokens_per_s"] for w in res["workloads"].values()]
        if all(v_ is not None for v_ in vals):
            res["geomean_fixed_varlen_tokens_per_s"] = round(float(np.exp(np.mean(np.log(vals)))), 1)
    print(json.dumps(res), flush=True)
    if not ok:
        log("PARITY FAILED: no speed reported")
        sys.exit(1)


if __name__ == "__main__":
    main()
