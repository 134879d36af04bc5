#!/usr/bin/env python3
"""Benchmark: chunkwise DeltaProduct forward on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input
already resident in HBM: for the symmetric workloads the prep/UT launch and
the chunk-scan launch; for the asymmetric-write-key workload the OSDN phase-1
scan first.  Prints ONE JSON line on stdout; diagnostics go to stderr.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c3]

Per-kernel durations come from HIP events recorded on the launch stream
around every launch inside the timed region.  The CPU baseline is the fp64
oracle on a bounded sample of heads of the same workload, on this host.  The
same line also carries a packed variable-length batch (`varlen`) and the
packed OSDN layer forward on it (`varlen_osdn`), the
one-token decode step at batch 1 and 64 (`decode`), the chunkwise backward on
the default workload's shape (`bwd`), each with its own figures, and what the
GPU sustains on a plain copy and a library GEMM (`ceilings`).
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "tokens/sec & MFMA TFLOP/s, DeltaProduct fwd n_h=2/3, dk=dv=128, L=4096"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
PIPELINE_SEGMENTS = 4          # token runs of the pipelined write-key forward
BF16_PEAK_TFLOPS = 2516.6      # MI355X dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3       # MI355X dense fp32 MFMA


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # the GPU's clocks ramp up over the first ~50 forwards of a cold run (~0.5 ms
    # each at c3); 100 warm-up steps put the timed steps in the steady state
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--settle", type=float, default=1.0, metavar="SECONDS",
                    help="untimed steps for at least this long before the warm-up, so that the "
                         "timed steps run at settled clocks (reported in the line; 0 = none)")
    ap.add_argument("--no-other-path", action="store_true",
                    help="skip timing the bf16 symmetric-key workload on the path the library "
                         "does not pick by default (fused kernel or prep / chain pair)")
    ap.add_argument("--workload", default="c3", help="c1, c2, c3, c3b, c4 or c5")
    ap.add_argument("--also", default="c3b",
                    help="comma-separated extra workloads timed in the same run ('' = none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode-step timing")
    ap.add_argument("--no-varlen", action="store_true", help="skip the packed variable-length timing")
    ap.add_argument("--no-bwd", action="store_true", help="skip the backward timing")
    ap.add_argument("--no-osdn-bwd", action="store_true", help="skip the OSDN layer backward timing")
    ap.add_argument("--no-kda", action="store_true", help="skip the per-channel-gate forward timing")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the copy / GEMM ceiling measurements")
    ap.add_argument("--cpu-heads", type=int, default=0, help="heads in the CPU sample (0: auto)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="only run device-to-device copies of BYTES (counter calibration)")
    return ap.parse_args()


def copy_probe(nbytes):
    """Device-to-device copies of a known size: what the HBM read / write
    counters report for them calibrates the counters of the forward's kernels."""
    import torch

    n = nbytes // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n * 4, "copies": 3}), flush=True)


def source_digest(kernel=None):
    """sha256 over the sources a forward kernel is built from (csrc/*.hip,
    *.hpp, in name order, without the backward and decode files, and without
    the fused kernel's header unless `kernel` is the fused kernel)."""
    import glob
    import hashlib

    hsh = hashlib.sha256()
    for f in sorted(glob.glob(os.path.join(ROOT, "linear_rnn_sequence_amd", "csrc", "*"))):
        base = os.path.basename(f)
        if base.startswith(("dp_bwd", "dp_decode")):
            continue
        if base == "dp_fused.hpp" and kernel != "dp_fused_kernel":
            continue
        if f.endswith((".hip", ".hpp")):
            hsh.update(os.path.basename(f).encode())
            with open(f, "rb") as fh:
                hsh.update(fh.read())
    return hsh.hexdigest()


def counter_record(kind, workload, kernel):
    """The committed counter record profiles/<kind>_<kernel>_<workload>.json,
    or None when there is none or the kernel's sources changed since."""
    path = os.path.join(ROOT, "profiles", f"{kind}_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha256") != source_digest(kernel):
        return None
    return rec


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` for `workload` from the committed counter
    summary, or None when there is none or the kernel sources changed since."""
    rec = counter_record("traffic", workload, kernel)
    return None if rec is None else rec.get("bytes_per_launch")


def measured_mfma_busy(workload, kernel):
    """Fraction of the chip's SIMD cycles the MFMA units were busy during
    `kernel` (SQ_VALU_MFMA_BUSY_CYCLES over GRBM_GUI_ACTIVE / 8 XCDs x 1024
    SIMDs), from the committed counter record, or None."""
    rec = counter_record("mfma", workload, kernel)
    return None if rec is None else rec.get("mfma_busy_frac")


# ---------------------------------------------------------------- accounting

def elem_bytes(w):
    return 4 if w.dtype == "f32" else 2


def alg_bytes(w):
    """Algorithmic HBM bytes of one forward (single pass over inputs and outputs).

    Per head and sub-step: k (dk), v (dv), beta (4 B) and, for the write-key
    workload, kt (dk); per head and token: q (dk), out (dv) and g (4 B) when
    gated; per head: the fp32 state out (and in, when there is an initial state).
    The output counts at its stored width (fp32 for workloads run with fp32 out).
    """
    s = elem_bytes(w)
    N = w.L * w.n_h
    so = 4 if w.out_f32 else s
    per_head = N * (w.dk * s + w.dv * s + 4) + w.L * (w.dk * s + w.dv * so)
    if w.asym:
        per_head += N * w.dk * s
    if w.gate:
        per_head += w.L * 4
    per_head += w.dk * w.dv * 4 * (2 if w.h0_std > 0 else 1)
    return w.B * w.H * per_head


def precond_bytes(w):
    """Phase 1: read k and beta, write kt, per token and head; d in and out."""
    s = elem_bytes(w)
    return w.B * w.H * (w.L * (2 * w.dk * s + 4) + 2 * w.dk * 4)


def chunk_flops(w):
    """Chunkwise MFMA flops of the forward, dense C x C blocks (the standard
    accounting: A, W and U products, W*H and the state update, Q*H, scores and
    scores times pseudo-values), summed over chunks."""
    C = w.chunk
    N = w.L * w.n_h
    nc = -(-N // C)
    R = C / w.n_h
    per = (2 * C * C * (2 * w.dk + w.dv) + 4 * C * w.dk * w.dv + 2 * R * w.dk * w.dv
           + 2 * R * C * (w.dk + w.dv))
    return w.B * w.H * nc * per


def recurrent_flops(w):
    """Flops of the sequential recurrence: per token n_h * 4 dk dv + 2 dk dv (+ dk dv gate)."""
    per_tok = w.n_h * 4 * w.dk * w.dv + 2 * w.dk * w.dv + (w.dk * w.dv if w.gate else 0)
    return w.B * w.L * w.H * per_tok


def fused_possible(w):
    """Can this workload run the single fused kernel (DP_FWD_FUSED)?"""
    return w.dtype == "bf16" and not w.asym and w.dk % 32 == 0 and w.chunk % 32 == 0


def kernel_names(w):
    """(prep / UT kernel, scan kernel) names of the two-launch path a workload
    runs on; the fused path is the one kernel dp_fused_kernel."""
    if w.dtype == "bf16" and (not w.asym or (w.dk % 32 == 0 and w.chunk % 32 == 0)):
        return "dp_prep_kernel", "dp_chain_kernel"
    if w.dtype == "bf16":
        return "dp_ut_kernel", "dp_scan16_kernel"
    return "dp_ut_kernel", "dp_scan_kernel"


def fused_issued_flops(w, plan):
    """MFMA flops dp_fused_kernel issues per forward (tile-padded).  Every
    workgroup of a head builds the chunk's operands itself: the Gram matrix's
    lower 16 x 16 tiles (bf16), the readout scores (fp16) and the two
    off-diagonal T blocks as split-fp16 products (two 32-deep steps per
    product, two products per 32-row half); the consumers, per 16 value
    columns: Kn H, Q H, the three 32 x 32 solve steps per half pair, P Up and
    the state update."""
    C, dk, dv, BV, RT = w.chunk, w.dk, w.dv, plan["BV"], plan["readout_rows"]
    nc = -(-(w.L * w.n_h) // C)
    NT, CH = C // 16, C // 32
    prod = (NT * (NT + 1) // 2) * 2 * 16 * 16 * dk + 2 * RT * C * dk + CH * 2 * 2 * 2 * 16 * 16 * 32
    solve = (2 + 4 * (CH - 1)) * 2 * 16 * 16 * 32
    cons16 = 2 * 16 * (C * dk + RT * dk + RT * C + dk * C) + solve
    heads = w.B * w.H
    return heads * nc * ((dv // BV) * prod + (dv // 16) * cons16)


def issued_flops(w, plan):
    """MFMA flops the two kernels of the two-launch path issue (tile-padded), per forward."""
    C, dk, dv, BV, RT = w.chunk, w.dk, w.dv, plan["BV"], plan["readout_rows"]
    N = w.L * w.n_h
    nc = -(-N // C)
    NT = C // 16
    ut = (NT * (NT + 1) // 2) * 16 * 16 * dk * 2
    for dist in range(1, NT):  # blocked inverse, fp32
        ut += (NT - dist) * (dist + 1) * 16 * 16 * 16 * 2
    heads = w.B * w.H
    if kernel_names(w)[0] == "dp_prep_kernel":
        ut += 2 * RT * C * dk  # scores of the readout rows
        per16 = 2 * 16 * (C * dk + C * C + RT * dk + RT * C + dk * C)  # per 16 value columns
        return heads * nc * ut, heads * nc * per16 * (dv // 16)
    scan = 2 * (C * BV * dk + C * RT * dk + RT * BV * dk + C * C * BV + RT * C * BV + dk * C * BV)
    return heads * nc * ut, heads * nc * scan * (dv // BV)


def roofline_fields(kernel, kernel_ms, kernel_bytes, step_bytes, step_ms, traffic):
    """The line's roofline object: the dominant kernel's algorithmic bytes over
    its event-timed duration against the HBM peak, and the whole step's
    algorithmic bytes over ms_per_step beside it."""
    achieved = kernel_bytes / (kernel_ms * 1e6)
    step = step_bytes / (step_ms * 1e6)
    return {"kernel": kernel, "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
            "alg_bytes_per_launch": kernel_bytes, "step_achieved": step,
            "step_frac": step / HBM_PEAK_GBS,
            "note": "achieved: the kernel's own algorithmic bytes over its event-timed "
                    "duration; step_*: the whole step's algorithmic bytes over ms_per_step"}


# ---------------------------------------------------------------- GPU timing

def settle_clocks(step, seconds):
    """Run untimed steps for at least `seconds` of wall time: a cold MI355X
    raises its clocks over the first ~50 forwards, and a short warm-up would
    time that ramp.  Returns (steps run, seconds)."""
    import torch

    if seconds <= 0:
        return 0, 0.0
    n, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(10):
            step()
        torch.cuda.synchronize()
        n += 10
    return n, time.perf_counter() - t0


def time_gpu(w, steps, warmup, settle=0.0, path="auto"):
    """Time `steps` forwards of workload w on the path the library picks by
    default (path="auto"), or on the one named ("split", "fused").  The fused
    kernel runs as one call; the two-kernel paths (prep / chain for bf16
    symmetric keys, UT / scan otherwise) as two staged calls, so that each
    kernel is timed on its own."""
    import torch

    import linear_rnn_sequence_amd as dp
    from linear_rnn_sequence_amd.inputs import make

    dev = torch.device("cuda:0")
    t0 = time.perf_counter()
    inp = make(w)
    log(f"[bench] {w.name}: inputs drawn in {time.perf_counter() - t0:.1f}s")
    d = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    dt = d["q"].dtype
    plan = dp.launch_info(w.n_h, w.B, w.H, w.L, w.dk, w.dv, w.chunk, dt, asym=w.asym)
    # launch_info reports the default call's plan (no UT workgroups: the fused kernel)
    fused = path == "fused" or (path == "auto" and plan["ut_wgs"] == 0)
    ws = None if fused else dp.alloc_workspace(w.n_h, w.B, w.H, w.L, w.dk, w.dv, w.chunk, dt, dev)
    out = torch.empty(w.B, w.L, w.H, w.dv, dtype=inp["out_dtype"], device=dev)
    fs = torch.empty(w.B, w.H, w.dk, w.dv, dtype=torch.float32, device=dev)
    k1 = b1 = kt = dstate = d1 = None
    if w.asym:
        k1 = d["k"][:, :, :, 0, :].contiguous()
        b1 = d["beta"][..., 0].contiguous()
        kt = torch.empty_like(k1)
        d1 = torch.ones(w.B, w.H, w.dk, dtype=torch.float32, device=dev)
        dstate = torch.empty_like(d1)
    args = (d["q"], d["k"], d["v"], d["beta"], d["g"])
    split_flag = "split" if fused_possible(w) else "auto"
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if w.asym:
            dstate.copy_(d1)
            if ev is not None:
                ev[0].record(stream)
            dp.osdn_precond(k1, b1, d_state=dstate, kt=kt)
        kk = None if kt is None else kt.unsqueeze(3)
        if ev is not None:
            ev[1].record(stream)
        if fused:
            dp.fwd(*args, chunk=w.chunk, h0=d["h0"], kt=kk, out=out, final_state=fs, path="fused")
            if ev is not None:
                ev[2].record(stream)
        else:
            dp.fwd(*args, chunk=w.chunk, h0=d["h0"], kt=kk, out=out, final_state=fs, workspace=ws,
                   stages=dp.STAGE_UT, path=split_flag)
            if ev is not None:
                ev[2].record(stream)
            dp.fwd(*args, chunk=w.chunk, h0=d["h0"], kt=kk, out=out, final_state=fs, workspace=ws,
                   stages=dp.STAGE_SCAN, path=split_flag)
        if ev is not None:
            ev[3].record(stream)

    settled = settle_clocks(step, settle)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ut_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / steps
    scan_ms = sum(e[2].elapsed_time(e[3]) for e in evs) / steps
    pre_ms = (sum(e[0].elapsed_time(e[1]) for e in evs) / steps) if w.asym else 0.0
    res = dict(elapsed=elapsed, ms_per_step=1e3 * elapsed / steps, ut_ms=ut_ms, scan_ms=scan_ms,
               pre_ms=pre_ms, plan=plan, inputs=inp, fused=fused, settled=settled)
    if w.asym:
        # the same step as one pipelined call (phase 1 of a token run overlaps the
        # forward of the previous run); the per-kernel times above are the two-call path's
        S = PIPELINE_SEGMENTS
        q, kk, vv = d["q"], k1, d["v"][:, :, :, 0, :].contiguous()
        pws = torch.empty(dp.osdn_fwd_workspace_size(w.B, w.H, w.L, w.dk, w.dv, w.chunk, S),
                          dtype=torch.uint8, device=dev)
        fs2 = torch.empty_like(fs)
        out2 = torch.empty_like(out)
        pipe = dp.Pipeline()

        def pstep():
            dstate.copy_(d1)
            dp.osdn_fwd(q, kk, vv, b1, chunk=w.chunk, segments=S, d_state=dstate, kt=kt, out=out2,
                        final_state=fs2, workspace=pws, pipeline=pipe)

        for _ in range(warmup):
            pstep()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            pstep()
        torch.cuda.synchronize()
        pel = time.perf_counter() - t0
        pipe.close()
        res["two_call_ms_per_step"] = res["ms_per_step"]
        res["elapsed"], res["ms_per_step"], res["segments"] = pel, 1e3 * pel / steps, S
    return res


def decode_bytes(B, H, n_h, dk, dv, elem=2):
    """Algorithmic bytes of one decode step: the fp32 state read and written,
    plus q, k, v (elem bytes each), beta and out per head."""
    return B * H * (2 * dk * dv * 4 + (n_h * (dk + dv) + dk + dv) * elem + n_h * 4)


def time_decode(B, H, n_h, dk, dv, tokens=128, reps=5):
    """Recurrent decode: `tokens` consecutive one-token launches on a resident
    state (the pages' protocol decodes 128 tokens after a prefill), timed with
    HIP events on the launch stream; best of `reps` runs."""
    import torch

    import linear_rnn_sequence_amd as dp
    from linear_rnn_sequence_amd.inputs import WORKLOADS, make

    dev = torch.device("cuda:0")
    w = WORKLOADS["c3"].scaled(B=B, H=H, L=tokens, n_h=n_h, dk=dk, dv=dv)
    inp = make(w)
    toks = [{n: inp[n][:, t].contiguous().to(dev) for n in ("q", "k", "v", "beta")}
            for t in range(tokens)]
    state = torch.zeros(B, H, dk, dv, dtype=torch.float32, device=dev)
    out = torch.empty(B, H, dv, dtype=torch.bfloat16, device=dev)
    stream = torch.cuda.current_stream()

    def run():
        for x in toks:
            dp.decode(x["q"], x["k"], x["v"], x["beta"], state, out=out, stream=stream)

    run()
    torch.cuda.synchronize()
    best = None
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        run()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        best = ms if best is None else min(best, ms)
    us = 1e3 * best / tokens
    nbytes = decode_bytes(B, H, n_h, dk, dv)
    return {"workload": f"decode: B={B} H={H} n_h={n_h} dk={dk} dv={dv} bf16, fp32 state, "
                        f"{tokens} one-token launches",
            "us_per_token": us, "tokens_per_s": B * 1e6 / us,
            "roofline": {"kernel": "dp_decode_kernel", "bound": "hbm",
                         "achieved": nbytes / (us * 1e3), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": nbytes / (us * 1e3) / HBM_PEAK_GBS,
                         "alg_bytes_per_launch": nbytes}}


def time_varlen(steps, warmup, T=65536):
    """Packed variable-length forward: T tokens of log-normal document lengths
    (H=16, dk=dv=128, n_h=2, bf16), each document its own sequence and state."""
    import itertools

    import torch

    import linear_rnn_sequence_amd as dp
    from linear_rnn_sequence_amd.inputs import WORKLOADS, make, packed_lengths

    dev = torch.device("cuda:0")
    w = WORKLOADS["c3b"]
    lengths = packed_lengths(T, seed=11)
    inp = make(w.scaled(B=1, L=T))
    d = {n: inp[n][0].contiguous().to(dev) for n in ("q", "k", "v", "beta")}
    cu = torch.tensor([0] + list(itertools.accumulate(lengths)), dtype=torch.int32, device=dev)
    nseq = len(lengths)
    ws = torch.empty(dp.varlen_workspace_size(w.n_h, nseq, w.H, T, w.dk, w.dv, w.chunk),
                     dtype=torch.uint8, device=dev)
    out = torch.empty(T, w.H, w.dv, dtype=torch.bfloat16, device=dev)
    fs = torch.empty(nseq, w.H, w.dk, w.dv, dtype=torch.float32, device=dev)

    def step():
        dp.fwd_varlen(d["q"], d["k"], d["v"], d["beta"], cu, chunk=w.chunk, out=out, final_state=fs,
                      workspace=ws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms = 1e3 * (time.perf_counter() - t0) / steps
    return {"workload": f"varlen: {nseq} packed documents, T={T} tokens, H={w.H} n_h={w.n_h} "
                        f"dk={w.dk} dv={w.dv} chunk={w.chunk} bf16",
            "value": T / (ms / 1e3), "unit": "tokens/s", "ms_per_step": ms}


def time_varlen_osdn(steps, warmup, T=65536):
    """Packed OSDN layer forward: T tokens of log-normal document lengths at the
    write-key workload's head shape (H=16, dk=dv=128, n_h=1, bf16); every
    document runs phase 1 from d = 1 (a fill of d is part of the step; the
    chunked form, 64-token chunks from each document's start) and then the
    write-key forward from a zero state."""
    import itertools

    import torch

    import linear_rnn_sequence_amd as dp
    from linear_rnn_sequence_amd.inputs import WORKLOADS, make, packed_lengths

    dev = torch.device("cuda:0")
    w = WORKLOADS["c5"]
    lengths = packed_lengths(T, seed=11)
    inp = make(w.scaled(B=1, L=T))
    d = {n: inp[n][0].contiguous().to(dev) for n in ("q", "k", "v", "beta")}
    k1, b1 = d["k"][:, :, 0].contiguous(), d["beta"][:, :, 0].contiguous()
    cu = torch.tensor([0] + list(itertools.accumulate(lengths)), dtype=torch.int32, device=dev)
    nseq = len(lengths)
    ws = torch.empty(dp.varlen_workspace_size(w.n_h, nseq, w.H, T, w.dk, w.dv, w.chunk),
                     dtype=torch.uint8, device=dev)
    dst = torch.empty(nseq, w.H, w.dk, dtype=torch.float32, device=dev)
    pws = torch.empty(max(dp.osdn_precond_varlen_workspace_size(nseq, w.H, T, w.dk), 1),
                      dtype=torch.uint8, device=dev)
    kt = torch.empty(T, w.H, w.dk, dtype=torch.bfloat16, device=dev)
    out = torch.empty(T, w.H, w.dv, dtype=torch.bfloat16, device=dev)
    fs = torch.empty(nseq, w.H, w.dk, w.dv, dtype=torch.float32, device=dev)

    def phase1():
        dst.fill_(1.0)
        dp.osdn_precond_varlen(k1, b1, cu, d_state=dst, kt=kt, workspace=pws)

    def step():
        phase1()
        dp.fwd_varlen(d["q"], d["k"], d["v"], d["beta"], cu, chunk=w.chunk, kt=kt.unsqueeze(2),
                      out=out, final_state=fs, workspace=ws)

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            fn()
        torch.cuda.synchronize()
        return 1e3 * (time.perf_counter() - t0) / steps

    ms, ms1 = timed(step), timed(phase1)
    return {"workload": f"packed OSDN layer forward: {nseq} documents, T={T} tokens, H={w.H} "
                        f"n_h={w.n_h} dk={w.dk} dv={w.dv} chunk={w.chunk} bf16, phase 1 per document "
                        f"(chunked; longest {max(lengths)} tokens) then the write-key forward",
            "value": T / (ms / 1e3), "unit": "tokens/s", "ms_per_step": ms, "phase1_ms": ms1}


def time_bwd(w, steps, warmup):
    """Chunkwise backward (dp_bwd_*) on the forward workload ``w``'s shape:
    gradients w.r.t. q, k, v, beta (and g, h0) for a seeded output gradient,
    with inputs, gradients and workspace resident in HBM."""
    import torch

    import linear_rnn_sequence_amd as dp
    from linear_rnn_sequence_amd.inputs import make, make_grads

    dev = torch.device("cuda:0")
    inp = make(w)
    gr = make_grads(w)
    d = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    dout = gr["dout"].to(dev)
    dfinal = gr["dfinal"].to(dev)
    ws = torch.empty(dp.bwd_workspace_size(w.n_h, w.B, w.H, w.L, w.dk, w.dv), dtype=torch.uint8, device=dev)
    grads = dp.bwd(d["q"], d["k"], d["v"], d["beta"], dout, d["g"], h0=d["h0"], dfinal=dfinal, workspace=ws)

    def step():
        dp.bwd(d["q"], d["k"], d["v"], d["beta"], dout, d["g"], h0=d["h0"], dfinal=dfinal, workspace=ws,
               grads=grads)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    return {"workload": f"backward of {describe(w)}; fp32 state and accumulation, fp16 MFMA operands, 32-sub-step chunks",
            "value": w.B * w.L / (ms / 1e3), "unit": "tokens/s", "ms_per_step": ms,
            "workspace_bytes": ws.numel()}


def _event_time(step, steps, warmup):
    import torch

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def time_osdn_bwd(steps, warmup):
    """Backward of the whole OSDN layer (dp_osdn_bwd_bf16: phase 1 again with
    its trajectory of d, the write-key backward, phase 1's reverse scan) on the
    write-key workload's shape, inputs and workspace resident in HBM."""
    import torch

    import linear_rnn_sequence_amd as dp
    from linear_rnn_sequence_amd.inputs import WORKLOADS, make, make_grads

    w = WORKLOADS["c5"]
    dev = torch.device("cuda:0")
    inp = make(w)
    gr = make_grads(w, final=False)
    q = inp["q"].to(dev)
    k = inp["k"][:, :, :, 0].contiguous().to(dev)
    v = inp["v"][:, :, :, 0].contiguous().to(dev)
    beta = inp["beta"][..., 0].contiguous().to(dev)
    dout = gr["dout"].to(dev)
    ws = torch.empty(dp.osdn_bwd_workspace_size(w.B, w.H, w.L, w.dk, w.dv), dtype=torch.uint8, device=dev)
    grads = dp.osdn_bwd(q, k, v, beta, dout, workspace=ws)
    ms = _event_time(lambda: dp.osdn_bwd(q, k, v, beta, dout, workspace=ws, grads=grads), steps, warmup)
    return {"workload": f"OSDN layer backward (phase 1 + write-key forward) of {describe(w)}; "
                        "fp32 state and accumulation, fp16 MFMA operands, 32-token chunks",
            "value": w.B * w.L / (ms / 1e3), "unit": "tokens/s", "ms_per_step": ms,
            "workspace_bytes": ws.numel()}


def time_kda(steps, warmup):
    """Chunkwise forward with the KDA host's per-key-channel gate on the
    LM-layer shape (alpha uniform in [0.9, 1] per channel and token)."""
    import torch

    import linear_rnn_sequence_amd as dp
    from linear_rnn_sequence_amd.inputs import WORKLOADS, channel_gate, make

    w = WORKLOADS["c3"]
    dev = torch.device("cuda:0")
    inp = make(w)
    d = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    ga = channel_gate(w.B, w.L, w.H, w.dk, seed=w.seed + 17, lo=0.9).to(dev)
    ws = dp.alloc_workspace(w.n_h, w.B, w.H, w.L, w.dk, w.dv, w.chunk, d["q"].dtype, dev)
    out, fs = dp.fwd(d["q"], d["k"], d["v"], d["beta"], chunk=w.chunk, ga=ga, workspace=ws)
    ms = _event_time(lambda: dp.fwd(d["q"], d["k"], d["v"], d["beta"], chunk=w.chunk, ga=ga, out=out,
                                    final_state=fs, workspace=ws), steps, warmup)
    return {"workload": f"{describe(w)} with a per-key-channel gate alpha [B,L,H,dk] (KDA host)",
            "value": w.B * w.L / (ms / 1e3), "unit": "tokens/s", "ms_per_step": ms,
            "kernels": "dp_ut_kernel + dp_scan_kernel in their per-channel-gate form"}


def measure_ceilings():
    """What this GPU sustains on plain library work, next to the published
    peaks: a 1 GiB device-to-device copy (read + write bytes / time) and an
    8192^3 bf16 GEMM (torch.matmul)."""
    import torch

    dev = torch.device("cuda:0")
    out = {}
    src = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(20):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    out["d2d_copy_gbs"] = 2 * src.numel() * 4 * 20 / (e0.elapsed_time(e1) * 1e6)
    del src, dst
    n = 8192
    a = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    b = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    for _ in range(5):
        c = a @ b
    e0.record()
    for _ in range(20):
        c = a @ b
    e1.record()
    torch.cuda.synchronize()
    out["bf16_gemm_tflops"] = 2 * n ** 3 * 20 / (e0.elapsed_time(e1) * 1e9)
    del a, b, c
    return out


# ---------------------------------------------------------------- CPU baseline

def cpu_baseline(w, inp, nheads, min_seconds=10.0, max_pass_seconds=30.0, max_passes=100):
    """Time the fp64 oracle on this host's cores on the same input bytes.

    The sample is the whole workload (every head, full length) when one pass
    is estimated to take at most ``max_pass_seconds``; otherwise the largest
    set of evenly spread heads that fits about half of that.  Passes repeat
    until ``min_seconds`` of wall time have accumulated; the rate is taken
    from the median pass.
    """
    import statistics

    import numpy as np
    import torch

    import oracle
    from linear_rnn_sequence_amd.inputs import sampled_heads, select_heads, select_state

    threads = oracle.num_threads()
    total = w.B * w.H
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass

    def prepare(heads):
        sub = {k: (None if inp[k] is None else select_heads(inp[k], heads, w.H))
               for k in ("q", "k", "v", "beta", "g")}
        conv = {k: (None if v is None else np.ascontiguousarray(v.to(torch.float64).numpy()))
                for k, v in sub.items()}
        conv["h0"] = (None if inp["h0"] is None else
                      np.ascontiguousarray(select_state(inp["h0"], heads, w.H)
                                           .to(torch.float64).numpy()))
        return conv

    def one_pass(c, nthreads=0):
        t0 = time.perf_counter()
        if w.asym:
            kt, _ = oracle.precond(c["k"][:, :, :, 0, :], c["beta"][..., 0], nthreads=nthreads)
            oracle.fwd(c["q"], c["k"], c["v"], c["beta"], g=c["g"], kt=kt[:, :, :, None, :],
                       h0=c["h0"], nthreads=nthreads)
        else:
            oracle.fwd(c["q"], c["k"], c["v"], c["beta"], g=c["g"], h0=c["h0"], nthreads=nthreads)
        return time.perf_counter() - t0

    if nheads:
        heads = sampled_heads(w.B, w.H, nheads)
    else:
        pilot = sampled_heads(w.B, w.H, min(total, threads))
        t_pilot = one_pass(prepare(pilot))
        waves = -(-total // threads)
        if t_pilot * waves <= max_pass_seconds:
            heads = list(range(total))
        else:
            fit = max(1, int(0.5 * max_pass_seconds / max(t_pilot, 1e-9)))
            heads = sampled_heads(w.B, w.H, min(total, fit * threads))
    conv = prepare(heads)
    times = []
    t_start = time.perf_counter()
    while True:
        times.append(one_pass(conv))
        if time.perf_counter() - t_start >= min_seconds or len(times) >= max_passes:
            break
    t = statistics.median(times)
    value = len(heads) * w.L / w.H / t   # whole-workload tokens/s at this rate
    what = ("the whole workload" if len(heads) == total
            else f"{len(heads)} of {total} heads (b,h)")
    # the same oracle on one thread, on a few heads (about two seconds)
    few = sampled_heads(w.B, w.H, min(total, 2))
    c1 = prepare(few)
    t1s, t_start = [], time.perf_counter()
    while not t1s or (time.perf_counter() - t_start < 2.0 and len(t1s) < 5):
        t1s.append(one_pass(c1, nthreads=1))
    t1 = statistics.median(t1s)
    return {"value": value, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{what} of {w.name}, full L={w.L}, all {w.n_h} sub-steps per token"
                      f"{', phase 1 included' if w.asym else ''}; fp64 sequential recurrence; "
                      f"median of {len(times)} passes ({sum(times):.1f}s wall) on {threads} threads",
            "seconds_per_pass": t, "cpu_model": model,
            "one_thread": {"value": len(few) * w.L / w.H / t1, "unit": "tokens/s",
                           "sample": f"{len(few)} heads of {w.name}, full L, median of {len(t1s)} passes "
                                     f"on 1 thread",
                           "speedup_of_cores": value / (len(few) * w.L / w.H / t1)}}


# ---------------------------------------------------------------- main

def describe(w):
    extra = (", gated, h0" if w.gate else "") + (", write key (OSDN phase 1 + 2)" if w.asym else "")
    return (f"{w.name}: DeltaProduct fwd B={w.B} H={w.H} L={w.L} n_h={w.n_h} dk={w.dk} dv={w.dv} "
            f"chunk={w.chunk} {w.dtype}{extra}")


def main():
    a = parse()
    if a.copy_probe:
        copy_probe(a.copy_probe)
        return
    if a.gpus != 1 or os.environ.get("WORLD_SIZE", "1") not in ("1", ""):
        print("bench.py measures one GPU only: there is no multi-GPU path here (the forward "
              "shards over heads or value columns with no communication). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)
    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(3)
    from __graft_entry__ import _ensure_built

    _ensure_built()
    from linear_rnn_sequence_amd.inputs import WORKLOADS

    w = WORKLOADS[a.workload]
    r = time_gpu(w, a.steps, a.warmup, settle=a.settle)
    tokens = w.B * w.L
    value = tokens / (r["ms_per_step"] / 1e3)
    cf = chunk_flops(w)
    rf = recurrent_flops(w)
    ab = alg_bytes(w)
    peak_mfma = FP32_PEAK_TFLOPS if w.dtype == "f32" else BF16_PEAK_TFLOPS
    if r["fused"]:
        fi = fused_issued_flops(w, r["plan"])
        kernels = {"dp_fused_kernel": {"ms": r["ut_ms"], "issued_tflops": fi / (r["ut_ms"] * 1e9),
                                       "issued_frac": fi / (r["ut_ms"] * 1e9) / peak_mfma,
                                       "mfma_busy_counter": measured_mfma_busy(w.name, "dp_fused_kernel"),
                                       "workgroups": r["plan"]["scan_wgs"],
                                       "value_columns": r["plan"]["BV"]}}
    else:
        ut_issued, scan_issued = issued_flops(w, r["plan"])
        ut_name, scan_name = kernel_names(w)
        kernels = {
            ut_name: {"ms": r["ut_ms"], "issued_tflops": ut_issued / (r["ut_ms"] * 1e9),
                      "issued_frac": ut_issued / (r["ut_ms"] * 1e9) / peak_mfma,
                      "mfma_busy_counter": measured_mfma_busy(w.name, ut_name),
                      "workgroups": r["plan"]["ut_wgs"]},
            scan_name: {"ms": r["scan_ms"], "issued_tflops": scan_issued / (r["scan_ms"] * 1e9),
                        "issued_frac": scan_issued / (r["scan_ms"] * 1e9) / peak_mfma,
                        "mfma_busy_counter": measured_mfma_busy(w.name, scan_name),
                        "workgroups": r["plan"]["scan_wgs"], "value_columns": r["plan"]["BV"]},
        }
    if w.asym:
        kernels["dp_precond_kernel"] = {"ms": r["pre_ms"],
                                        "gbs": precond_bytes(w) / (r["pre_ms"] * 1e6)}

    # dominant kernel and its own algorithmic bytes: the fused kernel (or, on the
    # two-launch paths, the scan) reads every input and writes every output of
    # the forward once; phase 1 reads k and beta and writes kt
    dom = max(kernels, key=lambda k: kernels[k]["ms"])
    dom_ms = kernels[dom]["ms"]
    dom_bytes = ab if dom != "dp_precond_kernel" else precond_bytes(w)
    step_bytes = ab + (precond_bytes(w) if w.asym else 0)
    line = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": r["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded, shapes and distributions of the pages' workloads)",
        "config": {"workload": describe(w), "B": w.B, "H": w.H, "L": w.L, "n_h": w.n_h,
                   "dk": w.dk, "dv": w.dv, "chunk": w.chunk, "gate": w.gate, "asym": w.asym,
                   "global_batch": w.B, "seq_len": w.L, "parallelism": "none (1 GPU)"},
        "mfma_tflops": cf / (r["ms_per_step"] * 1e9),
        "mfma_tflops_frac": cf / (r["ms_per_step"] * 1e9) / peak_mfma,
        "recurrent_tflops": rf / (r["ms_per_step"] * 1e9),
        "alg_gbs": ab / (r["ms_per_step"] * 1e6),
        "kernels": kernels,
        "roofline": roofline_fields(dom, dom_ms, dom_bytes, step_bytes, r["ms_per_step"],
                                    measured_traffic(w.name, dom)),
        "clock_settle": {"steps": r["settled"][0], "seconds": r["settled"][1],
                         "note": "untimed steps run before the warm-up so that the timed steps see "
                                 "settled clocks"},
    }
    if fused_possible(w) and not a.no_other_path:
        other = "split" if r["fused"] else "fused"
        rs = time_gpu(w, a.steps, a.warmup, settle=min(a.settle, 0.3), path=other)
        if other == "split":
            line["other_path"] = {"path": "split (DP_FWD_SPLIT)", "ms_per_step": rs["ms_per_step"],
                                  "dp_prep_kernel_ms": rs["ut_ms"], "dp_chain_kernel_ms": rs["scan_ms"],
                                  "note": "the same workload on the two-kernel path: operand blocks "
                                          "written to HBM by the prep kernel"}
        else:
            line["other_path"] = {"path": "fused (DP_FWD_FUSED)", "ms_per_step": rs["ms_per_step"],
                                  "dp_fused_kernel_ms": rs["ut_ms"],
                                  "note": "the same workload on the single fused kernel: every "
                                          "value-column workgroup of a head builds the chunk's "
                                          "operands itself"}
        del rs
    if w.asym:
        line["pipeline"] = {"call": "dp_osdn_fwd_bf16", "segments": r["segments"],
                            "two_call_ms_per_step": r["two_call_ms_per_step"],
                            "note": "the step is one pipelined call; kernels.* are the two-call path's"}
    also = {}
    for name in [x for x in a.also.split(",") if x and x != a.workload]:
        w2 = WORKLOADS[name]
        r2 = time_gpu(w2, a.steps, a.warmup, settle=min(a.settle, 0.3))
        also[name] = {"workload": describe(w2),
                      "value": w2.B * w2.L / (r2["ms_per_step"] / 1e3), "unit": "tokens/s",
                      "ms_per_step": r2["ms_per_step"],
                      "mfma_tflops": chunk_flops(w2) / (r2["ms_per_step"] * 1e9)}
        if r2["fused"]:
            also[name]["dp_fused_kernel_ms"] = r2["ut_ms"]
        else:
            also[name]["ut_ms"], also[name]["scan_ms"] = r2["ut_ms"], r2["scan_ms"]
        del r2
    if also:
        line["also"] = also
    if not a.no_varlen:
        line["varlen"] = time_varlen(a.steps, a.warmup)
        line["varlen_osdn"] = time_varlen_osdn(a.steps, a.warmup)
    if not a.no_decode:
        # the pages' decode protocol (batch 1) and a serving-size batch, head shape of c3
        line["decode"] = {"b1": time_decode(1, 16, 3, 128, 128),
                          "b64": time_decode(64, 16, 3, 128, 128)}
    if not a.no_bwd:
        line["bwd"] = time_bwd(w, max(5, a.steps // 10), max(3, a.warmup // 10))
    if not a.no_osdn_bwd:
        line["osdn_bwd"] = time_osdn_bwd(max(5, a.steps // 10), max(3, a.warmup // 10))
    if not a.no_kda:
        line["kda"] = time_kda(max(5, a.steps // 10), max(2, a.warmup // 10))
    if not a.no_ceilings:
        line["ceilings"] = measure_ceilings()
    if not a.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, r["inputs"], a.cpu_heads)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
