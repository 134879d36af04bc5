"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Every case compares, element by element, the GPU result with the oracle run
on the same stored bytes, with err = max|x_gpu - x_oracle| / RMS(x_oracle)
per tensor, bounded by 1e-4 on the fp32 path and 2e-2 on the bf16 path (bf16
inputs, fp32 state and accumulation).  Full-size workloads run exactly as the
benchmark launches them and are checked on sampled heads, which the oracle
computes one by one (heads are independent).
"""
import math

import numpy as np
import pytest
import torch

import linear_rnn_sequence_amd as dp
import oracle
from linear_rnn_sequence_amd.inputs import WORKLOADS, make, write_keys
from parity import TOL, f64, gpu_forward, oracle_heads, rel_err, sampled_heads, say, \
    select_heads, select_state

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    dp.load()  # raises when libdp.so is missing: no silent fallback


def run_pair(inp, chunk=None, dtype="bf16"):
    """GPU forward (with the phase-1 scan for asymmetric workloads) and the oracle."""
    asym = inp.get("asym", False)
    if asym:
        k1 = inp["k"][:, :, :, 0, :].contiguous()
        b1 = inp["beta"][..., 0].contiguous()
        ktg, dg = dp.osdn_precond(k1.cuda(), b1.cuda())
        out, fs = gpu_forward(inp, chunk=chunk, kt=ktg.unsqueeze(3))
        kto, do = oracle.precond(k1, b1)
        oo, fo = oracle.fwd(inp["q"], inp["k"], inp["v"], inp["beta"], g=inp["g"],
                            kt=kto[:, :, :, None, :], h0=inp["h0"])
        return dict(out=(f64(out), oo), fs=(f64(fs), fo), kt=(f64(ktg), kto), d=(f64(dg), do))
    out, fs = gpu_forward(inp, chunk=chunk)
    oo, fo = oracle.fwd(inp["q"], inp["k"], inp["v"], inp["beta"], g=inp["g"], h0=inp["h0"])
    return dict(out=(f64(out), oo), fs=(f64(fs), fo))


def check(res, tol, label):
    for name, (x, ref) in res.items():
        e = rel_err(x, ref)
        say(f"  {label} {name}: err {e:.3e} (tol {tol:.0e})")
        assert np.all(np.isfinite(x)), f"{label} {name}: non-finite values"
        assert e <= tol, f"{label} {name}: err {e:.3e} > {tol}"


# ------------------------------------------------------------------ small, full parity

SMALL = [
    ("c1", {}),
    ("c1", dict(B=2, H=3, L=77)),
    ("c2", dict(B=2, H=3, L=203)),
    ("c3", dict(B=1, H=2, L=150)),
    ("c3b", dict(B=1, H=2, L=161)),
    ("c4", dict(B=2, H=2, L=300)),
    ("c5", dict(B=2, H=3, L=257)),
    ("c4", dict(B=1, H=2, L=130, n_h=3)),  # gated, h0, 22 readout rows of 32 per chunk
]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("name,kw", SMALL, ids=[f"{n}-{i}" for i, (n, _) in enumerate(SMALL)])
def test_small_workloads(name, kw, dtype):
    w = WORKLOADS[name].scaled(dtype=dtype, **kw)
    say(f"case {name} {kw} dtype={dtype} seed={w.seed} n_h={w.n_h} dk={w.dk} dv={w.dv} C={w.chunk}")
    inp = make(w)
    inp["asym"] = w.asym
    check(run_pair(inp, dtype=dtype), TOL[dtype], f"{name}/{dtype}")


# ------------------------------------------------------------------ full sizes, sampled heads

@pytest.mark.parametrize("name,nsel", [("c2", 32), ("c3", 6), ("c3b", 8), ("c4", 6), ("c5", 12)])
def test_full_size_sampled_heads(name, nsel):
    w = WORKLOADS[name]
    say(f"case full {name}: B={w.B} H={w.H} L={w.L} n_h={w.n_h} d={w.dk} C={w.chunk} {w.dtype}")
    inp = make(w)
    heads = sampled_heads(w.B, w.H, nsel)
    H = w.H
    if w.asym:
        k1 = inp["k"][:, :, :, 0, :].contiguous()
        b1 = inp["beta"][..., 0].contiguous()
        ktg, dg = dp.osdn_precond(k1.cuda(), b1.cuda())
        out, fs = gpu_forward(inp, kt=ktg.unsqueeze(3))
        # the oracle runs phase 1 and phase 2 itself, on the sampled heads only
        kto, do = oracle.precond(select_heads(k1, heads, H), select_heads(b1, heads, H))
        sub = {kk: select_heads(inp[kk], heads, H) for kk in ("q", "k", "v", "beta")}
        oo, fo = oracle.fwd(sub["q"], sub["k"], sub["v"], sub["beta"], kt=kto[:, :, :, None, :])
        ktg_s = select_heads(ktg.cpu(), heads, H)
        dg_s = select_state(dg.cpu(), heads, H)
        res = dict(kt=(f64(ktg_s), kto), d=(f64(dg_s), do))
    else:
        out, fs = gpu_forward(inp)
        oo, fo = oracle_heads(inp, heads)
        res = {}
    res["out"] = (f64(select_heads(out.cpu(), heads, H)), oo)
    res["fs"] = (f64(select_state(fs.cpu(), heads, H)), fo)
    check(res, TOL[w.dtype], f"full-{name}")
    assert torch.isfinite(out.float()).all()


def test_full_size_c5_pipelined_call():
    """The c5 step as bench.py times it: one dp_osdn_fwd_bf16 call over the
    bench's token runs with a pipeline handle, phase 1 in its chunked form
    (dk = 128), against the oracle's phase 1 and forward on sampled heads."""
    import bench
    w = WORKLOADS["c5"]
    S = bench.PIPELINE_SEGMENTS
    say(f"case full c5 pipelined: B={w.B} H={w.H} L={w.L} runs={S}")
    inp = make(w)
    heads = sampled_heads(w.B, w.H, 12)
    H = w.H
    k1 = inp["k"][:, :, :, 0, :].contiguous()
    v1 = inp["v"][:, :, :, 0, :].contiguous()
    b1 = inp["beta"][..., 0].contiguous()
    pipe = dp.Pipeline()
    out, fs, kt, d = dp.osdn_fwd(inp["q"].cuda(), k1.cuda(), v1.cuda(), b1.cuda(), chunk=w.chunk, segments=S,
                                 pipeline=pipe)
    torch.cuda.synchronize()
    pipe.close()
    kto, do = oracle.precond(select_heads(k1, heads, H), select_heads(b1, heads, H))
    sub = {kk: select_heads(inp[kk], heads, H) for kk in ("q", "k", "v", "beta")}
    oo, fo = oracle.fwd(sub["q"], sub["k"], sub["v"], sub["beta"], kt=kto[:, :, :, None, :])
    res = dict(kt=(f64(select_heads(kt.cpu(), heads, H)), kto), d=(f64(select_state(d.cpu(), heads, H)), do),
               out=(f64(select_heads(out.cpu(), heads, H)), oo), fs=(f64(select_state(fs.cpu(), heads, H)), fo))
    check(res, TOL["bf16"], "full-c5-pipelined")
    assert torch.isfinite(out.float()).all()


# ------------------------------------------------------------------ write keys on every shape

WK = [  # workload, overrides: head dims 32..128, chunk 32 and 64, n_h 1..3, gate and h0
    ("c5", dict(B=2, H=2, L=190)),
    ("c5", dict(B=1, H=3, L=150, n_h=2)),
    ("c5", dict(B=1, H=2, L=101, n_h=3, dk=64, dv=32)),
    ("c4", dict(B=1, H=2, L=140, dk=64, dv=64)),               # gated, h0, fp32 out
    ("c4", dict(B=2, H=1, L=77, n_h=1, dk=32, dv=128, chunk=32)),
    ("c2", dict(B=1, H=2, L=66, n_h=3, chunk=32)),
    ("c1", dict(B=1, H=2, L=40, dtype="bf16", dk=16, dv=32)),  # dk 16: the UT / scan16 kernels
]


@pytest.mark.parametrize("name,kw", WK, ids=[f"{n}-{i}" for i, (n, _) in enumerate(WK)])
def test_write_key_forward_shapes(name, kw):
    """The write-key forward (kt as given, not normalised) against the oracle,
    with seeded write keys of the phase-1 shape and range.  These outputs are
    heavy-tailed (max/RMS 7-9), so a bf16 output alone carries up to ~2.5e-2 of
    rounding error (the oracle's own output rounded to bf16 measures the same):
    the computation is checked with fp32 output, and the bf16 output must be
    exactly that output rounded to nearest even."""
    w = WORKLOADS[name].scaled(**kw)
    say(f"case write-key {name} {kw}")
    inp = make(w)
    kt = write_keys(w, seed=w.seed + 5)
    out, fs = gpu_forward(inp, kt=kt, out_dtype=torch.float32)
    o16, f16 = gpu_forward(inp, kt=kt, out_dtype=torch.bfloat16)
    oo, fo = oracle.fwd(inp["q"], inp["k"], inp["v"], inp["beta"], g=inp["g"], kt=kt, h0=inp["h0"])
    check(dict(out=(f64(out), oo), fs=(f64(fs), fo)), TOL[w.dtype], f"wk-{name}")
    assert torch.equal(out.to(torch.bfloat16), o16) and torch.equal(fs, f16)


def test_c4_bf16_output_is_the_rounded_fp32_output():
    """c4 at full size (sampled heads): the fp32 output meets the bound; the
    bf16 output is that output rounded, so its error is the rounding of
    heavy-tailed outputs plus the fp32 error -- the limit dp.h states for bf16
    out, which is why the c4 workload runs with fp32 out."""
    w = WORKLOADS["c4"]
    inp = make(w)
    heads = sampled_heads(w.B, w.H, 4)
    o32, f32 = gpu_forward(inp, out_dtype=torch.float32)
    o16, _ = gpu_forward(inp, out_dtype=torch.bfloat16)
    assert torch.equal(o32.to(torch.bfloat16), o16)
    oo, fo = oracle_heads(inp, heads)
    g32 = f64(select_heads(o32.cpu(), heads, w.H))
    g16 = f64(select_heads(o16.cpu(), heads, w.H))
    e32, e16 = rel_err(g32, oo), rel_err(g16, oo)
    floor = rel_err(torch.from_numpy(oo).to(torch.bfloat16).double().numpy(), oo)
    say(f"  c4 fp32 out err {e32:.3e}, bf16 out err {e16:.3e}, oracle rounded to bf16 {floor:.3e}")
    check(dict(out=(g32, oo), fs=(f64(select_state(f32.cpu(), heads, w.H)), fo)), TOL["bf16"], "c4-f32out")
    # rounding to bf16 moves each element by at most 2^-8 of its magnitude
    assert e16 <= e32 + 2.0 ** -8 * np.abs(g32).max() / np.sqrt((oo ** 2).mean()) + 1e-12


# ------------------------------------------------------------------ chunk invariance, resume, stages

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_chunk_invariance(dtype):
    w = WORKLOADS["c4"].scaled(B=1, H=2, L=333, dtype=dtype, dk=64, dv=64)
    inp = make(w)
    oo, fo = oracle.fwd(inp["q"], inp["k"], inp["v"], inp["beta"], g=inp["g"], h0=inp["h0"])
    outs = {}
    for C in (16, 32, 64):
        say(f"case chunk-invariance dtype={dtype} C={C}")
        out, fs = gpu_forward(inp, chunk=C)
        check(dict(out=(f64(out), oo), fs=(f64(fs), fo)), TOL[dtype], f"C={C}")
        outs[C] = f64(out)
    assert rel_err(outs[16], outs[64]) <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_resume_split_equals_single_call(dtype):
    w = WORKLOADS["c4"].scaled(B=2, H=2, L=250, dtype=dtype)
    inp = make(w)
    m = 97  # 194 sub-steps: not a chunk boundary
    say(f"case resume dtype={dtype} split at token {m}")
    out, fs = gpu_forward(inp)
    first = {k: (v[:, :m].contiguous() if isinstance(v, torch.Tensor) and v.dim() >= 3 and k != "h0"
                 else v) for k, v in inp.items()}
    second = {k: (v[:, m:].contiguous() if isinstance(v, torch.Tensor) and v.dim() >= 3 and k != "h0"
                  else v) for k, v in inp.items()}
    o1, f1 = gpu_forward(first)
    o2, f2 = gpu_forward(second, h0=f1)
    oo, fo = oracle.fwd(inp["q"], inp["k"], inp["v"], inp["beta"], g=inp["g"], h0=inp["h0"])
    cat = torch.cat([o1, o2], dim=1)
    check(dict(out=(f64(cat), oo), fs=(f64(f2), fo)), TOL[dtype], "resume")
    assert rel_err(f64(cat), f64(out)) <= TOL[dtype]
    # in-place resume: h0 and final_state may be the same buffer
    st = f1.clone()
    o2b, _ = dp.fwd(*(second[k].cuda() for k in ("q", "k", "v", "beta")), second["g"].cuda(),
                    chunk=w.chunk, h0=st, final_state=st, out_dtype=second["out_dtype"])
    torch.cuda.synchronize()
    assert torch.equal(o2b, o2) and torch.equal(st, f2)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_staged_equals_single_launch_and_is_deterministic(dtype):
    """The default call is deterministic; the two-launch path (prep / UT kernel,
    then the scan) run as two staged calls equals the same path in one call.
    On the bf16 path with symmetric keys the fused kernel is a different
    summation order: it is checked against the oracle."""
    w = WORKLOADS["c3"].scaled(B=1, H=3, L=123, dtype=dtype)
    inp = make(w)
    d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    ws = dp.alloc_workspace(w.n_h, w.B, w.H, w.L, w.dk, w.dv, w.chunk, d["q"].dtype, "cuda")
    args = (d["q"], d["k"], d["v"], d["beta"], d["g"])
    o_all, f_all = dp.fwd(*args, chunk=w.chunk, workspace=ws)
    o_all2, f_all2 = dp.fwd(*args, chunk=w.chunk, workspace=ws)
    o_sp, f_sp = dp.fwd(*args, chunk=w.chunk, workspace=ws, path="split")
    o_fu = f_fu = None
    if dtype == "bf16":
        o_fu, f_fu = dp.fwd(*args, chunk=w.chunk, workspace=ws, path="fused")
    dp.fwd(*args, chunk=w.chunk, workspace=ws, stages=dp.STAGE_UT)
    o_st, f_st = dp.fwd(*args, chunk=w.chunk, workspace=ws, stages=dp.STAGE_SCAN)
    torch.cuda.synchronize()
    assert torch.equal(o_all, o_all2) and torch.equal(f_all, f_all2)
    assert torch.equal(o_sp, o_st) and torch.equal(f_sp, f_st)
    oo, fo = oracle.fwd(inp["q"], inp["k"], inp["v"], inp["beta"], g=inp["g"], h0=inp["h0"])
    res = dict(out=(f64(o_all), oo), fs=(f64(f_all), fo), out_split=(f64(o_sp), oo), fs_split=(f64(f_sp), fo))
    if o_fu is not None:
        res.update(out_fused=(f64(o_fu), oo), fs_fused=(f64(f_fu), fo))
    check(res, TOL[dtype], f"staged/{dtype}")


@pytest.mark.parametrize("name,kw", [
    ("c2", dict(B=2, H=3, L=203)), ("c3", dict(B=1, H=3, L=150)), ("c3b", dict(B=2, H=2, L=161)),
    ("c4", dict(B=2, H=2, L=300)), ("c3", dict(B=1, H=2, L=150, n_h=1)), ("c3", dict(B=1, H=2, L=99, n_h=5)),
    ("c4", dict(B=1, H=3, L=200, dk=32, dv=64)), ("c4", dict(B=1, H=2, L=200, dk=128, dv=32, chunk=32)),
    ("c3", dict(B=1, H=2, L=77, dk=64, dv=16, chunk=32, n_h=1)),
])
def test_fused_and_split_paths_agree(name, kw):
    """The fused kernel (DP_FWD_FUSED) and the prep / chain pair (DP_FWD_SPLIT)
    are two schedules of the same chunk form: both meet the bound against the
    oracle, across head dims 32..128, chunk 32 and 64, n_h 1..5, gate and h0,
    and the default call equals one of them bit for bit."""
    w = WORKLOADS[name].scaled(**kw)
    say(f"case fused-vs-split {name} {kw}")
    inp = make(w)
    d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    odt = inp.get("out_dtype")
    res = {}
    for path in ("fused", "split", "auto"):
        o, f = dp.fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], chunk=w.chunk, h0=d["h0"],
                      out_dtype=odt, path=path)
        torch.cuda.synchronize()
        res[path] = (f64(o), f64(f))
    auto = "fused" if w.dv <= 32 else "split"
    assert np.array_equal(res["auto"][0], res[auto][0]) and np.array_equal(res["auto"][1], res[auto][1])
    oo, fo = oracle.fwd(inp["q"], inp["k"], inp["v"], inp["beta"], g=inp["g"], h0=inp["h0"])
    check(dict(out=(res["fused"][0], oo), fs=(res["fused"][1], fo), out_split=(res["split"][0], oo),
               fs_split=(res["split"][1], fo)), TOL["bf16"], f"{name}")


def test_out_f32_flag_is_the_unrounded_output():
    """DP_OUT_F32 writes the same values the bf16 output rounds (to nearest even)."""
    w = WORKLOADS["c3"].scaled(B=2, H=2, L=200)
    inp = make(w)
    o16, f16 = gpu_forward(inp, out_dtype=torch.bfloat16)
    o32, f32 = gpu_forward(inp, out_dtype=torch.float32)
    assert o16.dtype == torch.bfloat16 and o32.dtype == torch.float32
    assert torch.equal(o32.to(torch.bfloat16), o16)
    assert torch.equal(f16, f32)


# ------------------------------------------------------------------ exact constructions (fp32 path)

def _f32(*shape):
    return torch.zeros(*shape, dtype=torch.float32)


def test_mod3_rotation_embedded():
    """DeltaProduct notes sec. 2.4 teaching example, zero-padded into dk = dv = 16."""
    L, n = 9, 16
    k = _f32(1, L, 1, 2, n)
    k[..., 0, 0] = 1.0
    k[..., 1, 0] = 0.5
    k[..., 1, 1] = math.sqrt(3) / 2
    beta = torch.full((1, L, 1, 2), 2.0)
    v = _f32(1, L, 1, 2, n)
    h0 = _f32(1, 1, n, n)
    h0[0, 0, 0, 0] = 1.0
    h0[0, 0, 1, 1] = 1.0
    R = np.array([[-0.5, -math.sqrt(3) / 2], [math.sqrt(3) / 2, -0.5]])
    rows = []
    for r in range(2):
        q = _f32(1, L, 1, n)
        q[..., r] = 1.0
        out, fs = dp.fwd(q.cuda(), k.cuda(), v.cuda(), beta.cuda(), chunk=16, h0=h0.cuda())
        torch.cuda.synchronize()
        rows.append(out.cpu().numpy()[0, :, 0, :2])
    for t in range(L):
        At = np.linalg.matrix_power(R, t + 1)
        got = np.stack([rows[0][t], rows[1][t]])
        np.testing.assert_allclose(got, At, atol=2e-6)
        if (t + 1) % 3 == 0:
            np.testing.assert_allclose(got, np.eye(2), atol=2e-6)


def test_swap_reflections_embedded():
    """DeltaProduct notes sec. 3.1: reflections k = (e_a - e_b)/sqrt2, beta = 2 permute rows."""
    n, dk = 5, 16
    perm = [3, 0, 4, 1, 2]
    cur = list(range(n))
    swaps = []
    for i in range(n - 1):
        j = cur.index(perm[i])
        if j != i:
            swaps.append((i, j))
            cur[i], cur[j] = cur[j], cur[i]
    n_h = n - 1
    k = _f32(1, 1, 1, n_h, dk)
    beta = _f32(1, 1, 1, n_h)
    for s, pair in enumerate(swaps):
        a, b = pair
        k[0, 0, 0, s, a] = 1 / math.sqrt(2)
        k[0, 0, 0, s, b] = -1 / math.sqrt(2)
        beta[0, 0, 0, s] = 2.0
    for s in range(len(swaps), n_h):
        k[0, 0, 0, s, 0] = 1.0  # beta = 0: identity factor
    h0 = _f32(1, 1, dk, 16)
    h0[0, 0, :n, 0] = torch.arange(1.0, n + 1)
    out, fs = dp.fwd(_f32(1, 1, 1, dk).cuda(), k.cuda(), _f32(1, 1, 1, n_h, 16).cuda(),
                     beta.cuda(), chunk=16, h0=h0.cuda())
    torch.cuda.synchronize()
    got = fs.cpu().numpy()[0, 0, :n, 0]
    np.testing.assert_allclose(got, np.arange(1.0, n + 1)[perm], atol=1e-5)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gate_zero_reset(dtype):
    """DeltaProduct notes sec. 3.3: g = 0 erases the history (here mid-chunk)."""
    w = WORKLOADS["c4"].scaled(B=1, H=2, L=120, dk=32, dv=32, dtype=dtype)
    base = make(w)
    base["g"][:, 45] = 0.0
    outs = []
    for seed in (0, 1):
        inp = {k: (v.clone() if isinstance(v, torch.Tensor) else v) for k, v in base.items()}
        gen = torch.Generator().manual_seed(77 + seed)
        inp["k"][:, :45] = torch.randn(inp["k"][:, :45].shape, generator=gen).to(inp["k"].dtype)
        inp["v"][:, :45] = torch.randn(inp["v"][:, :45].shape, generator=gen).to(inp["v"].dtype)
        say(f"case gate-reset dtype={dtype} history={seed}")
        res = run_pair(inp)
        check(res, TOL[dtype], f"reset-{seed}")
        outs.append(res["out"][0])
    after = slice(45, None)
    assert rel_err(outs[0][:, after], outs[1][:, after]) <= (1e-5 if dtype == "f32" else 1e-2)


# ------------------------------------------------------------------ edge cases

EDGE = [
    dict(B=1, H=1, L=1, n_h=4, dk=16, dv=128, chunk=64),     # one token, one partial chunk
    dict(B=1, H=3, L=40, n_h=1, dk=128, dv=16, chunk=32),    # B*H not a multiple of 8
    dict(B=2, H=1, L=29, n_h=5, dk=32, dv=64, chunk=64),     # n_h = 5: 13 readouts / chunk
    dict(B=1, H=2, L=9, n_h=17, dk=16, dv=32, chunk=16),     # n_h > chunk
    dict(B=1, H=1, L=64, n_h=2, dk=64, dv=32, chunk=16),     # exact multiple of chunk
    dict(B=1, H=2, L=45, n_h=3, dk=64, dv=64, chunk=32),     # 11 readouts in a 16-row tile
    dict(B=2, H=1, L=37, n_h=7, dk=128, dv=32, chunk=64),    # 10 readouts in a 16-row tile
]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", EDGE, ids=[f"e{i}" for i in range(len(EDGE))])
def test_edge_shapes(shape, dtype):
    w = WORKLOADS["c2"].scaled(dtype=dtype, **shape)
    say(f"case edge {shape} {dtype}")
    inp = make(w)
    check(run_pair(inp), TOL[dtype], "edge")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_degenerate_inputs(dtype):
    """beta outside [0, 2] is clamped, zero keys are no-op sub-steps."""
    w = WORKLOADS["c2"].scaled(B=1, H=2, L=70, dk=32, dv=32, dtype=dtype)
    inp = make(w)
    inp["beta"][:, ::5] = 3.5
    inp["beta"][:, 1::7] = -1.0
    inp["k"][:, 2::9, :, 1] = 0
    check(run_pair(inp), TOL[dtype], "degenerate")


def test_empty_sequence_copies_state():
    w = WORKLOADS["c4"].scaled(B=2, H=3, L=0, dk=32, dv=16, dtype="bf16")
    inp = make(w)
    out, fs = gpu_forward(inp)
    assert out.numel() == 0
    assert torch.equal(fs.cpu(), inp["h0"])
    out, fs = gpu_forward(inp, h0=None)
    assert torch.equal(fs.cpu(), torch.zeros_like(inp["h0"]))


def test_errors_surface_as_exceptions():
    w = WORKLOADS["c2"].scaled(B=1, H=1, L=8)
    d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in make(w).items()}
    tiny = torch.empty(16, dtype=torch.uint8, device="cuda")
    # the two-kernel path keeps its operand blocks in the workspace
    with pytest.raises(dp.DPError) as ei:
        dp.fwd(d["q"], d["k"], d["v"], d["beta"], chunk=64, workspace=tiny, path="split")
    assert ei.value.code == dp.binding.DP_EWORKSPACE
    # the fused kernel needs none
    dp.fwd(d["q"], d["k"], d["v"], d["beta"], chunk=64, workspace=tiny, path="fused")
    torch.cuda.synchronize()
    with pytest.raises(dp.DPError):
        dp.fwd(d["q"], d["k"], d["v"], d["beta"], chunk=48)


# ------------------------------------------------------------------ phase 1 alone

@pytest.mark.parametrize("dtype,dk", [("f32", 16), ("bf16", 32), ("f32", 32), ("bf16", 64), ("bf16", 128),
                                      ("f32", 128)])
def test_precond_parity(dtype, dk):
    w = WORKLOADS["c5"].scaled(B=2, H=5, L=301, dk=dk, dv=dk, dtype=dtype)
    inp = make(w)
    k1 = inp["k"][:, :, :, 0, :].contiguous()
    b1 = inp["beta"][..., 0].contiguous()
    say(f"case precond {dtype} dk={dk}")
    ktg, dg = dp.osdn_precond(k1.cuda(), b1.cuda(), eta=0.05)
    torch.cuda.synchronize()
    kto, do = oracle.precond(k1, b1, eta=0.05)
    check(dict(kt=(f64(ktg), kto), d=(f64(dg), do)), TOL[dtype], "precond")
    assert float(dg.min()) >= 0.5 and float(dg.max()) <= 2.0


# the scan works in blocks of 64 tokens (bf16) or 32 (fp32) at dk >= 64 and in
# blocks of 16 / 8 with 16 or 32 lanes per head below: sequences shorter than,
# equal to and one past a block, and an odd number of heads per wavefront
@pytest.mark.parametrize("dtype,dk,B,H,L", [("bf16", 128, 1, 3, 1), ("bf16", 128, 2, 1, 7), ("bf16", 128, 1, 2, 64),
                                            ("bf16", 128, 1, 2, 65), ("f32", 128, 1, 2, 33), ("f32", 64, 3, 1, 32),
                                            ("bf16", 32, 1, 3, 17), ("f32", 16, 1, 5, 9), ("bf16", 16, 2, 3, 16)])
def test_precond_block_edges(dtype, dk, B, H, L):
    w = WORKLOADS["c5"].scaled(B=B, H=H, L=L, dk=dk, dv=dk, dtype=dtype)
    inp = make(w)
    k1 = inp["k"][:, :, :, 0, :].contiguous()
    b1 = inp["beta"][..., 0].contiguous()
    say(f"case precond edges {dtype} dk={dk} B={B} H={H} L={L}")
    ktg, dg = dp.osdn_precond(k1.cuda(), b1.cuda(), eta=0.05)
    torch.cuda.synchronize()
    kto, do = oracle.precond(k1, b1, eta=0.05)
    check(dict(kt=(f64(ktg), kto), d=(f64(dg), do)), TOL[dtype], "precond edges")
