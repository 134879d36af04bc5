"""GPU parity of the OSDN backward with the fp64 oracle's gradient.

Three pieces, each against its oracle (pinned on the CPU by finite
differences, tests/test_oracle_bwd_pins.py):

* the write-key forward's gradient (dp.bwd with kt: dp_bwd_wk_*) against
  oracle.bwd with the same write keys, for every input and for kt;
* phase 1's gradient (dp.osdn_precond_bwd) against oracle.precond_bwd, with
  retention, the beta-free step, a clamping box, d0 and a final-d gradient
  (for dk >= 64 the forward pass inside it runs in 64-token chunks and hands
  a head to the sequential scan where the box comes near: cases where that
  happens on some heads late in the sequence, and on every head at once);
* the whole layer (dp.osdn_bwd: phase 1, then the write-key forward, n_h = 1)
  against oracle.osdn_bwd, small and at the full c5 shape on sampled heads.

Errors are max|x_gpu - x_oracle| / RMS(x_oracle) per gradient, bounded by 1e-4
for fp32 inputs and 2e-2 for bf16 inputs (all arithmetic is fp32).
"""
import numpy as np
import pytest
import torch

import linear_rnn_sequence_amd as dp
import oracle
from linear_rnn_sequence_amd.inputs import WORKLOADS, make, make_grads, retention, select_heads, \
    select_state, write_keys
from parity import TOL, f64, rel_err, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    dp.load()  # raises when libdp.so is missing: no silent fallback


def check(got, ref, tol, label, names=None):
    for n in (names or ref):
        x, r = f64(got[n]), ref[n]
        assert x.shape == r.shape, f"{label} d{n}: shape {x.shape} vs {r.shape}"
        assert np.all(np.isfinite(x)), f"{label} d{n}: non-finite values"
        e = rel_err(x, r)
        say(f"  {label} d{n}: err {e:.3e} (tol {tol:.0e})")
        assert e <= tol, f"{label} d{n}: err {e:.3e} > {tol}"


def cuda(x):
    return None if x is None else x.cuda()


# ------------------------------------------------------------------ write-key forward's gradient

WK = [  # workload, overrides, final-state gradient: n_h 1..3, head dims 16..128, gate and h0
    ("c5", dict(B=2, H=1, L=70, dk=64, dv=64), True),
    ("c5", dict(B=1, H=2, L=45, n_h=3, dk=128, dv=32, dtype="f32"), False),
    ("c4", dict(B=1, H=2, L=50, dk=32, dv=128, asym=True), True),        # gate, h0
    ("c1", dict(B=1, H=2, L=40, dk=16, dv=16, asym=True), True),
    ("c4", dict(B=1, H=1, L=33, n_h=2, dk=128, dv=128, dtype="f32", asym=True), True),
]


@pytest.mark.parametrize("name,kw,final", WK, ids=[f"{c[0]}-{i}" for i, c in enumerate(WK)])
def test_write_key_backward_matches_oracle(name, kw, final):
    w = WORKLOADS[name].scaled(**kw)
    say(f"case bwd-wk {name} {kw} dtype={w.dtype}")
    inp = make(w)
    gr = make_grads(w, final=final)
    kt = write_keys(w, seed=w.seed + 7)
    out = dp.bwd(cuda(inp["q"]), cuda(inp["k"]), cuda(inp["v"]), cuda(inp["beta"]), cuda(gr["dout"]),
                 g=cuda(inp["g"]), h0=cuda(inp["h0"]), dfinal=cuda(gr["dfinal"]), kt=cuda(kt))
    torch.cuda.synchronize()
    got = {n: t.cpu() for n, t in out.items()}
    ref = oracle.bwd(inp["q"], inp["k"], inp["v"], inp["beta"], gr["dout"], g=inp["g"], kt=kt, h0=inp["h0"],
                     dfinal=gr["dfinal"])
    assert set(got) == set(ref)
    check(got, ref, TOL[w.dtype], f"wk-{name}/{w.dtype}")


# ------------------------------------------------------------------ phase 1's gradient

def p1_inputs(B, L, H, dk, dtype, seed):
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    k = torch.randn(B, L, H, dk, generator=gen).to(dtype)
    beta = torch.sigmoid(torch.randn(B, L, H, generator=gen))
    dkt = torch.randn(B, L, H, dk, generator=gen)
    d0 = 0.8 + 0.6 * torch.rand(B, H, dk, generator=gen)
    ddf = torch.randn(B, H, dk, generator=gen)
    return k, beta, dkt, d0, ddf


P1 = [  # (B, L, H, dk), options
    ((2, 150, 2, 128), dict()),
    ((1, 70, 3, 64), dict(ret=True, d0=True, final=True)),
    ((2, 90, 1, 32), dict(beta_free=True, ret=True)),
    ((1, 40, 5, 16), dict(eta=0.5, dmin=0.9, dmax=1.1, d0=True)),        # clamps bind
    ((1, 64, 2, 128), dict(eta=0.05, dmin=float("-inf"), dmax=float("inf"), final=True)),  # open box
    # dk >= 64 replays phase 1 in 64-token chunks and hands a head to the
    # sequential scan from the chunk where a step first comes near the box.
    # The bound is crossed by a decay of 1% (or ~5%) a token, so no step ends
    # within rounding of it (there the clamp's gradient, 0 or 1, would be
    # decided by rounding alone):
    ((2, 300, 3, 128), dict(ret="late")),           # heads 0 and 2 reach dmin near token 69
    ((2, 300, 3, 128), dict(ret=True, d0=True)),    # every head, in the first chunk
]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape,opt", P1, ids=[str(i) for i in range(len(P1))])
def test_phase1_backward_matches_oracle(shape, opt, dtype):
    B, L, H, dk = shape
    say(f"case p1-bwd {shape} {opt} {dtype}")
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    k, beta, dkt, d0, ddf = p1_inputs(B, L, H, dk, tdt, seed=31 + L)
    r = retention(B, L, H, seed=5 + L) if opt.get("ret") else None
    if opt.get("ret") == "late":
        r = torch.ones(B, L, H)
        r[:, :, 0::2] = 0.99
    d0 = d0 if opt.get("d0") else None
    ddf = ddf if opt.get("final") else None
    kw = dict(eta=opt.get("eta", 3e-3), dmin=opt.get("dmin", 0.5), dmax=opt.get("dmax", 2.0),
              beta_aware=not opt.get("beta_free", False))
    out = dp.osdn_precond_bwd(k.cuda(), beta.cuda(), dkt.cuda(), d0=cuda(d0), dd_final=cuda(ddf), r=cuda(r), **kw)
    torch.cuda.synchronize()
    got = {n: t.cpu() for n, t in out.items()}
    ref = oracle.precond_bwd(k, beta, dkt, d0=d0, dd_final=ddf, r=r, **kw)
    assert set(got) == set(ref)
    check(got, ref, TOL[dtype], f"p1/{dtype}")
    if not kw["beta_aware"]:
        assert torch.all(got["beta"] == 0)


def test_phase1_backward_accumulates_and_handles_empty():
    """dk and dbeta are added into (they may hold the write-key forward's
    gradients already); with L = 0 the gradient on d_1 is the final d's."""
    B, L, H, dk = 1, 50, 2, 64
    k, beta, dkt, d0, ddf = p1_inputs(B, L, H, dk, torch.float32, seed=77)
    base_k = torch.randn(B, L, H, dk)
    base_b = torch.randn(B, L, H)
    out = dp.osdn_precond_bwd(k.cuda(), beta.cuda(), dkt.cuda(), dk=base_k.clone().cuda(),
                              dbeta=base_b.clone().cuda())
    torch.cuda.synchronize()
    ref = oracle.precond_bwd(k, beta, dkt)
    for n, base in (("k", base_k), ("beta", base_b)):
        # out = base + gradient, rounded once in fp32: the bound is the fp32
        # tolerance of the gradient plus the rounding of the sum
        err = np.max(np.abs(f64(out[n]) - f64(base) - ref[n]))
        bound = TOL["f32"] * np.sqrt(np.mean(ref[n] ** 2)) + 2.0 ** -22 * np.max(np.abs(f64(base) + ref[n]))
        say(f"  p1-acc d{n}: err {err:.3e} (bound {bound:.3e})")
        assert err <= bound
    e = dp.osdn_precond_bwd(torch.zeros(B, 0, H, dk).cuda(), torch.zeros(B, 0, H).cuda(),
                            torch.zeros(B, 0, H, dk).cuda(), dd_final=ddf.cuda())
    torch.cuda.synchronize()
    assert torch.equal(e["d0"].cpu(), ddf)


# ------------------------------------------------------------------ the whole OSDN layer

def osdn_inputs(w, gate=False, h0=False, final=False, ret=False, d0=False):
    inp = make(w)
    gr = make_grads(w, final=final)
    x = dict(q=inp["q"], k=inp["k"][:, :, :, 0].contiguous(), v=inp["v"][:, :, :, 0].contiguous(),
             beta=inp["beta"][..., 0].contiguous(), dout=gr["dout"], dfinal=gr["dfinal"])
    gen = torch.Generator(device="cpu")
    gen.manual_seed(w.seed + 99)
    x["g"] = (0.9 + 0.1 * torch.rand(w.B, w.L, w.H, generator=gen)) if gate else None
    x["h0"] = 0.1 * torch.randn(w.B, w.H, w.dk, w.dv, generator=gen) if h0 else None
    x["r"] = retention(w.B, w.L, w.H, seed=w.seed + 3) if ret else None
    x["d0"] = (0.8 + 0.6 * torch.rand(w.B, w.H, w.dk, generator=gen)) if d0 else None
    return x


def gpu_osdn_bwd(x, **kw):
    out = dp.osdn_bwd(cuda(x["q"]), cuda(x["k"]), cuda(x["v"]), cuda(x["beta"]), cuda(x["dout"]),
                      g=cuda(x["g"]), h0=cuda(x["h0"]), dfinal=cuda(x["dfinal"]), r=cuda(x["r"]),
                      d0=cuda(x["d0"]), **kw)
    torch.cuda.synchronize()
    return {n: t.cpu() for n, t in out.items()}


OSDN = [  # overrides, options
    (dict(B=2, H=2, L=100, dk=64, dv=64), dict()),
    (dict(B=1, H=2, L=130, dk=128, dv=128, dtype="f32"), dict(gate=True, h0=True, final=True)),
    (dict(B=1, H=3, L=77, dk=32, dv=16), dict(ret=True, d0=True, final=True)),
    (dict(B=2, H=1, L=64, dk=128, dv=32, dtype="f32"), dict(ret=True, beta_free=True)),
    (dict(B=1, H=2, L=40, dk=16, dv=64), dict(gate=True)),
]


@pytest.mark.parametrize("kw,opt", OSDN, ids=[str(i) for i in range(len(OSDN))])
def test_osdn_layer_backward_matches_oracle(kw, opt):
    w = WORKLOADS["c5"].scaled(**kw)
    say(f"case osdn-bwd {kw} {opt} dtype={w.dtype}")
    x = osdn_inputs(w, **{k: v for k, v in opt.items() if k != "beta_free"})
    ba = not opt.get("beta_free", False)
    got = gpu_osdn_bwd(x, beta_aware=ba)
    ref = oracle.osdn_bwd(x["q"], x["k"], x["v"], x["beta"], x["dout"], g=x["g"], h0=x["h0"], dfinal=x["dfinal"],
                          d0=x["d0"], r=x["r"], beta_aware=ba)
    assert set(got) == set(ref)
    check(got, ref, TOL[w.dtype], f"osdn/{w.dtype}")


def test_osdn_layer_backward_full_size_sampled_heads():
    """The full write-key workload B=8, H=16, L=4096, dk=dv=128 (bf16) in one
    call, against the oracle on three sampled heads."""
    w = WORKLOADS["c5"]
    x = osdn_inputs(w)
    say(f"case osdn-bwd full c5: B={w.B} H={w.H} L={w.L}")
    got = gpu_osdn_bwd(x)
    heads = [0, 61, 127]
    sel = lambda t: None if t is None else select_heads(t, heads, w.H)
    ref = oracle.osdn_bwd(sel(x["q"]), sel(x["k"]), sel(x["v"]), sel(x["beta"]), sel(x["dout"]), nthreads=3)
    pick = {n: select_heads(got[n], heads, w.H) for n in ("q", "k", "v", "beta")}
    pick["h0"] = select_state(got["h0"], heads, w.H)
    pick["d0"] = select_state(got["d0"], heads, w.H)
    check(pick, ref, TOL["bf16"], "c5-full", names=["q", "k", "v", "beta", "h0", "d0"])
