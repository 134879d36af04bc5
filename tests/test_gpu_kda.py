"""GPU parity of the chunkwise forward with the KDA host's per-key-channel gate.

OSDN notes sec. 2.7: before token t's sub-steps the state's row c (key channel c)
is multiplied by alpha_t[c] (then by the scalar gate g_t when given).  The oracle
applies that definition token by token (`oracle.fwd(..., ga=...)`, pinned on the
CPU by the per-channel gate pins); the GPU runs the UT and scan kernels in their
per-channel-gate form.  Errors are max|x_gpu - x_oracle| / RMS(x_oracle), bounded
by 1e-4 (fp32) and 2e-2 (bf16).  bf16 cases are checked with fp32 output (the
computation) and their bf16 output must be exactly that output rounded.
"""
import numpy as np
import pytest
import torch

import linear_rnn_sequence_amd as dp
import oracle
from linear_rnn_sequence_amd.inputs import WORKLOADS, channel_gate, make, sampled_heads, select_heads, \
    select_state, write_keys
from parity import TOL, f64, rel_err, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    dp.load()  # raises when libdp.so is missing: no silent fallback


def check(pairs, tol, label):
    for name, (x, ref) in pairs.items():
        e = rel_err(x, ref)
        say(f"  {label} {name}: err {e:.3e} (tol {tol:.0e})")
        assert np.all(np.isfinite(x)), f"{label} {name}: non-finite values"
        assert e <= tol, f"{label} {name}: err {e:.3e} > {tol}"


def run_case(w, ga, kt=None, label=""):
    inp = make(w)
    d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    kk = None if kt is None else kt.cuda()
    o32, f32 = dp.fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], chunk=w.chunk, h0=d["h0"], kt=kk,
                      ga=ga.cuda(), out_dtype=torch.float32)
    if w.dtype == "bf16":
        o16, f16 = dp.fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], chunk=w.chunk, h0=d["h0"], kt=kk,
                          ga=ga.cuda(), out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    oo, fo = oracle.fwd(inp["q"], inp["k"], inp["v"], inp["beta"], g=inp["g"], kt=kt, h0=inp["h0"], ga=ga)
    check(dict(out=(f64(o32), oo), fs=(f64(f32), fo)), TOL[w.dtype], label)
    if w.dtype == "bf16":
        assert torch.equal(o32.to(torch.bfloat16), o16) and torch.equal(f32, f16)


# (workload, overrides, gate floor lo, write keys): head dims 16..128, chunk 16/32/64,
# n_h 1..3, scalar gate and h0, ragged tails, fast-decaying channels
CASES = [
    ("c3", dict(B=1, H=2, L=150), 0.6, False),
    ("c3", dict(B=2, H=1, L=77, n_h=1, chunk=32), 0.6, False),
    ("c4", dict(B=1, H=2, L=130, dk=64, dv=64), 0.6, False),            # with g and h0
    ("c2", dict(B=1, H=3, L=91, n_h=2, dk=32, dv=64, chunk=64), 0.05, False),  # fast decay
    ("c5", dict(B=2, H=2, L=100, dk=64, dv=32), 0.6, True),             # write keys
    ("c1", dict(B=1, H=2, L=45, n_h=3), 0.6, False),                    # dk 16, chunk 16
]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("name,kw,lo,wk", CASES, ids=[f"{c[0]}-{i}" for i, c in enumerate(CASES)])
def test_channel_gate_forward_matches_oracle(name, kw, lo, wk, dtype):
    w = WORKLOADS[name].scaled(dtype=dtype, **kw)
    say(f"case kda {name} {kw} lo={lo} wk={wk} dtype={dtype}")
    ga = channel_gate(w.B, w.L, w.H, w.dk, seed=w.seed + 11, lo=lo)
    kt = write_keys(w, seed=w.seed + 5) if wk else None
    run_case(w, ga, kt, f"kda-{name}/{dtype}")


def test_channel_gate_of_ones_is_the_ungated_forward():
    """alpha = 1 everywhere leaves only the scalar gate: the result equals the
    ungated forward's oracle (and the decay machinery multiplies by exactly 1)."""
    w = WORKLOADS["c4"].scaled(B=1, H=2, L=140, dk=64, dv=64, dtype="f32")
    inp = make(w)
    ga = torch.ones(w.B, w.L, w.H, w.dk)
    d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    o, f = dp.fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], chunk=w.chunk, h0=d["h0"], ga=ga.cuda())
    torch.cuda.synchronize()
    oo, fo = oracle.fwd(inp["q"], inp["k"], inp["v"], inp["beta"], g=inp["g"], h0=inp["h0"])
    check(dict(out=(f64(o), oo), fs=(f64(f), fo)), TOL["f32"], "ga=1")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_channel_gate_prefill_then_decode(dtype):
    """A chunkwise prefill with the channel gate hands its final state to the
    decode step, which continues with the same gate: together they equal the
    oracle over the whole sequence."""
    w = WORKLOADS["c3"].scaled(B=1, H=2, L=140, dk=64, dv=64, dtype=dtype)
    inp = make(w)
    ga = channel_gate(w.B, w.L, w.H, w.dk, seed=w.seed + 13)
    L0 = 128
    d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    cut = lambda x, a, b: None if x is None else x[:, a:b].contiguous()
    o1, st = dp.fwd(cut(d["q"], 0, L0), cut(d["k"], 0, L0), cut(d["v"], 0, L0), cut(d["beta"], 0, L0),
                    chunk=w.chunk, ga=cut(ga, 0, L0).cuda(), out_dtype=torch.float32)
    outs = []
    for t in range(L0, w.L):
        tok = lambda x: x[:, t].contiguous()
        outs.append(dp.decode(tok(d["q"]), tok(d["k"]), tok(d["v"]), tok(d["beta"]), st,
                              ga=tok(ga).cuda(), out_dtype=torch.float32))
    torch.cuda.synchronize()
    oo, fo = oracle.fwd(inp["q"], inp["k"], inp["v"], inp["beta"], ga=ga)
    got = torch.cat([o1.cpu(), torch.stack([o.cpu() for o in outs], dim=1)], dim=1)
    check(dict(out=(f64(got), oo), fs=(f64(st), fo)), TOL[dtype], f"kda-prefill/{dtype}")


def test_channel_gate_full_size_sampled_heads():
    """The LM-layer shape (B=4, H=16, L=4096, n_h=3, dk=dv=128, bf16) with the
    channel gate, checked on sampled heads (fp32 output)."""
    w = WORKLOADS["c3"]
    inp = make(w)
    ga = channel_gate(w.B, w.L, w.H, w.dk, seed=w.seed + 17, lo=0.9)
    d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}
    say("case kda full size c3")
    o, f = dp.fwd(d["q"], d["k"], d["v"], d["beta"], chunk=w.chunk, ga=ga.cuda(), out_dtype=torch.float32)
    torch.cuda.synchronize()
    heads = sampled_heads(w.B, w.H, 4)
    sel = lambda t: select_heads(t, heads, w.H)
    oo, fo = oracle.fwd(sel(inp["q"]), sel(inp["k"]), sel(inp["v"]), sel(inp["beta"]), ga=sel(ga))
    got_o = f64(sel(o.cpu()))
    got_f = f64(select_state(f.cpu(), heads, w.H))
    check(dict(out=(got_o, oo), fs=(got_f, fo)), TOL["bf16"], "kda-full")


def test_channel_gate_rejects_the_fused_path():
    w = WORKLOADS["c3"].scaled(B=1, H=1, L=64, dv=32)
    d = {k: (v.cuda() if isinstance(v, torch.Tensor) else v) for k, v in make(w).items()}
    ga = torch.ones(1, 64, 1, 128, device="cuda")
    with pytest.raises(dp.DPError) as ei:
        dp.fwd(d["q"], d["k"], d["v"], d["beta"], chunk=64, ga=ga, path="fused")
    assert ei.value.code == dp.binding.DP_ENOTSUP
