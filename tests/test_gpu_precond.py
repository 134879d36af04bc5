"""GPU parity of the phase-1 variants (OSDN notes sec. 2.6: the APF retention
gate of d; sec. 2.7: the beta-free step of the 1.3B configuration, with the
box kept or dropped) against the fp64 oracle, alone and feeding the
write-key forward.  Errors: max|x_gpu - x_oracle| / RMS(x_oracle) per tensor,
bounded by 1e-4 (fp32) and 2e-2 (bf16)."""
import numpy as np
import pytest
import torch

import linear_rnn_sequence_amd as dp
import oracle
from linear_rnn_sequence_amd.inputs import WORKLOADS, make, retention, sampled_heads, \
    select_heads, select_state
from parity import TOL, check_bf16_stored, f64, gpu_forward, rel_err, say

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


def check_phase1(ktg, kto, dg, do, dtype, label):
    if dtype == "bf16":
        check_bf16_stored(f64(ktg), kto, label)
        check(dict(d=(f64(dg), do)), TOL[dtype], label)
    else:
        check(dict(kt=(f64(ktg), kto), d=(f64(dg), do)), TOL[dtype], label)


VARIANTS = [
    # (retention, beta_aware, box)
    (True, True, (0.5, 2.0)),          # APF
    (False, False, (0.5, 2.0)),        # beta-free step
    (True, False, (0.5, 2.0)),         # both (the 1.3B configuration with the box)
    (True, False, (-np.inf, np.inf)),  # the 1.3B update as printed, no projection
]


@pytest.mark.parametrize("dtype,dk", [("f32", 16), ("f32", 128), ("bf16", 64), ("bf16", 128)])
@pytest.mark.parametrize("ret,aware,box", VARIANTS, ids=["apf", "betafree", "both", "open"])
def test_precond_variant_parity(dtype, dk, ret, aware, box):
    w = WORKLOADS["c5"].scaled(B=2, H=5, L=301, dk=dk, dv=dk, dtype=dtype)
    inp = make(w)
    k1 = inp["k"][:, :, :, 0, :].contiguous()
    b1 = inp["beta"][..., 0].contiguous()
    # with the box dropped, the retention is drawn near 1 (sigmoid(N(0,1) + 6) ~ 0.9975,
    # the 1.3B configuration initialises its gate at about 0.999); r ~ 0.95 with no floor
    # would shrink d, and the stored bf16 write keys with it, by two orders of magnitude
    # within the sequence, and the bf16 rounding of the early keys alone would then
    # exceed the error bound relative to the RMS
    bias = 3.0 if np.isfinite(box[0]) else 6.0
    r = retention(w.B, w.L, w.H, seed=w.seed + 7, bias=bias) if ret else None
    say(f"case precond-variant {dtype} dk={dk} retention={ret} beta_aware={aware} box={box}")
    ktg, dg = dp.osdn_precond(k1.cuda(), b1.cuda(), eta=0.05, dmin=box[0], dmax=box[1],
                              r=None if r is None else r.cuda(), beta_aware=aware)
    torch.cuda.synchronize()
    kto, do = oracle.precond(k1, b1, eta=0.05, dmin=box[0], dmax=box[1], r=r, beta_aware=aware)
    check_phase1(ktg, kto, dg, do, dtype, "precond-variant")
    if np.isfinite(box[0]):
        assert float(dg.min()) >= box[0] and float(dg.max()) <= box[1]


def test_precond_retention_one_is_the_plain_scan():
    """r = 1 everywhere goes through the variant entry point and must give
    exactly (bit for bit) what the plain entry point gives."""
    w = WORKLOADS["c5"].scaled(B=2, H=3, L=200)
    inp = make(w)
    k1 = inp["k"][:, :, :, 0, :].contiguous().cuda()
    b1 = inp["beta"][..., 0].contiguous().cuda()
    kt0, d0 = dp.osdn_precond(k1, b1)
    kt1, d1 = dp.osdn_precond(k1, b1, r=torch.ones(2, 200, 3, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(kt0, kt1) and torch.equal(d0, d1)


def test_apf_phase1_feeds_the_write_key_forward():
    """APF phase 1 then the write-key forward (bf16), end to end, against the
    oracle running both phases."""
    w = WORKLOADS["c5"].scaled(B=2, H=3, L=257)
    inp = make(w)
    k1 = inp["k"][:, :, :, 0, :].contiguous()
    b1 = inp["beta"][..., 0].contiguous()
    r = retention(w.B, w.L, w.H, seed=w.seed + 9)
    ktg, dg = dp.osdn_precond(k1.cuda(), b1.cuda(), r=r.cuda())
    out, fs = gpu_forward(inp, kt=ktg.unsqueeze(3))
    kto, do = oracle.precond(k1, b1, r=r)
    oo, fo = oracle.fwd(inp["q"], inp["k"], inp["v"], inp["beta"], kt=kto[:, :, :, None, :])
    check_phase1(ktg, kto, dg, do, "bf16", "apf+fwd")
    check(dict(out=(f64(out), oo), fs=(f64(fs), fo)), TOL["bf16"], "apf+fwd")


def test_precond_variants_full_size_sampled_heads():
    """The write-key workload's phase-1 size (B=8, H=16, L=4096, dk=128, bf16)
    with the retention gate and the beta-free step, checked on sampled heads."""
    w = WORKLOADS["c5"]
    inp = make(w)
    k1 = inp["k"][:, :, :, 0, :].contiguous()
    b1 = inp["beta"][..., 0].contiguous()
    r = retention(w.B, w.L, w.H, seed=w.seed + 11)
    ktg, dg = dp.osdn_precond(k1.cuda(), b1.cuda(), r=r.cuda(), beta_aware=False)
    torch.cuda.synchronize()
    heads = sampled_heads(w.B, w.H, 12)
    kto, do = oracle.precond(select_heads(k1, heads, w.H), select_heads(b1, heads, w.H),
                             r=select_heads(r, heads, w.H), beta_aware=False)
    check_phase1(select_heads(ktg.cpu(), heads, w.H), kto, select_state(dg.cpu(), heads, w.H), do,
                 "bf16", "full-c5-variant")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_precond_clamps_and_nans_inside_full_blocks(dtype):
    """The dk >= 64 scan runs each full block of tokens speculatively (no
    coordinate clamped) and falls back to the exact step when a clamp or a NaN
    shows up.  With eta = 0.5 the box [0.5, 2] binds inside full blocks, and a
    NaN beta in the middle of a block of one head must poison that head from
    the next token on exactly as the oracle's clamp (which keeps NaN) does,
    while the other heads meet the bound.  With eta = 0.5 and the box [0.9,
    1.1] the clean heads first clamp at tokens 74 and 95, inside full blocks,
    and clamp on most tokens after that."""
    w = WORKLOADS["c5"].scaled(B=1, H=3, L=256, dk=128, dv=128, dtype=dtype)
    inp = make(w)
    k1 = inp["k"][:, :, :, 0, :].contiguous()
    b1 = inp["beta"][..., 0].contiguous().clone()
    b1[0, 100, 1] = float("nan")
    say(f"case precond clamps/NaN {dtype}")
    ktg, dg = dp.osdn_precond(k1.cuda(), b1.cuda(), eta=0.5, dmin=0.9, dmax=1.1)
    torch.cuda.synchronize()
    kto, do = oracle.precond(k1, b1, eta=0.5, dmin=0.9, dmax=1.1)
    g, o = f64(ktg), kto
    assert np.array_equal(np.isnan(g), np.isnan(o)), "NaN positions of the write keys differ"
    assert np.array_equal(np.isnan(f64(dg)), np.isnan(do))
    assert np.isnan(o[0, 101:, 1]).all() and not np.isnan(o[0, :101, 1]).any()
    keep = [0, 2]
    check_phase1(ktg[:, :, keep], kto[:, :, keep], dg[:, keep], do[:, keep], dtype, "clamps")
    # the box binds: some coordinates of the clean heads end on a bound
    dd = do[:, keep]
    assert (np.abs(dd - 0.9) < 1e-9).any() or (np.abs(dd - 1.1) < 1e-9).any()
