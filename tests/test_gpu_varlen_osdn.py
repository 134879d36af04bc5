"""GPU parity of the packed variable-length OSDN path: phase 1 on packed
sequences (each from its own d) and the write-key forward on them.

The pages pack training documents into one token tensor and restart the
recurrent state at every document boundary; the plain reading for OSDN is that
both the memory S and the preconditioner d restart, so each packed sequence is
an independent phase 1 + phase 2.  Each sequence is therefore checked against
the fp64 oracle run on it alone (max|x_gpu - x_oracle| / RMS(x_oracle), bounded
by 1e-4 for f32 and 2e-2 for bf16; write keys stored in bf16 element by element
within bf16 rounding of the oracle's) and against the fixed-length entry points
run on it alone, bit for bit.
"""
import numpy as np
import pytest
import torch

import linear_rnn_sequence_amd as dp
import oracle
from linear_rnn_sequence_amd.inputs import WORKLOADS, make, retention
from parity import TOL, check_bf16_stored, f64, rel_err, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    dp.load()  # raises when libdp.so is missing: no silent fallback


def offsets(lengths):
    return torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int32)


def packed_keys(H, dk, lengths, dtype, seed=0):
    """Keys k [T,H,dk], beta [T,H] of the write-key workload's distributions,
    T = sum(lengths), plus a retention gate r [T,H] (the APF recipe) and a
    start d per sequence [nseq,H,dk] in [0.5, 2]."""
    T = int(sum(lengths))
    w = WORKLOADS["c5"].scaled(B=1, L=T, H=H, dk=dk, dtype=dtype)
    inp = make(w, seed=w.seed + seed)
    k = inp["k"][0, :, :, 0].contiguous()
    b = inp["beta"][0, :, :, 0].contiguous()
    r = retention(1, T, H, seed=w.seed + 7 + seed)[0].contiguous()
    gen = torch.Generator().manual_seed(41 + seed)
    d0 = 0.5 + 1.5 * torch.rand(len(lengths), H, dk, generator=gen)
    return k, b, r, d0


PRE_CASES = [  # dtype, H, dk, lengths
    ("f32", 3, 16, [0, 1, 70, 129, 5, 0, 200]),   # 4 heads per wavefront: heads of two sequences share one
    ("bf16", 3, 32, [33, 0, 64, 1, 97]),
    ("bf16", 2, 64, [130, 1, 0, 65]),
    ("bf16", 2, 128, [0, 200, 7, 64, 129]),
    ("f32", 1, 128, [300, 2]),
]
VARIANTS = ["plain", "apf", "beta_free"]


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("dtype,H,dk,lengths", PRE_CASES, ids=[f"{c[0]}-dk{c[2]}-{i}" for i, c in enumerate(PRE_CASES)])
def test_precond_varlen_matches_each_sequence_alone(dtype, H, dk, lengths, variant):
    """Packed phase 1 against phase 1 on each sequence alone: the exact scan of
    dp_osdn_precond_ex_* to the bit, and the oracle within the tolerance."""
    say(f"case precond varlen {dtype} H={H} dk={dk} lengths={lengths} {variant}")
    k, b, r, d0 = packed_keys(H, dk, lengths, dtype)
    cu = offsets(lengths)
    rr = r if variant == "apf" else None
    aware = variant != "beta_free"
    cuda = lambda x: None if x is None else x.cuda()
    kt, d = dp.osdn_precond_varlen(k.cuda(), b.cuda(), cu.cuda(), d_state=d0.clone().cuda(),
                                   r=cuda(rr), beta_aware=aware)
    torch.cuda.synchronize()
    kt, d = kt.cpu(), d.cpu()
    errs = {"d": 0.0} if dtype == "bf16" else {"kt": 0.0, "d": 0.0}
    for s, n in enumerate(lengths):
        a = int(cu[s])
        if n == 0:
            assert torch.equal(d[s], d0[s]), f"sequence {s}: an empty sequence changed its d"
            continue
        one = lambda x: None if x is None else x[a:a + n].unsqueeze(0)
        kt1, d1 = dp.osdn_precond(one(k).cuda(), one(b).cuda(), d_state=d0[s:s + 1].clone().cuda(),
                                  r=cuda(one(rr)), beta_aware=aware)
        torch.cuda.synchronize()
        assert torch.equal(kt[a:a + n], kt1[0].cpu()), f"sequence {s}: kt differs from the single run"
        assert torch.equal(d[s], d1[0].cpu()), f"sequence {s}: d differs from the single run"
        kto, do = oracle.precond(one(k), one(b), d0=d0[s:s + 1], r=one(rr), beta_aware=aware)
        if dtype == "bf16":
            check_bf16_stored(f64(kt[a:a + n]), kto[0], f"sequence {s}")
        else:
            errs["kt"] = max(errs["kt"], rel_err(f64(kt[a:a + n]), kto[0]))
        errs["d"] = max(errs["d"], rel_err(f64(d[s]), do[0]))
    for name, e in errs.items():
        say(f"  {name}: worst err {e:.3e} (tol {TOL[dtype]:.0e})")
        assert e <= TOL[dtype], f"{name}: err {e:.3e} > {TOL[dtype]}"


def test_precond_varlen_malformed_offsets_read_nothing():
    """A sequence whose offsets leave [0, T] or run backwards is empty: no kt row
    of it is written and its d stays as it was; offsets whose last entry is not
    T make every sequence empty."""
    k, b, _, d0 = packed_keys(2, 64, [30, 30], "bf16")  # T = 60, two sequences
    for bad in ([0, 70, 60], [0, 30, 50]):  # past T and backwards; last offset not T
        cu = torch.tensor(bad, dtype=torch.int32).cuda()
        kt = torch.full((60, 2, 64), 7.0, dtype=torch.bfloat16, device="cuda")
        d = d0.clone().cuda()
        dp.osdn_precond_varlen(k.cuda(), b.cuda(), cu, d_state=d, kt=kt)
        torch.cuda.synchronize()
        assert bool((kt == 7.0).all()), f"offsets {bad}: kt was written"
        assert torch.equal(d.cpu(), d0), f"offsets {bad}: d changed"


def oracle_osdn_seq(q, k, v, b, kt_used, h0, a, n):
    """On tokens a .. a+n-1 alone: the oracle's phase 1 from d = 1, and the
    oracle's write-key forward on the write keys the forward was given."""
    one = lambda x: x[a:a + n].unsqueeze(0)
    kto, do = oracle.precond(one(k), one(b))
    oo, fo = oracle.fwd(one(q), one(k).unsqueeze(3), one(v).unsqueeze(3), one(b).unsqueeze(3),
                        kt=one(kt_used).unsqueeze(3), h0=h0)
    return oo[0], fo[0], kto[0], do[0]


OSDN_CASES = [  # H, dk, dv, chunk, lengths, h0
    (2, 128, 128, 64, [0, 1, 64, 65, 130, 7, 0, 200], False),
    (3, 64, 32, 32, [90, 1, 33, 0, 257], True),
]


@pytest.mark.parametrize("H,dk,dv,chunk,lengths,with_h0", OSDN_CASES,
                         ids=[f"dk{c[1]}-{i}" for i, c in enumerate(OSDN_CASES)])
def test_osdn_packed_layer_matches_each_sequence_alone(H, dk, dv, chunk, lengths, with_h0):
    """Packed phase 1 (d = 1 at every sequence start) then the packed write-key
    forward, each sequence against the same two calls on it alone (bit for
    bit) and against the oracle: phase 1's stored keys within bf16 rounding of
    the oracle's and its d within the bound; the forward on the bf16 write keys
    it was given (the layer hands them over in bf16), within the bound."""
    say(f"case osdn varlen H={H} dk={dk} dv={dv} chunk={chunk} lengths={lengths} h0={with_h0}")
    T, nseq = int(sum(lengths)), len(lengths)
    w = WORKLOADS["c5"].scaled(B=1, L=T, H=H, dk=dk, dv=dv, chunk=chunk)
    inp = make(w)
    q = inp["q"][0].contiguous()
    k = inp["k"][0, :, :, 0].contiguous()
    v = inp["v"][0, :, :, 0].contiguous()
    b = inp["beta"][0, :, :, 0].contiguous()
    h0 = (0.1 * torch.randn(nseq, H, dk, dv, generator=torch.Generator().manual_seed(3))) if with_h0 else None
    cu = offsets(lengths)
    kt, d = dp.osdn_precond_varlen(k.cuda(), b.cuda(), cu.cuda())
    out, fs = dp.fwd_varlen(q.cuda(), k.unsqueeze(2).cuda(), v.unsqueeze(2).cuda(), b.unsqueeze(2).cuda(),
                            cu.cuda(), chunk=chunk, h0=None if h0 is None else h0.cuda(),
                            kt=kt.unsqueeze(2))
    torch.cuda.synchronize()
    out, fs, ktc, d = out.cpu(), fs.cpu(), kt.cpu(), d.cpu()
    errs = {"out": 0.0, "fs": 0.0, "d": 0.0}
    for s, n in enumerate(lengths):
        a = int(cu[s])
        hs = None if h0 is None else h0[s:s + 1]
        if n == 0:
            assert torch.equal(fs[s], torch.zeros_like(fs[s]) if hs is None else hs[0])
            continue
        one = lambda x: x[a:a + n].unsqueeze(0).cuda()
        o1, f1 = dp.fwd(one(q), one(k).unsqueeze(3), one(v).unsqueeze(3), one(b).unsqueeze(3),
                        chunk=chunk, h0=None if hs is None else hs.cuda(), kt=one(ktc).unsqueeze(3))
        torch.cuda.synchronize()
        assert torch.equal(out[a:a + n], o1[0].cpu()), f"sequence {s}: out differs from the single run"
        assert torch.equal(fs[s], f1[0].cpu()), f"sequence {s}: final state differs from the single run"
        oo, fo, kto, do = oracle_osdn_seq(q, k, v, b, ktc, hs, a, n)
        errs["out"] = max(errs["out"], rel_err(f64(out[a:a + n]), oo))
        errs["fs"] = max(errs["fs"], rel_err(f64(fs[s]), fo))
        check_bf16_stored(f64(ktc[a:a + n]), kto, f"sequence {s}")
        errs["d"] = max(errs["d"], rel_err(f64(d[s]), do))
    for name, e in errs.items():
        say(f"  {name}: worst err {e:.3e} (tol {TOL['bf16']:.0e})")
        assert e <= TOL["bf16"], f"{name}: err {e:.3e} > {TOL['bf16']}"


def test_varlen_wk_general_write_keys_gate_and_n_h():
    """The packed write-key forward with n_h = 2, a gate, h0 and write keys that
    are not phase 1's, against the oracle on each sequence alone."""
    w = WORKLOADS["c4"].scaled(B=1, H=2, dk=64, dv=64, n_h=2)
    lengths = [90, 0, 257, 33, 1]
    T = int(sum(lengths))
    inp = make(w.scaled(L=T))
    q, k, v, b, g = (inp[n][0].contiguous() for n in ("q", "k", "v", "beta", "g"))
    kt = (0.5 * make(w.scaled(L=T), seed=w.seed + 9)["k"][0]).to(torch.bfloat16).contiguous()
    h0 = 0.1 * torch.randn(len(lengths), w.H, w.dk, w.dv, generator=torch.Generator().manual_seed(8))
    cu = offsets(lengths)
    say(f"case varlen wk n_h=2 gated lengths={lengths}")
    out, fs = dp.fwd_varlen(q.cuda(), k.cuda(), v.cuda(), b.cuda(), cu.cuda(), g=g.cuda(),
                            chunk=w.chunk, h0=h0.cuda(), kt=kt.cuda(), out_dtype=torch.float32)
    torch.cuda.synchronize()
    out, fs = out.cpu(), fs.cpu()
    errs = {"out": 0.0, "fs": 0.0}
    for s, n in enumerate(lengths):
        a = int(cu[s])
        one = lambda x: x[a:a + n].unsqueeze(0)
        oo, fo = oracle.fwd(one(q), one(k), one(v), one(b), g=one(g), kt=one(kt), h0=h0[s:s + 1])
        if n > 0:
            errs["out"] = max(errs["out"], rel_err(f64(out[a:a + n]), oo[0]))
        errs["fs"] = max(errs["fs"], rel_err(f64(fs[s]), fo[0]))
    for name, e in errs.items():
        say(f"  {name}: worst err {e:.3e} (tol {TOL['bf16']:.0e})")
        assert e <= TOL["bf16"], f"{name}: err {e:.3e} > {TOL['bf16']}"


CHUNK_CASES = [  # dtype, H, dk, lengths
    ("bf16", 2, 128, [0, 200, 7, 64, 129, 1, 65]),
    ("bf16", 3, 64, [130, 1, 0, 65, 300]),
    ("f32", 2, 128, [100, 0, 64, 257]),
]


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("dtype,H,dk,lengths", CHUNK_CASES, ids=[f"{c[0]}-dk{c[2]}-{i}" for i, c in enumerate(CHUNK_CASES)])
def test_precond_varlen_chunked_matches_oracle(dtype, H, dk, lengths, variant):
    """The chunked form on packed sequences (64-token chunks from each sequence's
    start) against the oracle on each sequence alone: d at the bound, the keys
    at the bound (f32) or within bf16 rounding (bf16)."""
    say(f"case precond varlen chunked {dtype} H={H} dk={dk} lengths={lengths} {variant}")
    k, b, r, d0 = packed_keys(H, dk, lengths, dtype, seed=3)
    cu = offsets(lengths)
    rr = r if variant == "apf" else None
    aware = variant != "beta_free"
    cuda = lambda x: None if x is None else x.cuda()
    kt, d = dp.osdn_precond_varlen(k.cuda(), b.cuda(), cu.cuda(), d_state=d0.clone().cuda(),
                                   r=cuda(rr), beta_aware=aware, chunked=True)
    torch.cuda.synchronize()
    kt, d = kt.cpu(), d.cpu()
    errs = {"d": 0.0} if dtype == "bf16" else {"kt": 0.0, "d": 0.0}
    for s, n in enumerate(lengths):
        a = int(cu[s])
        if n == 0:
            assert torch.equal(d[s], d0[s]), f"sequence {s}: an empty sequence changed its d"
            continue
        one = lambda x: None if x is None else x[a:a + n].unsqueeze(0)
        kto, do = oracle.precond(one(k), one(b), d0=d0[s:s + 1], r=one(rr), beta_aware=aware)
        if dtype == "bf16":
            check_bf16_stored(f64(kt[a:a + n]), kto[0], f"sequence {s}")
        else:
            errs["kt"] = max(errs["kt"], rel_err(f64(kt[a:a + n]), kto[0]))
        errs["d"] = max(errs["d"], rel_err(f64(d[s]), do[0]))
    for name, e in errs.items():
        say(f"  {name}: worst err {e:.3e} (tol {TOL[dtype]:.0e})")
        assert e <= TOL[dtype], f"{name}: err {e:.3e} > {TOL[dtype]}"


def test_precond_varlen_chunked_equals_the_layer_phase1_bit_for_bit():
    """Each packed sequence's chunked phase 1 is the chunked phase 1 that
    dp_osdn_fwd_bf16 runs on that sequence alone (one run): same chunks, same
    kernels, so the same bits."""
    H, dk, dv = 2, 128, 64
    lengths = [200, 1, 0, 64, 129]
    k, b, _, _ = packed_keys(H, dk, lengths, "bf16", seed=5)
    cu = offsets(lengths)
    kt, d = dp.osdn_precond_varlen(k.cuda(), b.cuda(), cu.cuda(), chunked=True)
    torch.cuda.synchronize()
    kt, d = kt.cpu(), d.cpu()
    gen = torch.Generator().manual_seed(6)
    for s, n in enumerate(lengths):
        if n == 0:
            continue
        a = int(cu[s])
        one = lambda x: x[a:a + n].unsqueeze(0).contiguous().cuda()
        q = torch.randn(1, n, H, dk, generator=gen).to(torch.bfloat16).cuda()
        v = torch.randn(1, n, H, dv, generator=gen).to(torch.bfloat16).cuda()
        _, _, kt1, d1 = dp.osdn_fwd(q, one(k), v, one(b), segments=1)
        torch.cuda.synchronize()
        assert torch.equal(kt[a:a + n], kt1[0].cpu()), f"sequence {s}: kt differs from the layer's phase 1"
        assert torch.equal(d[s], d1[0].cpu()), f"sequence {s}: d differs from the layer's phase 1"


def test_precond_varlen_chunked_hands_clamped_heads_to_the_exact_scan():
    """A large step size makes the box bind inside some chunks: those heads
    continue with the exact scan from their first such chunk (per sequence,
    from the chunk's start d), and every sequence still meets the oracle."""
    H, dk = 3, 128
    lengths = [150, 0, 70, 300, 5]
    k, b, _, _ = packed_keys(H, dk, lengths, "f32", seed=7)
    cu = offsets(lengths)
    box = dict(eta=0.8, dmin=0.95, dmax=1.05)  # a narrow box: coordinates end on its bounds
    kt, d = dp.osdn_precond_varlen(k.cuda(), b.cuda(), cu.cuda(), chunked=True, **box)
    torch.cuda.synchronize()
    kt, d = kt.cpu(), d.cpu()
    clamped = 0
    for s, n in enumerate(lengths):
        if n == 0:
            assert bool((d[s] == 1.0).all())
            continue
        a = int(cu[s])
        one = lambda x: x[a:a + n].unsqueeze(0)
        kto, do = oracle.precond(one(k), one(b), **box)
        clamped += int(np.sum((do[0] <= 0.95) | (do[0] >= 1.05)))
        e_kt, e_d = rel_err(f64(kt[a:a + n]), kto[0]), rel_err(f64(d[s]), do[0])
        say(f"  sequence {s}: kt err {e_kt:.3e}, d err {e_d:.3e}")
        assert e_kt <= TOL["f32"] and e_d <= TOL["f32"]
    assert clamped > 0, "the case should make the box bind"


def test_precond_varlen_chunked_malformed_offsets_read_nothing():
    """In the chunked form, offsets that are not a valid packing make every
    sequence empty: kt is left as it was and d keeps its value."""
    k, b, _, d0 = packed_keys(2, 128, [30, 30], "bf16", seed=9)  # T = 60, two sequences
    for bad in ([0, 70, 60], [0, 30, 50]):
        cu = torch.tensor(bad, dtype=torch.int32).cuda()
        kt = torch.full((60, 2, 128), 7.0, dtype=torch.bfloat16, device="cuda")
        d = d0.clone().cuda()
        dp.osdn_precond_varlen(k.cuda(), b.cuda(), cu, d_state=d, kt=kt, chunked=True)
        torch.cuda.synchronize()
        assert bool((kt == 7.0).all()), f"offsets {bad}: kt was written"
        assert torch.equal(d.cpu(), d0), f"offsets {bad}: d changed"
