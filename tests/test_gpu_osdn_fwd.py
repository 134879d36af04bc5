"""GPU checks of the pipelined write-key forward (dp_osdn_fwd_bf16).

It runs OSDN phase 1 followed by the write-key forward, cut into token runs
(the state and d pass between runs in fp32).  With the pipeline and without it
the results are the same bit for bit.  For dk < 64 phase 1 is the sequential
scan of dp_osdn_precond_bf16, so they also equal the two-call path bit for
bit; for dk >= 64 phase 1 takes the chunked form (solved 64-token chunks, with
the sequential scan again from the first chunk where a clamp comes near),
which rounds differently: there d meets the two-call path's to fp32 rounding
and every result meets the oracle.  Clamping cases check that hand-over.
"""
import pytest
import torch

import linear_rnn_sequence_amd as dp
import oracle
from linear_rnn_sequence_amd.inputs import WORKLOADS, make
from parity import TOL, f64, rel_err, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    dp.load()  # raises when libdp.so is missing: no silent fallback


def two_calls(q, k1, v1, b1, h0, chunk):
    kt, d = dp.osdn_precond(k1, b1)
    out, fs = dp.fwd(q, k1.unsqueeze(3), v1.unsqueeze(3), b1.unsqueeze(3), chunk=chunk, h0=h0,
                     kt=kt.unsqueeze(3))
    return out, fs, kt, d


def oracle_layer(q, k1, v1, b1, h0=None, **box):
    kto, do = oracle.precond(k1.cpu(), b1.cpu(), **box)
    oo, fo = oracle.fwd(q.cpu(), k1.cpu().unsqueeze(3), v1.cpu().unsqueeze(3), b1.cpu().unsqueeze(3),
                        kt=kto[:, :, :, None, :], h0=None if h0 is None else h0.cpu())
    return oo, fo, kto, do


def inputs(B, H, L, dk, dv, with_h0=False):
    w = WORKLOADS["c5"].scaled(B=B, H=H, L=L, dk=dk, dv=dv)
    inp = make(w)
    dev = torch.device("cuda:0")
    q = inp["q"].to(dev)
    k1 = inp["k"][:, :, :, 0, :].contiguous().to(dev)
    v1 = inp["v"][:, :, :, 0, :].contiguous().to(dev)
    b1 = inp["beta"][..., 0].contiguous().to(dev)
    h0 = (0.1 * torch.randn(B, H, dk, dv, generator=torch.Generator().manual_seed(5))).to(dev) if with_h0 else None
    return q, k1, v1, b1, h0


CASES = [  # B, H, L, dk, dv, chunk, segments, h0
    (2, 3, 300, 128, 128, 64, 1, False),
    (2, 3, 300, 128, 128, 64, 2, False),
    (2, 3, 300, 128, 128, 64, 4, True),
    (1, 2, 300, 128, 128, 64, 16, False),  # more runs asked for than chunks
    (1, 2, 50, 128, 64, 64, 4, False),     # shorter than one chunk
    (2, 1, 257, 64, 32, 32, 3, True),
    (1, 3, 130, 32, 32, 32, 2, False),     # dk = 32: two heads per phase-1 wavefront
    (1, 2, 100, 16, 16, 16, 5, True),      # dk = 16, chunk 16
]


@pytest.mark.parametrize("B,H,L,dk,dv,chunk,segments,with_h0", CASES)
def test_pipelined_equals_two_calls(B, H, L, dk, dv, chunk, segments, with_h0):
    say(f"case osdn_fwd B={B} H={H} L={L} dk={dk} dv={dv} C={chunk} segments={segments} h0={with_h0}")
    q, k1, v1, b1, h0 = inputs(B, H, L, dk, dv, with_h0)
    ref = two_calls(q, k1, v1, b1, h0, chunk)
    pipe = dp.Pipeline()
    got = dp.osdn_fwd(q, k1, v1, b1, h0=h0, chunk=chunk, segments=segments, pipeline=pipe)
    seq = dp.osdn_fwd(q, k1, v1, b1, h0=h0, chunk=chunk, segments=segments)
    torch.cuda.synchronize()
    pipe.close()
    for name, x, y, r in zip(("out", "final_state", "kt", "d"), got, seq, ref):
        assert torch.equal(x, y), f"{name}: the pipelined and in-order runs differ"
        if dk < 64:
            assert torch.equal(x, r), f"{name} differs from the two-call path"
    if dk >= 64:
        # d is fp32 throughout: it meets the sequential scan's to fp32 rounding;
        # the bf16 results meet the oracle (two bf16 roundings of nearly equal
        # values may differ by an ulp, so they are not compared to each other)
        e = rel_err(f64(got[3]), f64(ref[3]))
        say(f"  d: vs two calls {e:.3e}")
        assert e <= TOL["f32"]
        orc = oracle_layer(q, k1, v1, b1, h0=h0)
        for name, x, r in zip(("out", "final_state", "kt", "d"), got, orc):
            e = rel_err(f64(x), r)
            say(f"  {name}: err {e:.3e}")
            assert e <= TOL["bf16"], f"{name}: err {e:.3e}"


def test_one_pipeline_serves_calls_from_two_threads():
    """A handle may be shared: each call holds it for its enqueue sequence, so
    calls from two host threads on their own streams give the results of one
    call without a pipeline."""
    import threading

    B, H, L, dk, dv = 1, 2, 300, 128, 128
    q, k1, v1, b1, _ = inputs(B, H, L, dk, dv)
    ref = dp.osdn_fwd(q, k1, v1, b1, segments=4)
    torch.cuda.synchronize()
    pipe = dp.Pipeline()
    results = [None, None]

    def run(i):
        st = torch.cuda.Stream()
        with torch.cuda.stream(st):
            for _ in range(3):
                r = dp.osdn_fwd(q, k1, v1, b1, segments=4, pipeline=pipe, stream=st)
            st.synchronize()
            results[i] = r

    ts = [threading.Thread(target=run, args=(i,)) for i in range(2)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    torch.cuda.synchronize()
    pipe.close()
    for got in results:
        for name, x, r in zip(("out", "final_state", "kt", "d"), got, ref):
            assert torch.equal(x, r), f"{name} differs from the call without a pipeline"


def test_failed_call_leaves_outputs_untouched():
    """Every run is checked before the first is enqueued: a misaligned v (which
    only the forward of a run reads) fails the call with d, kt, out and the
    final state as they were."""
    B, H, L, dk, dv = 1, 2, 300, 128, 128
    q, k1, v1, b1, _ = inputs(B, H, L, dk, dv)
    raw = torch.empty(v1.numel() + 1, dtype=v1.dtype, device=v1.device)
    v_mis = raw[1:].view(v1.shape)
    v_mis.copy_(v1)
    assert v_mis.is_contiguous() and v_mis.data_ptr() % 16 != 0
    d = torch.full((B, H, dk), 1.25, device=q.device)
    kt = torch.full((B, L, H, dk), 3.0, dtype=torch.bfloat16, device=q.device)
    out = torch.full((B, L, H, dv), -2.0, dtype=torch.bfloat16, device=q.device)
    fs = torch.full((B, H, dk, dv), 7.0, device=q.device)
    snap = [t.clone() for t in (d, kt, out, fs)]
    pipe = dp.Pipeline()
    for p in (pipe, None):
        with pytest.raises(dp.DPError) as ei:
            dp.osdn_fwd(q, k1, v_mis, b1, segments=4, d_state=d, kt=kt, out=out, final_state=fs,
                        pipeline=p)
        assert ei.value.code == dp.binding.DP_EINVAL
    torch.cuda.synchronize()
    pipe.close()
    for t, s in zip((d, kt, out, fs), snap):
        assert torch.equal(t, s)


def test_pipelined_matches_oracle():
    B, H, L, dk, dv = 2, 2, 200, 128, 128
    say(f"case osdn_fwd vs oracle B={B} H={H} L={L}")
    q, k1, v1, b1, _ = inputs(B, H, L, dk, dv)
    pipe = dp.Pipeline()
    out, fs, kt, d = dp.osdn_fwd(q, k1, v1, b1, segments=3, pipeline=pipe)
    torch.cuda.synchronize()
    pipe.close()
    kto, do = oracle.precond(k1.cpu(), b1.cpu())
    oo, fo = oracle.fwd(q.cpu(), k1.cpu().unsqueeze(3), v1.cpu().unsqueeze(3), b1.cpu().unsqueeze(3),
                        kt=kto[:, :, :, None, :])
    for name, x, r in (("out", out, oo), ("final_state", fs, fo), ("kt", kt, kto), ("d", d, do)):
        e = rel_err(f64(x), r)
        say(f"  {name}: err {e:.3e}")
        assert e <= TOL["bf16"], f"{name}: err {e:.3e}"


def test_argument_errors():
    q, k1, v1, b1, _ = inputs(1, 1, 130, 128, 128)
    with pytest.raises(dp.DPError):
        dp.osdn_fwd(q, k1, v1, b1, segments=0)
    with pytest.raises(dp.DPError):
        dp.osdn_fwd(q, k1, v1, b1, segments=17)


CLAMP = [  # eta, dmax; the phase-1 clamp binds in: (dk 128, L 300, c5 inputs)
    (1e-2, 1.0059),   # some heads only, late in the sequence
    (1e-2, 1.002),    # every head, after the first chunk
    (3e-2, 1.002),    # every head, within the first chunk
]


@pytest.mark.parametrize("eta,dmax", CLAMP)
def test_clamping_box_matches_oracle(eta, dmax):
    """With the upper bound of the box binding (on some heads or all, late or
    within the first chunk) the chunked phase 1 hands those heads to the
    sequential scan from the chunk where a step first came near the bound:
    the call meets the oracle, clamps included, and the two-call path's d."""
    B, H, L, dk, dv = 2, 3, 300, 128, 128
    say(f"case osdn_fwd clamps B={B} H={H} L={L} eta={eta} dmax={dmax}")
    q, k1, v1, b1, _ = inputs(B, H, L, dk, dv)
    box = dict(eta=eta, dmin=0.5, dmax=dmax)
    ref = oracle_layer(q, k1, v1, b1, **box)
    at_bound = (ref[3] >= dmax).any(axis=-1)
    say(f"  heads ending at the bound: {int(at_bound.sum())} of {B * H}")
    assert at_bound.any()
    got = dp.osdn_fwd(q, k1, v1, b1, segments=2, **box)
    kt, d = dp.osdn_precond(k1, b1, **box)
    torch.cuda.synchronize()
    for name, x, r in zip(("out", "final_state", "kt", "d"), got, ref):
        e = rel_err(f64(x), r)
        say(f"  {name}: err {e:.3e}")
        assert e <= TOL["bf16"], f"{name}: err {e:.3e}"
    assert torch.all(got[3] <= dmax) and torch.all(got[3] >= 0.5)
    assert rel_err(f64(got[3]), f64(d)) <= TOL["f32"]


def test_nan_beta_hands_over_to_the_sequential_scan():
    """A NaN beta at token 150 of head 1 (dk = 128, two runs): the chunked
    phase 1 meets the NaN in that chunk's check and runs the sequential scan
    from the chunk's start, so d and the write keys are NaN exactly where the
    oracle's are (head 1 from token 151 on, through the second run), and the
    other heads still meet the oracle."""
    import numpy as np
    B, H, L, dk, dv = 1, 3, 300, 128, 128
    q, k1, v1, b1, _ = inputs(B, H, L, dk, dv)
    b1 = b1.clone()
    b1[0, 150, 1] = float("nan")
    kto, do = oracle.precond(k1.cpu(), b1.cpu())
    out, fs, kt, d = dp.osdn_fwd(q, k1, v1, b1, segments=2)
    torch.cuda.synchronize()
    ktn, dn = f64(kt), f64(d)
    assert np.array_equal(np.isnan(ktn), np.isnan(kto)), "NaN pattern of the write keys"
    assert np.array_equal(np.isnan(dn), np.isnan(do)), "NaN pattern of d"
    assert np.isnan(ktn[0, 151:, 1]).all() and np.isfinite(ktn[0, :151, 1]).all()
    for h in (0, 2):
        e = max(rel_err(ktn[0, :, h], kto[0, :, h]), rel_err(dn[0, h], do[0, h]))
        say(f"  head {h}: err {e:.3e}")
        assert e <= TOL["bf16"]
    e = rel_err(ktn[0, :151, 1], kto[0, :151, 1])
    say(f"  head 1 before the NaN: err {e:.3e}")
    assert e <= TOL["bf16"]
    oo, fo = oracle.fwd(q.cpu()[:, :, 0::2], k1.cpu()[:, :, 0::2].unsqueeze(3), v1.cpu()[:, :, 0::2].unsqueeze(3),
                        b1.cpu()[:, :, 0::2].unsqueeze(3), kt=kto[:, :, 0::2, None, :])
    e = max(rel_err(f64(out)[:, :, 0::2], oo), rel_err(f64(fs)[:, 0::2], fo))
    say(f"  outputs of heads 0 and 2: err {e:.3e}")
    assert e <= TOL["bf16"]
