"""GPU checks of the no-alloc packed forward (dp_fwd_varlen_noalloc_bf16).

It runs the same kernels as dp_fwd_varlen_bf16 with DP_FWD_FUSED, with the
per-sequence chunk-offset table in the library's fixed scratch array instead
of a caller's workspace, so its results must equal that entry point's bit for
bit.  Two calls in a row, the second with fewer sequences and tokens, check
that what the first call left in the shared array is never read; sampled
sequences are also checked against the fp64 oracle.
"""
import numpy as np
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


def packed(w, lengths, seed_shift):
    """Packed [T, ...] inputs of workload w (T = sum(lengths)) and the offsets."""
    T = int(sum(lengths))
    inp = make(w.scaled(B=1, L=T), seed=w.seed + seed_shift)
    pk = {n: (None if inp[n] is None else inp[n][0].contiguous()) for n in ("q", "k", "v", "beta", "g")}
    h0 = None
    if w.h0_std > 0:
        gen = torch.Generator().manual_seed(w.seed + 77 + seed_shift)
        h0 = torch.randn(len(lengths), w.H, w.dk, w.dv, generator=gen) * w.h0_std
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int32)
    return pk, h0, cu


def both_entry_points(w, lengths, seed_shift):
    """(no-alloc results, workspace entry point's fused results, inputs) on the GPU."""
    pk, h0, cu = packed(w, lengths, seed_shift)
    dev = lambda x: None if x is None else x.cuda()
    q, k, v, b, g = (dev(pk[n]) for n in ("q", "k", "v", "beta", "g"))
    h0d, cud = dev(h0), cu.cuda()
    T, nseq = int(cu[-1]), len(lengths)
    odt = torch.float32 if w.out_f32 else torch.bfloat16
    # outputs pre-filled with NaN: any element the call does not write shows
    out_na = torch.full((T, w.H, w.dv), float("nan"), dtype=odt, device="cuda")
    fs_na = torch.full((nseq, w.H, w.dk, w.dv), float("nan"), device="cuda")
    dp.fwd_varlen_noalloc(q, k, v, b, cud, out_na, g=g, chunk=w.chunk, h0=h0d, final_state=fs_na)
    out_ws, fs_ws = dp.fwd_varlen(q, k, v, b, cud, g=g, chunk=w.chunk, h0=h0d, out_dtype=odt, path="fused")
    torch.cuda.synchronize()
    return (out_na.cpu(), fs_na.cpu()), (out_ws.cpu(), fs_ws.cpu()), (pk, h0, cu)


def check_oracle(out, fs, pk, h0, cu, seqs, label):
    for d in seqs:
        a, e = int(cu[d]), int(cu[d + 1])
        sl = lambda x: None if x is None else x[a:e].unsqueeze(0)
        oo, fo = oracle.fwd(sl(pk["q"]), sl(pk["k"]), sl(pk["v"]), sl(pk["beta"]), g=sl(pk["g"]),
                            h0=None if h0 is None else h0[d:d + 1])
        ef = rel_err(f64(fs[d]), fo[0])
        eo = rel_err(f64(out[a:e]), oo[0]) if e > a else 0.0
        say(f"  {label} seq {d} ({e - a} tokens): out err {eo:.3e}, state err {ef:.3e}")
        assert eo <= TOL["bf16"] and ef <= TOL["bf16"], f"{label} seq {d}"


# (workload, overrides, first call's lengths, second call's lengths): the second
# call has fewer sequences and tokens than the first
CASES = [
    ("c3b", dict(H=4), [300, 1, 0, 129, 64, 513, 7], [65, 0, 40]),
    ("c4", dict(H=2, dk=64, dv=32), [90, 0, 257, 33, 1, 200], [31, 64]),   # gated, h0, fp32 out
    ("c3", dict(H=3, dk=32, dv=16, chunk=32, n_h=1), [17, 99, 2, 0, 45], [5]),
]


@pytest.mark.parametrize("name,kw,first,second", CASES, ids=[c[0] for c in CASES])
def test_noalloc_equals_workspace_entry_point_two_calls(name, kw, first, second):
    w = WORKLOADS[name].scaled(**kw)
    assert sum(second) < sum(first) and len(second) < len(first)
    for call, lengths in enumerate((first, second)):
        say(f"case no-alloc {name} {kw} call {call + 1}: {len(lengths)} sequences, T={sum(lengths)}")
        (o_na, f_na), (o_ws, f_ws), (pk, h0, cu) = both_entry_points(w, lengths, seed_shift=call)
        assert torch.equal(o_na, o_ws), f"call {call + 1}: out differs from dp_fwd_varlen_bf16"
        assert torch.equal(f_na, f_ws), f"call {call + 1}: final state differs"
        assert not torch.isnan(o_na).any() and not torch.isnan(f_na).any()
        order = np.argsort(lengths)
        check_oracle(o_na, f_na, pk, h0, cu, sorted({int(order[0]), int(order[-1])}), f"{name}#{call + 1}")


def test_noalloc_limits_and_flags():
    """More sequences than the scratch holds is DP_ESCRATCH; shapes without a
    fused kernel are DP_ENOTSUP; both before anything is enqueued."""
    w = WORKLOADS["c3b"].scaled(H=1, dk=128, dv=32)
    n = dp.binding.NOALLOC_MAX_SEQS + 1
    T = n
    q = torch.zeros(T, 1, 128, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(T, 1, 2, 128, dtype=torch.bfloat16, device="cuda")
    v = torch.zeros(T, 1, 2, 32, dtype=torch.bfloat16, device="cuda")
    b = torch.zeros(T, 1, 2, device="cuda")
    cu = torch.arange(n + 1, dtype=torch.int32, device="cuda")
    out = torch.empty(T, 1, 32, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(dp.DPError) as ei:
        dp.fwd_varlen_noalloc(q, k, v, b, cu, out, chunk=w.chunk)
    assert ei.value.code == dp.binding.DP_ESCRATCH
    with pytest.raises(dp.DPError) as ei:
        dp.fwd_varlen_noalloc(q[:16], k[:16], v[:16], b[:16], cu[:3].clone().clamp_(max=16), out[:16], chunk=16)
    assert ei.value.code == dp.binding.DP_ENOTSUP
    # the largest allowed count works: every sequence one token long
    q2, k2, v2, b2 = q[:n - 1], k[:n - 1], v[:n - 1], b[:n - 1]
    cu2 = torch.arange(n, dtype=torch.int32, device="cuda")
    o2 = torch.full((n - 1, 1, 32), float("nan"), dtype=torch.bfloat16, device="cuda")
    dp.fwd_varlen_noalloc(q2, k2, v2, b2, cu2, o2, chunk=w.chunk)
    torch.cuda.synchronize()
    # zero inputs, zero initial state: the output is exactly zero everywhere
    assert torch.count_nonzero(o2) == 0
