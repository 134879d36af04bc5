"""The fp16 operand range of the bf16 path (include/dp.h, "Precision").

On the bf16 path the MFMA operands the kernels compute (queries, write keys,
pseudo-values, the state copy, scores) are fp16, so a value beyond +-65504
there becomes +-Inf.  These tests pin what the header states: the results that
depend on such a value are not finite (nothing is silently repaired), every
other head is unaffected and still meets the oracle bound, and the fp32 path
computes the same inputs without loss.
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


def run(inp, dtype):
    dt = torch.float32 if dtype == "f32" else torch.bfloat16
    c = lambda x: None if x is None else x.cuda()
    out, fs = dp.fwd(c(inp["q"].to(dt)), c(inp["k"].to(dt)), c(inp["v"].to(dt)), c(inp["beta"]), c(inp["g"]),
                     chunk=64, h0=c(inp["h0"]), out_dtype=torch.float32)
    torch.cuda.synchronize()
    return f64(out), f64(fs)


def base_inputs():
    w = WORKLOADS["c3"].scaled(B=1, H=2, L=130, dtype="f32")
    return make(w)


def test_query_beyond_fp16_range():
    """|q| = 2^17 at one token of head 1: that token's output row is not finite
    on the bf16 path; the state, head 0 and head 1's other tokens are
    unaffected; the fp32 path matches the oracle everywhere."""
    inp = base_inputs()
    inp["q"][0, 70, 1, 5] = 131072.0  # 2^17: exact in bf16 and fp32, beyond fp16
    q16 = inp["q"].to(torch.bfloat16)
    ref_in = dict(inp, q=q16.float(), k=inp["k"].to(torch.bfloat16).float(), v=inp["v"].to(torch.bfloat16).float())
    oo, fo = oracle.fwd(ref_in["q"], ref_in["k"], ref_in["v"], inp["beta"])
    out, fs = run(inp, "bf16")
    say(f"  bf16: non-finite outputs {np.count_nonzero(~np.isfinite(out))}")
    assert not np.all(np.isfinite(out[0, 70, 1])), "the overflowing query's output should not be finite"
    mask = np.ones(out.shape[:3], bool)
    mask[0, 70, 1] = False
    assert np.all(np.isfinite(out[mask])) and np.all(np.isfinite(fs))
    e_out, e_fs = rel_err(out[mask], oo[mask]), rel_err(fs, fo)
    say(f"  bf16 others: out err {e_out:.3e}, fs err {e_fs:.3e}")
    assert e_out <= TOL["bf16"] and e_fs <= TOL["bf16"]
    o32, f32 = run(inp, "f32")
    ox, fx = oracle.fwd(inp["q"], inp["k"], inp["v"], inp["beta"])
    assert np.all(np.isfinite(o32)) and rel_err(o32, ox) <= TOL["f32"] and rel_err(f32, fx) <= TOL["f32"]


def test_pseudo_value_beyond_fp16_range():
    """|v| = 2^20 on one sub-step of head 1 with beta = 1: its pseudo-value
    leaves fp16 range, so head 1's results from that chunk on are not finite
    on the bf16 path (inside the chunk the masked scores multiply it by zero,
    which is not finite either) while head 0 and head 1's earlier chunks are
    unaffected; the fp32 path matches the oracle."""
    inp = base_inputs()
    inp["v"][0, 70, 1, 0, 3] = 1048576.0  # 2^20, sub-step 210: the fourth 64-sub-step chunk
    inp["beta"][0, 70, 1, 0] = 1.0
    ref_in = dict(q=inp["q"].to(torch.bfloat16).float(), k=inp["k"].to(torch.bfloat16).float(),
                  v=inp["v"].to(torch.bfloat16).float())
    oo, fo = oracle.fwd(ref_in["q"], ref_in["k"], ref_in["v"], inp["beta"])
    out, fs = run(inp, "bf16")
    assert not (np.all(np.isfinite(out[0, 70:, 1])) and np.all(np.isfinite(fs[0, 1])))
    assert np.all(np.isfinite(out[0, :64, 1]))  # the chunks before it never see it
    assert np.all(np.isfinite(out[0, :, 0])) and np.all(np.isfinite(fs[0, 0]))
    e0 = max(rel_err(out[0, :, 0], oo[0, :, 0]), rel_err(fs[0, 0], fo[0, 0]))
    say(f"  bf16 head 0: err {e0:.3e}")
    assert e0 <= TOL["bf16"]
    o32, f32 = run(inp, "f32")
    ox, fx = oracle.fwd(inp["q"], inp["k"], inp["v"], inp["beta"])
    assert np.all(np.isfinite(o32)) and rel_err(o32, ox) <= TOL["f32"] and rel_err(f32, fx) <= TOL["f32"]
