"""Helpers of the GPU parity tests: run the HIP path through the C ABI and the
fp64 oracle on the same stored bytes, and measure the error the way the
tolerances are stated: max |x_gpu - x_oracle| / RMS(x_oracle), per tensor."""
import sys

import numpy as np
import torch

import linear_rnn_sequence_amd as dp
import oracle
from linear_rnn_sequence_amd.inputs import sampled_heads, select_heads, select_state  # noqa: F401

TOL = {"f32": 1e-4, "bf16": 2e-2}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_err(x, ref) -> float:
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(ref * ref)))
    if rms == 0.0:
        return float(np.max(np.abs(x - ref)))
    return float(np.max(np.abs(x - ref)) / rms)


def f64(t):
    return t.detach().to("cpu").to(torch.float64).numpy()


def to_dev(inp, device="cuda"):
    return {k: (v.to(device) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}


def gpu_forward(inp, chunk=None, kt=None, h0="input", stream=None, out_dtype="input"):
    """Run dp.fwd on the GPU copies of `inp`; returns (out, final_state) on the device."""
    d = to_dev(inp)
    h0t = d["h0"] if h0 == "input" else h0
    ktt = None if kt is None else kt.to("cuda")
    odt = inp.get("out_dtype") if out_dtype == "input" else out_dtype
    out, fs = dp.fwd(d["q"], d["k"], d["v"], d["beta"], d["g"], chunk=chunk or inp["chunk"],
                     h0=h0t, kt=ktt, stream=stream, out_dtype=odt)
    torch.cuda.synchronize()
    return out, fs


def oracle_heads(inp, heads, kt=None):
    """Oracle forward of the listed heads only (stacked along H, B = 1)."""
    H = inp["q"].shape[2]
    sel = lambda t: None if t is None else select_heads(t, heads, H)
    h0 = None if inp["h0"] is None else select_state(inp["h0"], heads, H)
    return oracle.fwd(sel(inp["q"]), sel(inp["k"]), sel(inp["v"]), sel(inp["beta"]),
                      g=sel(inp["g"]), kt=None if kt is None else sel(kt), h0=h0)


def check_bf16_stored(x, ref, label):
    """Write keys stored in bf16: each element is d_t * k_t (fp32, ~1e-6 relative
    from the oracle's fp64 value) rounded to nearest even, so it lies within
    2^-8 |ref| of the reference (half a unit in the last place at the bottom of
    a binade), plus the fp32 part.  The scan is judged on d (fp32, max/RMS
    bound); max/RMS of the stored keys measures their rounding, which for
    keys spread over a decade exceeds 2e-2 by itself."""
    ref = np.asarray(ref, np.float64)
    rms = float(np.sqrt(np.mean(ref * ref)))
    bound = 2.0 ** -8 * np.abs(ref) * (1 + 1e-3) + 1e-5 * rms
    excess = float(np.max(np.abs(x - ref) - bound))
    say(f"  {label} kt: max/RMS {rel_err(x, ref):.3e}; worst |err| - 2^-8 |ref| bound {excess:.3e}")
    assert np.all(np.isfinite(x)), f"{label} kt: non-finite values"
    assert excess <= 0.0, f"{label} kt: an element is off by more than bf16 rounding"
