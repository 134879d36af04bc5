"""Pins of the oracle's gradient (CPU only).

The gradient is pinned to the forward alone, never to its own formulas:

* central finite differences of the fp64 forward, for every coordinate of
  every input of small problems (gated, with an initial state and a
  final-state gradient, symmetric and with write keys, n_h = 1..3, a
  clamped beta);
* a closed form: one token, one sub-step, zero initial state, where
  out = beta <kh, q> v with kh = k / |k|;
* invariances the definition fixes: the output does not change when a key is
  scaled, so each key gradient is orthogonal to its key; the gradient is
  linear in (dout, dfinal); beta = 0 sub-steps pass no gradient to v; g = 0
  passes no gradient to h0.
"""
import numpy as np
import pytest

import oracle


def problem(B=1, L=4, H=2, n_h=2, dk=4, dv=3, gate=True, h0=True, asym=False, seed=0):
    rng = np.random.default_rng(seed)
    x = dict(q=rng.normal(size=(B, L, H, dk)), k=rng.normal(size=(B, L, H, n_h, dk)),
             v=rng.normal(size=(B, L, H, n_h, dv)), beta=rng.uniform(0.1, 1.9, size=(B, L, H, n_h)),
             g=rng.uniform(0.5, 1.0, size=(B, L, H)) if gate else None,
             h0=rng.normal(size=(B, H, dk, dv)) if h0 else None,
             kt=rng.normal(size=(B, L, H, n_h, dk)) if asym else None)
    w_out = rng.normal(size=(B, L, H, dv))
    w_fin = rng.normal(size=(B, H, dk, dv))
    return x, w_out, w_fin


def loss(x, w_out, w_fin):
    o, f = oracle.fwd(x["q"], x["k"], x["v"], x["beta"], g=x["g"], kt=x["kt"], h0=x["h0"])
    return float(np.sum(o * w_out) + np.sum(f * w_fin))


def grads(x, w_out, w_fin):
    return oracle.bwd(x["q"], x["k"], x["v"], x["beta"], w_out, g=x["g"], kt=x["kt"], h0=x["h0"],
                      dfinal=w_fin)


def fd(x, w_out, w_fin, name, eps=1e-6):
    base = x[name]
    out = np.zeros_like(base)
    for idx in np.ndindex(base.shape):
        saved = base[idx]
        base[idx] = saved + eps
        lp = loss(x, w_out, w_fin)
        base[idx] = saved - eps
        lm = loss(x, w_out, w_fin)
        base[idx] = saved
        out[idx] = (lp - lm) / (2 * eps)
    return out


CASES = [
    dict(n_h=1, gate=False, h0=False),
    dict(n_h=2, gate=True, h0=True),
    dict(n_h=3, gate=True, h0=True, L=3, dk=3, dv=4),
    dict(n_h=2, gate=True, h0=True, asym=True),
    dict(n_h=3, gate=False, h0=True, asym=True, L=3),
]


@pytest.mark.parametrize("case", CASES, ids=[str(i) for i in range(len(CASES))])
def test_gradient_matches_finite_differences(case):
    x, wo, wf = problem(**case, seed=len(str(case)))
    gr = grads(x, wo, wf)
    names = ["q", "k", "v", "beta"] + [n for n in ("g", "h0", "kt") if x[n] is not None]
    for n in names:
        ref = fd(x, wo, wf, n)
        got = gr[n]
        scale = max(1.0, float(np.max(np.abs(ref))))
        err = float(np.max(np.abs(got - ref))) / scale
        assert err < 2e-7, f"{n}: finite-difference mismatch {err:.2e}"


def test_clamped_beta_passes_no_gradient():
    x, wo, wf = problem(n_h=2, seed=5)
    x["beta"][0, 1, 0, 0] = 2.5    # clamped to 2
    x["beta"][0, 2, 1, 1] = -0.3   # clamped to 0
    gr = grads(x, wo, wf)
    ref = fd(x, wo, wf, "beta")
    assert gr["beta"][0, 1, 0, 0] == 0.0 and gr["beta"][0, 2, 1, 1] == 0.0
    assert abs(ref[0, 1, 0, 0]) < 1e-9 and abs(ref[0, 2, 1, 1]) < 1e-9
    assert np.max(np.abs(gr["beta"] - ref)) < 2e-7 * max(1.0, np.max(np.abs(ref)))


def test_one_sub_step_closed_form():
    """L = 1, n_h = 1, no gate, zero initial state: out = beta <kh, q> v."""
    rng = np.random.default_rng(3)
    dk, dv = 5, 4
    q = rng.normal(size=(1, 1, 1, dk))
    k = rng.normal(size=(1, 1, 1, 1, dk))
    v = rng.normal(size=(1, 1, 1, 1, dv))
    beta = np.full((1, 1, 1, 1), 0.7)
    do = rng.normal(size=(1, 1, 1, dv))
    gr = oracle.bwd(q, k, v, beta, do)
    kv, qv, vv, dov = k.reshape(dk), q.reshape(dk), v.reshape(dv), do.reshape(dv)
    nk = np.linalg.norm(kv)
    kh = kv / nk
    a = kh @ qv
    np.testing.assert_allclose(gr["v"].reshape(dv), 0.7 * a * dov, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(gr["beta"].reshape(()), a * (vv @ dov), rtol=1e-13)
    np.testing.assert_allclose(gr["q"].reshape(dk), 0.7 * (vv @ dov) * kh, rtol=1e-13, atol=1e-14)
    dkh = 0.7 * (vv @ dov) * qv
    np.testing.assert_allclose(gr["k"].reshape(dk), (dkh - kh * (kh @ dkh)) / nk, rtol=1e-12,
                               atol=1e-14)
    # the final state's gradient was zero and h0 was zero: h0 gets
    # (I - beta kh kh^T) q dout^T from the readout of H0 through the sub-step
    dh0 = np.outer(qv - 0.7 * kh * (kh @ qv), dov)
    np.testing.assert_allclose(gr["h0"].reshape(dk, dv), dh0, rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("asym", [False, True])
def test_key_gradient_orthogonal_to_key(asym):
    x, wo, wf = problem(L=6, n_h=3, dk=8, dv=5, asym=asym, seed=9)
    gr = grads(x, wo, wf)
    dots = np.einsum("blhjd,blhjd->blhj", gr["k"], x["k"])
    assert np.max(np.abs(dots)) < 1e-12 * max(1.0, np.max(np.abs(gr["k"])))
    assert np.max(np.abs(gr["k"])) > 1e-3


def test_gradient_linear_in_output_gradients():
    x, wo, wf = problem(L=5, n_h=2, dk=6, dv=4, seed=4)
    g1 = grads(x, wo, wf)
    g2 = grads(x, 2.0 * wo, -wf)
    g3 = grads(x, 4.0 * wo, -2.0 * wf)   # = 2 * g2
    ga = grads(x, wo, 0.0 * wf)
    gb = grads(x, 0.0 * wo, wf)
    for n in g1:
        np.testing.assert_allclose(ga[n] + gb[n], g1[n], rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(g3[n], 2.0 * g2[n], rtol=1e-11, atol=1e-12)


def test_beta_zero_and_gate_zero():
    x, wo, wf = problem(L=4, n_h=2, seed=6)
    x["beta"][0, :, 0, 1] = 0.0
    x["g"][0, 0, 1] = 0.0     # head 1's first token erases h0
    gr = grads(x, wo, wf)
    assert np.all(gr["v"][0, :, 0, 1] == 0.0)
    assert np.all(gr["h0"][0, 1] == 0.0)
    assert np.max(np.abs(gr["h0"][0, 0])) > 1e-3


def test_heads_subset_equals_full():
    x, wo, wf = problem(B=2, L=5, H=3, n_h=2, dk=4, dv=3, seed=8)
    full = grads(x, wo, wf)
    heads = [4, 1]
    sub = oracle.bwd_heads(x["q"], x["k"], x["v"], x["beta"], wo, heads, g=x["g"], h0=x["h0"],
                           dfinal=wf)
    for i, bh in enumerate(heads):
        b, h = divmod(bh, 3)
        assert np.array_equal(sub["q"][i], full["q"][b, :, h])
        assert np.array_equal(sub["k"][i], full["k"][b, :, h])
        assert np.array_equal(sub["v"][i], full["v"][b, :, h])
        assert np.array_equal(sub["beta"][i], full["beta"][b, :, h])
        assert np.array_equal(sub["g"][i], full["g"][b, :, h])
        assert np.array_equal(sub["h0"][i], full["h0"][b, h])
