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


# ------------------------------------------------------------------ phase-1 gradient
# OSDN notes sec. 2.5 (closing paragraph): in training the write key
# kt_t = d_t * kh_t passes its gradient into d_t and k_t, and the gradient of
# d runs back through the phase-1 recursion.  Pinned to the phase-1 forward
# alone (finite differences, a closed form, invariances), and the composed
# layer (phase 1 then the write-key forward) to finite differences of the
# composed forward.

def p1_problem(L=6, H=2, dk=4, seed=0, ret=True, d0=True, tiny=False):
    rng = np.random.default_rng(seed)
    k = rng.normal(size=(1, L, H, dk))
    if tiny:  # |k| < 1e-6: kh = k / 1e-6 is not a unit vector, n varies with k
        k *= 5e-7 / np.linalg.norm(k, axis=-1, keepdims=True)
    x = dict(k=k, beta=rng.uniform(0.1, 1.9, size=(1, L, H)),
             r=rng.uniform(0.6, 1.0, size=(1, L, H)) if ret else None,
             d0=rng.uniform(0.8, 1.5, size=(1, H, dk)) if d0 else None)
    wk = rng.normal(size=(1, L, H, dk))
    wd = rng.normal(size=(1, H, dk))
    return x, wk, wd


def p1_loss(x, wk, wd, **kw):
    kt, d = oracle.precond(x["k"], x["beta"], r=x["r"], d0=x["d0"], **kw)
    return float(np.sum(kt * wk) + np.sum(d * wd))


def p1_fd(x, wk, wd, name, step, **kw):
    base = x[name]
    out = np.zeros_like(base)
    for idx in np.ndindex(base.shape):
        saved = base[idx]
        base[idx] = saved + step
        lp = p1_loss(x, wk, wd, **kw)
        base[idx] = saved - step
        lm = p1_loss(x, wk, wd, **kw)
        base[idx] = saved
        out[idx] = (lp - lm) / (2 * step)
    return out


P1_CASES = [
    dict(kw=dict(eta=0.3), prob=dict()),                                          # box open in practice
    dict(kw=dict(eta=0.5, dmin=0.9, dmax=1.1), prob=dict(seed=1)),                # clamps bind
    dict(kw=dict(eta=0.4, beta_aware=False), prob=dict(seed=2, dk=5)),            # beta-free step
    dict(kw=dict(eta=0.2), prob=dict(seed=3, ret=False, d0=False)),               # Alg.1 as printed
    dict(kw=dict(eta=0.3, eps=0.1, dmin=-1e9, dmax=1e9), prob=dict(seed=4, tiny=True)),  # n < 1 keys
]


@pytest.mark.parametrize("case", P1_CASES, ids=[str(i) for i in range(len(P1_CASES))])
def test_phase1_gradient_matches_finite_differences(case):
    kw, prob = case["kw"], case["prob"]
    x, wk, wd = p1_problem(**prob)
    gr = oracle.precond_bwd(x["k"], x["beta"], wk, d0=x["d0"], dd_final=wd, r=x["r"], **kw)
    steps = dict(k=1e-13 if prob.get("tiny") else 1e-6, beta=1e-6, r=1e-6, d0=1e-6)
    names = ["k", "beta"] + [n for n in ("r", "d0") if x[n] is not None]
    for n in names:
        ref = p1_fd(x, wk, wd, n, steps[n], **kw)
        got = gr[n]
        scale = max(1.0, float(np.max(np.abs(ref))))
        err = float(np.max(np.abs(got - ref))) / scale
        assert err < 1e-6, f"{n}: finite-difference mismatch {err:.2e}"
    if kw.get("dmin") == 0.9:  # the case is meant to clamp: some d_t must sit on the box
        kt, _ = oracle.precond(x["k"], x["beta"], r=x["r"], d0=x["d0"], **kw)
        assert np.any(np.isclose(kt / (x["k"] / np.linalg.norm(x["k"], axis=-1, keepdims=True)), 0.9)) \
            or np.any(np.isclose(kt / (x["k"] / np.linalg.norm(x["k"], axis=-1, keepdims=True)), 1.1))


def test_phase1_gradient_closed_form():
    """k = e1 on every token, constant beta and retention r, box open:
    d_{t+1}[0] = (r - eta beta^2) d_t[0] + eta beta and kt_t[0] = d_t[0].  For
    the loss sum_t kt_t[0], the gradient on d_{t+1}[0] is
    G_{t+1} = sum_{u=0}^{L-t-2} rho^u (rho = r - eta beta^2); dd0[0] = G_0,
    dbeta_t = eta (1 - 2 beta d_t[0]) G_{t+1}, dr_t = d_t[0] G_{t+1}."""
    L, dk, eta, b, r = 7, 3, 0.2, 0.8, 0.9
    k = np.zeros((1, L, 1, dk))
    k[..., 0] = 1.0
    beta = np.full((1, L, 1), b)
    rr = np.full((1, L, 1), r)
    wk = np.zeros((1, L, 1, dk))
    wk[..., 0] = 1.0
    gr = oracle.precond_bwd(k, beta, wk, eta=eta, dmin=-1e9, dmax=1e9, r=rr)
    rho = r - eta * b * b
    d = [1.0]
    for _ in range(L):
        d.append(rho * d[-1] + eta * b)
    G = [sum(rho ** u for u in range(L - t)) for t in range(L + 1)]  # G[t]: gradient on d_t
    np.testing.assert_allclose(gr["d0"][0, 0, 0], G[0], rtol=1e-13)
    np.testing.assert_allclose(gr["d0"][0, 0, 1:], 1.0 * 0, atol=0)
    np.testing.assert_allclose(gr["beta"][0, :, 0], [eta * (1 - 2 * b * d[t]) * G[t + 1] for t in range(L)],
                               rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(gr["r"][0, :, 0], [d[t] * G[t + 1] for t in range(L)], rtol=1e-12, atol=1e-15)
    assert np.all(gr["k"] == 0.0)  # kh = e1 is the only direction that matters, and |kh| is fixed


def test_phase1_gradient_invariances():
    x, wk, wd = p1_problem(L=8, H=2, dk=6, seed=7)
    kw = dict(eta=0.3, r=x["r"], d0=x["d0"])
    g1 = oracle.precond_bwd(x["k"], x["beta"], wk, dd_final=wd, **kw)
    # phase 1 reads k only through kh = k / |k|: each key gradient is orthogonal to its key
    dots = np.einsum("blhd,blhd->blh", g1["k"], x["k"])
    assert np.max(np.abs(dots)) < 1e-12 * max(1.0, np.max(np.abs(g1["k"])))
    assert np.max(np.abs(g1["k"])) > 1e-3
    # linear in (dkt, dd_final)
    ga = oracle.precond_bwd(x["k"], x["beta"], wk, dd_final=0 * wd, **kw)
    gb = oracle.precond_bwd(x["k"], x["beta"], 0 * wk, dd_final=wd, **kw)
    g2 = oracle.precond_bwd(x["k"], x["beta"], 3 * wk, dd_final=3 * wd, **kw)
    for n in g1:
        np.testing.assert_allclose(ga[n] + gb[n], g1[n], rtol=1e-11, atol=1e-13)
        np.testing.assert_allclose(g2[n], 3 * g1[n], rtol=1e-11, atol=1e-13)
    # the beta-free step has no beta gradient; a clamped beta passes none
    gf = oracle.precond_bwd(x["k"], x["beta"], wk, dd_final=wd, beta_aware=False, **kw)
    assert np.all(gf["beta"] == 0.0)
    b2 = x["beta"].copy()
    b2[0, 2, 1] = 2.5
    b2[0, 4, 0] = -0.5
    gc = oracle.precond_bwd(x["k"], b2, wk, dd_final=wd, **kw)
    assert gc["beta"][0, 2, 1] == 0.0 and gc["beta"][0, 4, 0] == 0.0
    # no retention gate equals a gate of ones
    gn = oracle.precond_bwd(x["k"], x["beta"], wk, dd_final=wd, eta=0.3, d0=x["d0"])
    go = oracle.precond_bwd(x["k"], x["beta"], wk, dd_final=wd, eta=0.3, d0=x["d0"],
                            r=np.ones_like(x["beta"]))
    for n in gn:
        np.testing.assert_array_equal(gn[n], go[n])


def osdn_loss(x, wo, wf, **kw):
    kt, _ = oracle.precond(x["k"], x["beta"], r=x["r"], d0=x["d0"], **kw)
    o, f = oracle.fwd(x["q"], x["k"][:, :, :, None], x["v"][:, :, :, None], x["beta"][..., None], g=x["g"],
                      kt=kt[:, :, :, None], h0=x["h0"])
    return float(np.sum(o * wo) + np.sum(f * wf))


@pytest.mark.parametrize("gate", [False, True])
def test_osdn_layer_gradient_matches_finite_differences(gate):
    """The whole layer: phase 1 emits the write keys from (k, beta), the
    write-key forward reads (q, k, v, beta) with them.  oracle.osdn_bwd sums
    the two routes into k and beta; finite differences of the composed forward
    pin that sum."""
    rng = np.random.default_rng(11 + gate)
    B, L, H, dk, dv = 1, 5, 2, 4, 3
    x = dict(q=rng.normal(size=(B, L, H, dk)), k=rng.normal(size=(B, L, H, dk)),
             v=rng.normal(size=(B, L, H, dv)), beta=rng.uniform(0.1, 1.9, size=(B, L, H)),
             g=rng.uniform(0.5, 1.0, size=(B, L, H)) if gate else None, h0=rng.normal(size=(B, H, dk, dv)),
             r=rng.uniform(0.7, 1.0, size=(B, L, H)), d0=rng.uniform(0.8, 1.4, size=(B, H, dk)))
    wo, wf = rng.normal(size=(B, L, H, dv)), rng.normal(size=(B, H, dk, dv))
    kw = dict(eta=0.4)
    gr = oracle.osdn_bwd(x["q"], x["k"], x["v"], x["beta"], wo, g=x["g"], h0=x["h0"], dfinal=wf,
                         d0=x["d0"], r=x["r"], **kw)
    names = ["q", "k", "v", "beta", "h0", "r", "d0"] + (["g"] if gate else [])
    for n in names:
        base = x[n]
        ref = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            saved = base[idx]
            base[idx] = saved + 1e-6
            lp = osdn_loss(x, wo, wf, **kw)
            base[idx] = saved - 1e-6
            lm = osdn_loss(x, wo, wf, **kw)
            base[idx] = saved
            ref[idx] = (lp - lm) / 2e-6
        scale = max(1.0, float(np.max(np.abs(ref))))
        err = float(np.max(np.abs(gr[n] - ref))) / scale
        assert err < 1e-6, f"{n}: finite-difference mismatch {err:.2e}"
