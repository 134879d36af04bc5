"""Pins of the fp64 oracle to what the pages and the mathematics fix (CPU only).

Each test names the passage it checks.  [DP] = DeltaProduct study notes
(arXiv 2502.10297v7), [OSDN] = OSDN study notes (arXiv 2605.13473v1).
The oracle is driven only through its public functions; the expected values
come from printed examples, closed forms, invariants or an independent
product-form brute force (tests/brute.py).
"""
import json
import math
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
from brute import brute_fwd, token_transition
from chunkform import chunk_fwd

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def transition(keys, betas, g=None, kt=None):
    """A_i of one token, read back from the oracle: H0 = I (dv = dk), v = 0."""
    keys = np.asarray(keys, np.float64)
    n_h, dk = keys.shape
    k = keys.reshape(1, 1, 1, n_h, dk)
    v = np.zeros((1, 1, 1, n_h, dk))
    q = np.zeros((1, 1, 1, dk))
    beta = np.asarray(betas, np.float64).reshape(1, 1, 1, n_h)
    gg = None if g is None else np.full((1, 1, 1), float(g))
    ktt = None if kt is None else np.asarray(kt, np.float64).reshape(1, 1, 1, n_h, dk)
    h0 = np.eye(dk).reshape(1, 1, dk, dk)
    _, fs = oracle.fwd(q, k, v, beta, g=gg, kt=ktt, h0=h0)
    return fs[0, 0]


def write_term(keys, betas, vals, kt=None):
    """B_i of one token, read back from the oracle: H0 = 0."""
    keys = np.asarray(keys, np.float64)
    vals = np.asarray(vals, np.float64)
    n_h, dk = keys.shape
    dv = vals.shape[1]
    k = keys.reshape(1, 1, 1, n_h, dk)
    v = vals.reshape(1, 1, 1, n_h, dv)
    q = np.zeros((1, 1, 1, dk))
    beta = np.asarray(betas, np.float64).reshape(1, 1, 1, n_h)
    ktt = None if kt is None else np.asarray(kt, np.float64).reshape(1, 1, 1, n_h, dk)
    _, fs = oracle.fwd(q, k, v, beta, kt=ktt)
    return fs[0, 0]


def rand_unit(rng, n, dk):
    x = rng.standard_normal((n, dk))
    return x / np.linalg.norm(x, axis=1, keepdims=True)


# ---------------------------------------------------------------- [DP] sec. 2.4


def test_mod3_worked_example_matrix():
    """[DP] sec. 2.4 (Fig.3, App.B.2): F2 F1 is the printed 120-degree rotation."""
    fx = _load("mod3_rotation.json")
    A = transition([fx["k1"], fx["k2"]], [fx["beta"], fx["beta"]])
    np.testing.assert_allclose(A, np.array(fx["F2F1_printed"]), atol=1e-15)
    ang = math.degrees(math.atan2(A[1, 0], A[0, 0]))
    assert abs(ang - fx["rotation_degrees"]) < 1e-12


def test_mod3_worked_example_orbit():
    """[DP] sec. 2.4: from (1,0), the state returns after exactly 3 tokens."""
    fx = _load("mod3_rotation.json")
    L = 9
    k = np.tile(np.array([fx["k1"], fx["k2"]]), (L, 1, 1)).reshape(1, L, 1, 2, 2)
    v = np.zeros((1, L, 1, 2, 1))
    beta = np.full((1, L, 1, 2), fx["beta"])
    h0 = np.array(fx["start_state"]).reshape(1, 1, 2, 1)
    states = []
    for e in (np.array([1.0, 0.0]), np.array([0.0, 1.0])):
        q = np.tile(e, (L, 1)).reshape(1, L, 1, 2)
        out, _ = oracle.fwd(q, k, v, beta, h0=h0)
        states.append(out[0, :, 0, 0])
    S = np.stack(states, axis=1)  # [L, 2]: the state after each token
    start = np.array(fx["start_state"])
    for t in range(L):
        if (t + 1) % fx["period_tokens"] == 0:
            np.testing.assert_allclose(S[t], start, atol=1e-14)
        else:
            assert np.linalg.norm(S[t] - start) > 1.0
    np.testing.assert_allclose(S[0], [-0.5, math.sqrt(3) / 2], atol=1e-15)
    np.testing.assert_allclose(S[1], [-0.5, -math.sqrt(3) / 2], atol=1e-15)


@pytest.mark.parametrize("b", [0.0, 0.3, 1.0, 1.7, 2.0])
def test_householder_spectrum(b):
    """[DP] sec. 2.4: F k = (1 - beta) k and F u = u for u orthogonal to k."""
    rng = np.random.default_rng(1)
    dk = 6
    k = rand_unit(rng, 1, dk)[0]
    A = transition([k], [b])
    np.testing.assert_allclose(A @ k, (1 - b) * k, atol=1e-14)
    u = rng.standard_normal(dk)
    u -= (u @ k) * k
    np.testing.assert_allclose(A @ u, u, atol=1e-14)


def test_identical_keys_collapse():
    """[DP] sec. 2.4: identical keys give one factor, beta_eff = 1 - prod(1 - beta_j)."""
    rng = np.random.default_rng(2)
    dk = 5
    for n_h in (2, 3, 4):
        k = rand_unit(rng, 1, dk)[0]
        betas = rng.uniform(0, 2, n_h)
        A = transition([k] * n_h, betas)
        beff = 1 - np.prod(1 - betas)
        np.testing.assert_allclose(A, np.eye(dk) - beff * np.outer(k, k), atol=1e-14)


def test_orthogonal_keys_commute():
    """[DP] sec. 2.4: orthogonal keys commute, A = I - sum beta_j k_j k_j^T (symmetric)."""
    rng = np.random.default_rng(3)
    dk, n_h = 6, 3
    Q, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    keys = Q[:, :n_h].T
    betas = rng.uniform(0, 2, n_h)
    A = transition(keys, betas)
    expect = np.eye(dk) - sum(b * np.outer(kk, kk) for b, kk in zip(betas, keys))
    np.testing.assert_allclose(A, expect, atol=1e-14)
    np.testing.assert_allclose(A, A.T, atol=1e-14)
    A_rev = transition(keys[::-1], betas[::-1])
    np.testing.assert_allclose(A_rev, A, atol=1e-14)


def test_complex_eigenvalue_criterion():
    """[DP] sec. 2.4 (App.A, Prop.1): tau = trace, delta = det; complex iff tau^2 < 4 delta."""
    rng = np.random.default_rng(4)
    seen = {True: 0, False: 0}
    for _ in range(200):
        k1, k2 = rand_unit(rng, 2, 2)
        b1, b2 = rng.uniform(0, 2, 2)
        A = transition([k1, k2], [b1, b2])
        c = k1 @ k2
        tau = 2 - b1 - b2 + b1 * b2 * c * c
        delta = (1 - b1) * (1 - b2)
        assert abs(np.trace(A) - tau) < 1e-13
        assert abs(np.linalg.det(A) - delta) < 1e-13
        disc = tau * tau - 4 * delta
        if abs(disc) < 1e-9:
            continue
        ev = np.linalg.eigvals(A)
        is_complex = bool(np.max(np.abs(ev.imag)) > 1e-12)
        assert is_complex == (disc < 0)
        seen[is_complex] += 1
    assert seen[True] > 5 and seen[False] > 5


# ---------------------------------------------------------------- [DP] sec. 2.3


def test_nh2_cross_term():
    """[DP] sec. 2.3: A_i = I - b1 k1k1^T - b2 k2k2^T + b1 b2 (k2^T k1) k2 k1^T,
    and H_i = F2 F1 H + F2 C1 + C2."""
    rng = np.random.default_rng(5)
    dk, dv = 5, 3
    for _ in range(10):
        k1, k2 = rand_unit(rng, 2, dk)
        b1, b2 = rng.uniform(0, 2, 2)
        A = transition([k1, k2], [b1, b2])
        expect = (np.eye(dk) - b1 * np.outer(k1, k1) - b2 * np.outer(k2, k2)
                  + b1 * b2 * (k2 @ k1) * np.outer(k2, k1))
        np.testing.assert_allclose(A, expect, atol=1e-14)
        assert np.max(np.abs(A - A.T)) > 1e-3  # the cross term breaks symmetry
        vals = rng.standard_normal((2, dv))
        Bw = write_term([k1, k2], [b1, b2], vals)
        F2 = np.eye(dk) - b2 * np.outer(k2, k2)
        C1 = b1 * np.outer(k1, vals[0])
        C2 = b2 * np.outer(k2, vals[1])
        np.testing.assert_allclose(Bw, F2 @ C1 + C2, atol=1e-14)


@pytest.mark.parametrize("n_h", [1, 2, 3, 4])
def test_rank_bound(n_h):
    """[DP] sec. 2.3: rank(A_i - I) <= n_h; [DP] sec. 2.6: rank(A_i - g I) <= n_h."""
    rng = np.random.default_rng(10 + n_h)
    dk = 8
    keys = rand_unit(rng, n_h, dk)
    betas = rng.uniform(0.1, 2, n_h)
    sv = np.linalg.svd(transition(keys, betas) - np.eye(dk), compute_uv=False)
    assert np.all(sv[n_h:] < 1e-12)
    assert sv[n_h - 1] > 1e-6
    g = 0.37
    sv = np.linalg.svd(transition(keys, betas, g=g) - g * np.eye(dk), compute_uv=False)
    assert np.all(sv[n_h:] < 1e-12)


def test_norm_bound_products():
    """[DP] sec. 2.5 (App.B.6): unit keys and beta in [0,2] give ||A_t...A_1||_2 <= 1."""
    rng = np.random.default_rng(6)
    dk, n_h, L = 6, 3, 40
    k = rng.standard_normal((1, L, 1, n_h, dk))
    beta = rng.uniform(0, 2, (1, L, 1, n_h))
    beta[0, ::7, 0, :] = 2.0  # include pure reflections
    v = np.zeros((1, L, 1, n_h, dk))
    q = np.zeros((1, L, 1, dk))
    for t in range(1, L + 1):
        _, fs = oracle.fwd(q[:, :t], k[:, :t], v[:, :t], beta[:, :t],
                           h0=np.eye(dk).reshape(1, 1, dk, dk))
        assert np.linalg.norm(fs[0, 0], 2) <= 1 + 1e-12
    A1 = transition(k[0, 0, 0], beta[0, 0, 0])
    assert np.linalg.norm(A1, 2) <= 1 + 1e-12


def test_product_not_sum_closed_form():
    """[DP] sec. 2.5: identical keys with beta1 = beta2 = 2 give A = I (the sum would give
    eigenvalue -3); writes still grow: H_t = H0 + t * 2 k (v2 - v1)^T."""
    rng = np.random.default_rng(7)
    dk, dv, L = 4, 3, 6
    kk = rand_unit(rng, 1, dk)[0]
    A = transition([kk, kk], [2.0, 2.0])
    np.testing.assert_allclose(A, np.eye(dk), atol=1e-14)
    summed = np.eye(dk) - 2 * np.outer(kk, kk) - 2 * np.outer(kk, kk)
    assert abs(np.min(np.linalg.eigvalsh(summed)) + 3) < 1e-12
    v1, v2 = rng.standard_normal((2, dv))
    k = np.tile(kk, (L, 2, 1)).reshape(1, L, 1, 2, dk)
    v = np.tile(np.stack([v1, v2]), (L, 1, 1)).reshape(1, L, 1, 2, dv)
    beta = np.full((1, L, 1, 2), 2.0)
    h0 = rng.standard_normal((1, 1, dk, dv))
    step = 2 * np.outer(kk, v2 - v1)
    for t in range(1, L + 1):
        _, fs = oracle.fwd(np.zeros((1, t, 1, dk)), k[:, :t], v[:, :t], beta[:, :t], h0=h0)
        np.testing.assert_allclose(fs[0, 0], h0[0, 0] + t * step, atol=1e-12)


# ---------------------------------------------------------------- [DP] sec. 2.1 / 3.1


def test_exact_recall_beta_one():
    """[DP] sec. 2.1 (Eq.(2)): with a unit key and beta = 1, H^T k = v after the step."""
    rng = np.random.default_rng(8)
    dk, dv = 7, 5
    h0 = rng.standard_normal((1, 1, dk, dv))
    kraw = rng.standard_normal(dk) * 3.7  # unnormalised: the forward normalises it
    kh = kraw / np.linalg.norm(kraw)
    v = rng.standard_normal(dv)
    out, _ = oracle.fwd(kh.reshape(1, 1, 1, dk), kraw.reshape(1, 1, 1, 1, dk),
                        v.reshape(1, 1, 1, 1, dv), np.ones((1, 1, 1, 1)), h0=h0)
    np.testing.assert_allclose(out[0, 0, 0], v, atol=1e-13)


def test_orthonormal_keys_recall_all_pairs():
    """Orthonormal keys with beta = 1 store every one of the n_h pairs exactly
    ([DP] sec. 2.1 exact recall, combined with the commuting case of sec. 2.4)."""
    rng = np.random.default_rng(9)
    dk, dv, n_h = 8, 4, 4
    Q, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    keys = Q[:, :n_h].T
    vals = rng.standard_normal((n_h, dv))
    h0 = rng.standard_normal((1, 1, dk, dv))
    _, fs = oracle.fwd(np.zeros((1, 1, 1, dk)), keys.reshape(1, 1, 1, n_h, dk),
                       vals.reshape(1, 1, 1, n_h, dv), np.ones((1, 1, 1, n_h)), h0=h0)
    np.testing.assert_allclose(keys @ fs[0, 0], vals, atol=1e-13)


def test_swap_reflection_permutes_rows():
    """[DP] sec. 3.1: k = (e_a - e_b)/sqrt2 with beta = 2 swaps coordinates a and b;
    n - 1 such reflections in one token realise any permutation (Theorem 1, 1 layer)."""
    n = 5
    e = np.eye(n)
    h0 = np.arange(1.0, n + 1).reshape(1, 1, n, 1)  # H0 = (1, ..., n)^T
    perm = [3, 0, 4, 1, 2]  # target: new[i] = old[perm[i]]
    # build transpositions that sort identity into perm
    cur = list(range(n))
    swaps = []
    for i in range(n - 1):
        jj = cur.index(perm[i])
        if jj != i:
            swaps.append((i, jj))
            cur[i], cur[jj] = cur[jj], cur[i]
    while len(swaps) < n - 1:  # pad with identity factors (beta = 0)
        swaps.append(None)
    keys, betas = [], []
    for s in swaps:
        if s is None:
            keys.append(e[0])
            betas.append(0.0)
        else:
            keys.append((e[s[0]] - e[s[1]]) / math.sqrt(2))
            betas.append(2.0)
    _, fs = oracle.fwd(np.zeros((1, 1, 1, n)), np.array(keys).reshape(1, 1, 1, n - 1, n),
                       np.zeros((1, 1, 1, n - 1, 1)), np.array(betas).reshape(1, 1, 1, n - 1),
                       h0=h0)
    np.testing.assert_allclose(fs[0, 0, :, 0], np.arange(1.0, n + 1)[perm], atol=1e-13)


# ---------------------------------------------------------------- [DP] sec. 2.6 / 3.3 / 4.1


def test_gate_zero_resets_history():
    """[DP] sec. 3.3 (App.B.3): g_t = 0 erases the history; the state after token t is
    B_t whatever came before."""
    rng = np.random.default_rng(11)
    dk, dv, n_h, L = 6, 4, 2, 8
    k = rng.standard_normal((1, L, 1, n_h, dk))
    v = rng.standard_normal((1, L, 1, n_h, dv))
    beta = rng.uniform(0, 2, (1, L, 1, n_h))
    q = rng.standard_normal((1, L, 1, dk))
    g = rng.uniform(0.2, 1.0, (1, L, 1))
    g[0, 4, 0] = 0.0
    outs = []
    for seed in (0, 1):
        r2 = np.random.default_rng(100 + seed)
        k2 = k.copy()
        v2 = v.copy()
        k2[:, :4] = r2.standard_normal(k2[:, :4].shape)
        v2[:, :4] = r2.standard_normal(v2[:, :4].shape)
        out, fs = oracle.fwd(q, k2, v2, beta, g=g, h0=r2.standard_normal((1, 1, dk, dv)))
        outs.append((out, fs))
    np.testing.assert_allclose(outs[0][0][:, 4:], outs[1][0][:, 4:], atol=1e-13)
    np.testing.assert_allclose(outs[0][1], outs[1][1], atol=1e-13)
    assert np.max(np.abs(outs[0][0][:, :4] - outs[1][0][:, :4])) > 1e-3
    _, Bt = token_transition(k[0, 4, 0], beta[0, 4, 0], v=v[0, 4, 0])
    out5, fs5 = oracle.fwd(q[:, 4:5], k[:, 4:5], v[:, 4:5], beta[:, 4:5])
    np.testing.assert_allclose(fs5[0, 0], Bt, atol=1e-13)


def test_expansion_equals_deltanet_on_expanded_sequence():
    """[DP] sec. 4.1 (Sec.5.1): DeltaProduct(n_h) equals DeltaNet (n_h = 1) over the
    interleaved sub-step sequence with gate (g, 1, ..., 1), reading each token's last
    sub-step."""
    rng = np.random.default_rng(12)
    B, L, H, n_h, dk, dv = 2, 7, 3, 3, 5, 4
    q = rng.standard_normal((B, L, H, dk))
    k = rng.standard_normal((B, L, H, n_h, dk))
    v = rng.standard_normal((B, L, H, n_h, dv))
    beta = rng.uniform(0, 2, (B, L, H, n_h))
    g = rng.uniform(0.1, 1.0, (B, L, H))
    h0 = rng.standard_normal((B, H, dk, dv))
    out, fs = oracle.fwd(q, k, v, beta, g=g, h0=h0)
    N = L * n_h
    ke = k.transpose(0, 2, 1, 3, 4).reshape(B, H, N, dk).transpose(0, 2, 1, 3)[:, :, :, None]
    ve = v.transpose(0, 2, 1, 3, 4).reshape(B, H, N, dv).transpose(0, 2, 1, 3)[:, :, :, None]
    be = beta.transpose(0, 2, 1, 3).reshape(B, H, N).transpose(0, 2, 1)[..., None]
    ge = np.ones((B, N, H))
    ge[:, 0::n_h] = g
    qe = np.zeros((B, N, H, dk))
    qe[:, n_h - 1::n_h] = q
    oute, fse = oracle.fwd(qe, ke, ve, be, g=ge, h0=h0)
    np.testing.assert_allclose(oute[:, n_h - 1::n_h], out, atol=1e-12)
    np.testing.assert_allclose(fse, fs, atol=1e-12)


def test_resume_split_equals_single_call():
    """[DP] sec. 2.2: H_{i,0} = H_{i-1}; the carried state is everything, so two calls
    with the state passed on equal one call."""
    rng = np.random.default_rng(13)
    B, L, H, n_h, dk, dv = 1, 11, 2, 2, 4, 3
    q = rng.standard_normal((B, L, H, dk))
    k = rng.standard_normal((B, L, H, n_h, dk))
    v = rng.standard_normal((B, L, H, n_h, dv))
    beta = rng.uniform(0, 2, (B, L, H, n_h))
    g = rng.uniform(0.1, 1.0, (B, L, H))
    out, fs = oracle.fwd(q, k, v, beta, g=g)
    m = 5
    o1, f1 = oracle.fwd(q[:, :m], k[:, :m], v[:, :m], beta[:, :m], g=g[:, :m])
    o2, f2 = oracle.fwd(q[:, m:], k[:, m:], v[:, m:], beta[:, m:], g=g[:, m:], h0=f1)
    np.testing.assert_allclose(np.concatenate([o1, o2], 1), out, atol=1e-13)
    np.testing.assert_allclose(f2, fs, atol=1e-13)


def test_fwd_heads_matches_full():
    rng = np.random.default_rng(14)
    B, L, H, n_h, dk, dv = 2, 6, 3, 2, 4, 5
    q = rng.standard_normal((B, L, H, dk))
    k = rng.standard_normal((B, L, H, n_h, dk))
    v = rng.standard_normal((B, L, H, n_h, dv))
    beta = rng.uniform(0, 2, (B, L, H, n_h))
    out, fs = oracle.fwd(q, k, v, beta)
    heads = [5, 0, 3]
    oh, fh = oracle.fwd_heads(q, k, v, beta, heads)
    for i, bh in enumerate(heads):
        b, h = divmod(bh, H)
        np.testing.assert_array_equal(oh[i], out[b, :, h])
        np.testing.assert_array_equal(fh[i], fs[b, h])


# ---------------------------------------------------------------- brute force / chunk form


@settings(max_examples=60, deadline=None)
@given(dk=st.integers(1, 8), dv=st.integers(1, 8), n_h=st.integers(1, 4),
       L=st.integers(1, 12), gated=st.booleans(), asym=st.booleans(), with_h0=st.booleans(),
       seed=st.integers(0, 2 ** 31 - 1))
def test_oracle_equals_product_form(dk, dv, n_h, L, gated, asym, with_h0, seed):
    """Oracle (sub-step updates) vs explicit per-token products A_i, B_i ([DP] sec. 2.3)."""
    rng = np.random.default_rng(seed)
    B, H = 1, 2
    q = rng.standard_normal((B, L, H, dk))
    k = rng.standard_normal((B, L, H, n_h, dk))
    v = rng.standard_normal((B, L, H, n_h, dv))
    beta = rng.uniform(-0.5, 2.5, (B, L, H, n_h))  # exercises the [0, 2] clamp
    g = rng.uniform(0, 1, (B, L, H)) if gated else None
    kt = rng.standard_normal((B, L, H, n_h, dk)) * 0.5 if asym else None
    h0 = rng.standard_normal((B, H, dk, dv)) if with_h0 else None
    out, fs = oracle.fwd(q, k, v, beta, g=g, kt=kt, h0=h0)
    ob, fb = brute_fwd(q, k, v, beta, g=g, kt=kt, h0=h0)
    scale = max(1.0, np.max(np.abs(ob)), np.max(np.abs(fb)))
    assert np.max(np.abs(out - ob)) <= 1e-12 * scale
    assert np.max(np.abs(fs - fb)) <= 1e-12 * scale


@pytest.mark.parametrize("n_h,L,C,gated,asym", [
    (1, 40, 16, False, False), (2, 37, 16, True, False), (3, 30, 16, False, True),
    (3, 33, 32, True, True), (2, 64, 64, True, False), (4, 9, 16, False, False),
])
def test_chunk_form_equals_oracle(n_h, L, C, gated, asym):
    """The chunkwise WY / UT form ([OSDN] sec. 2.5, App.A.2) with gates and padding
    reproduces the sequential oracle; tokens straddle chunks when n_h does not divide C."""
    rng = np.random.default_rng(1000 + n_h * 100 + L)
    B, H, dk, dv = 1, 2, 8, 6
    q = rng.standard_normal((B, L, H, dk))
    k = rng.standard_normal((B, L, H, n_h, dk))
    v = rng.standard_normal((B, L, H, n_h, dv))
    beta = rng.uniform(0, 2, (B, L, H, n_h))
    g = rng.uniform(0.3, 1.0, (B, L, H)) if gated else None
    kt = rng.standard_normal((B, L, H, n_h, dk)) * 0.3 if asym else None
    h0 = rng.standard_normal((B, H, dk, dv))
    out, fs = oracle.fwd(q, k, v, beta, g=g, kt=kt, h0=h0)
    oc, fc = chunk_fwd(q, k, v, beta, C, g=g, kt=kt, h0=h0)
    scale = max(1.0, np.max(np.abs(out)))
    assert np.max(np.abs(out - oc)) <= 1e-12 * scale
    assert np.max(np.abs(fs - fc)) <= 1e-12 * max(1.0, np.max(np.abs(fs)))


# ---------------------------------------------------------------- [OSDN]


def test_osdn_one_step_identity_and_teaching_example():
    """[OSDN] sec. 2.3-2.4: with write key d*k, S_t k - v = -u (1 - a), a = beta <d, k*k>,
    and the printed teaching example q = (1 - a)^2 = 0.25 / 0.0625."""
    fx = _load("osdn_teaching_example.json")
    rng = np.random.default_rng(15)
    dk = len(fx["k"])
    dv = 3
    k = np.array(fx["k"])
    v = rng.standard_normal(dv)
    h0 = rng.standard_normal((1, 1, dk, dv))
    for case in fx["cases"]:
        d = np.array(case["d"])
        kt = d * k
        out, _ = oracle.fwd(k.reshape(1, 1, 1, dk), k.reshape(1, 1, 1, 1, dk),
                            v.reshape(1, 1, 1, 1, dv), np.full((1, 1, 1, 1), fx["beta"]),
                            kt=kt.reshape(1, 1, 1, 1, dk), h0=h0)
        u = v - h0[0, 0].T @ k
        a = fx["beta"] * np.dot(d, k * k)
        np.testing.assert_allclose(out[0, 0, 0] - v, -u * (1 - a), atol=1e-14)
        ratio = np.sum((out[0, 0, 0] - v) ** 2) / np.sum(u ** 2)
        assert abs(ratio - case["q"]) < 1e-14


def test_osdn_oscillation_counterexample():
    """[OSDN] sec. 3.3 (App.D.4): K = V = 1, k = 1, exact writes, v_t = (-1)^t give
    S_t = (-1)^t.  Phase 1 keeps d = 1 here because a_t = 1."""
    fx = _load("osdn_oscillation.json")
    L = 10
    k = np.full((1, L, 1, 1), fx["k"])
    beta = np.full((1, L, 1), fx["beta_exact_write"])
    kt, d = oracle.precond(k, beta)
    np.testing.assert_allclose(d, 1.0, atol=0)
    np.testing.assert_allclose(kt, 1.0, atol=0)
    v = np.array([(-1.0) ** t for t in range(1, L + 1)]).reshape(1, L, 1, 1, 1)
    out, fs = oracle.fwd(np.ones((1, L, 1, 1)), k.reshape(1, L, 1, 1, 1), v,
                         beta.reshape(1, L, 1, 1), kt=kt.reshape(1, L, 1, 1, 1))
    np.testing.assert_allclose(out[0, :, 0, 0], v.reshape(L), atol=0)
    assert fs[0, 0, 0, 0] == (-1.0) ** L


@pytest.mark.parametrize("b", [0.6, 0.9, 1.3])
def test_phase1_closed_form_inside_box(b):
    """[OSDN] sec. 2.4: k = e1, beta constant: d_{t,1} = 1/b + (1 - eta b^2)^(t-1) (1 - 1/b)
    while inside the box (1/b in [0.5, 2]); other coordinates stay 1; the emitted key
    uses d_t (before the update)."""
    eta, dk, L = 0.05, 4, 60
    k = np.zeros((1, L, 1, dk))
    k[..., 0] = 2.5  # raw, normalised inside to e1
    beta = np.full((1, L, 1), b)
    kt, d = oracle.precond(k, beta, eta=eta)
    t = np.arange(1, L + 1)
    d1 = 1 / b + (1 - eta * b * b) ** (t - 1) * (1 - 1 / b)
    np.testing.assert_allclose(kt[0, :, 0, 0], d1, rtol=0, atol=1e-13)
    np.testing.assert_allclose(kt[0, :, 0, 1:], 0.0, atol=0)
    dL1 = 1 / b + (1 - eta * b * b) ** L * (1 - 1 / b)
    assert abs(d[0, 0, 0] - dL1) < 1e-13
    np.testing.assert_allclose(d[0, 0, 1:], 1.0, atol=0)


def test_phase1_saturates_at_box():
    """[OSDN] sec. 2.4 / 3.2: beta < 0.5 puts the target 1/beta above the box; d climbs by
    the closed form, then sits exactly at dmax = 2."""
    b, eta, dk, L = 0.3, 0.5, 3, 40
    k = np.zeros((1, L, 1, dk))
    k[..., 0] = 1.0
    kt, d = oracle.precond(k, np.full((1, L, 1), b), eta=eta)
    traj = kt[0, :, 0, 0]
    t = np.arange(1, L + 1)
    free = 1 / b + (1 - eta * b * b) ** (t - 1) * (1 - 1 / b)
    first = int(np.argmax(free > 2.0))
    assert first > 1
    np.testing.assert_allclose(traj[:first], free[:first], atol=1e-13)
    np.testing.assert_allclose(traj[first:], 2.0, atol=0)
    assert d[0, 0, 0] == 2.0
    # and the lower face: beta = 1.8 pulls d towards 1/1.8 < dmin = 0.8
    kt2, d2 = oracle.precond(k, np.full((1, L, 1), 1.8), eta=eta, dmin=0.8)
    assert np.min(kt2[0, :, 0, 0]) >= 0.8 and d2[0, 0, 0] == 0.8


def test_phase1_fixed_point_and_box_invariant():
    """[OSDN] sec. 2.4: a_t = 1 leaves d unchanged; d always stays in [0.5, 2]."""
    rng = np.random.default_rng(16)
    dk, L = 16, 50
    k = rng.standard_normal((1, L, 1, dk))
    kt, d = oracle.precond(k, np.ones((1, L, 1)))
    np.testing.assert_allclose(d, 1.0, atol=1e-13)
    k = rng.standard_normal((2, 200, 3, dk))
    beta = rng.uniform(0, 1, (2, 200, 3))
    kt, d = oracle.precond(k, beta, eta=0.8)
    kh = k / np.linalg.norm(k, axis=-1, keepdims=True)
    ratio = kt / np.where(np.abs(kh) > 1e-9, kh, np.nan)
    assert np.nanmin(ratio) >= 0.5 - 1e-12 and np.nanmax(ratio) <= 2 + 1e-12
    assert np.min(d) >= 0.5 and np.max(d) <= 2.0


# ---------------------------------------------------------------- [OSDN] phase-1 variants


def test_phase1_retention_closed_form():
    """[OSDN] sec. 2.6 (APF, Sec.4.4): the retention gate scales d_t, the step still uses
    d_t.  k = e1, constant beta and r: d_{t+1,1} = (r - eta b^2) d_t + eta b, so
    d_{t,1} = d* + (r - eta b^2)^(t-1) (1 - d*), d* = eta b / (1 - r + eta b^2), while
    inside the box; the other coordinates only decay, d_t = r^(t-1), until the
    projection's floor dmin holds them (the gate does not reset d to 1)."""
    eta, b, r, dk, L = 0.05, 0.9, 0.97, 3, 60
    k = np.zeros((1, L, 1, dk))
    k[..., 0] = 0.7
    kt, d = oracle.precond(k, np.full((1, L, 1), b), eta=eta, r=np.full((1, L, 1), r))
    t = np.arange(1, L + 1)
    ds = eta * b / (1 - r + eta * b * b)
    assert 0.5 < ds < 2.0
    np.testing.assert_allclose(kt[0, :, 0, 0], ds + (r - eta * b * b) ** (t - 1) * (1 - ds),
                               rtol=0, atol=1e-13)
    np.testing.assert_allclose(d[0, 0, 0], ds + (r - eta * b * b) ** L * (1 - ds), atol=1e-13)
    # coordinates with s = 0: pure decay, then the floor (the emitted key is 0 there)
    np.testing.assert_allclose(d[0, 0, 1:], max(r ** L, 0.5), atol=0)
    for T in (5, 20, 40):
        _, dT = oracle.precond(k[:, :T], np.full((1, T, 1), b), eta=eta, r=np.full((1, T, 1), r))
        np.testing.assert_allclose(dT[0, 0, 1:], max(r ** T, 0.5), rtol=1e-14, atol=0)
    # r = 1 is exactly the gate-free scan
    kt1, d1 = oracle.precond(k, np.full((1, L, 1), b), eta=eta, r=np.ones((1, L, 1)))
    kt0, d0 = oracle.precond(k, np.full((1, L, 1), b), eta=eta)
    assert np.array_equal(kt1, kt0) and np.array_equal(d1, d0)


def test_phase1_beta_free_closed_form():
    """[OSDN] sec. 2.7 (App.B/C, the 1.3B configuration): the phase-1 step carries no
    beta, d_{t+1} = d_t + eta (1 - <d_t, k^2>) k^2 for unit keys.  With k = e1 the first
    coordinate follows d_t = 1 + (1 - eta)^(t-1) (d_1 - 1) whatever beta is; with the box
    dropped (dmin = -inf, dmax = inf) and a retention r it follows the affine map
    d_{t+1} = (r - eta) d_t + eta below the old floor."""
    rng = np.random.default_rng(21)
    eta, dk, L = 0.08, 4, 50
    k = np.zeros((1, L, 1, dk))
    k[..., 0] = 3.0
    beta = rng.uniform(0.05, 1.95, (1, L, 1))
    d0 = np.full((1, 1, dk), 0.6)
    kt, d = oracle.precond(k, beta, eta=eta, d0=d0, beta_aware=False)
    t = np.arange(1, L + 1)
    np.testing.assert_allclose(kt[0, :, 0, 0], 1 + (1 - eta) ** (t - 1) * (0.6 - 1), atol=1e-13)
    np.testing.assert_allclose(d[0, 0, 1:], 0.6, atol=0)
    # the beta-aware scan on the same input moves differently
    kta, _ = oracle.precond(k, beta, eta=eta, d0=d0)
    assert np.max(np.abs(kta - kt)) > 1e-3
    # no box, retention 0.9: fixed point eta / (1 - r + eta) = 0.444.. < 0.5
    r = 0.9
    kt2, d2 = oracle.precond(k, beta, eta=eta, d0=d0, beta_aware=False, dmin=-np.inf,
                             dmax=np.inf, r=np.full((1, L, 1), r))
    fp = eta / (1 - r + eta)
    np.testing.assert_allclose(kt2[0, :, 0, 0], fp + (r - eta) ** (t - 1) * (0.6 - fp), atol=1e-13)
    np.testing.assert_allclose(d2[0, 0, 1:], 0.6 * r ** L, rtol=1e-13)


# ---------------------------------------------------------------- [OSDN] KDA host: per-channel gate


def test_channel_gate_without_writes_is_a_diagonal_decay():
    """[OSDN] sec. 2.7: the KDA host decays the state per key channel, H <- Diag(alpha_t) H,
    before the token's update.  With beta = 0 nothing is written, so H_t =
    Diag(prod_{s <= t} alpha_s) H_0 row by row, and out_t = H_t^T q_t."""
    rng = np.random.default_rng(31)
    B, L, H, n_h, dk, dv = 1, 7, 2, 2, 5, 3
    q = rng.standard_normal((B, L, H, dk))
    k = rng.standard_normal((B, L, H, n_h, dk))
    v = rng.standard_normal((B, L, H, n_h, dv))
    beta = np.zeros((B, L, H, n_h))
    ga = rng.uniform(0.2, 1.0, (B, L, H, dk))
    h0 = rng.standard_normal((B, H, dk, dv))
    out, fs = oracle.fwd(q, k, v, beta, ga=ga, h0=h0)
    decay = np.cumprod(ga, axis=1)  # [B, L, H, dk]
    for t in range(L):
        Ht = decay[0, t][:, :, None] * h0[0]  # [H, dk, dv]
        np.testing.assert_allclose(out[0, t], np.einsum("hkv,hk->hv", Ht, q[0, t]), atol=1e-13)
    np.testing.assert_allclose(fs[0], decay[0, -1][:, :, None] * h0[0], atol=1e-14)


def test_channel_gate_kda_step_closed_form():
    """[OSDN] sec. 2.7: H_1 = (I - b kt k^T) Diag(alpha) H_0 + b kt v^T.  With k = e_1,
    kt = c e_1 and b = 1, row 0 becomes (1 - c) alpha_0 H_0[0] + c v and every other row
    r is alpha_r H_0[r]: the decay acts on rows (key channels), before the write."""
    rng = np.random.default_rng(32)
    dk, dv, c = 4, 3, 0.7
    h0 = rng.standard_normal((1, 1, dk, dv))
    alpha = np.array([0.9, 0.5, 0.25, 0.8])
    v = rng.standard_normal(dv)
    k = np.zeros((1, 1, 1, 1, dk))
    k[..., 0] = 2.0  # normalised inside to e_1
    kt = np.zeros_like(k)
    kt[..., 0] = c
    q = rng.standard_normal((1, 1, 1, dk))
    _, fs = oracle.fwd(q, k, v.reshape(1, 1, 1, 1, dv), np.ones((1, 1, 1, 1)), kt=kt, h0=h0,
                       ga=alpha.reshape(1, 1, 1, dk))
    want = alpha[:, None] * h0[0, 0]
    want[0] = (1 - c) * alpha[0] * h0[0, 0, 0] + c * v
    np.testing.assert_allclose(fs[0, 0], want, atol=1e-14)


def test_uniform_channel_gate_is_the_scalar_gate():
    """A per-channel gate equal in every channel is the scalar gate of [DP] sec. 2.6, and
    the two compose by product."""
    rng = np.random.default_rng(33)
    B, L, H, n_h, dk, dv = 2, 9, 2, 3, 6, 4
    q = rng.standard_normal((B, L, H, dk))
    k = rng.standard_normal((B, L, H, n_h, dk))
    v = rng.standard_normal((B, L, H, n_h, dv))
    beta = rng.uniform(0, 2, (B, L, H, n_h))
    g = rng.uniform(0.3, 1.0, (B, L, H))
    o1, f1 = oracle.fwd(q, k, v, beta, g=g)
    o2, f2 = oracle.fwd(q, k, v, beta, ga=np.repeat(g[..., None], dk, axis=-1))
    np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(f2, f1, rtol=1e-12, atol=1e-13)
    g2 = rng.uniform(0.3, 1.0, (B, L, H))
    o3, _ = oracle.fwd(q, k, v, beta, g=g, ga=np.repeat(g2[..., None], dk, axis=-1))
    o4, _ = oracle.fwd(q, k, v, beta, g=g * g2)
    np.testing.assert_allclose(o3, o4, rtol=1e-12, atol=1e-13)
