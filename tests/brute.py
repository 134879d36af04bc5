"""Product-form brute force (fp64 NumPy) for tiny shapes: a pin for the oracle.

Instead of the oracle's sub-step update, each token's transition is built as
explicit matrices, following the expansion in the DeltaProduct study notes,
sec. 2.3 (Eq.(3) written out in execution order):

    F_j = I - beta_j w_j k_j^T          (w_j = k_j, or the write key)
    C_j = beta_j w_j v_j^T
    A_i = g_i F_{n_h} ... F_1           (sec. 2.6: the gate multiplies A only)
    B_i = sum_j F_{n_h} ... F_{j+1} C_j (empty product = I)
    H_i = A_i H_{i-1} + B_i,   o_i = H_i^T q_i.

The asymmetric factor I - beta w k^T is the OSDN transition (OSDN study notes,
sec. 2.2, Eq.(5), written for H = S^T).  Independent code from the oracle: a
test helper only.
"""
import numpy as np


def unit(x, eps=1e-6):
    n = np.linalg.norm(x)
    return x / max(n, eps)


def token_transition(k, beta, g=None, kt=None, v=None):
    """A_i and B_i of one token.

    k: [n_h, dk] raw keys; beta: [n_h]; g: scalar or None; kt: [n_h, dk] write
    keys or None; v: [n_h, dv] or None (then B_i is returned as None).
    """
    n_h, dk = k.shape
    eye = np.eye(dk)
    Fs, Cs = [], []
    for j in range(n_h):
        kh = unit(k[j])
        b = min(max(float(beta[j]), 0.0), 2.0)
        w = kh if kt is None else kt[j]
        Fs.append(eye - b * np.outer(w, kh))
        if v is not None:
            Cs.append(b * np.outer(w, v[j]))
    A = eye.copy()
    for F in Fs:            # later factors multiply on the left
        A = F @ A
    if g is not None:
        A = g * A
    if v is None:
        return A, None
    Bm = np.zeros((dk, v.shape[1]))
    for j in range(n_h):
        P = eye.copy()
        for F in Fs[j + 1:]:
            P = F @ P
        Bm += P @ Cs[j]
    return A, Bm


def brute_fwd(q, k, v, beta, g=None, kt=None, h0=None):
    """Whole forward by explicit per-token products; same layouts as the oracle."""
    q, k, v, beta = (np.asarray(a, np.float64) for a in (q, k, v, beta))
    B, L, H, n_h, dk = k.shape
    dv = v.shape[-1]
    out = np.zeros((B, L, H, dv))
    fs = np.zeros((B, H, dk, dv))
    for b in range(B):
        for h in range(H):
            S = np.zeros((dk, dv)) if h0 is None else np.array(h0[b, h], np.float64)
            for t in range(L):
                A, Bm = token_transition(k[b, t, h], beta[b, t, h],
                                         None if g is None else float(g[b, t, h]),
                                         None if kt is None else np.asarray(kt[b, t, h], np.float64),
                                         v[b, t, h])
                S = A @ S + Bm
                out[b, t, h] = S.T @ q[b, t, h]
            fs[b, h] = S
    return out, fs
