"""fp64 NumPy chunk form of the forward: pins the algebra the GPU kernels use.

A test helper, not the oracle.  It is checked against the sequential oracle
to 1e-12, which shows that the chunkwise (WY / UT) formulation computes the
same recurrence.  The ungated symmetric form is the one the OSDN study notes
print (sec. 2.5, App.A.2 / App.C):

    T = (I + tril(B K Kt^T, -1))^{-1},  W = T B K,  U = T B V,
    S_next = S + (U - W S^T)^T Kt,  scores Q Kt^T.

Here it is written for H = S^T (dk x dv), for the expanded sequence of
DeltaProduct sub-steps (DeltaProduct study notes sec. 4.1 / Sec.5.1: keys
interleaved token by token, gate expanded to (g, 1, ..., 1), readout only at
each token's last sub-step), with the per-sub-step log-gate lambda and its
chunk-local inclusive cumsum G, E_ij = exp(G_i - G_j):

    M   = strict_tril(diag(beta) (E o K Kt^T))      T = (I + M)^{-1}
    Up  = T diag(beta) (V - diag(e^G) K H0)          (pseudo-values)
    O   = diag(e^G) Q H0 + (tril_incl(Q Kt^T) o E) Up   (readout rows only)
    H1  = e^{G_last} H0 + (diag(e^{G_last - G}) Kt)^T Up

A sequence whose length N = L*n_h is not a multiple of the chunk C is padded
with beta = 0, k = 0, lambda = 0 sub-steps (beta = 0 makes a factor the
identity, DeltaProduct notes sec. 2.4), which is exact.
"""
import numpy as np


def _expand(k, kt, v, beta, g, b, h, n_h, eps=1e-6):
    L = k.shape[1]
    N = L * n_h
    K = k[b, :, h].reshape(N, -1).astype(np.float64)
    nrm = np.maximum(np.linalg.norm(K, axis=1), eps)
    Kh = K / nrm[:, None]
    Kt = Kh if kt is None else kt[b, :, h].reshape(N, -1).astype(np.float64)
    V = v[b, :, h].reshape(N, -1).astype(np.float64)
    bet = np.clip(beta[b, :, h].reshape(N).astype(np.float64), 0.0, 2.0)
    lam = np.zeros(N)
    if g is not None:
        with np.errstate(divide="ignore"):
            lam[0::n_h] = np.log(np.maximum(g[b, :, h].astype(np.float64), 1e-300))
    return Kh, Kt, V, bet, lam


def chunk_fwd(q, k, v, beta, chunk, g=None, kt=None, h0=None, return_intermediates=False):
    """Chunkwise forward in fp64; same layouts and results as the oracle."""
    q, k, v, beta = (np.asarray(a, np.float64) for a in (q, k, v, beta))
    B, L, H, n_h, dk = k.shape
    dv = v.shape[-1]
    N = L * n_h
    C = chunk
    nc = -(-N // C)
    Np = nc * C
    out = np.zeros((B, L, H, dv))
    fs = np.zeros((B, H, dk, dv))
    inter = []
    for b in range(B):
        for h in range(H):
            Kh, Kt, V, bet, lam = _expand(k, kt, v, beta, g, b, h, n_h)
            pad = Np - N
            if pad:
                Kh = np.vstack([Kh, np.zeros((pad, dk))])
                Kt = np.vstack([Kt, np.zeros((pad, dk))])
                V = np.vstack([V, np.zeros((pad, dv))])
                bet = np.concatenate([bet, np.zeros(pad)])
                lam = np.concatenate([lam, np.zeros(pad)])
            S = np.zeros((dk, dv)) if h0 is None else np.array(h0[b, h], np.float64)
            for c in range(nc):
                sl = slice(c * C, (c + 1) * C)
                Kc, Ktc, Vc, bc = Kh[sl], Kt[sl], V[sl], bet[sl]
                G = np.cumsum(lam[sl])
                D = G[:, None] - G[None, :]
                E = np.where(np.tril(np.ones((C, C))) > 0, np.exp(np.minimum(D, 0.0)), 0.0)
                M = np.tril(bc[:, None] * (E * (Kc @ Ktc.T)), -1)
                T = np.linalg.inv(np.eye(C) + M)
                Up = T @ (bc[:, None] * (Vc - np.exp(G)[:, None] * (Kc @ S)))
                # readout rows: sub-steps s with s % n_h == n_h - 1 inside this chunk
                for i in range(C):
                    s = c * C + i
                    if s >= N or s % n_h != n_h - 1:
                        continue
                    t = s // n_h
                    qq = q[b, t, h]
                    P = (Ktc[: i + 1] @ qq) * E[i, : i + 1]
                    out[b, t, h] = np.exp(G[i]) * (qq @ S) + P @ Up[: i + 1]
                if return_intermediates:
                    inter.append(dict(b=b, h=h, c=c, T=T, Up=Up, G=G, S0=S.copy()))
                S = np.exp(G[-1]) * S + (np.exp(G[-1] - G)[:, None] * Ktc).T @ Up
            fs[b, h] = S
    if return_intermediates:
        return out, fs, inter
    return out, fs
