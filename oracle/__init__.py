"""fp64 CPU oracle for the DeltaProduct forward and the OSDN phase-1 scan.

TEST INFRASTRUCTURE ONLY.  Only the tests, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this package.  The product path
(``linear_rnn_sequence_amd``) never imports it and shares no code with it.

The arithmetic lives in ``dp_oracle.c`` (plain sequential loops in IEEE
double, one sub-step at a time); this module only converts arrays to
contiguous float64 and calls it through ctypes.  Sources, by page title:

* "DeltaProduct: Improving State-Tracking in Linear RNNs via Householder
  Products" -- sec. 2.1 Eq.(2) (delta rule), sec. 2.2 Eq.(3) (n_h ordered
  generalized-Householder sub-steps), sec. 2.6 (per-token gate applied before
  the sub-steps; readout H^T q), sec. 4.1 / Sec.5.1 (only each token's last
  sub-step is read out).
* the gradient of that forward w.r.t. all of its inputs, by reverse-mode
  differentiation of the same sequential definition (``bwd``).
* "OSDN: Improving Delta Rule with Provable Online Preconditioning in Linear
  Attention" -- sec. 2.2 Eqs.(2)/(5) (asymmetric write key), sec. 2.4 Alg.1
  (phase-1 preconditioner, emit-then-update), and its gradient (sec. 2.5,
  closing paragraph: through the write key into d and k, then back through
  the recursion; ``precond_bwd``, ``osdn_bwd``).
"""
import ctypes
import os

import numpy as np

from . import build as _build

_LIB = None
_D = ctypes.POINTER(ctypes.c_double)
_LP = ctypes.POINTER(ctypes.c_long)


def _load():
    global _LIB
    if _LIB is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        lib = ctypes.CDLL(_build.LIB)
        lib.oracle_fwd.restype = ctypes.c_int
        lib.oracle_fwd.argtypes = [_D, _D, _D, _D, _D, _D, _D, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   _D, _D, _D, ctypes.c_int]
        lib.oracle_fwd_heads.restype = ctypes.c_int
        lib.oracle_fwd_heads.argtypes = [_D, _D, _D, _D, _D, _D, _D, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int, _D, _LP, ctypes.c_int, _D, _D,
                                         ctypes.c_int]
        lib.oracle_precond.restype = ctypes.c_int
        lib.oracle_precond.argtypes = [_D, _D, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_int, ctypes.c_double, ctypes.c_double,
                                       ctypes.c_double, ctypes.c_double, _D, _D,
                                       ctypes.c_int]
        lib.oracle_precond_ex.restype = ctypes.c_int
        lib.oracle_precond_ex.argtypes = [_D, _D, _D, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_int, ctypes.c_int, ctypes.c_double,
                                          ctypes.c_double, ctypes.c_double, ctypes.c_double,
                                          _D, _D, ctypes.c_int]
        lib.oracle_precond_bwd.restype = ctypes.c_int
        lib.oracle_precond_bwd.argtypes = [_D, _D, _D, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                           ctypes.c_int, ctypes.c_int, ctypes.c_double,
                                           ctypes.c_double, ctypes.c_double, ctypes.c_double,
                                           _D, _D, _D, _D, _D, _D, _D, ctypes.c_int]
        lib.oracle_bwd.restype = ctypes.c_int
        lib.oracle_bwd.argtypes = [_D, _D, _D, _D, _D, _D, ctypes.c_int, ctypes.c_int,
                                   ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                   _D, _D, _D, _D, _D, _D, _D, _D, _D, _D, ctypes.c_int]
        lib.oracle_bwd_heads.restype = ctypes.c_int
        lib.oracle_bwd_heads.argtypes = [_D, _D, _D, _D, _D, _D, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                         _D, _D, _D, _LP, ctypes.c_int, _D, _D, _D, _D, _D, _D,
                                         _D, ctypes.c_int]
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_num_threads.argtypes = []
        _LIB = lib
    return _LIB


def _f64(x):
    """Contiguous float64 numpy copy (exact upcast of fp32 / bf16 values)."""
    if x is None:
        return None
    if hasattr(x, "detach"):  # torch tensor
        x = x.detach().to("cpu")
        import torch
        x = x.to(torch.float64).numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(_D)


def num_threads() -> int:
    """Threads the oracle's OpenMP loops use by default."""
    return _load().oracle_num_threads()


def _shapes(q, k, v, beta, g, kt, h0, ga=None):
    if q.ndim != 4 or k.ndim != 5 or v.ndim != 5 or beta.ndim != 4:
        raise ValueError("expected q[B,L,H,dk], k[B,L,H,n_h,dk], v[B,L,H,n_h,dv], beta[B,L,H,n_h]")
    B, L, H, dk = q.shape
    n_h = k.shape[3]
    dv = v.shape[4]
    if k.shape != (B, L, H, n_h, dk) or v.shape != (B, L, H, n_h, dv):
        raise ValueError("shape mismatch between q, k, v")
    if beta.shape != (B, L, H, n_h):
        raise ValueError("beta must be [B,L,H,n_h]")
    if g is not None and g.shape != (B, L, H):
        raise ValueError("g must be [B,L,H]")
    if kt is not None and kt.shape != k.shape:
        raise ValueError("kt must have the shape of k")
    if ga is not None and ga.shape != (B, L, H, dk):
        raise ValueError("ga must be [B,L,H,dk]")
    if h0 is not None and h0.shape != (B, H, dk, dv):
        raise ValueError("h0 must be [B,H,dk,dv]")
    return B, L, H, n_h, dk, dv


def fwd(q, k, v, beta, g=None, kt=None, h0=None, nthreads=0, ga=None):
    """Sequential fp64 forward over every head.

    ``ga [B,L,H,dk]``: optional per-key-channel gate (the KDA host).
    Returns ``(out [B,L,H,dv], final_state [B,H,dk,dv])`` as float64 arrays.
    """
    q, k, v, beta, g, kt, h0, ga = (_f64(a) for a in (q, k, v, beta, g, kt, h0, ga))
    B, L, H, n_h, dk, dv = _shapes(q, k, v, beta, g, kt, h0, ga)
    out = np.zeros((B, L, H, dv), np.float64)
    fs = np.zeros((B, H, dk, dv), np.float64)
    rc = _load().oracle_fwd(_ptr(q), _ptr(k), _ptr(kt), _ptr(v), _ptr(beta), _ptr(g), _ptr(ga),
                            n_h, B, H, L, dk, dv, _ptr(h0), _ptr(out), _ptr(fs), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_fwd failed ({rc})")
    return out, fs


def fwd_heads(q, k, v, beta, heads, g=None, kt=None, h0=None, nthreads=0, ga=None):
    """Forward for the listed flattened heads ``b*H + h`` only.

    Returns compact ``(out [n,L,dv], final_state [n,dk,dv])``; each head is
    computed exactly as :func:`fwd` computes it.
    """
    q, k, v, beta, g, kt, h0, ga = (_f64(a) for a in (q, k, v, beta, g, kt, h0, ga))
    B, L, H, n_h, dk, dv = _shapes(q, k, v, beta, g, kt, h0, ga)
    hs = np.ascontiguousarray(np.asarray(heads, dtype=np.int64))
    n = hs.size
    out = np.zeros((n, L, dv), np.float64)
    fs = np.zeros((n, dk, dv), np.float64)
    rc = _load().oracle_fwd_heads(_ptr(q), _ptr(k), _ptr(kt), _ptr(v), _ptr(beta), _ptr(g),
                                  _ptr(ga), n_h, B, H, L, dk, dv, _ptr(h0), hs.ctypes.data_as(_LP), n,
                                  _ptr(out), _ptr(fs), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_fwd_heads failed ({rc})")
    return out, fs


def precond(k, beta, eta=3e-3, dmin=0.5, dmax=2.0, eps=1e-6, d0=None, nthreads=0, r=None,
            beta_aware=True):
    """OSDN phase 1 over ``k [B,L,H,dk]`` (raw keys) and ``beta [B,L,H]``.

    ``r [B,L,H]`` is the optional APF retention gate on d; ``beta_aware=False``
    takes the beta-free phase-1 step.  Returns ``(kt [B,L,H,dk], d_final
    [B,H,dk])``; ``d0`` defaults to ones.
    """
    k = _f64(k)
    beta = _f64(beta)
    if k.ndim != 4 or beta.shape != k.shape[:3]:
        raise ValueError("expected k[B,L,H,dk] and beta[B,L,H]")
    B, L, H, dk = k.shape
    r = None if r is None else _f64(r)
    if r is not None and r.shape != beta.shape:
        raise ValueError("r must be [B,L,H]")
    d = np.ones((B, H, dk), np.float64) if d0 is None else _f64(d0).copy()
    if d.shape != (B, H, dk):
        raise ValueError("d0 must be [B,H,dk]")
    kt = np.zeros((B, L, H, dk), np.float64)
    rc = _load().oracle_precond_ex(_ptr(k), _ptr(beta), _ptr(r), int(bool(beta_aware)), B, H, L,
                                   dk, float(eta), float(dmin), float(dmax), float(eps), _ptr(d),
                                   _ptr(kt), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_precond_ex failed ({rc})")
    return kt, d


def precond_bwd(k, beta, dkt, eta=3e-3, dmin=0.5, dmax=2.0, eps=1e-6, d0=None, dd_final=None,
                nthreads=0, r=None, beta_aware=True):
    """Gradient of :func:`precond` for a loss with gradient ``dkt [B,L,H,dk]``
    on the emitted write keys and ``dd_final [B,H,dk]`` (None: zero) on the
    final d.  Returns a dict of float64 arrays: ``k [B,L,H,dk]`` (raw keys),
    ``beta [B,L,H]``, ``d0 [B,H,dk]`` and ``r [B,L,H]`` when a retention gate
    is given."""
    k, beta, dkt = _f64(k), _f64(beta), _f64(dkt)
    if k.ndim != 4 or beta.shape != k.shape[:3] or dkt.shape != k.shape:
        raise ValueError("expected k[B,L,H,dk], beta[B,L,H] and dkt[B,L,H,dk]")
    B, L, H, dk = k.shape
    r = None if r is None else _f64(r)
    if r is not None and r.shape != beta.shape:
        raise ValueError("r must be [B,L,H]")
    d0 = None if d0 is None else _f64(d0)
    dd_final = None if dd_final is None else _f64(dd_final)
    for name, a in (("d0", d0), ("dd_final", dd_final)):
        if a is not None and a.shape != (B, H, dk):
            raise ValueError(f"{name} must be [B,H,dk]")
    out = dict(k=np.zeros((B, L, H, dk)), beta=np.zeros((B, L, H)), d0=np.zeros((B, H, dk)))
    if r is not None:
        out["r"] = np.zeros((B, L, H))
    rc = _load().oracle_precond_bwd(_ptr(k), _ptr(beta), _ptr(r), int(bool(beta_aware)), B, H, L,
                                    dk, float(eta), float(dmin), float(dmax), float(eps), _ptr(d0),
                                    _ptr(dkt), _ptr(dd_final), _ptr(out["k"]), _ptr(out["beta"]),
                                    _ptr(out.get("r")), _ptr(out["d0"]), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_precond_bwd failed ({rc})")
    return out


def osdn_bwd(q, k, v, beta, dout, g=None, h0=None, dfinal=None, eta=3e-3, dmin=0.5, dmax=2.0,
             eps=1e-6, d0=None, r=None, beta_aware=True, nthreads=0):
    """Gradient of the whole OSDN layer for n_h = 1: phase 1 over ``k [B,L,H,dk]``
    and ``beta [B,L,H]`` gives the write keys, then the write-key forward over
    q, k, v, beta (``v [B,L,H,dv]``) -- the two gradients of :func:`bwd` (write
    keys as inputs) and :func:`precond_bwd` (the write-key gradient carried
    back through phase 1), summed where they meet (the raw keys and beta).
    Returns float64 ``q, k, v, beta, h0, d0`` (+ ``g``, ``r`` when given)."""
    k, beta = _f64(k), _f64(beta)
    kt, _ = precond(k, beta, eta, dmin, dmax, eps, d0=d0, nthreads=nthreads, r=r,
                    beta_aware=beta_aware)
    g2 = bwd(q, k[:, :, :, None, :], _f64(v)[:, :, :, None, :], beta[..., None], dout, g=g,
             kt=kt[:, :, :, None, :], h0=h0, dfinal=dfinal, nthreads=nthreads)
    g1 = precond_bwd(k, beta, g2["kt"][:, :, :, 0, :], eta, dmin, dmax, eps, d0=d0,
                     nthreads=nthreads, r=r, beta_aware=beta_aware)
    res = dict(q=g2["q"], k=g2["k"][:, :, :, 0, :] + g1["k"], v=g2["v"][:, :, :, 0, :],
               beta=g2["beta"][..., 0] + g1["beta"], h0=g2["h0"], d0=g1["d0"])
    if g is not None:
        res["g"] = g2["g"]
    if r is not None:
        res["r"] = g1["r"]
    return res


def _bwd_args(q, k, v, beta, dout, g, kt, h0, dfinal):
    q, k, v, beta, dout, g, kt, h0, dfinal = (_f64(a) for a in (q, k, v, beta, dout, g, kt, h0,
                                                                  dfinal))
    B, L, H, n_h, dk, dv = _shapes(q, k, v, beta, g, kt, h0)
    if dout.shape != (B, L, H, dv):
        raise ValueError("dout must be [B,L,H,dv]")
    if dfinal is not None and dfinal.shape != (B, H, dk, dv):
        raise ValueError("dfinal must be [B,H,dk,dv]")
    return (q, k, v, beta, dout, g, kt, h0, dfinal), (B, L, H, n_h, dk, dv)


def bwd(q, k, v, beta, dout, g=None, kt=None, h0=None, dfinal=None, nthreads=0):
    """Gradient of the sequential fp64 forward, for a loss with gradient
    ``dout [B,L,H,dv]`` on the outputs and ``dfinal [B,H,dk,dv]`` (None: zero)
    on the final state.

    Returns a dict of float64 arrays in the inputs' layouts: ``q, k, v, beta,
    h0`` always, ``g`` when a gate is given, ``kt`` when write keys are given.
    """
    (q, k, v, beta, dout, g, kt, h0, dfinal), (B, L, H, n_h, dk, dv) = _bwd_args(
        q, k, v, beta, dout, g, kt, h0, dfinal)
    r = dict(q=np.zeros((B, L, H, dk)), k=np.zeros((B, L, H, n_h, dk)),
             v=np.zeros((B, L, H, n_h, dv)), beta=np.zeros((B, L, H, n_h)),
             h0=np.zeros((B, H, dk, dv)))
    if g is not None:
        r["g"] = np.zeros((B, L, H))
    if kt is not None:
        r["kt"] = np.zeros((B, L, H, n_h, dk))
    rc = _load().oracle_bwd(_ptr(q), _ptr(k), _ptr(kt), _ptr(v), _ptr(beta), _ptr(g), n_h, B, H,
                            L, dk, dv, _ptr(h0), _ptr(dout), _ptr(dfinal), _ptr(r["q"]),
                            _ptr(r["k"]), _ptr(r.get("kt")), _ptr(r["v"]), _ptr(r["beta"]),
                            _ptr(r.get("g")), _ptr(r["h0"]), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_bwd failed ({rc})")
    return r


def bwd_heads(q, k, v, beta, dout, heads, g=None, kt=None, h0=None, dfinal=None, nthreads=0):
    """:func:`bwd` for the listed flattened heads ``b*H + h`` only; gradients
    compact per head: ``q [n,L,dk]``, ``k``/``kt [n,L,n_h,dk]``, ``v
    [n,L,n_h,dv]``, ``beta [n,L,n_h]``, ``g [n,L]``, ``h0 [n,dk,dv]``."""
    (q, k, v, beta, dout, g, kt, h0, dfinal), (B, L, H, n_h, dk, dv) = _bwd_args(
        q, k, v, beta, dout, g, kt, h0, dfinal)
    hs = np.ascontiguousarray(np.asarray(heads, dtype=np.int64))
    n = hs.size
    r = dict(q=np.zeros((n, L, dk)), k=np.zeros((n, L, n_h, dk)), v=np.zeros((n, L, n_h, dv)),
             beta=np.zeros((n, L, n_h)), h0=np.zeros((n, dk, dv)))
    if g is not None:
        r["g"] = np.zeros((n, L))
    if kt is not None:
        r["kt"] = np.zeros((n, L, n_h, dk))
    rc = _load().oracle_bwd_heads(_ptr(q), _ptr(k), _ptr(kt), _ptr(v), _ptr(beta), _ptr(g), n_h,
                                  B, H, L, dk, dv, _ptr(h0), _ptr(dout), _ptr(dfinal),
                                  hs.ctypes.data_as(_LP), n, _ptr(r["q"]), _ptr(r["k"]),
                                  _ptr(r.get("kt")), _ptr(r["v"]), _ptr(r["beta"]),
                                  _ptr(r.get("g")), _ptr(r["h0"]), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_bwd_heads failed ({rc})")
    return r
