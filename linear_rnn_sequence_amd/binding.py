"""Thin ctypes binding of libdp.so (the C ABI in include/dp.h).

Argument marshalling only: shapes are read off the tensors, outputs and the
workspace are allocated with torch on the inputs' device, and every step of
the forward runs in the library's HIP kernels on torch's current stream.
There is no fallback: if libdp.so is missing or a call fails, this raises.
"""
import ctypes
import os
from typing import Optional, Tuple

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdp.so")

DP_OK, DP_EINVAL, DP_ENOTSUP, DP_EWORKSPACE, DP_EHIP, DP_ESCRATCH = 0, -1, -2, -3, -4, -5
NOALLOC_MAX_SEQS = 65535
STAGE_UT, STAGE_SCAN, STAGE_ALL, OUT_F32, FWD_SPLIT, FWD_FUSED = 1, 2, 3, 4, 8, 16
_PATH_FLAGS = {"auto": 0, "split": FWD_SPLIT, "fused": FWD_FUSED}


def _path_flag(path):
    if path not in _PATH_FLAGS:
        raise ValueError(f"path must be one of {sorted(_PATH_FLAGS)}, not {path!r}")
    return _PATH_FLAGS[path]
PRECOND_BETA_FREE = 1

# every symbol include/dp.h declares
EXPORTS = (
    "dp_status_str", "dp_fwd_workspace_size", "dp_fwd_launch_info",
    "dp_fwd_f32", "dp_fwd_bf16", "dp_fwd_wk_f32", "dp_fwd_wk_bf16",
    "dp_fwd_ex_f32", "dp_fwd_ex_bf16",
    "dp_osdn_precond_f32", "dp_osdn_precond_bf16",
    "dp_decode_f32", "dp_decode_bf16",
    "dp_osdn_precond_ex_f32", "dp_osdn_precond_ex_bf16",
    "dp_fwd_varlen_workspace_size", "dp_fwd_varlen_bf16",
    "dp_bwd_workspace_size", "dp_bwd_f32", "dp_bwd_bf16",
    "dp_osdn_fwd_workspace_size", "dp_osdn_fwd_bf16", "dp_pipeline_create", "dp_pipeline_destroy",
    "dp_fwd_varlen_noalloc_bf16",
    "dp_bwd_wk_f32", "dp_bwd_wk_bf16",
    "dp_osdn_precond_bwd_workspace_size", "dp_osdn_precond_bwd_f32", "dp_osdn_precond_bwd_bf16",
    "dp_osdn_bwd_workspace_size", "dp_osdn_bwd_f32", "dp_osdn_bwd_bf16",
    "dp_fwd_varlen_wk_bf16", "dp_osdn_precond_varlen_f32", "dp_osdn_precond_varlen_bf16",
    "dp_osdn_precond_varlen_workspace_size", "dp_fwd_varlen_f32", "dp_fwd_varlen_wk_f32",
)

_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int
_F = ctypes.c_float


class DPError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {status_str(code)} ({code})")


def load() -> ctypes.CDLL:
    """Load libdp.so from the package directory (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(LIB_PATH)
        lib.dp_status_str.restype = ctypes.c_char_p
        lib.dp_status_str.argtypes = [_I]
        lib.dp_fwd_workspace_size.restype = _I
        lib.dp_fwd_workspace_size.argtypes = [_I] * 8 + [ctypes.POINTER(ctypes.c_size_t)]
        lib.dp_fwd_launch_info.restype = _I
        lib.dp_fwd_launch_info.argtypes = [_I] * 9 + [ctypes.POINTER(ctypes.c_int)]
        fwd_args = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P,
                    ctypes.c_size_t, _P]
        for name in ("dp_fwd_f32", "dp_fwd_bf16"):
            getattr(lib, name).restype = _I
            getattr(lib, name).argtypes = fwd_args
        wk_args = [_P] + fwd_args
        for name in ("dp_fwd_wk_f32", "dp_fwd_wk_bf16"):
            getattr(lib, name).restype = _I
            getattr(lib, name).argtypes = wk_args
        ex = [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P, _P, _P, _P,
              ctypes.c_size_t, _I, _P]
        for name in ("dp_fwd_ex_f32", "dp_fwd_ex_bf16"):
            getattr(lib, name).restype = _I
            getattr(lib, name).argtypes = ex
        pre = [_P, _P, _I, _I, _I, _I, _F, _F, _F, _F, _P, _P, _P]
        for name in ("dp_osdn_precond_f32", "dp_osdn_precond_bf16"):
            getattr(lib, name).restype = _I
            getattr(lib, name).argtypes = pre
        pre_ex = [_P, _P, _P, _I, _I, _I, _I, _I, _F, _F, _F, _F, _P, _P, _P]
        for name in ("dp_osdn_precond_ex_f32", "dp_osdn_precond_ex_bf16"):
            getattr(lib, name).restype = _I
            getattr(lib, name).argtypes = pre_ex
        # k, beta, r, flags, cu_seqlens, nseq, H, T, dk, eta, dmin, dmax, eps, d, kt, ws, bytes, stream
        pre_var = [_P, _P, _P, _I, _P, _I, _I, _I, _I, _F, _F, _F, _F, _P, _P, _P, ctypes.c_size_t, _P]
        lib.dp_osdn_precond_varlen_workspace_size.restype = _I
        lib.dp_osdn_precond_varlen_workspace_size.argtypes = [_I] * 4 + [ctypes.POINTER(ctypes.c_size_t)]
        for name in ("dp_osdn_precond_varlen_f32", "dp_osdn_precond_varlen_bf16"):
            getattr(lib, name).restype = _I
            getattr(lib, name).argtypes = pre_var
        lib.dp_fwd_varlen_workspace_size.restype = _I
        lib.dp_fwd_varlen_workspace_size.argtypes = [_I] * 7 + [ctypes.POINTER(ctypes.c_size_t)]
        lib.dp_fwd_varlen_bf16.restype = _I
        lib.dp_fwd_varlen_bf16.argtypes = [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P, _P,
                                           _P, _P, ctypes.c_size_t, _I, _P]
        lib.dp_fwd_varlen_wk_bf16.restype = _I
        lib.dp_fwd_varlen_wk_bf16.argtypes = [_P] * 7 + [_I] * 7 + [_P] * 4 + [ctypes.c_size_t, _I, _P]
        lib.dp_fwd_varlen_f32.restype = _I
        lib.dp_fwd_varlen_f32.argtypes = lib.dp_fwd_varlen_bf16.argtypes
        lib.dp_fwd_varlen_wk_f32.restype = _I
        lib.dp_fwd_varlen_wk_f32.argtypes = lib.dp_fwd_varlen_wk_bf16.argtypes
        lib.dp_fwd_varlen_noalloc_bf16.restype = _I
        lib.dp_fwd_varlen_noalloc_bf16.argtypes = [_P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P,
                                                   _P, _P, _I, _P]
        dec = [_P, _P, _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _P, _I, _P]
        for name in ("dp_decode_f32", "dp_decode_bf16"):
            getattr(lib, name).restype = _I
            getattr(lib, name).argtypes = dec
        lib.dp_bwd_workspace_size.restype = _I
        lib.dp_bwd_workspace_size.argtypes = [_I] * 6 + [ctypes.POINTER(ctypes.c_size_t)]
        bwd = [_P] * 8 + [_I] * 6 + [_P] * 7 + [ctypes.c_size_t, _P]
        for name in ("dp_bwd_f32", "dp_bwd_bf16"):
            getattr(lib, name).restype = _I
            getattr(lib, name).argtypes = bwd
        bwd_wk = [_P] * 9 + [_I] * 6 + [_P] * 8 + [ctypes.c_size_t, _P]
        for name in ("dp_bwd_wk_f32", "dp_bwd_wk_bf16"):
            getattr(lib, name).restype = _I
            getattr(lib, name).argtypes = bwd_wk
        lib.dp_osdn_precond_bwd_workspace_size.restype = _I
        lib.dp_osdn_precond_bwd_workspace_size.argtypes = [_I] * 4 + [ctypes.POINTER(ctypes.c_size_t)]
        pbwd = [_P] * 6 + [_I] * 5 + [_F] * 4 + [_P] * 5 + [ctypes.c_size_t, _P]
        for name in ("dp_osdn_precond_bwd_f32", "dp_osdn_precond_bwd_bf16"):
            getattr(lib, name).restype = _I
            getattr(lib, name).argtypes = pbwd
        lib.dp_osdn_bwd_workspace_size.restype = _I
        lib.dp_osdn_bwd_workspace_size.argtypes = [_I] * 5 + [ctypes.POINTER(ctypes.c_size_t)]
        obwd = [_P] * 11 + [_I] * 6 + [_F] * 4 + [_P] * 9 + [ctypes.c_size_t, _P]
        for name in ("dp_osdn_bwd_f32", "dp_osdn_bwd_bf16"):
            getattr(lib, name).restype = _I
            getattr(lib, name).argtypes = obwd
        lib.dp_osdn_fwd_workspace_size.restype = _I
        lib.dp_osdn_fwd_workspace_size.argtypes = [_I] * 7 + [ctypes.POINTER(ctypes.c_size_t)]
        lib.dp_osdn_fwd_bf16.restype = _I
        lib.dp_osdn_fwd_bf16.argtypes = [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _F, _F, _F, _P, _P,
                                         _P, _P, _P, ctypes.c_size_t, _I, _P, _P]
        lib.dp_pipeline_create.restype = _I
        lib.dp_pipeline_create.argtypes = [ctypes.POINTER(_P)]
        lib.dp_pipeline_destroy.restype = _I
        lib.dp_pipeline_destroy.argtypes = [_P]
        _lib = lib
    return _lib


def status_str(code: int) -> str:
    return load().dp_status_str(int(code)).decode()


def _check(code: int, where: str):
    if code != DP_OK:
        raise DPError(code, where)


def _suffix(dt: torch.dtype) -> str:
    if dt == torch.float32:
        return "f32"
    if dt == torch.bfloat16:
        return "bf16"
    raise TypeError(f"unsupported dtype {dt}; expected float32 or bfloat16")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _need(t, name, dtype, shape, device):
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def workspace_size(n_h, B, H, L, dk, dv, chunk, dtype) -> int:
    """Bytes of device workspace dp_fwd needs (dtype: torch.float32/bfloat16)."""
    elem = 4 if dtype == torch.float32 else 2
    out = ctypes.c_size_t(0)
    _check(load().dp_fwd_workspace_size(n_h, B, H, L, dk, dv, chunk, elem, ctypes.byref(out)),
           "dp_fwd_workspace_size")
    return int(out.value)


def launch_info(n_h, B, H, L, dk, dv, chunk, dtype, asym=False) -> dict:
    """The launch plan libdp would use for these sizes (nothing is launched)."""
    elem = 4 if dtype == torch.float32 else 2
    info = (ctypes.c_int * 6)()
    _check(load().dp_fwd_launch_info(n_h, B, H, L, dk, dv, chunk, elem, int(bool(asym)), info),
           "dp_fwd_launch_info")
    return dict(BV=info[0], scan_wgs=info[1], ut_wgs=info[2], scan_lds=info[3], ut_lds=info[4],
                readout_rows=info[5])


def alloc_workspace(n_h, B, H, L, dk, dv, chunk, dtype, device) -> torch.Tensor:
    nbytes = workspace_size(n_h, B, H, L, dk, dv, chunk, dtype)
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def fwd(q, k, v, beta, g=None, *, chunk: int = 64, h0=None, kt=None, ga=None, out=None,
        final_state=None, return_state: bool = True, workspace=None,
        stages: int = STAGE_ALL, out_dtype=None, path: str = "auto",
        stream=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """DeltaProduct forward through libdp.

    q [B,L,H,dk], k [B,L,H,n_h,dk], v [B,L,H,n_h,dv] (float32 or bfloat16, one
    dtype), beta [B,L,H,n_h] f32, g [B,L,H] f32 or None, h0 [B,H,dk,dv] f32 or
    None, kt (write keys, shape of k) or None, ga [B,L,H,dk] f32 (the per-key-
    channel gate of the KDA host) or None.  out_dtype: the input dtype
    (default) or torch.float32.  path (bf16 symmetric keys): "auto" lets the
    library choose, "split" runs the chunk-prep / chain kernel pair, "fused"
    the single fused kernel (same results up to rounding).  Returns (out, final_state); final_state is
    None when return_state is False and none was passed.
    """
    if q.dim() != 4 or k.dim() != 5 or v.dim() != 5:
        raise ValueError("expected q[B,L,H,dk], k[B,L,H,n_h,dk], v[B,L,H,n_h,dv]")
    B, L, H, dk = q.shape
    n_h, dv = k.shape[3], v.shape[4]
    dev, dt = q.device, q.dtype
    suf = _suffix(dt)
    _need(k, "k", dt, (B, L, H, n_h, dk), dev)
    _need(kt, "kt", dt, (B, L, H, n_h, dk), dev)
    _need(v, "v", dt, (B, L, H, n_h, dv), dev)
    _need(beta, "beta", torch.float32, (B, L, H, n_h), dev)
    _need(g, "g", torch.float32, (B, L, H), dev)
    _need(ga, "ga", torch.float32, (B, L, H, dk), dev)
    _need(h0, "h0", torch.float32, (B, H, dk, dv), dev)
    if not q.is_contiguous():
        raise ValueError("q must be contiguous")
    if out is not None and out_dtype is None:
        out_dtype = out.dtype
    odt = dt if out_dtype is None else out_dtype
    if odt not in (dt, torch.float32):
        raise TypeError(f"out_dtype must be {dt} or torch.float32")
    flags = stages | (OUT_F32 if odt == torch.float32 else 0) | _path_flag(path)
    if out is None:
        out = torch.empty(B, L, H, dv, dtype=odt, device=dev)
    _need(out, "out", odt, (B, L, H, dv), dev)
    if final_state is None and return_state:
        final_state = torch.empty(B, H, dk, dv, dtype=torch.float32, device=dev)
    _need(final_state, "final_state", torch.float32, (B, H, dk, dv), dev)
    if workspace is None:
        workspace = alloc_workspace(n_h, B, H, L, dk, dv, chunk, dt, dev)
    fn = getattr(load(), f"dp_fwd_ex_{suf}")
    rc = fn(_ptr(q), _ptr(k), _ptr(kt), _ptr(v), _ptr(beta), _ptr(g), _ptr(ga), n_h, B, H, L, dk, dv,
            chunk, _ptr(out), _ptr(final_state), _ptr(h0), _ptr(workspace),
            workspace.numel() * workspace.element_size(), flags, _stream(stream))
    _check(rc, f"dp_fwd_ex_{suf}")
    return out, final_state


def osdn_precond(k, beta, *, eta: float = 3e-3, dmin: float = 0.5, dmax: float = 2.0,
                 eps: float = 1e-6, d_state=None, kt=None, r=None, beta_aware: bool = True,
                 stream=None):
    """OSDN phase 1 through libdp: k [B,L,H,dk], beta [B,L,H] f32.

    d_state [B,H,dk] f32 is d_1 on entry (default ones) and d_{L+1} on return.
    r [B,L,H] f32: optional APF retention of d; beta_aware=False: the beta-free
    phase-1 step.  Either one selects dp_osdn_precond_ex_* (whose box may be
    open: dmin = -inf, dmax = inf).  Returns (kt [B,L,H,dk], d_state).
    """
    if k.dim() != 4:
        raise ValueError("expected k[B,L,H,dk]")
    B, L, H, dk = k.shape
    dev, dt = k.device, k.dtype
    suf = _suffix(dt)
    _need(beta, "beta", torch.float32, (B, L, H), dev)
    _need(r, "r", torch.float32, (B, L, H), dev)
    if not k.is_contiguous():
        raise ValueError("k must be contiguous")
    if d_state is None:
        d_state = torch.ones(B, H, dk, dtype=torch.float32, device=dev)
    _need(d_state, "d_state", torch.float32, (B, H, dk), dev)
    if kt is None:
        kt = torch.empty(B, L, H, dk, dtype=dt, device=dev)
    _need(kt, "kt", dt, (B, L, H, dk), dev)
    lib = load()
    if r is None and beta_aware:
        fn, name = getattr(lib, f"dp_osdn_precond_{suf}"), f"dp_osdn_precond_{suf}"
        rc = fn(_ptr(k), _ptr(beta), B, H, L, dk, eta, dmin, dmax, eps, _ptr(d_state), _ptr(kt),
                _stream(stream))
    else:
        fn, name = getattr(lib, f"dp_osdn_precond_ex_{suf}"), f"dp_osdn_precond_ex_{suf}"
        flags = 0 if beta_aware else PRECOND_BETA_FREE
        rc = fn(_ptr(k), _ptr(beta), _ptr(r), flags, B, H, L, dk, eta, dmin, dmax, eps,
                _ptr(d_state), _ptr(kt), _stream(stream))
    _check(rc, name)
    return kt, d_state


def osdn_precond_varlen_workspace_size(nseq, H, T, dk) -> int:
    n = ctypes.c_size_t(0)
    _check(load().dp_osdn_precond_varlen_workspace_size(nseq, H, T, dk, ctypes.byref(n)),
           "dp_osdn_precond_varlen_workspace_size")
    return n.value


def osdn_precond_varlen(k, beta, cu_seqlens, *, eta: float = 3e-3, dmin: float = 0.5,
                        dmax: float = 2.0, eps: float = 1e-6, d_state=None, kt=None, r=None,
                        beta_aware: bool = True, chunked: bool = False, workspace=None,
                        stream=None):
    """Packed variable-length OSDN phase 1 through libdp: k [T,H,dk], beta [T,H]
    f32, cu_seqlens [nseq+1] int32 on the device.  d_state [nseq,H,dk] f32 is
    each sequence's d_1 on entry (default ones) and its last d on return.  r
    [T,H] f32 and beta_aware as for :func:`osdn_precond`.  chunked (or a given
    workspace): the 64-token chunked form at dk >= 64, else the exact scan.
    Returns (kt [T,H,dk], d_state)."""
    if k.dim() != 3:
        raise ValueError("expected k[T,H,dk]")
    T, H, dk = k.shape
    dev, dt = k.device, k.dtype
    suf = _suffix(dt)
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise ValueError("cu_seqlens must be [nseq + 1]")
    nseq = cu_seqlens.numel() - 1
    _need(cu_seqlens, "cu_seqlens", torch.int32, (nseq + 1,), dev)
    _need(beta, "beta", torch.float32, (T, H), dev)
    _need(r, "r", torch.float32, (T, H), dev)
    if not k.is_contiguous():
        raise ValueError("k must be contiguous")
    if d_state is None:
        d_state = torch.ones(nseq, H, dk, dtype=torch.float32, device=dev)
    _need(d_state, "d_state", torch.float32, (nseq, H, dk), dev)
    if kt is None:
        kt = torch.empty(T, H, dk, dtype=dt, device=dev)
    _need(kt, "kt", dt, (T, H, dk), dev)
    if chunked and workspace is None:
        nbytes = osdn_precond_varlen_workspace_size(nseq, H, T, dk)
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    wsb = 0 if workspace is None else workspace.numel() * workspace.element_size()
    name = f"dp_osdn_precond_varlen_{suf}"
    flags = 0 if beta_aware else PRECOND_BETA_FREE
    rc = getattr(load(), name)(_ptr(k), _ptr(beta), _ptr(r), flags, _ptr(cu_seqlens), nseq, H, T,
                               dk, eta, dmin, dmax, eps, _ptr(d_state), _ptr(kt), _ptr(workspace), wsb,
                               _stream(stream))
    _check(rc, name)
    return kt, d_state


def osdn_fwd_workspace_size(B, H, L, dk, dv, chunk, segments) -> int:
    """Workspace bytes of :func:`osdn_fwd` (dp_osdn_fwd_workspace_size)."""
    n = ctypes.c_size_t(0)
    _check(load().dp_osdn_fwd_workspace_size(B, H, L, dk, dv, chunk, segments, ctypes.byref(n)),
           "dp_osdn_fwd_workspace_size")
    return n.value


class Pipeline:
    """A dp_pipeline: the second stream and events that let :func:`osdn_fwd`
    overlap phase 1 of one token run with the forward of the previous one.
    Made on the current device; released by close() or when collected."""

    def __init__(self):
        h = _P()
        _check(load().dp_pipeline_create(ctypes.byref(h)), "dp_pipeline_create")
        self._h = h

    @property
    def handle(self):
        return self._h

    def close(self):
        if self._h is not None and self._h.value is not None:
            h, self._h = self._h, None
            _check(load().dp_pipeline_destroy(h), "dp_pipeline_destroy")

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def osdn_fwd(q, k, v, beta, *, h0=None, chunk: int = 64, segments: int = 4, eta: float = 3e-3,
             dmin: float = 0.5, dmax: float = 2.0, eps: float = 1e-6, d_state=None, kt=None, out=None,
             final_state=None, workspace=None, pipeline: Optional[Pipeline] = None, stream=None):
    """OSDN phase 1 and the write-key forward in one call (dp_osdn_fwd_bf16),
    cut into `segments` token runs: q, k [B,L,H,dk], v [B,L,H,dv] bf16,
    beta [B,L,H] f32.  d_state [B,H,dk] is d_1 on entry (default ones).  With a
    :class:`Pipeline` the runs overlap (phase 1 of a run beside the forward of
    the previous one); without one they run in order on `stream`.
    Returns (out [B,L,H,dv], final_state [B,H,dk,dv], kt [B,L,H,dk], d_state)."""
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("expected q[B,L,H,dk], k[B,L,H,dk], v[B,L,H,dv]")
    B, L, H, dk = q.shape
    dv = v.shape[3]
    dev = q.device
    for t, n, shp in ((q, "q", (B, L, H, dk)), (k, "k", (B, L, H, dk)), (v, "v", (B, L, H, dv))):
        _need(t, n, torch.bfloat16, shp, dev)
        if not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous")
    _need(beta, "beta", torch.float32, (B, L, H), dev)
    _need(h0, "h0", torch.float32, (B, H, dk, dv), dev)
    if d_state is None:
        d_state = torch.ones(B, H, dk, dtype=torch.float32, device=dev)
    _need(d_state, "d_state", torch.float32, (B, H, dk), dev)
    if kt is None:
        kt = torch.empty(B, L, H, dk, dtype=torch.bfloat16, device=dev)
    _need(kt, "kt", torch.bfloat16, (B, L, H, dk), dev)
    if out is None:
        out = torch.empty(B, L, H, dv, dtype=torch.bfloat16, device=dev)
    _need(out, "out", torch.bfloat16, (B, L, H, dv), dev)
    if final_state is None:
        final_state = torch.empty(B, H, dk, dv, dtype=torch.float32, device=dev)
    _need(final_state, "final_state", torch.float32, (B, H, dk, dv), dev)
    if workspace is None:
        nbytes = osdn_fwd_workspace_size(B, H, L, dk, dv, chunk, segments)
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    rc = load().dp_osdn_fwd_bf16(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(h0), B, H, L, dk, dv, chunk,
                                 eta, dmin, dmax, eps, _ptr(d_state), _ptr(kt), _ptr(out), _ptr(final_state),
                                 _ptr(workspace), workspace.numel() * workspace.element_size(), segments,
                                 None if pipeline is None else pipeline.handle, _stream(stream))
    _check(rc, "dp_osdn_fwd_bf16")
    return out, final_state, kt, d_state


def decode(q, k, v, beta, state, g=None, *, kt=None, ga=None, out=None, out_dtype=None,
           stream=None):
    """One recurrent decode step through libdp, updating `state` in place.

    q [B,H,dk], k [B,H,n_h,dk], v [B,H,n_h,dv] (float32 or bfloat16, one
    dtype), beta [B,H,n_h] f32, g [B,H] f32 or None, ga [B,H,dk] f32 (the
    per-key-channel gate) or None, kt (write keys, shape of k) or None, state
    [B,H,dk,dv] f32 (H_{t-1} in, H_t out).  Returns out [B,H,dv] in the input
    dtype or out_dtype (torch.float32).
    """
    if q.dim() != 3 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("expected q[B,H,dk], k[B,H,n_h,dk], v[B,H,n_h,dv]")
    B, H, dk = q.shape
    n_h, dv = k.shape[2], v.shape[3]
    dev, dt = q.device, q.dtype
    suf = _suffix(dt)
    _need(k, "k", dt, (B, H, n_h, dk), dev)
    _need(kt, "kt", dt, (B, H, n_h, dk), dev)
    _need(v, "v", dt, (B, H, n_h, dv), dev)
    _need(beta, "beta", torch.float32, (B, H, n_h), dev)
    _need(g, "g", torch.float32, (B, H), dev)
    _need(ga, "ga", torch.float32, (B, H, dk), dev)
    _need(state, "state", torch.float32, (B, H, dk, dv), dev)
    if not q.is_contiguous():
        raise ValueError("q must be contiguous")
    if out is not None and out_dtype is None:
        out_dtype = out.dtype
    odt = dt if out_dtype is None else out_dtype
    if odt not in (dt, torch.float32):
        raise TypeError(f"out_dtype must be {dt} or torch.float32")
    if out is None:
        out = torch.empty(B, H, dv, dtype=odt, device=dev)
    _need(out, "out", odt, (B, H, dv), dev)
    flags = OUT_F32 if (odt == torch.float32 and dt != torch.float32) else 0
    fn = getattr(load(), f"dp_decode_{suf}")
    rc = fn(_ptr(q), _ptr(k), _ptr(kt), _ptr(v), _ptr(beta), _ptr(g), _ptr(ga), n_h, B, H, dk,
            dv, _ptr(out), _ptr(state), flags, _stream(stream))
    _check(rc, f"dp_decode_{suf}")
    return out


def varlen_workspace_size(n_h, nseq, H, T, dk, dv, chunk) -> int:
    """Bytes of device workspace dp_fwd_varlen_bf16 needs."""
    n = ctypes.c_size_t(0)
    _check(load().dp_fwd_varlen_workspace_size(n_h, nseq, H, T, dk, dv, chunk, ctypes.byref(n)),
           "dp_fwd_varlen_workspace_size")
    return n.value


def fwd_varlen(q, k, v, beta, cu_seqlens, g=None, *, chunk: int = 64, h0=None, kt=None, out=None,
               final_state=None, return_state: bool = True, workspace=None,
               stages: int = STAGE_ALL, out_dtype=None, path: str = "auto", stream=None):
    """Packed variable-length forward through libdp.

    q [T,H,dk], k [T,H,n_h,dk], v [T,H,n_h,dv] bfloat16 or float32, beta [T,H,n_h] f32,
    g [T,H] f32 or None, cu_seqlens [nseq+1] int32 on the device, h0
    [nseq,H,dk,dv] f32 or None.  kt [T,H,n_h,dk] bfloat16: the write keys
    (dp_fwd_varlen_wk_bf16), else symmetric keys.  path as for fwd.  Returns
    (out [T,H,dv], final_state).
    """
    if q.dim() != 3 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("expected q[T,H,dk], k[T,H,n_h,dk], v[T,H,n_h,dv]")
    T, H, dk = q.shape
    n_h, dv = k.shape[2], v.shape[3]
    dev, dt = q.device, q.dtype
    if dt not in (torch.bfloat16, torch.float32):
        raise TypeError("fwd_varlen takes bfloat16 or float32 q, k, v")
    suf = _suffix(dt)
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise ValueError("cu_seqlens must be [nseq + 1]")
    nseq = cu_seqlens.numel() - 1
    _need(cu_seqlens, "cu_seqlens", torch.int32, (nseq + 1,), dev)
    _need(k, "k", dt, (T, H, n_h, dk), dev)
    _need(kt, "kt", dt, (T, H, n_h, dk), dev)
    _need(v, "v", dt, (T, H, n_h, dv), dev)
    _need(beta, "beta", torch.float32, (T, H, n_h), dev)
    _need(g, "g", torch.float32, (T, H), dev)
    _need(h0, "h0", torch.float32, (nseq, H, dk, dv), dev)
    if not q.is_contiguous():
        raise ValueError("q must be contiguous")
    if out is not None and out_dtype is None:
        out_dtype = out.dtype
    odt = dt if out_dtype is None else out_dtype
    if odt not in (dt, torch.float32):
        raise TypeError(f"out_dtype must be {dt} or torch.float32")
    flags = stages | (OUT_F32 if odt == torch.float32 else 0) | _path_flag(path)
    if out is None:
        out = torch.empty(T, H, dv, dtype=odt, device=dev)
    _need(out, "out", odt, (T, H, dv), dev)
    if final_state is None and return_state:
        final_state = torch.empty(nseq, H, dk, dv, dtype=torch.float32, device=dev)
    _need(final_state, "final_state", torch.float32, (nseq, H, dk, dv), dev)
    if workspace is None:
        nbytes = varlen_workspace_size(n_h, nseq, H, T, dk, dv, chunk)
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    tail = (_ptr(v), _ptr(beta), _ptr(g), _ptr(cu_seqlens), nseq, n_h, H, T, dk, dv, chunk,
            _ptr(out), _ptr(final_state), _ptr(h0), _ptr(workspace),
            workspace.numel() * workspace.element_size(), flags, _stream(stream))
    if kt is None:
        name = f"dp_fwd_varlen_{suf}"
        rc = getattr(load(), name)(_ptr(q), _ptr(k), *tail)
    else:
        name = f"dp_fwd_varlen_wk_{suf}"
        rc = getattr(load(), name)(_ptr(q), _ptr(k), _ptr(kt), *tail)
    _check(rc, name)
    return out, final_state


def fwd_varlen_noalloc(q, k, v, beta, cu_seqlens, out, g=None, *, chunk: int = 64, h0=None,
                       final_state=None, stream=None):
    """The packed forward with no device allocation (dp_fwd_varlen_noalloc_bf16):
    the fused kernel, its chunk-offset table in the library's fixed scratch.
    Arguments as for :func:`fwd_varlen`, but `out` (bf16 or float32) must be
    given and nothing is allocated here either; final_state may be None.  At
    most NOALLOC_MAX_SEQS sequences; calls that overlap in time on one device
    race (they share the scratch)."""
    if q.dim() != 3 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("expected q[T,H,dk], k[T,H,n_h,dk], v[T,H,n_h,dv]")
    T, H, dk = q.shape
    n_h, dv = k.shape[2], v.shape[3]
    dev, dt = q.device, q.dtype
    if dt != torch.bfloat16:
        raise TypeError("fwd_varlen_noalloc takes bfloat16 q, k, v")
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise ValueError("cu_seqlens must be [nseq + 1]")
    nseq = cu_seqlens.numel() - 1
    _need(cu_seqlens, "cu_seqlens", torch.int32, (nseq + 1,), dev)
    _need(k, "k", dt, (T, H, n_h, dk), dev)
    _need(v, "v", dt, (T, H, n_h, dv), dev)
    _need(beta, "beta", torch.float32, (T, H, n_h), dev)
    _need(g, "g", torch.float32, (T, H), dev)
    _need(h0, "h0", torch.float32, (nseq, H, dk, dv), dev)
    _need(final_state, "final_state", torch.float32, (nseq, H, dk, dv), dev)
    if not q.is_contiguous():
        raise ValueError("q must be contiguous")
    if out is None or out.dtype not in (dt, torch.float32):
        raise TypeError("out must be a bfloat16 or float32 tensor [T, H, dv]")
    _need(out, "out", out.dtype, (T, H, dv), dev)
    flags = OUT_F32 if out.dtype == torch.float32 else 0
    rc = load().dp_fwd_varlen_noalloc_bf16(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g), _ptr(cu_seqlens),
                                           nseq, n_h, H, T, dk, dv, chunk, _ptr(out), _ptr(final_state),
                                           _ptr(h0), flags, _stream(stream))
    _check(rc, "dp_fwd_varlen_noalloc_bf16")
    return out, final_state


def bwd_workspace_size(n_h, B, H, L, dk, dv) -> int:
    """Workspace bytes of :func:`bwd` (dp_bwd_workspace_size)."""
    n = ctypes.c_size_t(0)
    _check(load().dp_bwd_workspace_size(n_h, B, H, L, dk, dv, ctypes.byref(n)),
           "dp_bwd_workspace_size")
    return n.value


def bwd(q, k, v, beta, dout, g=None, *, h0=None, dfinal=None, kt=None, workspace=None, grads=None,
        stream=None) -> dict:
    """Gradient of the forward through libdp (dp_bwd_* / dp_bwd_wk_*).

    Inputs as :func:`fwd` (q, k, v and dout in one dtype, float32 or
    bfloat16), dout [B,L,H,dv] the gradient on out and dfinal [B,H,dk,dv] f32
    (or None) the gradient on the final state; kt (the shape and dtype of k)
    selects the write-key forward's gradient.  Returns a dict of float32
    gradients ``q, k, v, beta, h0``, ``g`` when a gate is given and ``kt``
    with write keys; ``grads`` may hold preallocated tensors under those names.
    """
    if q.dim() != 4 or k.dim() != 5 or v.dim() != 5:
        raise ValueError("expected q[B,L,H,dk], k[B,L,H,n_h,dk], v[B,L,H,n_h,dv]")
    B, L, H, dk = q.shape
    n_h, dv = k.shape[3], v.shape[4]
    dev, dt = q.device, q.dtype
    suf = _suffix(dt)
    _need(k, "k", dt, (B, L, H, n_h, dk), dev)
    _need(v, "v", dt, (B, L, H, n_h, dv), dev)
    _need(dout, "dout", dt, (B, L, H, dv), dev)
    _need(beta, "beta", torch.float32, (B, L, H, n_h), dev)
    _need(g, "g", torch.float32, (B, L, H), dev)
    _need(h0, "h0", torch.float32, (B, H, dk, dv), dev)
    _need(dfinal, "dfinal", torch.float32, (B, H, dk, dv), dev)
    _need(kt, "kt", dt, (B, L, H, n_h, dk), dev)
    if not q.is_contiguous():
        raise ValueError("q must be contiguous")
    shapes = dict(q=(B, L, H, dk), k=(B, L, H, n_h, dk), v=(B, L, H, n_h, dv), beta=(B, L, H, n_h),
                  h0=(B, H, dk, dv))
    if g is not None:
        shapes["g"] = (B, L, H)
    if kt is not None:
        shapes["kt"] = (B, L, H, n_h, dk)
    out = dict(grads or {})
    for n, shp in shapes.items():
        if n not in out:
            out[n] = torch.empty(shp, dtype=torch.float32, device=dev)
        _need(out[n], "grad " + n, torch.float32, shp, dev)
    if workspace is None:
        nbytes = bwd_workspace_size(n_h, B, H, L, dk, dv)
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)
    wsb = workspace.numel() * workspace.element_size()
    if kt is None:
        fn = getattr(load(), f"dp_bwd_{suf}")
        rc = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g), _ptr(h0), _ptr(dout), _ptr(dfinal),
                n_h, B, H, L, dk, dv, _ptr(out["q"]), _ptr(out["k"]), _ptr(out["v"]), _ptr(out["beta"]),
                _ptr(out.get("g")), _ptr(out["h0"]), _ptr(workspace), wsb, _stream(stream))
        _check(rc, f"dp_bwd_{suf}")
    else:
        fn = getattr(load(), f"dp_bwd_wk_{suf}")
        rc = fn(_ptr(q), _ptr(k), _ptr(kt), _ptr(v), _ptr(beta), _ptr(g), _ptr(h0), _ptr(dout),
                _ptr(dfinal), n_h, B, H, L, dk, dv, _ptr(out["q"]), _ptr(out["k"]), _ptr(out["kt"]),
                _ptr(out["v"]), _ptr(out["beta"]), _ptr(out.get("g")), _ptr(out["h0"]), _ptr(workspace),
                wsb, _stream(stream))
        _check(rc, f"dp_bwd_wk_{suf}")
    return out


def osdn_precond_bwd_workspace_size(B, H, L, dk) -> int:
    """Workspace bytes of :func:`osdn_precond_bwd`."""
    n = ctypes.c_size_t(0)
    _check(load().dp_osdn_precond_bwd_workspace_size(B, H, L, dk, ctypes.byref(n)),
           "dp_osdn_precond_bwd_workspace_size")
    return n.value


def osdn_precond_bwd(k, beta, dkt, *, eta: float = 3e-3, dmin: float = 0.5, dmax: float = 2.0,
                     eps: float = 1e-6, d0=None, dd_final=None, r=None, beta_aware: bool = True,
                     dk=None, dbeta=None, workspace=None, stream=None) -> dict:
    """Gradient of OSDN phase 1 through libdp (dp_osdn_precond_bwd_*).

    k [B,L,H,dk] (float32 or bfloat16), beta [B,L,H] f32, dkt [B,L,H,dk] f32
    the gradient on the emitted write keys, dd_final [B,H,dk] f32 or None on
    the final d; d0, r, beta_aware and the constants as :func:`osdn_precond`.
    The key and beta gradients are ADDED into ``dk`` / ``dbeta`` when given
    (zero-filled tensors otherwise).  Returns float32 ``k, beta, d0`` and ``r``
    when a retention gate is given.
    """
    if k.dim() != 4:
        raise ValueError("expected k[B,L,H,dk]")
    B, L, H, dkk = k.shape
    dev, dt = k.device, k.dtype
    suf = _suffix(dt)
    _need(beta, "beta", torch.float32, (B, L, H), dev)
    _need(dkt, "dkt", torch.float32, (B, L, H, dkk), dev)
    _need(r, "r", torch.float32, (B, L, H), dev)
    _need(d0, "d0", torch.float32, (B, H, dkk), dev)
    _need(dd_final, "dd_final", torch.float32, (B, H, dkk), dev)
    if not k.is_contiguous():
        raise ValueError("k must be contiguous")
    if dk is None:
        dk = torch.zeros(B, L, H, dkk, dtype=torch.float32, device=dev)
    if dbeta is None:
        dbeta = torch.zeros(B, L, H, dtype=torch.float32, device=dev)
    _need(dk, "dk", torch.float32, (B, L, H, dkk), dev)
    _need(dbeta, "dbeta", torch.float32, (B, L, H), dev)
    out = dict(k=dk, beta=dbeta, d0=torch.empty(B, H, dkk, dtype=torch.float32, device=dev))
    if r is not None:
        out["r"] = torch.empty(B, L, H, dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = torch.empty(max(osdn_precond_bwd_workspace_size(B, H, L, dkk), 1), dtype=torch.uint8,
                                device=dev)
    flags = 0 if beta_aware else PRECOND_BETA_FREE
    fn = getattr(load(), f"dp_osdn_precond_bwd_{suf}")
    rc = fn(_ptr(k), _ptr(beta), _ptr(r), _ptr(d0), _ptr(dkt), _ptr(dd_final), flags, B, H, L, dkk, eta,
            dmin, dmax, eps, _ptr(out["k"]), _ptr(out["beta"]), _ptr(out.get("r")), _ptr(out["d0"]),
            _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream))
    _check(rc, f"dp_osdn_precond_bwd_{suf}")
    return out


def osdn_bwd_workspace_size(B, H, L, dk, dv) -> int:
    """Workspace bytes of :func:`osdn_bwd`."""
    n = ctypes.c_size_t(0)
    _check(load().dp_osdn_bwd_workspace_size(B, H, L, dk, dv, ctypes.byref(n)), "dp_osdn_bwd_workspace_size")
    return n.value


def osdn_bwd(q, k, v, beta, dout, g=None, *, h0=None, dfinal=None, r=None, d0=None, dd_final=None,
             eta: float = 3e-3, dmin: float = 0.5, dmax: float = 2.0, eps: float = 1e-6,
             beta_aware: bool = True, workspace=None, grads=None, stream=None) -> dict:
    """Gradient of the whole OSDN layer (n_h = 1) through libdp (dp_osdn_bwd_*).

    q, k [B,L,H,dk], v, dout [B,L,H,dv] in one dtype (float32 or bfloat16);
    beta [B,L,H] f32; g [B,L,H], h0/dfinal [B,H,dk,dv], r [B,L,H], d0/dd_final
    [B,H,dk] f32 or None; phase-1 constants as :func:`osdn_precond`.  Returns
    float32 ``q, k, v, beta, h0, d0`` (+ ``g``, ``r`` when given).
    """
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("expected q[B,L,H,dk], k[B,L,H,dk], v[B,L,H,dv]")
    B, L, H, dk = q.shape
    dv = v.shape[3]
    dev, dt = q.device, q.dtype
    suf = _suffix(dt)
    _need(k, "k", dt, (B, L, H, dk), dev)
    _need(v, "v", dt, (B, L, H, dv), dev)
    _need(dout, "dout", dt, (B, L, H, dv), dev)
    _need(beta, "beta", torch.float32, (B, L, H), dev)
    for name, x, shp in (("g", g, (B, L, H)), ("r", r, (B, L, H)), ("h0", h0, (B, H, dk, dv)),
                         ("dfinal", dfinal, (B, H, dk, dv)), ("d0", d0, (B, H, dk)), ("dd_final", dd_final, (B, H, dk))):
        _need(x, name, torch.float32, shp, dev)
    if not q.is_contiguous():
        raise ValueError("q must be contiguous")
    shapes = dict(q=(B, L, H, dk), k=(B, L, H, dk), v=(B, L, H, dv), beta=(B, L, H), h0=(B, H, dk, dv),
                  d0=(B, H, dk))
    if g is not None:
        shapes["g"] = (B, L, H)
    if r is not None:
        shapes["r"] = (B, L, H)
    out = dict(grads or {})
    for n, shp in shapes.items():
        if n not in out:
            out[n] = torch.empty(shp, dtype=torch.float32, device=dev)
        _need(out[n], "grad " + n, torch.float32, shp, dev)
    if workspace is None:
        workspace = torch.empty(max(osdn_bwd_workspace_size(B, H, L, dk, dv), 1), dtype=torch.uint8, device=dev)
    flags = 0 if beta_aware else PRECOND_BETA_FREE
    fn = getattr(load(), f"dp_osdn_bwd_{suf}")
    rc = fn(_ptr(q), _ptr(k), _ptr(v), _ptr(beta), _ptr(g), _ptr(h0), _ptr(r), _ptr(d0), _ptr(dout),
            _ptr(dfinal), _ptr(dd_final), flags, B, H, L, dk, dv, eta, dmin, dmax, eps, _ptr(out["q"]),
            _ptr(out["k"]), _ptr(out["v"]), _ptr(out["beta"]), _ptr(out.get("g")), _ptr(out["h0"]),
            _ptr(out.get("r")), _ptr(out["d0"]), _ptr(workspace), workspace.numel() * workspace.element_size(),
            _stream(stream))
    _check(rc, f"dp_osdn_bwd_{suf}")
    return out
