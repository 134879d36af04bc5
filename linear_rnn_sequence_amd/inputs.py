"""Seeded synthetic inputs for the DeltaProduct forward workloads.

This module only draws inputs.  It holds none of the forward's arithmetic
(no key normalisation, no beta range, no recurrence); both the HIP path and
the fp64 oracle consume the tensors it returns, byte for byte.

Recipe (shapes and distributions of the workloads the DeltaProduct and OSDN
study-note pages describe; no dataset or trained weight is involved):

* one CPU ``torch.Generator`` per workload, seeded ``1000 + id``;
* every draw is fp32 N(0, 1), taken in the fixed order q, k, v, beta, g, h0;
* q: N(0,1) scaled to unit L2 norm per (b, t, h)  -> ``[B, L, H, dk]``;
* k: SiLU(N(0,1)) per sub-step, passed *unnormalised* (the forward normalises
  read keys itself), or plain N(0,1) for the asymmetric-write-key workload
  -> ``[B, L, H, n_h, dk]``;
* v: N(0,1) (times ``v_scale``) -> ``[B, L, H, n_h, dv]``;
* beta: 2*sigmoid(N(0,1)) in (0, 2), or sigmoid(N(0,1)) in (0, 1) ->
  ``[B, L, H, n_h]`` fp32;
* g (gated workload only): exp(-softplus(N(0,1))) in (0, 1] -> ``[B, L, H]``
  fp32;
* h0 (where used): N(0,1) * 0.1 fp32 (variance 0.01) -> ``[B, H, dk, dv]``;
* q, k, v are then stored in the path dtype (fp32, or bf16 rounded to
  nearest-even by torch); beta, g and h0 always stay fp32.
"""
from dataclasses import dataclass, replace
from typing import Optional

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    cid: int            # workload id; seed = 1000 + cid
    B: int
    H: int
    L: int
    n_h: int
    dk: int
    dv: int
    chunk: int
    dtype: str          # "f32" or "bf16": storage type of q, k, v and out
    key: str = "silu"   # "silu": SiLU(N(0,1)) ; "normal": N(0,1)
    v_scale: float = 1.0
    beta: str = "2sig"  # "2sig": 2*sigmoid(N) ; "sig": sigmoid(N)
    gate: bool = False
    h0_std: float = 0.0  # 0: no initial state
    asym: bool = False   # write keys come from the OSDN phase-1 scan
    out_f32: bool = False  # output stored as fp32 (else in the input dtype)

    @property
    def seed(self) -> int:
        return 1000 + self.cid

    @property
    def tokens(self) -> int:
        return self.B * self.L

    def scaled(self, **kw) -> "Workload":
        """Same recipe, other sizes or seed (e.g. a small parity case)."""
        return replace(self, **kw)


WORKLOADS = {
    # tiny fp32 case: B1 H1 L64 n_h2 dk=dv=16 chunk16
    "c1": Workload("c1", 1, B=1, H=1, L=64, n_h=2, dk=16, dv=16, chunk=16, dtype="f32"),
    # bf16 inputs, fp32 state: B4 H8 L2048 n_h2 d64 chunk64
    "c2": Workload("c2", 2, B=4, H=8, L=2048, n_h=2, dk=64, dv=64, chunk=64, dtype="bf16"),
    # LM-layer shape: B4 H16 L4096 n_h3 d128 chunk64, v / sqrt(128)
    "c3": Workload("c3", 3, B=4, H=16, L=4096, n_h=3, dk=128, dv=128, chunk=64, dtype="bf16",
                   v_scale=128 ** -0.5),
    # the same shape with n_h = 2 (the headline metric names n_h = 2 and 3)
    "c3b": Workload("c3b", 32, B=4, H=16, L=4096, n_h=2, dk=128, dv=128, chunk=64,
                    dtype="bf16", v_scale=128 ** -0.5),
    # gated, with an initial state: B2 H16 L8192 n_h2 d128 chunk64.  Its outputs
    # are heavy-tailed (max/RMS ~ 8), so a bf16 output alone would carry a
    # rounding error of ~2e-2 of the RMS: the output is kept in fp32.
    "c4": Workload("c4", 4, B=2, H=16, L=8192, n_h=2, dk=128, dv=128, chunk=64, dtype="bf16",
                   gate=True, h0_std=0.1, out_f32=True),
    # asymmetric write key (OSDN phase 1 + phase 2): B8 H16 L4096 n_h1 d128 chunk64
    "c5": Workload("c5", 5, B=8, H=16, L=4096, n_h=1, dk=128, dv=128, chunk=64, dtype="bf16",
                   key="normal", beta="sig", asym=True),
}


def torch_dtype(name: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def make(w: Workload, seed: Optional[int] = None) -> dict:
    """Draw the inputs of workload ``w`` on the CPU.

    Returns a dict with ``q, k, v, beta, g, h0`` (g/h0 may be None) as CPU
    tensors in their stored dtypes, plus ``n_h``, ``chunk`` and ``out_dtype``
    (the output dtype the workload is run with).
    """
    gen = torch.Generator(device="cpu")
    gen.manual_seed(w.seed if seed is None else seed)
    B, L, H, n_h, dk, dv = w.B, w.L, w.H, w.n_h, w.dk, w.dv

    def normal(*shape):
        return torch.randn(*shape, generator=gen, dtype=torch.float32)

    q = normal(B, L, H, dk)
    q = q / q.norm(dim=-1, keepdim=True).clamp_min(1e-30)
    k = normal(B, L, H, n_h, dk)
    if w.key == "silu":
        k = torch.nn.functional.silu(k)
    v = normal(B, L, H, n_h, dv) * w.v_scale
    braw = normal(B, L, H, n_h)
    beta = 2.0 * torch.sigmoid(braw) if w.beta == "2sig" else torch.sigmoid(braw)
    g = None
    if w.gate:
        g = torch.exp(-torch.nn.functional.softplus(normal(B, L, H)))
    h0 = None
    if w.h0_std > 0:
        h0 = normal(B, H, dk, dv) * w.h0_std
    dt = torch_dtype(w.dtype)
    return {
        "q": q.to(dt).contiguous(),
        "k": k.to(dt).contiguous(),
        "v": v.to(dt).contiguous(),
        "beta": beta.contiguous(),
        "g": None if g is None else g.contiguous(),
        "h0": None if h0 is None else h0.contiguous(),
        "n_h": n_h,
        "chunk": w.chunk,
        "out_dtype": torch.float32 if (w.out_f32 or w.dtype == "f32") else dt,
    }


def make_grads(w: Workload, seed: Optional[int] = None, final: bool = True) -> dict:
    """Seeded output gradients for a backward of workload ``w``: ``dout
    [B,L,H,dv]`` (standard normal, in the workload's dtype) and ``dfinal
    [B,H,dk,dv]`` (f32, or None when ``final`` is False)."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed((w.seed if seed is None else seed) + 1000)
    dout = torch.randn(w.B, w.L, w.H, w.dv, generator=gen, dtype=torch.float32)
    dfinal = torch.randn(w.B, w.H, w.dk, w.dv, generator=gen, dtype=torch.float32) if final else None
    return {"dout": dout.to(torch_dtype(w.dtype)).contiguous(), "dfinal": dfinal}


# ------------------------------------------------------------------ head sampling
# Heads (b, h) are independent, so a large workload can be checked or timed on
# a sample of heads.  These helpers only index; they compute nothing.

def sampled_heads(B: int, H: int, n: int) -> list:
    """n flattened heads b*H + h spread evenly over the grid (first and last included)."""
    total = B * H
    if n >= total:
        return list(range(total))
    return sorted({round(i * (total - 1) / (n - 1)) for i in range(n)}) if n > 1 else [0]


def select_heads(t: torch.Tensor, heads, H: int) -> torch.Tensor:
    """Stack the listed heads of a token-major [B, L, H, ...] tensor into [1, L, n, ...]."""
    parts = []
    for bh in heads:
        b, h = divmod(int(bh), H)
        parts.append(t[b:b + 1, :, h:h + 1])
    return torch.cat(parts, dim=2).contiguous()


def select_state(t: torch.Tensor, heads, H: int) -> torch.Tensor:
    """Stack the listed heads of a [B, H, ...] tensor into [1, n, ...]."""
    parts = []
    for bh in heads:
        b, h = divmod(int(bh), H)
        parts.append(t[b:b + 1, h:h + 1])
    return torch.cat(parts, dim=1).contiguous()


def write_keys(w: Workload, seed: int) -> torch.Tensor:
    """Seeded write keys for the write-key forward, [B, L, H, n_h, dk] in the
    path dtype: a random direction N(0,1)/sqrt(dk) per sub-step times a
    per-channel factor drawn uniformly from [0.5, 2] per (b, h) -- the shape
    and range of the phase-1 write keys d * kn, without running phase 1."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    B, L, H, n_h, dk = w.B, w.L, w.H, w.n_h, w.dk
    kt = torch.randn(B, L, H, n_h, dk, generator=gen, dtype=torch.float32) / dk ** 0.5
    d = 0.5 + 1.5 * torch.rand(B, 1, H, 1, dk, generator=gen, dtype=torch.float32)
    return (kt * d).to(torch_dtype(w.dtype)).contiguous()


def channel_gate(B: int, L: int, H: int, dk: int, seed: int, lo: float = 0.6) -> torch.Tensor:
    """Per-key-channel gate alpha [B, L, H, dk] (fp32) for the KDA host: uniform
    in [lo, 1] per element on a seed of its own (lo = 0.6: a few percent of decay
    per token on average; a small lo gives fast-decaying channels)."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    return (lo + (1.0 - lo) * torch.rand(B, L, H, dk, generator=gen, dtype=torch.float32)).contiguous()


def retention(B: int, L: int, H: int, seed: int, bias: float = 3.0) -> torch.Tensor:
    """Per-token, per-head retention values in (0, 1) for the preconditioner
    (the APF gate is a sigmoid of a learned projection; here sigmoid(N(0,1) +
    bias), so values sit near sigmoid(bias) ~ 0.95) -> ``[B, L, H]`` fp32."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    return torch.sigmoid(torch.randn(B, L, H, generator=gen, dtype=torch.float32) + bias)


def packed_lengths(T: int, seed: int, median: float = 400.0, sigma: float = 1.0,
                   lmax: int = 8192) -> list:
    """Document lengths that pack exactly T tokens: log-normal draws (median
    `median`, log-sd `sigma`) clipped to [1, lmax], the last one cut to fit.
    The pages pack training text into fixed-size token tensors with the state
    reset at document boundaries but give no length distribution; this is a
    stand-in with a realistic spread of short and long documents."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(seed)
    out, total = [], 0
    while total < T:
        x = float(torch.exp(torch.randn(1, generator=gen) * sigma).item()) * median
        n = max(1, min(lmax, int(round(x))))
        n = min(n, T - total)
        out.append(n)
        total += n
    return out
