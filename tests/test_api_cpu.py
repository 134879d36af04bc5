"""C-ABI checks that need no GPU: every symbol include/dp.h declares is
exported by libdp.so, and every validation error is returned on the host
before any HIP call (so these run on a machine without a GPU)."""
import ctypes
import os
import re

import pytest

import linear_rnn_sequence_amd as dp
from linear_rnn_sequence_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        from linear_rnn_sequence_amd import build as b
        b.build()
    return dp.load()


def header_functions():
    src = open(os.path.join(ROOT, "include", "dp.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dp_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = header_functions()
    for required in ("dp_fwd_bf16", "dp_fwd_f32", "dp_fwd_wk_bf16", "dp_fwd_wk_f32",
                     "dp_osdn_precond_bf16", "dp_fwd_workspace_size", "dp_status_str"):
        assert required in names
    assert sorted(names) == sorted(dp.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    for name in header_functions():
        assert hasattr(lib, name), name


def test_library_is_gfx950_and_loads_on_cpu(lib):
    # the code object inside libdp.so targets gfx950 only
    blob = open(binding.LIB_PATH, "rb").read()
    assert b"gfx950" in blob
    for other in (b"gfx942", b"gfx90a", b"gfx1100"):
        assert other not in blob


def test_status_strings(lib):
    for code in (0, -1, -2, -3, -4, -5):
        assert dp.status_str(code).startswith("DP_")
    assert "unknown" in dp.status_str(7)


SZ = ctypes.c_size_t


def ws(n_h, B, H, L, dk, dv, chunk, elem):
    out = SZ(0)
    rc = dp.load().dp_fwd_workspace_size(n_h, B, H, L, dk, dv, chunk, elem, ctypes.byref(out))
    return rc, out.value


def bf16_chunk_block(dk, C, n_h, write_keys=False):
    """Bytes of one chunk's operand block on the bf16 path: T diag(beta), unit
    keys (C x dk), the write keys (C x dk, write-key form only), readout queries
    (RT x dk), scores (RT x C), all fp16, then e^G, e^{G_last - G} (C floats
    each), e^{G_loc} (RT floats) and the output offsets (RT int64, 8-byte
    aligned); RT = ceil(C / n_h) in 16s.  T diag(beta) is C x C, except that
    with dk and C multiples of 32 and C > 32 its 32-column tile t keeps only
    rows 32 t .. C-1 (the rows above are zero)."""
    r = -(-C // n_h)
    RT = C if r >= C else -(-r // 16) * 16
    scal = (8 * C + 4 * RT + 7) // 8 * 8 + 8 * RT
    if dk % 32 == 0 and C % 32 == 0 and C > 32:
        t_elems = sum(32 * (C - 32 * t) for t in range(C // 32))
    else:
        t_elems = C * C
    kw = C * dk if write_keys else 0
    return 2 * (t_elems + C * dk + kw + RT * dk + RT * C) + (scal + 15) // 16 * 16


def test_workspace_size_formula(lib):
    """One size serves the symmetric and the write-key forward: where the
    write-key form runs on the prep / chain pair (dk and chunk multiples of 32)
    the blocks are sized with the write keys."""
    rc, n = ws(3, 4, 16, 4096, 128, 128, 64, 2)
    assert rc == 0
    nc = 4096 * 3 // 64
    assert bf16_chunk_block(128, 64, 3) == 35712
    assert bf16_chunk_block(128, 64, 3, write_keys=True) == 35712 + 64 * 128 * 2
    sink = 4 * 16 * (128 // 16) * 64 * 4  # one fp32 slot per lane of every scan wavefront
    assert n == -(-4 * 16 * nc * (35712 + 16384) // 256) * 256 + sink
    # the per-channel-gate form keeps T (C x C), the per-sub-step scalars, the
    # readout scores (RT x C, RT = 16 here), gated read and write keys (the
    # layout of k), gated readout queries (the layout of q) and a dk-float decay
    # per chunk, each region 256-byte aligned; the size is the larger need
    up = lambda x: -(-x // 256) * 256

    def cg(elem, nch=5, C=16, RT=16, toks=33, n_h=2, dk=16):
        return (up(nch * C * C * elem) + up(nch * C * 8) + up(nch * RT * C * elem) + 2 * up(toks * n_h * dk * elem)
                + up(toks * dk * elem) + up(nch * dk * 4))

    rc, n = ws(2, 1, 1, 33, 16, 16, 16, 2)  # ragged: 66 sub-steps -> 5 chunks
    assert rc == 0 and n == max(-(-5 * bf16_chunk_block(16, 16, 2) // 256) * 256 + 256, cg(2))
    rc, n = ws(2, 1, 1, 33, 16, 16, 16, 4)  # ragged: 66 sub-steps -> 5 chunks
    assert rc == 0 and n == cg(4)
    assert ws(2, 1, 1, 0, 16, 16, 16, 4) == (0, 0)


@pytest.mark.parametrize("args,code", [
    ((0, 1, 1, 8, 16, 16, 16, 2), dp.binding.DP_EINVAL),     # n_h = 0
    ((2, 0, 1, 8, 16, 16, 16, 2), dp.binding.DP_EINVAL),     # B = 0
    ((2, 1, 1, -1, 16, 16, 16, 2), dp.binding.DP_EINVAL),    # L < 0
    ((2, 1, 1, 8, 48, 16, 16, 2), dp.binding.DP_ENOTSUP),    # dk not in the set
    ((2, 1, 1, 8, 16, 256, 16, 2), dp.binding.DP_ENOTSUP),   # dv not in the set
    ((2, 1, 1, 8, 16, 16, 128, 2), dp.binding.DP_ENOTSUP),   # chunk not in the set
    ((65, 1, 1, 8, 16, 16, 16, 2), dp.binding.DP_ENOTSUP),   # n_h too large
    ((2, 1, 1, 8, 16, 16, 16, 3), dp.binding.DP_EINVAL),     # elem bytes
])
def test_workspace_size_validation(lib, args, code):
    assert ws(*args)[0] == code


FAKE = 1 << 20  # a 256-aligned non-null address; validation fails before any use


def fwd_call(lib, suffix="bf16", q=FAKE, k=FAKE, v=FAKE, beta=FAKE, g=None, ga=None, n_h=2, B=1, H=1,
             L=8, dk=16, dv=16, chunk=16, out=FAKE, fs=None, h0=None, wsp=FAKE, wsb=1 << 30,
             kt=None, stages=3):
    fn = getattr(lib, f"dp_fwd_ex_{suffix}")
    return fn(q, k, kt, v, beta, g, ga, n_h, B, H, L, dk, dv, chunk, out, fs, h0, wsp, wsb, stages,
              None)


@pytest.mark.parametrize("suffix", ["bf16", "f32"])
def test_fwd_validation_errors_before_hip(lib, suffix):
    E = dp.binding
    assert fwd_call(lib, suffix, q=None) == E.DP_EINVAL
    assert fwd_call(lib, suffix, k=None) == E.DP_EINVAL
    assert fwd_call(lib, suffix, v=None) == E.DP_EINVAL
    assert fwd_call(lib, suffix, beta=None) == E.DP_EINVAL
    assert fwd_call(lib, suffix, out=None) == E.DP_EINVAL
    assert fwd_call(lib, suffix, q=FAKE + 8) == E.DP_EINVAL          # misaligned
    assert fwd_call(lib, suffix, kt=FAKE + 4) == E.DP_EINVAL
    assert fwd_call(lib, suffix, n_h=0) == E.DP_EINVAL
    assert fwd_call(lib, suffix, H=0) == E.DP_EINVAL
    assert fwd_call(lib, suffix, dk=24) == E.DP_ENOTSUP
    assert fwd_call(lib, suffix, dv=8) == E.DP_ENOTSUP
    assert fwd_call(lib, suffix, chunk=8) == E.DP_ENOTSUP
    assert fwd_call(lib, suffix, n_h=100) == E.DP_ENOTSUP
    assert fwd_call(lib, suffix, stages=0) == E.DP_EINVAL
    assert fwd_call(lib, suffix, stages=4) == E.DP_EINVAL            # no stage bit
    assert fwd_call(lib, suffix, stages=32 | 3) == E.DP_EINVAL       # unknown flag
    assert fwd_call(lib, suffix, stages=8 | 16 | 3) == E.DP_EINVAL   # both path overrides
    # the fused kernel exists for bf16, symmetric keys, dk and chunk multiples of 32, both stages
    assert fwd_call(lib, suffix, stages=16 | 3) == E.DP_ENOTSUP
    assert fwd_call(lib, suffix, stages=16 | 1, dk=32, chunk=32) == E.DP_ENOTSUP
    assert fwd_call(lib, suffix, stages=16 | 3, dk=32, chunk=32, kt=FAKE) == E.DP_ENOTSUP
    assert fwd_call(lib, suffix, stages=16 | 3, dk=32, chunk=32, ga=FAKE) == E.DP_ENOTSUP  # no channel gate
    if suffix == "f32":
        assert fwd_call(lib, suffix, stages=16 | 3, dk=32, chunk=32) == E.DP_ENOTSUP
    assert fwd_call(lib, suffix, wsb=16) == E.DP_EWORKSPACE           # too small
    assert fwd_call(lib, suffix, wsp=None) == E.DP_EWORKSPACE         # missing
    assert fwd_call(lib, suffix, wsp=FAKE + 16) == E.DP_EWORKSPACE    # misaligned


def test_wk_requires_write_key(lib):
    args = (FAKE, FAKE, None, FAKE, FAKE, None, 1, 1, 1, 8, 16, 16, 16, FAKE, None, None, FAKE,
            1 << 30, None)
    assert lib.dp_fwd_wk_bf16(*args) == dp.binding.DP_EINVAL
    assert lib.dp_fwd_wk_f32(*args) == dp.binding.DP_EINVAL


def test_precond_validation_errors_before_hip(lib):
    E = dp.binding
    f = lib.dp_osdn_precond_bf16

    def call(k=FAKE, beta=FAKE, B=1, H=1, L=4, dk=16, eta=3e-3, dmin=0.5, dmax=2.0, eps=1e-6,
             d=FAKE, kt=FAKE):
        return f(k, beta, B, H, L, dk, eta, dmin, dmax, eps, d, kt, None)

    assert call(k=None) == E.DP_EINVAL
    assert call(d=None) == E.DP_EINVAL
    assert call(kt=None) == E.DP_EINVAL
    assert call(B=0) == E.DP_EINVAL
    assert call(dk=48) == E.DP_ENOTSUP
    assert call(eps=0.0) == E.DP_EINVAL
    assert call(dmin=2.0, dmax=1.0) == E.DP_EINVAL
    assert call(dmin=0.0) == E.DP_EINVAL
    assert call(eta=float("nan")) == E.DP_EINVAL
    assert call(L=0) == E.DP_OK  # nothing to do, nothing enqueued


def test_binding_rejects_bad_tensors_on_cpu():
    import torch
    q = torch.zeros(1, 4, 1, 16)
    k = torch.zeros(1, 4, 1, 2, 16)
    v = torch.zeros(1, 4, 1, 2, 16)
    beta = torch.zeros(1, 4, 1, 2)
    with pytest.raises(TypeError):
        dp.fwd(q.double(), k, v, beta)
    with pytest.raises(ValueError):
        dp.fwd(q, k[:, :3], v, beta)


@pytest.mark.parametrize("suffix", ["bf16", "f32"])
def test_decode_validation_errors_before_hip(lib, suffix):
    E = dp.binding
    f = getattr(lib, f"dp_decode_{suffix}")

    def call(q=FAKE, k=FAKE, kt=None, v=FAKE, beta=FAKE, g=None, ga=None, n_h=2, B=1, H=1, dk=16,
             dv=16, out=FAKE, state=FAKE, flags=0):
        return f(q, k, kt, v, beta, g, ga, n_h, B, H, dk, dv, out, state, flags, None)

    assert call(q=None) == E.DP_EINVAL
    assert call(k=None) == E.DP_EINVAL
    assert call(v=None) == E.DP_EINVAL
    assert call(beta=None) == E.DP_EINVAL
    assert call(out=None) == E.DP_EINVAL
    assert call(state=None) == E.DP_EINVAL
    assert call(n_h=0) == E.DP_EINVAL
    assert call(B=0) == E.DP_EINVAL
    assert call(flags=8) == E.DP_EINVAL
    assert call(dk=24) == E.DP_ENOTSUP
    assert call(dv=256) == E.DP_ENOTSUP
    assert call(n_h=65) == E.DP_ENOTSUP


def test_decode_binding_rejects_bad_tensors_on_cpu():
    import torch
    q = torch.zeros(2, 3, 16)
    k = torch.zeros(2, 3, 2, 16)
    v = torch.zeros(2, 3, 2, 16)
    beta = torch.zeros(2, 3, 2)
    st = torch.zeros(2, 3, 16, 16)
    with pytest.raises(TypeError):
        dp.decode(q, k, v, beta, st.double())
    with pytest.raises(ValueError):
        dp.decode(q, k, v[:, :2], beta, st)
    with pytest.raises(ValueError):
        dp.decode(q, k, v, beta, st.transpose(2, 3))


def test_precond_ex_validation_errors_before_hip(lib):
    E = dp.binding
    f = lib.dp_osdn_precond_ex_f32

    def call(k=FAKE, beta=FAKE, r=None, flags=0, B=1, H=1, L=4, dk=16, eta=3e-3, dmin=0.5,
             dmax=2.0, eps=1e-6, d=FAKE, kt=FAKE):
        return f(k, beta, r, flags, B, H, L, dk, eta, dmin, dmax, eps, d, kt, None)

    assert call(k=None) == E.DP_EINVAL
    assert call(flags=2) == E.DP_EINVAL
    assert call(dmin=2.0, dmax=1.0) == E.DP_EINVAL
    assert call(dmin=float("nan")) == E.DP_EINVAL
    assert call(eps=0.0) == E.DP_EINVAL
    assert call(dk=40) == E.DP_ENOTSUP
    # the open box is allowed here (and only here)
    assert call(L=0, dmin=float("-inf"), dmax=float("inf"), flags=1) == E.DP_OK
    assert lib.dp_osdn_precond_f32(FAKE, FAKE, 1, 1, 0, 16, 3e-3, float("-inf"), 2.0, 1e-6,
                                   FAKE, FAKE, None) == E.DP_EINVAL


def test_varlen_validation_errors_before_hip(lib):
    E = dp.binding
    f = lib.dp_fwd_varlen_bf16

    def call(q=FAKE, k=FAKE, v=FAKE, beta=FAKE, g=None, cu=FAKE, nseq=2, n_h=2, H=1, T=8, dk=16,
             dv=16, chunk=16, out=FAKE, fs=None, h0=None, wsp=FAKE, wsb=1 << 30, flags=3):
        return f(q, k, v, beta, g, cu, nseq, n_h, H, T, dk, dv, chunk, out, fs, h0, wsp, wsb, flags,
                 None)

    assert call(cu=None) == E.DP_EINVAL
    assert call(nseq=0) == E.DP_EINVAL
    assert call(T=-1) == E.DP_EINVAL
    assert call(q=None) == E.DP_EINVAL
    assert call(q=FAKE + 8) == E.DP_EINVAL
    assert call(flags=0) == E.DP_EINVAL
    assert call(flags=32 | 3) == E.DP_EINVAL
    assert call(flags=8 | 16 | 3) == E.DP_EINVAL
    assert call(flags=16 | 3) == E.DP_ENOTSUP    # dk 16: no fused kernel
    assert call(dk=24) == E.DP_ENOTSUP
    assert call(chunk=8) == E.DP_ENOTSUP
    assert call(wsb=16) == E.DP_EWORKSPACE
    assert call(wsp=FAKE + 16) == E.DP_EWORKSPACE


def test_varlen_wk_validation_errors_before_hip(lib):
    E = dp.binding
    f = lib.dp_fwd_varlen_wk_bf16

    def call(q=FAKE, k=FAKE, kt=FAKE, v=FAKE, beta=FAKE, g=None, cu=FAKE, nseq=2, n_h=1, H=1, T=8,
             dk=32, dv=32, chunk=32, out=FAKE, fs=None, h0=None, wsp=FAKE, wsb=1 << 30, flags=3):
        return f(q, k, kt, v, beta, g, cu, nseq, n_h, H, T, dk, dv, chunk, out, fs, h0, wsp, wsb,
                 flags, None)

    assert call(kt=None) == E.DP_EINVAL
    assert call(kt=FAKE + 8) == E.DP_EINVAL       # misaligned
    assert call(cu=None) == E.DP_EINVAL
    assert call(nseq=0) == E.DP_EINVAL
    assert call(flags=16 | 3) == E.DP_ENOTSUP     # no fused write-key kernel
    assert call(dk=16) == E.DP_ENOTSUP            # the pair needs dk and chunk in 32s
    assert call(chunk=16) == E.DP_ENOTSUP
    assert call(wsb=16) == E.DP_EWORKSPACE


def test_precond_varlen_validation_errors_before_hip(lib):
    E = dp.binding
    for f in (lib.dp_osdn_precond_varlen_f32, lib.dp_osdn_precond_varlen_bf16):
        def call(k=FAKE, beta=FAKE, r=None, flags=0, cu=FAKE, nseq=2, H=1, T=8, dk=16, eta=3e-3,
                 dmin=0.5, dmax=2.0, eps=1e-6, d=FAKE, kt=FAKE, wsp=None, wsb=0):
            return f(k, beta, r, flags, cu, nseq, H, T, dk, eta, dmin, dmax, eps, d, kt, wsp, wsb,
                     None)

        assert call(cu=None) == E.DP_EINVAL
        assert call(nseq=0) == E.DP_EINVAL
        assert call(d=None) == E.DP_EINVAL
        assert call(kt=FAKE + 4) == E.DP_EINVAL
        assert call(flags=2) == E.DP_EINVAL
        assert call(eps=0.0) == E.DP_EINVAL
        assert call(dmin=3.0) == E.DP_EINVAL         # dmin > dmax
        assert call(dk=24) == E.DP_ENOTSUP
        assert call(T=0) == E.DP_OK                  # nothing to scan: no launch
        assert call(dk=64, wsp=FAKE, wsb=16) == E.DP_EWORKSPACE          # too small
        assert call(dk=64, wsp=FAKE + 16, wsb=1 << 30) == E.DP_EWORKSPACE  # misaligned


def test_precond_varlen_workspace_size(lib):
    """The chunked form's arrays sized for ceil(T / 64) + nseq chunks per head,
    then one restart slot per head and the nseq + 1 chunk offsets, each region
    256-byte aligned; dk < 64 has no chunked form (0 bytes)."""
    n = SZ(0)
    up = lambda x: -(-x // 256) * 256
    nseq, H, T, dk = 5, 3, 1000, 128
    nch = H * (-(-T // 64) + nseq)
    want = (up(nch * 64 * 64 * 4) + 2 * up(nch * 64 * 4) + up(nch * 64 * 16) + up(nch * 4)
            + up(nch * dk * 4) + up(nseq * H * 4) + up((nseq + 1) * 4))
    assert lib.dp_osdn_precond_varlen_workspace_size(nseq, H, T, dk, ctypes.byref(n)) == 0
    assert n.value == want
    assert lib.dp_osdn_precond_varlen_workspace_size(nseq, H, T, 32, ctypes.byref(n)) == 0
    assert n.value == 0
    assert lib.dp_osdn_precond_varlen_workspace_size(0, H, T, dk, ctypes.byref(n)) == \
        dp.binding.DP_EINVAL
    assert lib.dp_osdn_precond_varlen_workspace_size(nseq, H, T, 24, ctypes.byref(n)) == \
        dp.binding.DP_ENOTSUP


def test_varlen_workspace_size(lib):
    n = SZ(0)
    # 3 heads, 1000 tokens, n_h 3, chunk 64: blocks for 3 (ceil(3000 / 64) + 5) chunks,
    # then 6 ints of chunk offsets and the sink (5 x 3 x 8 wavefront slots).  The
    # blocks are sized with the write keys (dk and chunk multiples of 32), so one
    # size serves the symmetric and the write-key packed forward.
    assert lib.dp_fwd_varlen_workspace_size(3, 5, 3, 1000, 128, 128, 64, ctypes.byref(n)) == 0
    blocks = -(-3 * (47 + 5) * bf16_chunk_block(128, 64, 3, write_keys=True) // 256) * 256
    assert n.value == blocks + 256 + -(-5 * 3 * 8 * 64 * 4 // 256) * 256
    # the fp32 layout (T, C x C fp32, and C float2 per work item, then the chunk
    # offsets) is the larger one at dk 16; one size serves both input types
    up = lambda x: -(-x // 256) * 256
    nwork = 3 * (47 + 5)
    fp32 = up(nwork * 64 * 64 * 4) + up(nwork * 64 * 8) + 256
    assert fp32 < n.value  # dk 128: the bf16 blocks are larger
    # dk 16: no write-key form on the pair, blocks without write keys
    assert lib.dp_fwd_varlen_workspace_size(3, 5, 3, 1000, 16, 16, 64, ctypes.byref(n)) == 0
    blocks = -(-3 * (47 + 5) * bf16_chunk_block(16, 64, 3) // 256) * 256
    bf16 = blocks + 256 + -(-5 * 3 * 1 * 64 * 4 // 256) * 256
    assert n.value == max(bf16, fp32) == fp32
    assert lib.dp_fwd_varlen_workspace_size(3, 0, 3, 1000, 128, 128, 64, ctypes.byref(n)) == \
        dp.binding.DP_EINVAL


def test_packed_lengths_cover_the_batch_exactly():
    from linear_rnn_sequence_amd.inputs import packed_lengths
    ls = packed_lengths(65536, seed=5)
    assert sum(ls) == 65536 and min(ls) >= 1 and max(ls) <= 8192 and len(ls) > 20


def test_launch_info_reports_the_default_path(lib):
    """Symmetric bf16 keys take the fused kernel (no UT workgroups, one workgroup
    per head) where dv <= 32, and the prep / chain pair where a head's dv columns
    would span several workgroups; fp32 and write keys always take two kernels."""
    info = (ctypes.c_int * 6)()
    assert lib.dp_fwd_launch_info(2, 8, 32, 2048, 128, 32, 64, 2, 0, info) == 0
    assert info[2] == 0 and info[0] == 32 and info[1] == 8 * 32
    assert lib.dp_fwd_launch_info(2, 1, 4, 256, 64, 16, 32, 2, 0, info) == 0
    assert info[2] == 0 and info[0] == 16 and info[1] == 4
    assert lib.dp_fwd_launch_info(3, 8, 16, 4096, 128, 128, 64, 2, 0, info) == 0
    assert info[2] > 0 and info[1] == 8 * 16 * (128 // info[0])
    assert lib.dp_fwd_launch_info(2, 8, 32, 2048, 128, 32, 64, 4, 0, info) == 0
    assert info[2] > 0
    assert lib.dp_fwd_launch_info(2, 8, 32, 2048, 128, 32, 64, 2, 1, info) == 0
    assert info[2] > 0


def test_osdn_fwd_checks_every_run_before_the_first(lib):
    """dp_osdn_fwd_bf16 validates what each run's phase 1 and forward would
    check before it enqueues anything: with no GPU here, a failure found only
    after the first run's phase 1 had been enqueued would surface as DP_EHIP
    (a HIP launch on a machine without a device), not as the status below.
    So on a failed call d_state, kt, out and final_state are never written."""
    E = dp.binding
    f = lib.dp_osdn_fwd_bf16

    def call(q=FAKE, k=FAKE, v=FAKE, beta=FAKE, h0=None, B=1, H=2, L=300, dk=128, dv=128, chunk=64,
             eta=3e-3, dmin=0.5, dmax=2.0, eps=1e-6, d=FAKE, kt=FAKE, out=FAKE, fs=FAKE, wsp=FAKE,
             wsb=1 << 30, segments=4, pipe=None):
        return f(q, k, v, beta, h0, B, H, L, dk, dv, chunk, eta, dmin, dmax, eps, d, kt, out, fs, wsp,
                 wsb, segments, pipe, None)

    assert call(v=FAKE + 2) == E.DP_EINVAL      # read by the forward only
    assert call(q=FAKE + 8) == E.DP_EINVAL
    assert call(kt=FAKE + 4) == E.DP_EINVAL
    assert call(dmin=0.0) == E.DP_EINVAL        # phase-1 box must be positive here
    assert call(eps=0.0) == E.DP_EINVAL
    assert call(dmin=3.0) == E.DP_EINVAL        # dmin > dmax
    assert call(fs=None) == E.DP_EINVAL         # the state passes through it between runs
    assert call(d=None) == E.DP_EINVAL
    assert call(wsb=16) == E.DP_EWORKSPACE
    assert call(segments=0) == E.DP_EINVAL
    assert call(segments=17) == E.DP_EINVAL
    assert call(dk=24) == E.DP_ENOTSUP


def test_osdn_fwd_workspace_size(lib):
    """One run's forward (the run of ceil(ceil(L / segments) / chunk) chunks),
    then for dk >= 64 one run's chunked phase 1: per 64-token chunk the 64 x 64
    inverse, v, the token factors, the chunk's log-retention, its start d and
    gamma; one restart index per head; each region 256-byte aligned."""
    up = lambda x: -(-x // 256) * 256
    for B, H, L, dk, dv, C, S in ((8, 16, 4096, 128, 128, 64, 4), (2, 3, 300, 64, 32, 32, 3), (1, 2, 100, 32, 32, 32, 2)):
        n = ctypes.c_size_t(0)
        assert lib.dp_osdn_fwd_workspace_size(B, H, L, dk, dv, C, S, ctypes.byref(n)) == 0
        run = -(-(-(-L // S)) // C) * C
        f = ctypes.c_size_t(0)
        assert lib.dp_fwd_workspace_size(1, B, H, run, dk, dv, C, 2, ctypes.byref(f)) == 0
        nch = B * H * -(-run // 64)
        chunked = (up(nch * 64 * 64 * 4) + 2 * up(nch * 64 * 4) + up(nch * 64 * 16) + up(nch * 4)
                   + up(nch * dk * 4) + up(B * H * 4)) if dk >= 64 else 0
        assert n.value == up(f.value) + chunked, (B, H, L, dk)


def test_pipeline_handle_arguments(lib):
    E = dp.binding
    assert lib.dp_pipeline_create(None) == E.DP_EINVAL
    assert lib.dp_pipeline_destroy(None) == E.DP_OK


def test_noalloc_varlen_validation_before_hip(lib):
    """dp_fwd_varlen_noalloc_bf16 rejects what it cannot run before any HIP
    call (including the lookup of its scratch array's device address)."""
    E = dp.binding
    f = lib.dp_fwd_varlen_noalloc_bf16

    def call(q=FAKE, k=FAKE, v=FAKE, beta=FAKE, g=None, cu=FAKE, nseq=2, n_h=2, H=1, T=8, dk=32,
             dv=16, chunk=32, out=FAKE, fs=None, h0=None, flags=0):
        return f(q, k, v, beta, g, cu, nseq, n_h, H, T, dk, dv, chunk, out, fs, h0, flags, None)

    assert call(nseq=E.NOALLOC_MAX_SEQS + 1) == E.DP_ESCRATCH
    assert call(flags=1) == E.DP_EINVAL          # stage bits are not taken: both always run
    assert call(flags=8) == E.DP_EINVAL
    assert call(dk=16) == E.DP_ENOTSUP           # no fused kernel for dk 16
    assert call(chunk=16) == E.DP_ENOTSUP
    assert call(cu=None) == E.DP_EINVAL
    assert call(nseq=0) == E.DP_EINVAL
    assert call(q=FAKE + 8) == E.DP_EINVAL
    assert "scratch" in dp.status_str(E.DP_ESCRATCH)


def test_backward_entry_points_validate_before_hip(lib):
    """The write-key backward, phase 1's backward and the OSDN layer's backward
    return every validation status before any HIP call."""
    E = dp.binding

    def bwd_wk(q=FAKE, k=FAKE, kt=FAKE, v=FAKE, beta=FAKE, dout=FAKE, n_h=1, B=1, H=1, L=8, dk=16, dv=16,
               dkt=FAKE, wsp=FAKE, wsb=1 << 30):
        return lib.dp_bwd_wk_bf16(q, k, kt, v, beta, None, None, dout, None, n_h, B, H, L, dk, dv, FAKE, FAKE,
                                  dkt, FAKE, FAKE, None, None, wsp, wsb, None)

    assert bwd_wk(kt=None) == E.DP_EINVAL
    assert bwd_wk(dkt=None) == E.DP_EINVAL
    assert bwd_wk(kt=FAKE + 4) == E.DP_EINVAL      # misaligned
    assert bwd_wk(dout=FAKE + 8) == E.DP_EINVAL
    assert bwd_wk(dk=48) == E.DP_ENOTSUP
    assert bwd_wk(wsp=None) == E.DP_EWORKSPACE
    assert bwd_wk(wsb=16) == E.DP_EWORKSPACE
    # the symmetric backward now checks alignment too
    assert lib.dp_bwd_bf16(FAKE + 2, FAKE, FAKE, FAKE, None, None, FAKE, None, 1, 1, 1, 8, 16, 16, FAKE, FAKE,
                           FAKE, FAKE, None, None, FAKE, 1 << 30, None) == E.DP_EINVAL

    def pbwd(k=FAKE, beta=FAKE, dkt=FAKE, flags=0, B=1, H=1, L=4, dk=16, eta=3e-3, dmin=0.5, dmax=2.0,
             eps=1e-6, dko=FAKE, db=FAKE, wsp=FAKE, wsb=1 << 30):
        return lib.dp_osdn_precond_bwd_bf16(k, beta, None, None, dkt, None, flags, B, H, L, dk, eta, dmin, dmax,
                                            eps, dko, db, None, None, wsp, wsb, None)

    assert pbwd(k=None) == E.DP_EINVAL
    assert pbwd(k=FAKE + 2) == E.DP_EINVAL
    assert pbwd(dkt=None) == E.DP_EINVAL
    assert pbwd(dko=None) == E.DP_EINVAL
    assert pbwd(db=None) == E.DP_EINVAL
    assert pbwd(flags=4) == E.DP_EINVAL
    assert pbwd(dk=48) == E.DP_ENOTSUP
    assert pbwd(eps=0.0) == E.DP_EINVAL
    assert pbwd(wsp=None) == E.DP_EWORKSPACE
    assert pbwd(wsp=FAKE + 16) == E.DP_EWORKSPACE
    n = ctypes.c_size_t(0)
    assert lib.dp_osdn_precond_bwd_workspace_size(2, 3, 5, 32, ctypes.byref(n)) == E.DP_OK
    up = lambda x: (x + 255) // 256 * 256
    # d, the trajectory of d, the write keys, the mask bytes, the per-token factors, the received gradient
    assert n.value == up(2 * 3 * 32 * 4) + 3 * up(2 * 5 * 3 * 32 * 4) + up(2 * 5 * 3 * 32) + up(2 * 5 * 3 * 16)
    assert pbwd(wsb=n.value - 1, B=2, H=3, L=5, dk=32) == E.DP_EWORKSPACE
    # dk >= 64: the forward's chunked form (per 64-token chunk: the 64 x 64
    # inverse, v, the token factors, the chunk's log-retention, its start d and
    # gamma; one restart index per head) shares the reverse scan's region
    assert lib.dp_osdn_precond_bwd_workspace_size(2, 3, 5, 128, ctypes.byref(n)) == E.DP_OK
    nch = 2 * 3 * 1
    chunked = (up(nch * 64 * 64 * 4) + 2 * up(nch * 64 * 4) + up(nch * 64 * 16) + up(nch * 4)
               + up(nch * 128 * 4) + up(2 * 3 * 4))
    rev = up(2 * 5 * 3 * 128) + up(2 * 5 * 3 * 16) + up(2 * 5 * 3 * 128 * 4)
    assert chunked > rev
    assert n.value == up(2 * 3 * 128 * 4) + 2 * up(2 * 5 * 3 * 128 * 4) + max(rev, chunked)

    def obwd(q=FAKE, k=FAKE, v=FAKE, beta=FAKE, dout=FAKE, B=1, H=1, L=8, dk=16, dv=16, dq=FAKE, dko=FAKE,
             dvo=FAKE, db=FAKE, eps=1e-6, wsp=FAKE, wsb=1 << 30):
        return lib.dp_osdn_bwd_bf16(q, k, v, beta, None, None, None, None, dout, None, None, 0, B, H, L, dk, dv,
                                    3e-3, 0.5, 2.0, eps, dq, dko, dvo, db, None, None, None, None, wsp, wsb, None)

    for kw in (dict(q=None), dict(v=None), dict(dout=None), dict(dq=None), dict(dvo=None), dict(dko=None),
               dict(db=None), dict(k=FAKE + 2), dict(v=FAKE + 4), dict(eps=-1.0)):
        assert obwd(**kw) == E.DP_EINVAL, kw
    assert obwd(dk=48) == E.DP_ENOTSUP
    assert obwd(wsp=None) == E.DP_EWORKSPACE
    assert lib.dp_osdn_bwd_workspace_size(2, 3, 70, 32, 64, ctypes.byref(n)) == E.DP_OK
    pb, bw = ctypes.c_size_t(0), ctypes.c_size_t(0)
    lib.dp_osdn_precond_bwd_workspace_size(2, 3, 70, 32, ctypes.byref(pb))
    lib.dp_bwd_workspace_size(1, 2, 3, 70, 32, 64, ctypes.byref(bw))
    assert n.value == pb.value + 2 * up(2 * 70 * 3 * 32 * 4) + bw.value
    assert obwd(wsb=n.value - 1, B=2, H=3, L=70, dk=32, dv=64) == E.DP_EWORKSPACE


def test_backward_bindings_reject_bad_tensors_on_cpu():
    import torch
    k = torch.zeros(1, 4, 2, 16)
    beta = torch.zeros(1, 4, 2)
    with pytest.raises(TypeError):
        dp.osdn_precond_bwd(k, beta, torch.zeros(1, 4, 2, 16, dtype=torch.float64))
    with pytest.raises(ValueError):
        dp.osdn_bwd(k, k, torch.zeros(1, 4, 2, 16), beta[:, :3], torch.zeros(1, 4, 2, 16))
