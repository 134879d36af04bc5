"""CPU checks of bench.py's contract and accounting (no GPU needed).

The byte and flop counts the roofline line divides by are checked against
closed forms written out here, per workload shape:

* single-pass HBM bytes of a forward: per head and sub-step the read key, the
  value and beta; per head and token the query and the output; per head the
  fp32 state out (and in, with an initial state);
* chunkwise MFMA flops with dense C x C blocks: 2 C^2 (2 dk + dv) + 4 C dk dv
  per chunk, plus 2 dk dv + 2 C (dk + dv) per readout row (one per token);
* OSDN phase 1: k read, k~ written, beta read per token and head, d in and out.
"""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from linear_rnn_sequence_amd.inputs import WORKLOADS  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_forward_bytes_c3_closed_form():
    # B=4 H=16 L=4096 n_h=3 dk=dv=128, bf16 in and out, no gate, no initial state
    heads, L, n_h, d = 4 * 16, 4096, 3, 128
    per_sub = 2 * d + 2 * d + 4          # k, v, beta
    per_tok = 2 * d + 2 * d              # q, out
    state = d * d * 4                    # final state out
    expect = heads * (L * n_h * per_sub + L * per_tok + state)
    assert expect == 544_210_944
    assert bench.alg_bytes(WORKLOADS["c3"]) == expect


def test_forward_bytes_c4_counts_gate_initial_state_and_fp32_out():
    # B=2 H=16 L=8192 n_h=2 dk=dv=128, gate per token, initial state in, fp32 out
    heads, L, n_h, d = 2 * 16, 8192, 2, 128
    expect = heads * (L * n_h * (2 * d + 2 * d + 4) + L * (2 * d + 4 * d + 4) + 2 * d * d * 4)
    assert bench.alg_bytes(WORKLOADS["c4"]) == expect


@pytest.mark.parametrize("name,gflop", [("c3", 107.374), ("c3b", 77.309)])
def test_chunkwise_flops_closed_form(name, gflop):
    w = WORKLOADS[name]
    C, dk, dv = w.chunk, w.dk, w.dv
    chunks = w.B * w.H * (w.L * w.n_h // C)
    rows = w.B * w.H * w.L
    expect = chunks * (2 * C * C * (2 * dk + dv) + 4 * C * dk * dv) + rows * (2 * dk * dv + 2 * C * (dk + dv))
    assert bench.chunk_flops(w) == pytest.approx(expect, rel=1e-12)
    assert expect / 1e9 == pytest.approx(gflop, abs=1e-3)


def test_recurrent_flops_c3():
    # n_h (4 dk dv) per token for the sub-steps plus 2 dk dv for the readout
    w = WORKLOADS["c3"]
    expect = w.B * w.H * w.L * (w.n_h * 4 * 128 * 128 + 2 * 128 * 128)
    assert bench.recurrent_flops(w) == pytest.approx(expect, rel=1e-12)


def test_phase1_and_decode_bytes():
    w = WORKLOADS["c5"]  # B=8 H=16 L=4096 dk=128 bf16
    heads = w.B * w.H
    assert bench.precond_bytes(w) == heads * (w.L * (2 * 128 + 2 * 128 + 4) + 2 * 128 * 4) == 270_663_680
    # one decode token, B=1 H=16 n_h=3: the fp32 state read and written, q, k, v, out, beta
    assert bench.decode_bytes(1, 16, 3, 128, 128) == 16 * (2 * 128 * 128 * 4 + (3 * 256 + 256) * 2 + 3 * 4)


def test_traffic_record_is_dropped_when_the_kernels_change(tmp_path, monkeypatch):
    rec = {"source_sha256": "abc", "bytes_per_launch": 123.0}
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "traffic_k_w.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "source_digest", lambda kernel=None: "abc")
    assert bench.measured_traffic("w", "k") == 123.0
    monkeypatch.setattr(bench, "source_digest", lambda kernel=None: "def")
    assert bench.measured_traffic("w", "k") is None
    assert bench.measured_traffic("w", "missing") is None


def test_fused_header_only_enters_the_fused_kernels_digest():
    assert bench.source_digest("dp_chain_kernel") == bench.source_digest("dp_prep_kernel")
    assert bench.source_digest("dp_fused_kernel") != bench.source_digest("dp_chain_kernel")


def test_issued_flops_of_the_pair_c3():
    """Per chunk: the prep forms the 10 lower 16 x 16 Gram blocks over dk (fp16),
    the blocked fp32 inverse ((NT - dist)(dist + 1) 16^3 products per level)
    and the readout scores (RT x C x dk); the chain, per 16 value columns, Kn H,
    T X, Q H, P Up and the state update."""
    w = WORKLOADS["c3"]
    C, dk, RT = 64, 128, 32
    nc = w.B * w.H * (w.L * w.n_h // C)
    gram = 10 * 16 * 16 * dk * 2
    inverse = sum((4 - dist) * (dist + 1) * 16 ** 3 * 2 for dist in range(1, 4))
    scores = 2 * RT * C * dk
    per16 = 2 * 16 * (C * dk + C * C + RT * dk + RT * C + dk * C)
    prep, chain = bench.issued_flops(w, {"BV": 32, "readout_rows": RT})
    assert prep == nc * (gram + inverse + scores)
    assert chain == nc * per16 * (128 // 16)


def test_issued_flops_of_the_fused_kernel():
    """Every workgroup of a head builds its chunk's operands: the Gram's lower
    tiles, the scores, two split-fp16 off-diagonal T products per 32-row half;
    the consumers run Kn H, Q H, the solve steps, P Up and the state update."""
    w = WORKLOADS["c3"].scaled(B=1, H=2, L=64, n_h=2, dk=64, dv=32)
    C, dk, dv, BV, RT = 64, 64, 32, 32, 32
    nc = 2
    prod = 10 * 2 * 16 * 16 * dk + 2 * RT * C * dk + 2 * 2 * 2 * 2 * 16 * 16 * 32
    solve = (2 + 4) * 2 * 16 * 16 * 32
    cons16 = 2 * 16 * (C * dk + RT * dk + RT * C + dk * C) + solve
    expect = 2 * nc * ((dv // BV) * prod + (dv // 16) * cons16)
    assert bench.fused_issued_flops(w, {"BV": BV, "readout_rows": RT}) == expect


def test_roofline_fields():
    r = bench.roofline_fields("k", 0.2, 544e6, 600e6, 0.35, None)
    assert r["achieved"] == pytest.approx(544e6 / 0.2e6)
    assert r["frac"] == pytest.approx(544e6 / 0.2e6 / 8000)
    assert r["step_achieved"] == pytest.approx(600e6 / 0.35e6)
    assert r["step_frac"] == pytest.approx(600e6 / 0.35e6 / 8000)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0 and r["traffic"] is None


def test_mfma_record_is_read_only_for_the_current_sources(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "mfma_k_w.json").write_text(json.dumps({"source_sha256": "abc", "mfma_busy_frac": 0.164}))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "source_digest", lambda kernel=None: "abc")
    assert bench.measured_mfma_busy("w", "k") == 0.164
    monkeypatch.setattr(bench, "source_digest", lambda kernel=None: "def")
    assert bench.measured_mfma_busy("w", "k") is None


def test_cpu_baseline_reports_cores_model_and_one_thread():
    """The oracle timed on this host on a tiny workload: the fields the line carries."""
    from linear_rnn_sequence_amd.inputs import make
    w = WORKLOADS["c1"].scaled(B=2, H=2, L=32)
    r = bench.cpu_baseline(w, make(w), 0, min_seconds=0.05)
    assert r["kind"] == "oracle" and r["unit"] == "tokens/s" and r["cores"] >= 1
    assert r["value"] > 0 and r["one_thread"]["value"] > 0
    assert "cpu_model" in r
