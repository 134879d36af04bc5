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
