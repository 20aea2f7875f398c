"""Host logic of bench.py (no GPU): algorithmic bytes and flops per launch against hand counts, the
choice of the binding roof, the traffic summaries' source check, and the one-GPU guard."""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

import bench
from bidirectional_linear_attention_lion_amd import inputs as lin

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_algorithmic_full_vit_tiny():
    wl = lin.WORKLOADS["vit_tiny_lit"]            # B64 H3 L197 d64 bf16, LIT: no decay input
    nbytes, flops = bench.algorithmic("full", wl, 64)
    assert nbytes == 4 * 64 * 3 * 197 * 64 * 2    # q, k, v read, y written, bf16
    bh, L, d = 64 * 3, 197, 64
    assert flops == bh * (4 * L * L * d + 2 * L * L)


def test_algorithmic_decay_inputs():
    base = 4 * 32 * 16 * 512 * 64 * 2
    assert bench.algorithmic("full", lin.WORKLOADS["bert_large_s"], 64)[0] == base + 4 * 32 * 16 * 512   # LION-S
    wl = lin.WORKLOADS["vit_base_d"]
    assert bench.algorithmic("full", wl, 64)[0] == 4 * 64 * 12 * 197 * 64 * 2 + 4 * 12                # LION-D


def test_algorithmic_chunk_and_rnn():
    wl = lin.WORKLOADS["vit_base_d"]
    bh, L, d, C = 64 * 12, 197, 64, 64
    assert bench.algorithmic("chunk", wl, C)[1] == bh * (4 * L * C * d + 8 * L * d * d + 2 * L * C)
    # two recurrences per token: state update and q^T S, q.z (LION-D: 5 d^2 + 4 d each)
    assert bench.algorithmic("birnn", wl, C)[1] == bh * L * 2 * (5 * d * d + 4 * d)
    lit = lin.WORKLOADS["vit_tiny_lit"]
    assert bench.algorithmic("birnn", lit, C)[1] == 64 * 3 * 197 * 2 * (4 * d * d + 3 * d)


def test_algorithmic_chunk_bwd():
    wl = lin.WORKLOADS["hires_d"]                 # B8 H12 L4097 d64, LION-D
    bh, L, d = 8 * 12, 4097, 64
    nbytes, flops = bench.algorithmic("chunk_bwd", wl, 32)
    assert nbytes == 8 * bh * L * d * 2 + 4 * bh * L + 4 * 12
    assert flops == bh * (10 * L * 32 * d + 8 * L * 32 + L * 20 * d * d)
    assert bench.bound_of("chunk_bwd", wl, 32) == "alu"         # fp32 matrix cores
    assert bench.bound_of("chunk_bwd", wl, 64) != "alu"         # bf16 matrix cores


def test_algorithmic_causal_counts_the_lower_triangle():
    wl = lin.WORKLOADS["hires_d"]
    bh, L, d = 8 * 12, 4097, 64
    pairs = L * (L + 1) / 2
    assert bench.algorithmic("full", wl, 64, causal=True)[1] == bh * (4 * pairs * d + 2 * pairs)


def test_binding_roof():
    # below the bf16 ridge (312.5 flop/B) the full and chunk forms are HBM-bound, above it MFMA-bound;
    # the RNN is vector-ALU work
    assert bench.bound_of("full", lin.WORKLOADS["vit_tiny_lit"], 64) == "hbm"       # ~99 flop/B
    assert bench.bound_of("full", lin.WORKLOADS["bert_large_s"], 64) == "hbm"       # ~256 flop/B
    assert bench.bound_of("full", lin.WORKLOADS["hires_d"], 64) == "mfma"           # ~2065 flop/B
    assert bench.bound_of("chunk", lin.WORKLOADS["hires_d"], 256) == "hbm"
    assert bench.bound_of("birnn", lin.WORKLOADS["vit_base_d"], 64) == "alu"
    assert bench.peak_of("hbm") == (8000.0, "GB/s")
    assert bench.peak_of("mfma") == (2500.0, "TFLOP/s")
    assert bench.peak_of("alu") == (157.3, "TFLOP/s")


def test_traffic_summary_needs_the_current_source(tmp_path, monkeypatch):
    # bench.py reports counter-measured traffic only from a summary taken on the current kernel source
    current = bench.kernel_hash("full")
    prof = tmp_path / "profiles"
    prof.mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    path = prof / "traffic_full_vit_tiny_lit.txt"
    path.write_text(f"kernel_source_sha256_16: {current}\nhbm_bytes_per_launch: 19472411\n")
    assert bench.read_traffic("full", "vit_tiny_lit") == 19472411.0
    path.write_text("kernel_source_sha256_16: 0000000000000000\nhbm_bytes_per_launch: 19472411\n")
    assert bench.read_traffic("full", "vit_tiny_lit") is None
    assert bench.read_traffic("chunk", "vit_tiny_lit") is None        # no summary at all


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_form_keys_and_default_forms():
    assert bench.split_form("chunk128") == ("chunk", 128)
    assert bench.split_form("chunk", 64) == ("chunk", 64)
    assert bench.split_form("chunk_bwd") == ("chunk_bwd", 64)
    assert bench.split_form("birnn") == ("birnn", 64)
    with pytest.raises(SystemExit):
        bench.split_form("birnn64")
    with pytest.raises(SystemExit):
        bench.split_form("attention")
    # the 4097-token workload: the chunkwise form at each chunk size, the RNN, the full form as reference
    assert bench.default_forms(lin.WORKLOADS["hires_d"]) == ["chunk64", "chunk128", "chunk256", "birnn", "full"]
    assert bench.default_forms(lin.WORKLOADS["vit_tiny_lit"]) == ["full", "chunk64"]
    assert bench.default_forms(lin.WORKLOADS["hires_d"], chunk=128) == ["chunk128", "birnn", "full"]


def test_memory_counts_inputs_output_and_workspace():
    wl = lin.WORKLOADS["hires_d"]
    m = bench.memory_bytes("chunk", wl, 128, 1_000_000)
    io = 4 * 8 * 12 * 4097 * 64 * 2 + 4 * 12
    assert m["io_MB"] == io / 1e6 and m["workspace_MB"] == 1.0 and m["total_MB"] == (io + 1e6) / 1e6


def test_two_order_chunk_keys_do_not_swallow_the_chunk_size():
    assert bench.split_form("chunk256") == ("chunk", 256)
    assert bench.split_form("chunk2_128") == ("chunk2", 128)
    assert bench.split_form("chunk2", 64) == ("chunk2", 64)
    assert bench.split_form("chunk_bwd64") == ("chunk_bwd", 64)
