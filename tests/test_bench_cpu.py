"""CPU checks of bench.py's accounting: the algorithmic bytes and FLOPs it
divides by, the committed profile records it reads, the rule that a record
measured on other kernel sources is ignored, and the one-GPU refusal."""
import importlib.util
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_algorithmic_bytes_of_the_benchmark_workload(bench):
    # B=1, H=32, L=65536, d=128, bf16 tokens, one fp32 state in and out per head:
    # listed tensor by tensor
    B, H, L, d = 1, 32, 65536, 128
    tokens = {name: B * H * L * d * 2 for name in ("Q", "K", "V", "O")}
    states = {name: B * H * d * d * 4 for name in ("S0", "S_end")}
    assert bench.alg_bytes(B, H, L, d) == sum(tokens.values()) + sum(states.values())
    assert bench.alg_bytes(B, H, L, d) == 2151677952
    # without state I/O it is 1024 bytes per token-head
    assert bench.alg_bytes(B, H, L, d, state_in=False, state_out=False) == 1024 * B * H * L


def test_algorithmic_flops_per_token_head(bench):
    # per token-head at d = 128, chunk 64: 2 d^2 for k v^T, 2 d^2 for q^T S,
    # and the causal half of the intra-chunk products, (C + 1)(dk + dv):
    # 82,176 FLOP, the figure the metric is defined with
    d, C = 128, 64
    per = 2 * d * d + 2 * d * d + (C + 1) * (d + d)
    assert per == 82176
    assert bench.alg_flops(1, 32, 65536, d) == per * 32 * 65536
    assert bench.alg_flops(2, 16, 16384, d) == per * 2 * 16 * 16384


@pytest.mark.parametrize("name,key", [("k_chunk_fwd_segment_64k_hbm_bytes.md", "traffic_bytes"),
                                      ("k_chunk_fwd_segment_64k_mfma.md", "mfma_util_pct")])
def test_profile_records_parse(bench, name, key):
    rec = bench._profile_record(name)
    assert rec is not None, f"profiles/{name} holds no JSON record"
    assert key in rec
    sha = rec["sources_sha256"]
    assert len(sha) == 64 and all(c in "0123456789abcdef" for c in sha)


def test_traffic_record_is_consistent(bench):
    rec = bench._profile_record("k_chunk_fwd_segment_64k_hbm_bytes.md")
    from_counters = (rec["fetch_kib"] * rec["fetch_factor"] + rec["write_kib"] * rec["write_factor"]) * 1024
    assert abs(from_counters - rec["traffic_bytes"]) <= 1e-5 * rec["traffic_bytes"]
    # the main kernel moves its algorithmic bytes plus a few sub-segment states
    ratio = rec["traffic_bytes"] / bench.alg_bytes(1, 32, 65536, 128)
    assert 1.0 <= ratio < 1.05


def test_records_of_other_sources_are_ignored(bench, monkeypatch):
    rec_t = bench._profile_record("k_chunk_fwd_segment_64k_hbm_bytes.md")
    rec_m = bench._profile_record("k_chunk_fwd_segment_64k_mfma.md")
    monkeypatch.setattr(bench, "_fwd_kernel_sha", lambda: "0" * 64)
    assert bench.measured_traffic() is None
    assert bench.measured_mfma() is None
    monkeypatch.setattr(bench, "_fwd_kernel_sha", lambda: rec_t["sources_sha256"])
    assert bench.measured_traffic() == rec_t["traffic_bytes"]
    monkeypatch.setattr(bench, "_fwd_kernel_sha", lambda: rec_m["sources_sha256"])
    assert bench.measured_mfma() == rec_m["mfma_util_pct"]


def test_source_hash_covers_the_kernel_files(bench):
    csrc = os.path.join(ROOT, "long_sequence_causal_amd", "csrc")
    for name in bench.FWD_KERNEL_SOURCES:
        assert os.path.exists(os.path.join(csrc, name)), name
    assert len(bench._fwd_kernel_sha()) == 64


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""
