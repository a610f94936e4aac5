"""Host-side logic of bench.py, checked on the CPU: the algorithmic byte counts
behind the roofline, the gate that lets a committed counter summary feed the
line's `traffic` only while the attention sources are unchanged, and the
refusal of more than one GPU."""
import os
import subprocess
import sys

import pytest

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_attention_bytes_llama7b_layer():
    # per (request, head): K and V of 1024 prefix + 46 tree slots, 128 dims,
    # 2 bytes, plus Q read and O written for the 46 nodes
    w = synth.make_config(2)
    per_pair = (1024 + 46) * 128 * 2 * 2 + 2 * 46 * 128 * 2
    assert bench.attn_bytes(w) == 8 * 32 * per_pair == 146_276_352
    # parents in; ancestor masks, child masks (N + 1 words), depths and status out
    assert bench.mask_bytes(w) == 8 * (46 * 4 + 46 * 8 + 47 * 8 + 46 * 4 + 4) == 8_928
    # every target row of fp32 logits once
    assert bench.logit_bytes(w) == 8 * 47 * 32000 * 4 == 48_128_000


def test_traffic_gate_follows_the_sources(monkeypatch):
    path = os.path.join(ROOT, "profiles", "tree_attn_verify_llama7b_layer_traffic.md")
    fields = {}
    with open(path) as f:
        for line in f:
            if line.startswith("- ") and ":" in line:
                k, v = line[2:].split(":", 1)
                fields[k.strip()] = v.strip().strip("`")
    got = bench.measured_traffic("llama7b_layer")
    if fields["attn_source_sha256"] == bench.attn_source_hash():
        assert got == int(fields["traffic_bytes_per_launch"])
    else:
        assert got is None
    # a summary taken on other sources is not used
    monkeypatch.setattr(bench, "attn_source_hash", lambda: "0" * 64)
    assert bench.measured_traffic("llama7b_layer") is None
    assert bench.measured_traffic("no_such_workload") is None


def test_committed_traffic_matches_the_sources():
    """The committed summaries were taken on the attention sources as they are."""
    for wl in ("llama65b_layer", "llama7b_layer"):
        assert bench.measured_traffic(wl) is not None, wl


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_cpu_model_is_named():
    name = bench._cpu_model()
    assert isinstance(name, str) and name and name != "unknown" or not os.path.exists("/proc/cpuinfo")
