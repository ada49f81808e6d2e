"""bench.py's host-side arithmetic and contract, on the CPU: the single-GPU guard, the roofline
entry of the dominant kernel class, the counter-traffic lookup, and the phase roofline's work
counts for the LLaDA-8B workload against the figures derived by hand from the model shape."""

import hashlib
import importlib.util
import json
import os
import re
import subprocess
import sys

import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench():
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_roofline_takes_the_class_with_the_largest_time():
    b = _bench()
    prof = {"gemm_skinny": {"launches": 10, "ms": 1.0, "bytes": 4e9, "flops": 1e9},
            "gemm_tiled": {"launches": 4, "ms": 2.0, "bytes": 1e9, "flops": 2e12},
            "attention": {"launches": 8, "ms": 0.5, "bytes": 1e9, "flops": 1e11}}
    roof, name = b.roofline(prof, "bf16", None)
    assert name == "gemm_tiled" and roof["bound"] == "mfma" and roof["unit"] == "TFLOP/s"
    assert roof["achieved"] == pytest.approx(2e12 / 2e-3 / 1e12)
    assert roof["frac"] == pytest.approx(roof["achieved"] / 2500.0)
    assert roof["avg_us"] == pytest.approx(500.0)
    assert roof["traffic"] is None  # no workload: no counters apply
    prof["gemm_skinny"]["ms"] = 5.0
    roof, name = b.roofline(prof, "bf16", None)
    assert name == "gemm_skinny" and roof["bound"] == "hbm" and roof["unit"] == "GB/s"
    assert roof["achieved"] == pytest.approx(4e9 / 5e-3 / 1e9)
    assert roof["frac"] == pytest.approx(roof["achieved"] / 8000.0)


def test_counter_traffic_follows_the_committed_summary():
    """The traffic figure is the committed summary's while the kernel source still hashes to the
    recorded value, None otherwise, and only for the workload the counters were taken on."""
    b = _bench()
    path = os.path.join(ROOT, "profiles", "gemm_tiled_llada8b_traffic.md")
    d = json.loads(re.search(r"```json\n(.*?)\n```", open(path).read(), re.S).group(1))
    src = os.path.join(ROOT, d["source"])
    same = hashlib.sha256(open(src, "rb").read()).hexdigest() == d["source_sha256"]
    got = b.counter_traffic("gemm_tiled", d["workload"])
    assert got == (d["traffic_bytes_per_dispatch"] if same else None)
    assert b.counter_traffic("gemm_tiled", "dream7b") is None
    assert b.counter_traffic("gemm_skinny", d["workload"]) is None
    # the recorded figure is the dispatch-weighted mean of the per-kernel bytes
    ks = d["kernels"].values()
    mean = sum(k["bytes_per_dispatch"] * k["dispatches"] for k in ks) / sum(k["dispatches"] for k in ks)
    assert abs(mean - d["traffic_bytes_per_dispatch"]) <= 1 + 1e-6 * mean
    for k in ks:  # bytes = scaled FETCH_SIZE + scaled WRITE_SIZE
        est = (k["fetch_kib_per_dispatch"] * d["fetch_scale"] + k["write_kib_per_dispatch"] * d["write_scale"]) * 1024
        assert est == pytest.approx(k["bytes_per_dispatch"], rel=1e-3)


def test_phase_roofline_work_of_the_llada8b_workload():
    """Weights 2 B each (32 layers of q/k/v, o, gate/up, down, plus the lm_head), K/V as 4-byte
    pairs per cached element, 2 flops per multiply-add: the figures a reader can check by hand."""
    b = _bench()
    cfg = synth.configs.get("llada8b")
    r = b.phase_roofline(cfg, 20.0, 4.0)
    d, F, V, nl, L, Bs = 4096, 12288, 126464, 32, 768, 32
    layer = d * 3 * d + d * d + 3 * d * F
    wbytes = (nl * layer + V * d) * 2
    assert wbytes == 14_994_636_800
    kv_read = 2 * 32 * L * 128 * 4 * nl
    step = r["cached_step"]
    assert step["bytes"] == pytest.approx(wbytes + kv_read + 2 * Bs * 32 * 128 * 4 * nl)
    assert step["bound"] == "hbm"
    assert step["roofline_ms"] == pytest.approx(step["bytes"] / 8e12 * 1e3)
    ref = r["refresh"]
    flops = 2.0 * L * nl * layer + 2.0 * Bs * V * d + 4.0 * L * L * 32 * 128 * nl
    assert ref["flops"] == pytest.approx(flops)
    assert ref["flops"] == pytest.approx(11.06e12, rel=1e-3)
    assert ref["bound"] == "mfma"
    assert ref["frac"] == pytest.approx(ref["roofline_ms"] / 20.0)
    # modes whose context varies by block have no single phase roofline
    assert b.phase_roofline(dict(cfg, suffix_window=32), 20.0, 4.0) is None
