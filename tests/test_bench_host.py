"""bench.py's host logic, on the CPU: the one-GPU contract, the counter-traffic lookup
(a figure is reported only while every source file of the kernel is the profiled one)
and the algorithmic byte counts the roofline divides by."""
import json
import os
import shutil
import subprocess
import sys
import types

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def run_bench(*args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, env=env, timeout=120)


def test_more_than_one_gpu_is_refused_before_any_gpu_work():
    r = run_bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""  # no JSON line
    r = run_bench(env_extra={"WORLD_SIZE": "4"})
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_unknown_record_is_an_argument_error():
    r = run_bench("--only", "headline,no_such_record")
    assert r.returncode == 2 and "unknown record" in r.stderr


def test_traffic_is_reported_only_for_the_profiled_sources(tmp_path, monkeypatch):
    rec_all = json.load(open(os.path.join(ROOT, "profiles", "pmc_traffic.json")))
    keys = [k for k, v in rec_all.items() if isinstance(v, dict) and "sources" in v]
    assert "decode_attn" in keys
    # a private copy of the profiled record and of the kernel's sources
    os.makedirs(tmp_path / "profiles")
    shutil.copy(os.path.join(ROOT, "profiles", "pmc_traffic.json"), tmp_path / "profiles")
    rec = rec_all["decode_attn"]
    for f in rec["sources"]:
        os.makedirs(os.path.dirname(tmp_path / f), exist_ok=True)
        shutil.copy(os.path.join(ROOT, f), tmp_path / f)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    if bench.pmc_traffic("decode_attn") is None:
        pytest.skip("the committed counters predate the current decode-attention sources")
    assert bench.pmc_traffic("decode_attn") == rec["hbm_bytes_per_launch"]
    # any change to any source file of the kernel withdraws the figure
    last = tmp_path / rec["sources"][-1]
    last.write_bytes(last.read_bytes() + b"\n")
    assert bench.pmc_traffic("decode_attn") is None
    assert bench.pmc_traffic("no_such_kernel") is None


def test_counter_records_are_scaled_by_the_copy_calibration():
    rec_all = json.load(open(os.path.join(ROOT, "profiles", "pmc_traffic.json")))
    cal = rec_all["copy_calibration"]
    for k, v in rec_all.items():
        if isinstance(v, dict) and "fetch_kib_raw" in v:
            want = (v["fetch_kib_raw"] * cal["fetch_scale"] + v["write_kib_raw"] * cal["write_scale"]) * 1024
            assert abs(v["hbm_bytes_per_launch"] - want) <= 1e-6 * want, k


def _ctx(**wl):
    import torch
    base = dict(d=128, B=16, Hq=32, kv_dtype=torch.bfloat16, lp_bits=8)
    base.update(wl)
    return types.SimpleNamespace(wl=types.SimpleNamespace(**base))


def test_algorithmic_bytes_of_one_decode_attention():
    import torch
    q_out = 16 * 32 * 128 * (2 + 4)  # bf16 queries read, fp32 outputs written
    # bf16 token-heads: K and V rows, 512 B each at d = 128, and a block-table entry per 16
    got = bench.Context.attn_bytes(_ctx(), 1600, 0)
    assert got == 1600 * 512 + 1600 / 16 * 4 + q_out
    # int8 (and fp8) codes: 2 x (128 codes + one fp32 scale) = 264 B per token-head
    got = bench.Context.attn_bytes(_ctx(lp_bits=8), 0, 3200)
    assert got == 3200 * 264 + 3200 / 16 * 4 + q_out
    assert bench.Context.attn_bytes(_ctx(lp_bits="fp8"), 0, 3200) == got
    # int4 codes: two per byte, 2 x (64 + 4) = 136 B per token-head
    assert bench.Context.attn_bytes(_ctx(lp_bits=4), 0, 3200) == 3200 * 136 + 3200 / 16 * 4 + q_out
    # fp32 caches: 4-byte elements, fp32 queries
    got = bench.Context.attn_bytes(_ctx(d=64, B=1, Hq=4, kv_dtype=torch.float32), 640, 0)
    assert got == 640 * 512 + 640 / 16 * 4 + 1 * 4 * 64 * (4 + 4)


def test_rate_helpers():
    assert bench.gbs(8e9, 1000.0) == pytest.approx(8.0)
    assert bench.gbs(5.44e8, 0.1032) == pytest.approx(5271.3, rel=1e-4)
    assert bench.code_bytes(4) == 0.5 and bench.code_bytes(8) == 1.0 and bench.code_bytes("fp8") == 1.0
