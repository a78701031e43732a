"""bench.py's one JSON line on a short headline run: the keys, units and relations the
contract fixes (value = kept token-heads per second of decode-step time, the roofline of
the decode attention against 8 TB/s, the CPU baseline of the oracle)."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_headline_line_keeps_the_contract():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print("bench contract: headline, 3 steps, 1 warm-up, 1 CPU row", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--only", "headline",
                        "--steps", "3", "--warmup", "1", "--cpu-rows", "1"],
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.strip()]
    assert len(lines) == 1, r.stdout[-2000:]  # exactly one JSON line on stdout
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
              "roofline", "cpu_baseline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 1
    assert d["higher_is_better"] is True and d["dtype"] == "bf16"
    assert d["config"]["workload"] == "qwen3_8b_layer"
    # value = token-heads of the timed steps / their time
    th = d["config"]["token_heads_per_step"]
    assert d["value"] == pytest.approx(th / (d["ms_per_step"] * 1e-3), rel=1e-6)
    rf = d["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert rf["achieved"] == pytest.approx(rf["per_launch_work"] / (rf["launch_ms"] * 1e-3) / 1e9, rel=1e-6)
    assert rf["frac"] == pytest.approx(rf["achieved"] / rf["peak"], rel=1e-9)
    assert 0.3 < rf["frac"] < 1.0  # a plausible HBM fraction for this call
    assert rf["traffic"] is None or rf["traffic"] > 0.9 * rf["per_launch_work"]
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1
    assert cb["unit"] == d["unit"]
    # the decode step is slower than the attention alone, and both are sub-millisecond
    assert rf["launch_ms"] < d["ms_per_step"] < 1.0
