"""bench.py's output contract on the GPU: one JSON line with every key the
contract names, of the right types, and the roofline, copy-ceiling and cold
objects (a short run of the small workload, and of the operator)."""
import json
import subprocess
import sys
from pathlib import Path

import pytest

pytestmark = pytest.mark.gpu

ROOT = Path(__file__).resolve().parents[1]

KEYS = {"metric": str, "value": float, "unit": str, "n_gpus": int, "steps": int,
        "warmup": int, "ms_per_step": float, "higher_is_better": bool, "scaling": str,
        "dtype": str, "data": str, "config": dict, "roofline": dict}


def _run(*args):
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), *args], capture_output=True,
                       text=True, cwd=ROOT, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.startswith("{")]
    assert len(lines) == 1, r.stdout[-2000:]
    return json.loads(lines[0])


def _check(d, steps, warmup):
    for k, t in KEYS.items():
        assert isinstance(d[k], t), (k, d.get(k))
    assert "vs_baseline" in d and d["vs_baseline"] is None
    assert d["n_gpus"] == 1 and d["steps"] == steps and d["warmup"] == warmup
    assert d["higher_is_better"] is True and d["scaling"] == "weak"
    assert d["value"] > 0 and d["ms_per_step"] > 0
    assert "workload" in d["config"]
    r = d["roofline"]
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-9
    assert r["traffic"] is None or r["traffic"] > 0
    c = d["copy_ceiling"]
    assert c["achieved"] > 0 and c["cold_achieved"] > 0 and d["cold"]["ms_per_launch"] > 0
    assert abs(c["frac"] - r["achieved"] / c["achieved"]) < 1e-9
    for k in ("copy_512MiB", "read_512MiB", "mix_512MiB"):
        assert c[k] > 0 and abs(c["frac_of_" + k] - r["achieved"] / c[k]) < 1e-9
    assert c["mix"] in ("1:1", "2:1", "4:1") and c["empty_launch_us"] > 0
    assert r["algorithmic_read_bytes"] + r["algorithmic_write_bytes"] == \
        r["algorithmic_bytes_per_launch"]
    # the warm-up launches from the host; the timed region is a graph replay
    h = d["host_launched"]
    assert h["launches"] == warmup and h["ms_per_launch"] > 0
    assert d["cold"]["ms_per_launch_unscrubbed"] > 0


def test_epilog_bench_line():
    d = _run("--config", "0", "--steps", "3", "--warmup", "2")
    _check(d, 3, 2)
    assert d["host_launched"]["prepared_ms_per_launch"] > 0
    assert d["config"]["workload"] == "mode0_tiny_d256"
    assert d["metric"].endswith("mode0_tiny_d256")
    pat = d["copy_ceiling"]["pattern"]
    assert pat["ms_per_launch"] > 0 and pat["row_bytes"] == 352 and pat["src_row_bytes"] == 512
    cb = d["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["cores"] == 1 and cb["value"] > 0 and cb["gbps"] > 0
    assert d["parity_sample_bytes_equal"] is True


def test_operator_bench_line():
    d = _run("--drq", "drq_fp16_h2304", "--steps", "3", "--warmup", "2", "--no-cpu")
    _check(d, 3, 2)
    assert d["config"]["workload"] == "drq_fp16_h2304"
