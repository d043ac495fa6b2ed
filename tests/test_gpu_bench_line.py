"""bench.py's JSON line on a GPU: one short run of the default workload,
checked field by field against the output contract (one GPU, graph-timed
steps, the roofline object of the dominant kernel)."""
import json
import os
import subprocess
import sys

import pytest

from gpu_util import need_gpu, say

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_json_line():
    need_gpu()
    say("bench.py --steps 8 --warmup 2 --no-cpu-baseline --no-secondary")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "8", "--warmup", "2",
                        "--no-cpu-baseline", "--no-secondary"], capture_output=True, text=True, timeout=100,
                       env=dict(os.environ, WORLD_SIZE="1"))
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1
    d = json.loads(lines[0])
    assert d["metric"] == "dispatch+combine HBM GB/s and tokens/s on 1 MI355X (% of HBM peak)"
    assert d["unit"] == "GB/s" and d["n_gpus"] == 1 and d["steps"] == 8 and d["warmup"] == 2
    assert d["higher_is_better"] is True and d["scaling"] == "weak" and d["vs_baseline"] is None
    assert d["dtype"] == "f32" and d["data"].startswith("synthetic")
    assert d["config"]["workload"] == "ht_prefill_4096_plus_combine"
    ab = d["config"]["algorithmic_bytes_per_step"]
    assert ab == 955_810_496
    assert abs(d["value"] - ab / (d["ms_per_step"] * 1e-3) / 1e9) <= 0.01 * d["value"]
    assert abs(d["frac_of_hbm_peak"] - d["value"] / 8000.0) < 1e-3
    rf = d["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert rf["kernel"] in ("dispatch", "combine")
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-3
    assert rf["traffic"] is None or abs(rf["traffic"] / rf["algorithmic_bytes_per_launch"] - 1) < 0.05
    assert 0 < d["value"] < 8000.0 and 0 < rf["achieved"] < 8000.0
    assert "cpu_baseline" not in d and "secondary" not in d
    assert set(d["kernel_ms"]) == {"route_handle", "dispatch", "combine"}
    # three more replays of the timed graph, each a plausible step time
    reps = d["ms_per_step_replays"]
    assert len(reps) == 3 and all(0.2 * d["ms_per_step"] < r < 5 * d["ms_per_step"] for r in reps)


def test_bench_secondary_lines():
    """The default run adds the 64 x 128 LL decode and the 16384-token round
    trip, each with its own step time, GB/s and roofline kernel."""
    need_gpu()
    say("bench.py --steps 4 --warmup 1 --no-cpu-baseline (with the secondary workloads)")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "4", "--warmup", "1",
                        "--no-cpu-baseline"], capture_output=True, text=True, timeout=110,
                       env=dict(os.environ, WORLD_SIZE="1"))
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [l for l in r.stdout.splitlines() if l.startswith("{")]
    assert len(lines) == 1
    d = json.loads(lines[0])
    assert d["config"]["workload"] == "ht_prefill_4096_plus_combine"
    sec = d["secondary"]
    assert sec["ll_decode_64x128"]["workload"] == "ll_decode_64x128_plus_combine"
    assert sec["round_trip_16384_zipf"]["workload"] == "ht_round_trip_16384_zipf_plus_combine"
    for line in sec.values():
        assert abs(line["gbs"] - line["algorithmic_bytes_per_step"] / (line["ms_per_step"] * 1e-3) / 1e9) \
            <= 0.01 * line["gbs"]
        assert line["roofline"]["kernel"] in ("dispatch", "combine")
        assert 0 < line["gbs"] < 8000.0
        assert len(line["ms_per_step_replays"]) == 3
