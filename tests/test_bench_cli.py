"""bench.py's contract on the host: one GPU only, no silent run without a GPU,
the algorithmic byte counts of the measured workloads, and the stored PMC
traffic readings."""
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True,
                          text=True, timeout=300, env=dict(os.environ, WORLD_SIZE="1"))


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.skipif(__import__("torch").cuda.is_available(), reason="checks the no-GPU path")
def test_no_gpu_is_an_error():
    r = _run("--steps", "1", "--warmup", "0")
    assert r.returncode == 2
    assert "needs a GPU" in r.stderr


def test_ht_step_bytes():
    # 4096 tokens of the DeepEP routing study (seed 0): 16,248 stage-1 rows,
    # 32,768 stage-2 rows; scores 4,194,304 + tokens 58,720,256 + topk and
    # weights 262,144 + stage-1 rows and metadata 121,275,072 + stage-2 rows
    # and metadata 242,614,272 + combine 528,744,448 bytes
    ab = bench.algorithmic_bytes(4096, 8, 7168, 16248, 32768, 256)
    assert ab["combine"] == 469_762_048 + 131_072 + 131_072 + 58_720_256
    assert ab["dispatch"] == 58_720_256 + 262_144 + 16248 * (7392 + 72) + 32768 * (7392 + 12)
    assert ab["total"] == 955_810_496
    assert ab["total"] - ab["combine"] == 427_066_048          # the HT dispatch side, scores included


def test_ll_step_bytes():
    # 64 sources x 128 tokens: scores 8,388,608 + tokens 117,440,512 + topk and
    # slot map 524,288 + counts 65,536 + messages 485,490,688 = 611,909,632 on
    # the dispatch side
    ab = bench.ll_algorithmic_bytes(8192, 8, 7168, 256, 64)
    assert ab["total"] - ab["combine"] == 611_909_632
    assert ab["total"] == 1_669_398_528
    assert bench.ll_algorithmic_bytes(8192, 8, 7168, 256, 64, fp8=False)["total"] == 2_124_480_512


def test_stored_traffic_is_consistent():
    ab = bench.algorithmic_bytes(4096, 8, 7168, 16248, 32768, 256)
    for kernel in ("dispatch", "combine"):
        t = bench.stored_traffic(kernel)
        if t is not None:       # only while the kernel sources match the profiled ones
            assert abs(t / ab[kernel] - 1) < 0.05, (kernel, t, ab[kernel])


def test_cpu_baseline_object(monkeypatch):
    """The oracle leg, on a 256-token batch of the prefill workload's shape:
    one whole run on the host, reported as the oracle with the threads it
    used, what it ran, and value = the step's algorithmic bytes / time."""
    import ep_inputs as I
    import oracle
    monkeypatch.setattr(bench, "MIN_CPU_SECONDS", 0.0)
    n = 256
    scores = I.page_scores(n, 256, 0)
    w = I.normal_weights(n, 8, 0)
    cb = bench.cpu_baseline(scores, I.normal_bf16(n, 7168, 1), w, I.normal_bf16(n * 8, 7168, 2), n)
    assert cb["kind"] == "oracle" and cb["unit"] == "GB/s" and cb["runs"] == 1
    assert cb["cores"] == bench.host_threads() and cb["nproc"] == os.cpu_count()
    assert cb["value"] > 0 and f"{n} tokens" in cb["sample"]
    st = cb["single_thread"]
    assert st["cores"] == 1 and st["runs"] == 1 and st["value"] > 0
    lay = oracle.layout_ht(oracle.route(scores, 8, 8, 4), 1, 256, 8, 8)
    ab = bench.algorithmic_bytes(n, 8, 7168, int(lay["c1"].sum()), int(lay["c2"].sum()), 256)["total"]
    # seconds is rounded to the millisecond
    for leg in (cb, st):
        assert abs(leg["value"] - ab / leg["seconds"] / 1e9) <= leg["value"] * (0.01 + 0.0006 / leg["seconds"])


def test_oracle_on_token_ranges_equals_the_whole_batch():
    """The multi-core CPU baseline runs the oracle's per-token stages on
    disjoint token ranges: routing, packing (rows written into one set) and
    the combine over ranges give exactly the whole batch's results."""
    import ep_inputs as I
    import oracle
    n, H = 300, 256
    scores = I.page_scores(n, 256, 3).astype(np.float32)
    xb = I.bf16_bits(I.normal_bf16(n, H, 4))
    w = I.normal_weights(n, 8, 5)
    parts = [(0, 77), (77, 78), (78, 300)]
    topk = oracle.route(scores, 8, 8, 4)
    topk_p = np.concatenate([oracle.route(scores[a:b], 8, 8, 4) for a, b in parts])
    np.testing.assert_array_equal(topk_p, topk)
    lay = oracle.layout_ht(topk, 1, 256, 8, 8)
    r1, r2 = int(lay["c1"].sum()), int(lay["c2"].sum())
    whole = oracle.pack_ht(xb, topk, w, n, 8, True, lay["node_row"], lay["row2"], r1, r2)
    pk = oracle.pack_ht(xb[:0], topk[:0], w[:0], n, 8, True, lay["node_row"][:0], lay["row2"][:0], r1, r2)
    for a, b in parts:
        oracle.pack_ht(xb[a:b], topk[a:b], w[a:b], n, 8, True, lay["node_row"][a:b], lay["row2"][a:b],
                       r1, r2, out=pk, first_token=a)
    for k in whole:
        np.testing.assert_array_equal(pk[k], whole[k], err_msg=k)
    y = oracle.dequant_rows(whole["stage2"], H, True)
    out = oracle.combine(y, w, lay["row2"])
    out_p = np.concatenate([oracle.combine(y, w, lay["row2"], which=np.arange(a, b)) for a, b in parts])
    np.testing.assert_array_equal(out_p, out)


def test_stored_round_trip_traffic_is_consistent():
    # 16384 tokens, Zipf(1.1) routing (seed 5): 64,695 stage-1 and 131,072 stage-2 rows
    ab = bench.algorithmic_bytes(16384, 8, 7168, 64695, 131072, 256)
    for kernel in ("dispatch", "combine"):
        t = bench.stored_traffic(kernel, bench.TRAFFIC_FILE_ROUND_TRIP)
        if t is not None:
            assert abs(t / ab[kernel] - 1) < 0.05, (kernel, t, ab[kernel])


@pytest.mark.parametrize("fp8", [True, False])
def test_stored_ll_traffic_is_consistent(fp8):
    ab = bench.ll_algorithmic_bytes(8192, 8, 7168, 256, 64, fp8=fp8)
    path = bench.TRAFFIC_FILE_LL if fp8 else bench.TRAFFIC_FILE_LL_BF16
    for kernel in ("dispatch", "combine"):
        t = bench.stored_traffic(kernel, path)
        if t is not None:
            assert abs(t / ab[kernel] - 1) < 0.05, (kernel, t, ab[kernel])


def test_stored_backward_traffic_is_consistent():
    n, K, H, rows = 4096, 8, 7168, 32768
    alg = {"combine_backward": n * H * 2 + 2 * rows * H * 2 + 3 * n * K * 4,
           "dispatch_backward": rows * H * 2 + n * K * 4 + n * H * 2}
    for kernel, b in alg.items():
        t = bench.stored_traffic(kernel, bench.TRAFFIC_FILE_BWD)
        if t is not None:
            assert abs(t / b - 1) < 0.05, (kernel, t, b)


@pytest.mark.parametrize("rows1,rows2,per_rank,name", [(16248, 30574, True, "TRAFFIC_FILE_PER_RANK"),
                                                       (21622, 32768, False, "TRAFFIC_FILE_NO_LIMIT")])
def test_stored_prefill_variant_traffic_is_consistent(rows1, rows2, per_rank, name):
    ab = bench.algorithmic_bytes(4096, 8, 7168, rows1, rows2, 256, per_rank)
    for kernel in ("dispatch", "combine"):
        t = bench.stored_traffic(kernel, getattr(bench, name))
        if t is not None:
            assert abs(t / ab[kernel] - 1) < 0.05, (kernel, t, ab[kernel])
