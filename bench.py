#!/usr/bin/env python3
"""Benchmark: MoE EP dispatch + combine at the 4096-token DeepSeek-V3 shape on one MI355X.

One step = the whole hot path over one batch, all inputs resident in HBM:
  route_handle (A1+A2) scores [4096, 256] f32 -> topk_idx [4096, 8], then
                     counts, prefix sums and in-tile ranks (one call)
  dispatch (A3+A5+A6) FP8 quantisation, node-deduplicated same-position
                     stage-1 rows and expert-grouped stage-2 rows (+ metadata)
  combine  (A7)      32768 expert-output rows (bf16, hidden 7168) gathered,
                     weighted and reduced back to [4096, 7168] bf16
Workload: 8 nodes x 8 ranks, 256 experts, top-8, at most 4 nodes per token,
router scores U[0,1) + 0.5*U[0,1) per expert (seed 0) -- the DeepEP page's
routing study; tokens and expert outputs ~N(0,1) bf16; weights softmax of
N(0,1) logits.  Four input sets (scores, tokens, expert outputs, outputs)
rotate so that no step reads what the previous one left in the last-level
cache.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                    [--mode graph|eager]
                    [--workload ht_prefill|ht_prefill_rank|ht_prefill_nolimit|ll_decode|
                                ll_decode_1src|ll_decode_bf16|ht_backward|round_trip]

Prints one JSON line (rank 0).  value = algorithmic bytes of one step /
step time, in GB/s, with the step time from one replay of a HIP graph that
holds exactly K captured steps; tokens/s and the fraction of the 8 TB/s HBM
peak are reported beside it.  The default run also times the 64 x 128-token
LL decode and the 16384-token skewed round trip the same way and adds them
under "secondary" (value stays the 4096-token step's).  The roofline object describes the dominant
kernel with its own average duration from HIP events recorded on the launch
stream.  The other workloads (LL decode, per-rank stage 2, backward) report
the same fields for their own steps.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import ep_inputs as I  # noqa: E402

HBM_PEAK_GBS = 8000.0
N_SETS = 4
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_ht_prefill_combine_4096.txt")
TRAFFIC_FILE_ROUND_TRIP = os.path.join(ROOT, "profiles", "traffic_ht_round_trip_16384_zipf.txt")
TRAFFIC_FILE_LL = os.path.join(ROOT, "profiles", "traffic_ll_decode_64x128.txt")
TRAFFIC_FILE_LL_BF16 = os.path.join(ROOT, "profiles", "traffic_ll_decode_64x128_bf16.txt")
TRAFFIC_FILE_BWD = os.path.join(ROOT, "profiles", "traffic_ht_backward_4096.txt")
TRAFFIC_FILE_PER_RANK = os.path.join(ROOT, "profiles", "traffic_ht_prefill_4096_per_rank.txt")
TRAFFIC_FILE_NO_LIMIT = os.path.join(ROOT, "profiles", "traffic_ht_prefill_4096_no_node_limit.txt")
KERNEL_SOURCES = ("ep_dispatch.hip", "ep_combine.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic_bytes(n_tok, K, H, rows1, rows2, E, per_rank=False):
    """Bytes each step must move at least once (read + write), per kernel.

    route_handle : scores n*E*4 read, topk n*K*4 written (the handle's own
               counts and in-tile ranks are not counted)
    dispatch : tokens n*H*2 read, topk + weights 2*n*K*4 read,
               stage-1 rows1*(H + H/128*4) + metadata rows1*(2 + 2K)*4,
               stage-2 rows2*(H + H/128*4) + metadata rows2*3*4 written
    combine  : rows2*H*2 read, weights n*K*4 + row map n*K*4 read,
               n*H*2 written
    With the per-rank stage 2 a stage-2 row also carries the token's K local
    expert ids and weights (+2K*4), and the combine reads no weights.
    """
    row = H + H // 128 * 4
    route = n_tok * E * 4 + n_tok * K * 4
    meta2 = 3 + (2 * K if per_rank else 0)
    dispatch = (n_tok * H * 2 + 2 * n_tok * K * 4 + rows1 * row + rows1 * (2 + 2 * K) * 4
                + rows2 * row + rows2 * meta2 * 4)
    combine = rows2 * H * 2 + (1 if per_rank else 2) * n_tok * K * 4 + n_tok * H * 2
    # headline total = scores + tokens + topk + weights + stage rows/meta + combine
    total = n_tok * E * 4 + dispatch + combine
    return dict(route_handle=route, dispatch=dispatch, combine=combine, total=total)


def source_digest():
    """Digest of the dispatch and combine sources' code: line comments,
    trailing blanks and empty lines are left out, so that only a change of
    code makes the stored counter readings stale."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "combine_ep_route_amd", "csrc", name)) as f:
            for line in f:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def stored_traffic(kernel: str, path: str = TRAFFIC_FILE):
    """HBM bytes per launch measured with rocprofv3 PMC counters, if the
    stored measurement was taken on the current kernel sources."""
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        line = line.strip()
        if line and not line.startswith("#") and "=" in line:
            k, v = line.split("=", 1)
            vals[k.strip()] = v.strip()
    if vals.get("source_sha256_16") != source_digest():
        return None
    v = vals.get(f"{kernel}_bytes_per_launch")
    return float(v) if v else None


MIN_CPU_SECONDS = 8.0   # each leg of the CPU baseline runs at least this long (whole runs)


def host_threads():
    """Host threads the multi-core oracle leg uses: the CPUs this process may
    run on, capped by OMP_NUM_THREADS when it is set (a shared host may set
    it to this job's CPU share)."""
    avail = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    cap = int(os.environ.get("OMP_NUM_THREADS", "0") or 0)
    return max(1, min(avail, cap) if cap > 0 else avail)


def oracle_step(oracle, scores, xb, weights, yb, n_tok, pool, parts):
    """One pass of the whole step through the oracle.  Routing, packing and
    the combine are per token, so with a thread pool they run on disjoint
    token ranges at once (the oracle's C functions release the interpreter
    lock); the counting sort of the layout is one sequential pass.  Returns
    (seconds of the timed parts, rows1, rows2)."""
    def each(fn):
        if pool is None:
            return [fn(a, b) for a, b in parts]
        return list(pool.map(lambda ab: fn(*ab), parts))
    t0 = time.perf_counter()
    topk = np.empty((n_tok, 8), np.int32)
    def route(a, b):
        topk[a:b] = oracle.route(scores[a:b], 8, 8, 4)
    each(route)
    lay = oracle.layout_ht(topk, 1, 256, 8, 8)
    rows1, rows2 = int(lay["c1"].sum()), int(lay["c2"].sum())
    pk = oracle.pack_ht(xb[:0], topk[:0], weights[:0], n_tok, 8, True, lay["node_row"][:0], lay["row2"][:0],
                        rows1, rows2)
    def pack(a, b):
        oracle.pack_ht(xb[a:b], topk[a:b], weights[a:b], n_tok, 8, True, lay["node_row"][a:b],
                       lay["row2"][a:b], rows1, rows2, out=pk, first_token=a)
    each(pack)
    t1 = time.perf_counter()
    y = oracle.dequant_rows(pk["stage2"], 7168, True) if yb is None else yb   # identity expert, untimed
    del pk
    t2 = time.perf_counter()
    def comb(a, b):
        oracle.combine(y, weights, lay["row2"], which=np.arange(a, b))
    each(comb)
    return (t1 - t0) + (time.perf_counter() - t2), rows1, rows2


def cpu_baseline(scores, x, weights, Y, n_tok):
    """The oracle on the same workload (all n_tok tokens), repeated whole
    until MIN_CPU_SECONDS have passed: on all the host threads this process
    may use (token ranges in parallel; `value`), and single-threaded.  Y None:
    the combine takes the identity expert's output of the oracle's own
    stage-2 rows, made outside the timed parts, as on the GPU."""
    import oracle
    from concurrent.futures import ThreadPoolExecutor
    xb = I.bf16_bits(x)
    yb = None if Y is None else I.bf16_bits(Y)
    threads = host_threads()
    legs = {}
    for name, nthr in (("all_cores", threads), ("single_thread", 1)):
        parts = [(int(a), int(b)) for a, b in zip(np.linspace(0, n_tok, nthr + 1)[:-1],
                                                  np.linspace(0, n_tok, nthr + 1)[1:]) if b > a]
        pool = ThreadPoolExecutor(nthr) if nthr > 1 else None
        runs, busy = 0, 0.0
        try:
            while True:
                dt, rows1, rows2 = oracle_step(oracle, scores, xb, weights, yb, n_tok, pool, parts)
                busy += dt
                runs += 1
                if busy >= MIN_CPU_SECONDS:
                    break
        finally:
            if pool:
                pool.shutdown()
        legs[name] = (busy / runs, runs, nthr)
    b = algorithmic_bytes(n_tok, 8, 7168, rows1, rows2, 256)["total"]
    expert = " (identity expert untimed)" if Y is None else ""
    dt, runs, nthr = legs["all_cores"]
    dt1, runs1, _ = legs["single_thread"]
    return dict(value=round(b / dt / 1e9, 4), unit="GB/s", cores=nthr, kind="oracle",
                sample=f"the whole step workload ({n_tok} tokens: route, layout, FP8 quantise + HT pack, "
                       f"combine{expert}); per-token stages on {nthr} threads over token ranges, the layout's "
                       f"counting sort on one; {runs} runs of {dt:.2f} s",
                seconds=round(dt, 3), runs=runs, tokens_per_s=round(n_tok / dt, 1),
                nproc=os.cpu_count(), affinity=len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None,
                single_thread={"value": round(b / dt1 / 1e9, 4), "unit": "GB/s", "cores": 1,
                               "seconds": round(dt1, 3), "runs": runs1, "tokens_per_s": round(n_tok / dt1, 1)})


def ll_algorithmic_bytes(n_tok, K, H, E, S, fp8=True):
    """LL step bytes (every entry valid under the node limit):
    route    : scores n*E*4 read, topk n*K*4 written
    dispatch : tokens n*H*2 read, topk n*K*4 read, slot map n*K*4 written,
               counts E*S*4, messages n*K*(H + H/128*4 + 16) written
               (BF16 payload: n*K*(2H + 16))
    combine  : n*K*H*2 read, weights + slot map 2*n*K*4 read, n*H*2 written
    """
    msg = (H + H // 128 * 4 + 16) if fp8 else (2 * H + 16)
    route = n_tok * E * 4 + n_tok * K * 4
    dispatch = n_tok * H * 2 + 2 * n_tok * K * 4 + E * S * 4 + n_tok * K * msg
    combine = n_tok * K * H * 2 + 2 * n_tok * K * 4 + n_tok * H * 2
    total = n_tok * E * 4 + dispatch + combine
    return dict(route_handle=route, dispatch=dispatch, combine=combine, total=total)


def ll_cpu_baseline(T=128):
    """The oracle on the LL decode workload, one source's T tokens at a time
    (route, fixed-slot layout, pack, identity expert on the used slots,
    combine), through the sources in order until MIN_CPU_SECONDS have passed
    or all of them are done."""
    import oracle
    w = I.LL_DECODE
    S_all = w.num_src_ranks
    scores = I.scores_for(w)
    xb = I.bf16_bits(I.tokens_for(w))
    wts = I.normal_weights(w.num_tokens, 8, w.seed)
    done = 0
    t0 = time.perf_counter()
    for src in range(S_all):
        r = slice(src * T, (src + 1) * T)
        topk = oracle.route(scores[r], 8, 8, 4)
        _, slot, _ = oracle.layout_ll(topk, 1, 256, 128)
        msgs = oracle.pack_ll(xb[r], T, 8, True, slot, 256 * 128)
        used = np.unique(slot[slot >= 0])
        y = np.zeros((256 * 128, 7168), np.uint16)
        y[used] = oracle.dequant_rows(msgs[used], 7168, True)
        oracle.combine(y, wts[r], slot)
        done += 1
        if time.perf_counter() - t0 >= MIN_CPU_SECONDS:
            break
    dt = time.perf_counter() - t0
    b = ll_algorithmic_bytes(T * done, 8, 7168, 256, done)["total"]
    return dict(value=round(b / dt / 1e9, 4), unit="GB/s", cores=1, kind="oracle",
                sample=f"sources 0..{done - 1} of the {S_all} x {T}-token decode workload, one source at a time "
                       f"(route, fixed-slot layout, FP8 quantise + LL pack, identity expert on the used slots, "
                       f"combine), {dt:.2f} s single-threaded",
                seconds=round(dt, 3), sources=done, tokens_per_s=round(T * done / dt, 1))


def time_steps(step, args, stream, out_of, ep, g, n_calls=3, replays=None):
    """Warm-up, an eager pass with events around every call (per-call ms),
    then (graph mode) one captured step per input set, replayed; the graph's
    output must equal the eager output of the same step.  The first timed
    replay gives ms_per_step; with `replays` (a list) three more replays are
    timed the same way and appended to it, to show the run-to-run spread."""
    log(f"[bench] warmup {args.warmup}")
    for j in range(args.warmup):
        step(j)
    torch.cuda.synchronize()
    assert ep.ep_get_device_error(g) == 0
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(n_calls + 1)] for _ in range(args.steps)]
    log(f"[bench] eager: timing {args.steps} steps with per-call events")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for j in range(args.steps):
        step(j, events[j])
    torch.cuda.synchronize()
    ms_eager = (time.perf_counter() - t0) * 1e3 / args.steps
    assert ep.ep_get_device_error(g) == 0
    per = np.array([[events[j][q].elapsed_time(events[j][q + 1]) for q in range(n_calls)]
                    for j in range(args.steps)])  # ms
    mean_ms = per.mean(axis=0)
    pct = {q: np.percentile(per, q, axis=0) for q in (10, 50, 90)}
    ms_per_step = ms_eager
    if args.mode == "graph":
        graph = torch.cuda.CUDAGraph()
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(cap):
            step(0)            # warm the capture stream
        torch.cuda.current_stream().wait_stream(cap)
        torch.cuda.synchronize()
        # one graph of exactly `steps` steps (the input sets in turn), so the
        # timed region is exactly that many steps
        with torch.cuda.graph(graph, stream=cap):
            for j in range(args.steps):
                step(j)
        graph.replay()             # untimed: the graph's first launch
        torch.cuda.synchronize()
        log(f"[bench] graph: timing {args.steps} steps (one replay)")
        t0 = time.perf_counter()
        graph.replay()
        torch.cuda.synchronize()
        ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
        if replays is not None:
            for _ in range(3):
                t0 = time.perf_counter()
                graph.replay()
                torch.cuda.synchronize()
                replays.append((time.perf_counter() - t0) * 1e3 / args.steps)
        assert ep.ep_get_device_error(g) == 0
        ref = out_of(0).clone()
        step(0)
        torch.cuda.synchronize()
        assert torch.equal(ref.view(torch.int16), out_of(0).view(torch.int16))
    return mean_ms, ms_eager, ms_per_step, pct


def percentiles_ms(names, pct):
    """Per-call p10 / median / p90 of the eager event timings, in ms."""
    return {k: {f"p{q}": round(float(pct[q][i]), 5) for q in (10, 50, 90)} for i, k in enumerate(names)}


def time_cpu_sync(ep, g, s, reps=50):
    """The HT receive-count query, the pages' CPU synchronisation, timed on
    the host apart from the step: `wait` is the blocking call alone on a
    finished handle (stream sync + device-to-host copy of the counts);
    `route_handle_wait` runs from enqueueing route + handle until the count
    is on the host."""
    wait, full = [], []
    for _ in range(reps):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        h = ep.ep_route_handle(g, s["scores"], s["topk"])
        ep.ep_handle_get_num_recv(h, -1)
        t1 = time.perf_counter()
        ep.ep_handle_get_num_recv(h, -1)
        t2 = time.perf_counter()
        ep.ep_destroy_handle(h)
        full.append(t1 - t0)
        wait.append(t2 - t1)
    q = lambda a: {f"p{p}": round(float(np.percentile(a, p)) * 1e6, 2) for p in (10, 50, 90)}
    return {"wait": q(wait), "route_handle_wait": q(full)}


STEP_CALLS = ["route_handle", "dispatch", "combine"]


def result_line(args, ab, mean_ms, ms_eager, ms_per_step, n_tok, config, traffic_ok, pct,
                traffic_file=TRAFFIC_FILE, replays=None):
    names = STEP_CALLS
    ms = dict(zip(names, mean_ms))
    value = ab["total"] / (ms_per_step * 1e-3) / 1e9
    dom = "combine" if ms["combine"] >= ms["dispatch"] else "dispatch"
    achieved = ab[dom] / (ms[dom] * 1e-3) / 1e9
    i_d, i_c = names.index("dispatch"), names.index("combine")
    return {
        "metric": "dispatch+combine HBM GB/s and tokens/s on 1 MI355X (% of HBM peak)",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "execution": args.mode,
        "ms_per_step_eager": round(ms_eager, 5),
        # three more replays of the same graph after the timed one
        "ms_per_step_replays": [round(r, 5) for r in (replays or [])],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # the arithmetic type: quantisation and the combine's accumulation are
        # fp32; FP8 and BF16 are the storage formats of rows and tokens
        "dtype": "f32",
        "formats": "fp8_e4m3 payload + fp32 scales / bf16 combine, fp32 accumulate",
        "data": "synthetic (seeded; the DeepEP routing study's score distribution, N(0,1) tokens and expert outputs)",
        "config": config,
        "tokens_per_s": round(n_tok / (ms_per_step * 1e-3), 1),
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "kernel_ms": {k: round(float(v), 5) for k, v in ms.items()},
        "kernel_ms_percentiles": percentiles_ms(names, pct),
        # dispatch + combine alone at their median per-call times (route and
        # handle excluded): tokens / (t_dispatch + t_combine) and the bytes of
        # the two over the same time
        "dispatch_combine_median": {
            "tokens_per_s": round(n_tok / ((pct[50][i_d] + pct[50][i_c]) * 1e-3), 1),
            "gbs": round((ab["dispatch"] + ab["combine"]) / ((pct[50][i_d] + pct[50][i_c]) * 1e-3) / 1e9, 1)},
        "kernel_gbs": {k: round(ab[k] / (ms[k] * 1e-3) / 1e9, 1) for k in names},
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": stored_traffic(dom, traffic_file) if traffic_ok else None,
                     "algorithmic_bytes_per_launch": ab[dom]},
    }


def secondary_line(r):
    """The compact form of another workload's result line."""
    return {"workload": r["config"]["workload"], "ms_per_step": r["ms_per_step"],
            "ms_per_step_replays": r["ms_per_step_replays"], "gbs": r["value"],
            "frac_of_hbm_peak": r["frac_of_hbm_peak"], "tokens_per_s": r["tokens_per_s"],
            "algorithmic_bytes_per_step": r["config"]["algorithmic_bytes_per_step"],
            "kernel_ms": r["kernel_ms"], "roofline": r["roofline"]}


def run_ht(args, ep, per_rank=False, node_limit=4, w=I.HT_PREFILL):
    """HT dispatch + combine.  At the prefill shape the combine reads N(0,1)
    expert outputs; the round trip (16384 tokens, Zipf popularity) combines
    the identity expert's output of the dispatched stage-2 rows, made once
    before the timed steps (every step routes the same scores)."""
    round_trip = w is I.ROUND_TRIP
    n_tok, E, K, H = w.num_tokens, w.num_experts, w.top_k, w.hidden
    log(f"[bench] building inputs: {n_tok} tokens, hidden {H}, {E} experts, top-{K}, {w.scores} scores")
    scores = I.scores_for(w)
    x = I.tokens_for(w)
    weights = I.normal_weights(n_tok, K, w.seed)
    # (per rank: the first rows2 are used)
    Y = None if round_trip else I.normal_bf16(n_tok * K, H, I.COMBINE.seed)

    dev = torch.device("cuda")
    sets = []
    for j in range(N_SETS):
        # every set holds the same values in different memory, the expert
        # outputs included (470 MB each at the prefill shape)
        sets.append(dict(scores=torch.from_numpy(scores).to(dev), x=x.to(dev),
                         topk=torch.empty((n_tok, K), dtype=torch.int32, device=dev),
                         out=torch.empty((n_tok, H), dtype=torch.bfloat16, device=dev),
                         Y=None if Y is None else Y.to(dev)))
    w_d = torch.from_numpy(weights).to(dev)
    Y_d = None

    g = ep.ep_create_group(mode="ht", num_nodes=8, ranks_per_node=8, num_experts=E, top_k=K,
                           max_nodes_per_token=node_limit, hidden=H, max_tokens_per_rank=n_tok,
                           num_src_ranks=1, payload="fp8", num_cus=args.num_cus,
                           ht_stage2="rank" if per_rank else "expert")
    stream = torch.cuda.current_stream()
    w_comb = None if per_rank else w_d   # per-rank rows are the ranks' weighted sums

    def step(j, ev=None):
        s = sets[j % N_SETS]
        if ev is not None:
            ev[0].record(stream)
        h = ep.ep_route_handle(g, s["scores"], s["topk"])
        if ev is not None:
            ev[1].record(stream)
        ep.ep_dispatch(h, s["x"], topk_weights=w_d)
        if ev is not None:
            ev[2].record(stream)
        ep.ep_combine(h, s["Y"] if s["Y"] is not None else Y_d, w_comb, s["out"])
        if ev is not None:
            ev[3].record(stream)
        ep.ep_destroy_handle(h)

    # Exact row counts of this routing (the same every step).
    h = ep.ep_route_handle(g, sets[0]["scores"], sets[0]["topk"])
    rows2 = ep.ep_handle_get_num_recv(h, -1)
    rows1 = int(ep.ep_handle_get_map(h, ep._abi.EP_MAP_HT_RANK_COUNT).sum().item())
    if round_trip:
        # the identity expert: dequantised stage-2 rows, the combine's input
        log(f"[bench] identity expert on {rows2} stage-2 rows (untimed)")
        ep.ep_dispatch(h, sets[0]["x"], topk_weights=w_d)
        Y_d = torch.empty((rows2, H), dtype=torch.bfloat16, device=dev)
        ep.ep_dequantize_rows(g, ep.ep_get_buffer(g, ep._abi.EP_BUF_HT_STAGE2)[:rows2], Y_d)
    ep.ep_destroy_handle(h)
    ab = algorithmic_bytes(n_tok, K, H, rows1, rows2, E, per_rank)

    replays = []
    mean_ms, ms_eager, ms_per_step, pct = time_steps(step, args, stream, lambda j: sets[j]["out"], ep, g,
                                                     replays=replays)
    if round_trip:
        name = f"ht_round_trip_{n_tok}_zipf"
    else:
        name = f"ht_prefill_{n_tok}" + ("_per_rank" if per_rank else "") + ("" if node_limit else "_no_node_limit")
    config = {"workload": name + "_plus_combine",
              "tokens": n_tok, "hidden": H, "experts": E, "top_k": K, "nodes": 8, "ranks_per_node": 8,
              "max_nodes_per_token": node_limit, "stage2": "per_rank" if per_rank else "per_expert",
              "stage1_rows": rows1, "stage2_rows": rows2, "algorithmic_bytes_per_step": ab["total"]}
    headline = not per_rank and node_limit == 4 and not round_trip
    traffic_file = (TRAFFIC_FILE_ROUND_TRIP if round_trip else TRAFFIC_FILE_PER_RANK if per_rank
                    else TRAFFIC_FILE_NO_LIMIT if node_limit == 0 else TRAFFIC_FILE)
    result = result_line(args, ab, mean_ms, ms_eager, ms_per_step, n_tok, config,
                         traffic_ok=True, pct=pct, traffic_file=traffic_file, replays=replays)
    result["cpu_sync_us"] = time_cpu_sync(ep, g, sets[0])
    if per_rank:
        result["formats"] = "fp8_e4m3 payload / bf16 combine of per-rank partial rows, fp32 accumulate"
    if round_trip:
        result["data"] = ("synthetic (seeded; U[0,1) scores plus a normalised Zipf(1.1) expert popularity, "
                          "N(0,1) tokens; the combine input is the identity expert's output of the "
                          "dispatched rows, made once outside the timed steps)")
        # end to end: the round trip returns every token within FP8 error of itself
        xs, out = sets[0]["x"].float(), sets[0]["out"].float()
        amax = xs.abs().view(n_tok, H // 128, 128).amax(dim=2, keepdim=True).expand(-1, -1, 128).reshape(n_tok, H)
        bound = 2.0**-4 * xs.abs() + 2.0**-8 * xs.abs() + amax * 2.0**-9 + 1e-6
        result["round_trip_within_fp8_bound"] = bool(((out - xs).abs() <= bound).all().item())
        del xs, out, amax, bound
    if not args.no_cpu_baseline and (headline or round_trip):
        log("[bench] timing the CPU oracle on the same workload")
        result["cpu_baseline"] = cpu_baseline(scores, x, weights, Y, n_tok)
    ep.ep_destroy_group(g)
    return result


def run_ll(args, ep, S, payload="fp8"):
    """The LL decode path, staged as in the NCCL-EP pipeline: route, handle,
    dispatch(send_only) + complete, combine(send_only) + complete."""
    w = I.LL_DECODE.with_(num_src_ranks=S)
    T, E, K, H = w.tokens_per_rank, w.num_experts, w.top_k, w.hidden
    n_tok = S * T
    log(f"[bench] building inputs: {S} sources x {T} tokens, hidden {H}, {E} experts, top-{K}")
    scores = I.scores_for(w)
    x = I.tokens_for(w)
    weights = I.normal_weights(n_tok, K, w.seed)
    dev = torch.device("cuda")
    sets = []
    for j in range(N_SETS):
        sets.append(dict(scores=torch.from_numpy(scores).to(dev), x=x.to(dev),
                         topk=torch.empty((n_tok, K), dtype=torch.int32, device=dev),
                         counts=torch.empty(E, dtype=torch.int32, device=dev),
                         out=torch.empty((n_tok, H), dtype=torch.bfloat16, device=dev)))
    w_d = torch.from_numpy(weights).to(dev)
    # expert outputs at the dispatch geometry [E, S*T_max, H]; only the used
    # slots are read
    gen = torch.Generator(device=dev)
    gen.manual_seed(I.COMBINE.seed)
    Y_d = torch.empty((E, S * T, H), dtype=torch.bfloat16, device=dev)
    Y_d.normal_(generator=gen)

    g = ep.ep_create_group(mode="ll", num_nodes=8, ranks_per_node=8, num_experts=E, top_k=K,
                           max_nodes_per_token=4, hidden=H, max_tokens_per_rank=T,
                           num_src_ranks=S, payload=payload, num_cus=args.num_cus)
    stream = torch.cuda.current_stream()

    def step(j, ev=None):
        s = sets[j % N_SETS]
        if ev is not None:
            ev[0].record(stream)
        h = ep.ep_route_handle(g, s["scores"], s["topk"])
        if ev is not None:
            ev[1].record(stream)
        ep.ep_dispatch(h, s["x"], recv_counts=s["counts"], send_only=True)
        ep.ep_complete(h)
        if ev is not None:
            ev[2].record(stream)
        ep.ep_combine(h, Y_d, w_d, s["out"], send_only=True)
        ep.ep_complete(h)
        if ev is not None:
            ev[3].record(stream)
        ep.ep_destroy_handle(h)

    ab = ll_algorithmic_bytes(n_tok, K, H, E, S, fp8=payload == "fp8")
    replays = []
    mean_ms, ms_eager, ms_per_step, pct = time_steps(step, args, stream, lambda j: sets[j]["out"], ep, g,
                                                     replays=replays)
    suffix = "" if payload == "fp8" else "_bf16"
    config = {"workload": f"ll_decode_{S}x{T}{suffix}_plus_combine", "tokens": n_tok, "sources": S,
              "tokens_per_source": T, "hidden": H, "experts": E, "top_k": K, "nodes": 8,
              "ranks_per_node": 8, "max_nodes_per_token": 4, "slots": T,
              "algorithmic_bytes_per_step": ab["total"]}
    result = result_line(args, ab, mean_ms, ms_eager, ms_per_step, n_tok, config,
                         traffic_ok=S == 64, pct=pct,
                         traffic_file=TRAFFIC_FILE_LL if payload == "fp8" else TRAFFIC_FILE_LL_BF16,
                         replays=replays)
    if payload != "fp8":
        result["formats"] = "bf16 payload / bf16 combine, fp32 accumulate"
    result["us_per_call"] = {k: round(float(v) * 1e3, 2) for k, v in zip(STEP_CALLS, mean_ms)}
    if not args.no_cpu_baseline and payload == "fp8":
        log("[bench] timing the CPU oracle on one source's share")
        result["cpu_baseline"] = ll_cpu_baseline(T)
    ep.ep_destroy_group(g)
    return result


def run_ht_backward(args, ep):
    """The backward pass at the prefill shape, reusing forward handles (NCCL-EP
    training example): combine adjoint (bf16 row gradients + weight gradients)
    then dispatch adjoint (token gradients), per step."""
    w = I.HT_PREFILL
    n_tok, E, K, H = w.num_tokens, w.num_experts, w.top_k, w.hidden
    log(f"[bench] building inputs: backward of {n_tok} tokens, hidden {H}, {E} experts, top-{K}")
    scores = I.scores_for(w)
    x = I.tokens_for(w)
    weights = I.normal_weights(n_tok, K, w.seed)
    dev = torch.device("cuda")
    g = ep.ep_create_group(mode="ht", num_nodes=8, ranks_per_node=8, num_experts=E, top_k=K,
                           max_nodes_per_token=4, hidden=H, max_tokens_per_rank=n_tok,
                           num_src_ranks=1, payload="fp8", num_cus=args.num_cus, max_handles=N_SETS)
    w_d = torch.from_numpy(weights).to(dev)
    rows2 = n_tok * K
    Y_d = I.normal_bf16(rows2, H, I.COMBINE.seed).to(dev)
    dY = torch.empty((rows2, H), dtype=torch.bfloat16, device=dev)
    sets = []
    for j in range(N_SETS):
        s = dict(scores=torch.from_numpy(scores).to(dev),
                 topk=torch.empty((n_tok, K), dtype=torch.int32, device=dev),
                 grad=I.normal_bf16(n_tok, H, 800 + j).to(dev),
                 dw=torch.empty((n_tok, K), dtype=torch.float32, device=dev),
                 out=torch.empty((n_tok, H), dtype=torch.bfloat16, device=dev))
        # the forward pass that made the handle (not timed)
        ep.ep_route(g, s["scores"], s["topk"])
        s["h"] = ep.ep_create_handle(g, s["topk"])
        ep.ep_dispatch(s["h"], x.to(dev), topk_weights=w_d)
        sets.append(s)
    torch.cuda.synchronize()
    assert ep.ep_handle_get_num_recv(sets[0]["h"], -1) == rows2
    stream = torch.cuda.current_stream()

    def step(j, ev=None):
        s = sets[j % N_SETS]
        if ev is not None:
            ev[0].record(stream)
        ep.ep_combine_backward(s["h"], s["grad"], w_d, dY, expert_out=Y_d, grad_weights=s["dw"])
        if ev is not None:
            ev[1].record(stream)
        ep.ep_dispatch_backward(s["h"], dY, s["out"])
        if ev is not None:
            ev[2].record(stream)

    cb = n_tok * H * 2 + 2 * rows2 * H * 2 + 3 * n_tok * K * 4
    db = rows2 * H * 2 + n_tok * K * 4 + n_tok * H * 2
    mean_ms, ms_eager, ms_per_step, pct = time_steps(step, args, stream, lambda j: sets[j]["out"], ep, g,
                                                     n_calls=2)
    total = cb + db
    value = total / (ms_per_step * 1e-3) / 1e9
    dom, dom_b, dom_ms = ("combine_backward", cb, mean_ms[0]) if mean_ms[0] >= mean_ms[1] else \
        ("dispatch_backward", db, mean_ms[1])
    achieved = dom_b / (dom_ms * 1e-3) / 1e9
    result = {
        "metric": "dispatch+combine HBM GB/s and tokens/s on 1 MI355X (% of HBM peak)",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "execution": args.mode,
        "ms_per_step_eager": round(ms_eager, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "formats": "bf16 gradients, fp32 accumulate",
        "data": "synthetic (seeded; the DeepEP routing study's score distribution, N(0,1) gradients and expert outputs)",
        "config": {"workload": "ht_prefill_4096_backward", "tokens": n_tok, "hidden": H, "experts": E,
                   "top_k": K, "nodes": 8, "ranks_per_node": 8, "max_nodes_per_token": 4,
                   "rows": rows2, "algorithmic_bytes_per_step": total},
        "tokens_per_s": round(n_tok / (ms_per_step * 1e-3), 1),
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "kernel_ms": {"combine_backward": round(float(mean_ms[0]), 5),
                      "dispatch_backward": round(float(mean_ms[1]), 5)},
        "kernel_ms_percentiles": percentiles_ms(["combine_backward", "dispatch_backward"], pct),
        "kernel_gbs": {"combine_backward": round(cb / (mean_ms[0] * 1e-3) / 1e9, 1),
                       "dispatch_backward": round(db / (mean_ms[1] * 1e-3) / 1e9, 1)},
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": stored_traffic(dom, TRAFFIC_FILE_BWD),
                     "algorithmic_bytes_per_launch": dom_b},
    }
    for s in sets:
        ep.ep_destroy_handle(s["h"])
    ep.ep_destroy_group(g)
    return result


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true",
                    help="with the default workload, skip the LL decode and round-trip lines")
    ap.add_argument("--num-cus", type=int, default=0, help="CU cap for dispatch/combine (0 = all)")
    ap.add_argument("--mode", choices=["graph", "eager"], default="graph",
                    help="graph: the step is captured once per input set in a HIP graph and replayed; "
                         "eager: every step is enqueued from Python")
    ap.add_argument("--workload", choices=["ht_prefill", "ht_prefill_rank", "ht_prefill_nolimit", "ll_decode",
                                           "ll_decode_1src", "ll_decode_bf16", "ht_backward", "round_trip"],
                    default="ht_prefill",
                    help="ht_prefill: 4096 tokens, HT dispatch + combine (the headline); "
                         "ll_decode: 64 sources x 128 tokens, staged LL dispatch + combine; "
                         "ll_decode_1src: one source's 128 tokens; "
                         "ht_backward: the backward pass at the prefill shape on forward handles; "
                         "ht_prefill_rank: the prefill step with the per-rank stage 2; "
                         "ht_prefill_nolimit: the prefill step routed without the node limit; "
                         "ll_decode_bf16: the 64 x 128 decode step with BF16 messages (14352 B); "
                         "round_trip: 16384 tokens with Zipf(1.1) expert popularity, FP8 dispatch + "
                         "combine of the identity expert's output")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy three times (the reference "
                         "kernel for scaling HBM byte counters), then exit")
    ap.add_argument("--calibrate-fill", type=int, default=0, metavar="BYTES",
                    help="only run a plain device fill of BYTES bytes three times (a write-only "
                         "reference kernel for the dispatch's write rate), then exit")
    args = ap.parse_args(argv)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the 64 EP ranks are partitions of one MI355X's HBM; "
              "it has no multi-GPU mode", file=sys.stderr)
        return 2
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2

    if args.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "device copy", "bytes_read_per_launch": 1 << 30,
                          "bytes_written_per_launch": 1 << 30, "launches": 3}), flush=True)
        return 0
    if args.calibrate_fill > 0:
        dst = torch.empty(args.calibrate_fill // 4, dtype=torch.int32, device="cuda")
        for _ in range(3):
            dst.fill_(1)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "device fill", "bytes_written_per_launch": dst.numel() * 4,
                          "launches": 3}), flush=True)
        return 0

    import combine_ep_route_amd as ep

    if args.workload in ("ht_prefill", "ht_prefill_rank", "ht_prefill_nolimit"):
        result = run_ht(args, ep, per_rank=args.workload == "ht_prefill_rank",
                        node_limit=0 if args.workload == "ht_prefill_nolimit" else 4)
        if args.workload == "ht_prefill" and not args.no_secondary:
            # the LL decode and the skewed round trip, timed the same way on
            # the same GPU; value stays the headline's
            sub = argparse.Namespace(**{**vars(args), "no_cpu_baseline": True})
            result["secondary"] = {}
            for key, fn in (("ll_decode_64x128", lambda: run_ll(sub, ep, 64)),
                            ("round_trip_16384_zipf", lambda: run_ht(sub, ep, w=I.ROUND_TRIP))):
                torch.cuda.empty_cache()
                result["secondary"][key] = secondary_line(fn())
            torch.cuda.empty_cache()
    elif args.workload == "round_trip":
        result = run_ht(args, ep, w=I.ROUND_TRIP)
    elif args.workload == "ht_backward":
        result = run_ht_backward(args, ep)
    elif args.workload == "ll_decode_bf16":
        result = run_ll(args, ep, 64, payload="bf16")
    else:
        result = run_ll(args, ep, 64 if args.workload == "ll_decode" else 1)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
