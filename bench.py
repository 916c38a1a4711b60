"""Benchmark of paged-KV split-KV decode attention on one MI355X.

One step = the whole hot path for one layer of one decode step: build the step
metadata (page prefix sums + work plan), append this step's K/V token of every
request and run the split-KV decode (partials and their merge).  By default
all three are one launch (pkv_decode_plan: every workgroup plans the step in
LDS, then appends and decodes); --plan metadata builds the plan in its own
launch first (pkv_build_metadata + pkv_decode_append), and --append separate
runs pkv_build_metadata, pkv_append_kv and pkv_decode as three launches.  The
step planned the other way is timed beside it (step_other_plan).  Inputs are seeded synthetic
batches already resident in HBM.  Between steps the pool rotates over several
identical copies whose total size exceeds the 256 MB Infinity Cache, so every
step streams its K/V from HBM.

Timing: after W warm-up steps, a bounded spin kernel holds the GPU while the
host enqueues all K timed steps; two HIP events on the stream the kernels run
on bracket the K steps (step time).  The decode kernel alone is then timed
over at least 100 launches, each between its own pair of HIP events on that
stream (median and p10/p90, each launch's dispatch included), and as the
mean of as many back-to-back launches (us_per_call: the kernel's average
launch duration, the roofline figure); a cache-warm figure (no pool rotation)
is reported beside it, labelled.

Prints one JSON line.  `value` is algorithmic GB/s of the whole step:
bytes the method must move (K/V attended, q, output, page ids, appended rows)
divided by the step time.
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

PEAK_HBM_GBPS = 8000.0
METRIC = "paged decode attention µs/call + achieved HBM GB/s (% of peak), B=16 ragged"
COUNTERS_FILE = os.path.join(ROOT, "profiles", "decode_kernel_counters.json")
KERNEL_SOURCE = os.path.join(ROOT, "paged_kv_split_attn_amd", "csrc", "pkv_decode.hip")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=3, help="workload preset 1..5 (3 = B=16 ragged)")
    ap.add_argument("--groups", type=int, default=0, help="decode grid (0 = one workgroup per CU)")
    ap.add_argument("--min-tiles", type=int, default=0)
    ap.add_argument("--copies", type=int, default=0, help="pool copies to rotate (0 = enough for 768 MB)")
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="CPU work (seconds x worker processes) of the oracle CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--append", choices=("fused", "separate"), default="fused",
                    help="KV append fused into the decode launch, or its own launch")
    ap.add_argument("--plan", choices=("launch", "metadata"), default="launch",
                    help="plan the step inside the decode launch (pkv_decode_plan), or with "
                         "its own metadata launch first (pkv_build_metadata)")
    ap.add_argument("--graph", action="store_true",
                    help="replay each step from a captured hipGraph (one graph per pool copy)")
    ap.add_argument("--layers", type=int, default=0, metavar="N",
                    help="also time a model-like decode step: one metadata build, then N layers of "
                         "fused append + decode (each layer its own pool and q), issued eagerly and "
                         "replayed from one captured hipGraph, timed on the device and host-paced")
    ap.add_argument("--graph-buckets", type=int, default=0, metavar="N",
                    help="also time the step-graph harness: N layers of fused append + decode "
                         "per step, one graph per power-of-two batch 1..64 (ragged lengths "
                         "uniform in [1, 4096]), replay against eager, host-paced")
    ap.add_argument("--mask-keep", type=float, default=None, metavar="P",
                    help="also time pkv_decode_masked with a random keep mask of density P")
    ap.add_argument("--prefill", action="store_true",
                    help="also time pkv_prefill on a causal prefill batch (4 x 1024 new tokens, "
                         "no prefix, Hq=32, Hkv=8, D=128, P=16)")
    ap.add_argument("--tokens", action="store_true",
                    help="also time pkv_decode_tokens (token-major K/V): the ragged batch through "
                         "a page-size-1 token table, and one contiguous 32k-token request")
    ap.add_argument("--ceiling", action="store_true",
                    help="(the read-only launch is timed by default; kept for old command lines)")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the read-only launch over the decode call's byte count (the "
                         "achievable read rate of one launch of that size), timed by default")
    ap.add_argument("--no-kernel-loop", action="store_true",
                    help="time only whole steps (skip the decode-only loop)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (counter calibration)")
    ap.add_argument("--warm", action="store_true", help="no pool rotation (cache-warm numbers)")
    return ap.parse_args()


def algorithmic_bytes(batch):
    """Bytes the method must move for one decode call and for one whole step."""
    kv = int(batch.seq_lens.astype(np.int64).sum()) * batch.Hkv * batch.D * 2 * 2
    qo = 2 * batch.B * batch.Hq * batch.D * 2
    pages = sum(len(p) for p in batch.page_lists)
    meta = 4 * pages + 4 * (batch.B + 1) + 4 * batch.B
    append = batch.B * batch.Hkv * batch.D * 2 * 2 * 2  # read k_new/v_new, write the slots
    call = kv + qo + meta
    return call, call + append + 4 * (batch.B + 1)


def unique_kv_bytes(batch):
    """K/V bytes of one decode call with every physical page counted once (a
    page shared by several requests' prefixes is read by each of them)."""
    used = {}
    for b, pages in enumerate(batch.page_lists):
        L = int(batch.seq_lens[b])
        for j, p in enumerate(pages):
            n = min(batch.P, L - j * batch.P)
            if n > 0:
                used[int(p)] = max(used.get(int(p), 0), n)
    return sum(used.values()) * batch.Hkv * batch.D * 2 * 2


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_units(batch):
    """The per-request units of one decode call and the function that runs the
    oracle on one of them: oracle.decode of request b alone (an [1, Hq, D]
    output)."""
    import oracle

    ip = oracle.kv_indptr(batch.seq_lens, batch.P)
    idx = batch.kv_indices
    units = [b for b in range(batch.B) if batch.seq_lens[b] > 0]

    def unit(b):
        return oracle.decode(batch.q[b:b + 1], batch.k_pool, batch.v_pool, ip[b:b + 2] - ip[b],
                             idx[int(ip[b]):int(ip[b + 1])], batch.seq_lens[b:b + 1],
                             batch.sm_scale, batch.P)
    return units, unit


_WORKER = {}


def _worker_init(cfg):
    # A fresh interpreter: rebuild the same seeded batch (no data is shipped).
    import workloads as W

    batch = W.config(cfg, poison=False)
    _WORKER["unit"] = oracle_units(batch)[1]


def _worker_unit(b):
    t0 = time.perf_counter()
    _WORKER["unit"](b)
    return time.perf_counter() - t0


def cpu_baseline(batch, budget_s, cfg=None):
    """The fp64 oracle, as it is, timed on the host cores: one decode call is
    split into its requests, each an oracle.decode of that request, run by a
    pool of worker processes (each with one BLAS thread; they rebuild the same
    seeded batch when they start).  One warm-up call, then calls until about
    budget_s seconds of CPU work (wall time x worker processes), at least 3,
    median reported.  cfg=None runs the units in this process, one after
    another (small batches, tests)."""
    import multiprocessing as mp

    units, unit = oracle_units(batch)
    cores = min(len(os.sched_getaffinity(0)), 16, max(1, len(units)))  # box share: 16
    times = []
    if cfg is None:
        cores = 1
        run = lambda: [unit(b) for b in units]  # noqa: E731
        pool = None
    else:
        os.environ.setdefault("OMP_NUM_THREADS", "1")
        pool = mp.get_context("spawn").Pool(cores, initializer=_worker_init, initargs=(cfg,))
        run = lambda: pool.map(_worker_unit, units, chunksize=1)  # noqa: E731
    try:
        run()  # warm-up
        t_all = time.perf_counter()
        while len(times) < 1000:
            t0 = time.perf_counter()
            run()
            times.append(time.perf_counter() - t0)
            if len(times) >= 3 and (time.perf_counter() - t_all) * cores >= budget_s:
                break
    finally:
        if pool is not None:
            pool.close()
            pool.join()
    per_call = float(np.median(times))
    call_bytes, _ = algorithmic_bytes(batch)
    how = (f"{len(units)} per-request units on {cores} worker processes" if pool is not None
           else "its requests one after another in one process")
    return {"value": round(call_bytes / per_call / 1e9, 4), "unit": "GB/s", "cores": cores,
            "cpu": cpu_model(), "kind": "oracle", "us_per_call": round(per_call * 1e6, 1),
            "sample": f"median of {len(times)} full decode calls of the {batch.name} batch "
                      f"(fp64 numpy oracle, {how}, after one warm-up call), "
                      f"{sum(times):.1f} s wall, about {sum(times) * cores:.0f} s of CPU work"}


def counters_for_current_kernel():
    """rocprofv3 FETCH/WRITE per decode launch, if taken on the current kernel source."""
    if not os.path.exists(COUNTERS_FILE):
        return None
    try:
        rec = json.load(open(COUNTERS_FILE))
        sha = hashlib.sha256(open(KERNEL_SOURCE, "rb").read()).hexdigest()
        if rec.get("kernel_source_sha256") != sha:
            return None
        return rec
    except Exception:
        return None


def calibrate_copy(mib, reps=5):
    """A plain device-to-device copy of a known size, for scaling HBM counters."""
    import torch

    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": reps}), flush=True)


PEAK_BF16_TFLOPS = 2500.0


def bench_prefill(pkv, W, torch, dev, stream, K):
    """Causal prefill of 4 x 1024 new tokens (no prefix); rotating pool copies."""
    pb = W.make_prefill(name="prefill_b4_q1024", seed=7, Hq=32, Hkv=8, D=128, P=16,
                        q_lens=[1024] * 4, prefix_lens=[0] * 4, poison=False)
    t = W.to_device(pb, dev)
    desc = pkv.Desc(max_batch=pb.B, num_q_heads=pb.Hq, num_kv_heads=pb.Hkv, head_dim=pb.D,
                    page_size=pb.P)
    ws = torch.zeros(pkv.pkv_workspace_bytes(desc), dtype=torch.uint8, device=dev)
    ip = torch.zeros(pb.B + 1, dtype=torch.int32, device=dev)
    pkv.pkv_build_metadata(desc, t["seq_lens"], 0, ip, ws, stream)
    out = torch.empty(tuple(pb.q_rows.shape), dtype=torch.int16, device=dev)
    pools = [pkv.Pool(t["k_pool"], t["v_pool"])]
    pools += [pkv.Pool(t["k_pool"].clone(), t["v_pool"].clone()) for _ in range(3)]

    def call(i):
        pkv.pkv_prefill(pools[i % len(pools)], desc, t["q_rows"], t["qo_indptr"], ip,
                        t["kv_indices"], t["seq_lens"], 1024, True, pb.sm_scale, out, stream)
    for i in range(3):
        call(i)
    ms = timed(stream, K, call)
    # causal: row i of a request sees i + 1 keys; 4 * D flop per key per query head
    keys = sum(int(n) * (int(n) + 1) // 2 for n in np.diff(pb.qo_indptr))
    flop = keys * pb.Hq * 4 * pb.D
    tf = flop / (ms * 1e-3) / 1e12
    return {"workload": pb.name, "us_per_call": round(ms * 1e3, 2), "flop": int(flop),
            "TFLOPs": round(tf, 1), "bound": "mfma", "peak": PEAK_BF16_TFLOPS,
            "frac": round(tf / PEAK_BF16_TFLOPS, 4)}


def bench_tokens(pkv, W, torch, dev, stream, K):
    """Token-major decode at full size: the ragged batch stored token-major
    (table mode) and one 32,768-token request in the contiguous layout.  K/V
    copies rotate so that every call streams from HBM."""
    cases = [W.tokens_from_pages(W.config(3, poison=False)),
             W.make_tokens(name="contig_b1_32k", seed=4, B=1, Hq=32, Hkv=8, D=128,
                           lengths=np.array([32768]), table=False, poison=False)]
    res = []
    for tb in cases:
        t = W.tokens_to_device(tb, dev)
        desc = pkv.Desc(max_batch=tb.B, num_q_heads=tb.Hq, num_kv_heads=tb.Hkv, head_dim=tb.D,
                        page_size=16)
        ws = torch.zeros(pkv.pkv_workspace_bytes(desc), dtype=torch.uint8, device=dev)
        ip = torch.zeros(tb.B + 1, dtype=torch.int32, device=dev)
        pkv.pkv_build_metadata(desc, t["seq_lens"], 0, ip, ws, stream)
        out = torch.empty((tb.B, tb.Hq, tb.D), dtype=torch.int16, device=dev)
        cache_bytes = 2 * t["k_cache"].numel() * 2
        n = max(1, -(-(768 << 20) // cache_bytes))
        caches = [(t["k_cache"], t["v_cache"])]
        caches += [(t["k_cache"].clone(), t["v_cache"].clone()) for _ in range(n - 1)]

        def call(i):
            k, v = caches[i % n]
            pkv.pkv_decode_tokens(desc, k, v, t["slot_table"], tb.stride, t["q"], ip,
                                  t["seq_lens"], tb.sm_scale, ws, out, stream)
        for i in range(3):
            call(i)
        ms = timed(stream, K, call)
        tokens = int(tb.seq_lens.astype(np.int64).sum())
        byts = (tokens * tb.Hkv * tb.D * 2 * 2 + 2 * tb.B * tb.Hq * tb.D * 2 + 4 * tb.B
                + (4 * tokens if tb.slot_table is not None else 0))
        gbps = byts / (ms * 1e-3) / 1e9
        res.append({"workload": tb.name, "layout": "table" if tb.slot_table is not None
                    else "contiguous", "kv_tokens": tokens, "us_per_call": round(ms * 1e3, 2),
                    "bytes": int(byts), "GBps": round(gbps, 1),
                    "frac": round(gbps / PEAK_HBM_GBPS, 4), "copies": n})
    return res


def bench_ceiling(pkv, torch, dev, stream, K, nbytes):
    """pkv_debug_read_ceiling over nbytes, rotating copies so that every call
    reads from HBM."""
    n = max(16, nbytes // 16 * 16)
    copies = max(3, -(-(768 << 20) // n))
    bufs = [torch.full((n,), i + 1, dtype=torch.uint8, device=dev) for i in range(copies)]
    sink = torch.empty(pkv.READ_CEILING_GROUPS * 64 * pkv.WAVES_PER_GROUP, dtype=torch.int32,
                       device=dev)

    def call(i):
        pkv.pkv_debug_read_ceiling(bufs[i % copies], sink, stream)
    for i in range(3):
        call(i)
    med, p10, p90, _ = timed_each(stream, max(K, 100), call)
    ms = timed(stream, max(K, 100), call)
    gbps = n / (ms * 1e-3) / 1e9
    return {"bytes": n, "us_per_call": round(ms * 1e3, 2),
            "us_per_call_event_median": round(med * 1e3, 2), "us_event_p10": round(p10 * 1e3, 2),
            "us_event_p90": round(p90 * 1e3, 2), "GBps": round(gbps, 1),
            "frac": round(gbps / PEAK_HBM_GBPS, 4), "copies": copies}


def bench_layers(pkv, torch, stream, K, batch, desc, base, nl, plan="launch"):
    """A decode step of an nl-layer model's attention: the first layer's
    pkv_decode_plan (plan = "launch"; else pkv_build_metadata, then that
    layer's pkv_decode_append), then pkv_decode_append for every later layer
    (each its own pool and q), eager and as one hipGraph replay.  Device-timed
    (host enqueues ahead) and host-paced (GPU idle at the start, launch cost
    included)."""
    layers = [(pkv.Pool(base["k_pool"].clone(), base["v_pool"].clone()), base["q"].clone())
              for _ in range(nl)]
    ws = torch.zeros(pkv.pkv_workspace_bytes(desc), dtype=torch.uint8, device=stream.device)
    kv_indptr = torch.zeros(batch.B + 1, dtype=torch.int32, device=stream.device)
    out = torch.zeros((batch.B, batch.Hq, batch.D), dtype=torch.int16, device=stream.device)
    seq, idx = base["seq_lens"], base["kv_indices"]

    def step_on(st):
        for li, (pool, q) in enumerate(layers):
            if li == 0 and plan == "launch":
                pkv.pkv_decode_plan(pool, desc, q, base["k_new"], base["v_new"], seq, 0, kv_indptr,
                                    idx, batch.sm_scale, ws, out, st)
                continue
            if li == 0:
                pkv.pkv_build_metadata(desc, seq, 0, kv_indptr, ws, st)
            pkv.pkv_decode_append(pool, desc, q, base["k_new"], base["v_new"], kv_indptr, idx, seq,
                                  batch.sm_scale, ws, out, st)

    for _ in range(3):
        step_on(stream)
    torch.cuda.synchronize()
    cap = torch.cuda.Stream()
    cap.wait_stream(stream)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            step_on(cap)
    stream.wait_stream(cap)
    torch.cuda.synchronize()
    ref = out.clone()
    g.replay()
    torch.cuda.synchronize()
    if not torch.equal(out, ref):
        raise RuntimeError("graph replay of the layered step differs from the eager step")
    eager = lambda i: step_on(stream)  # noqa: E731
    replay = lambda i: g.replay()  # noqa: E731
    kl = max(5, K // 4)
    res = {"layers": nl, "workload": batch.name, "plan": plan,
           "eager_device_us": timed(stream, kl, eager) * 1e3,
           "graph_device_us": timed(stream, kl, replay) * 1e3,
           "eager_host_paced_us": paced(kl, eager) * 1e3,
           "graph_host_paced_us": paced(kl, replay) * 1e3}
    res = {k: (round(v, 1) if isinstance(v, float) else v) for k, v in res.items()}
    res["graph_speedup_host_paced"] = round(res["eager_host_paced_us"] / res["graph_host_paced_us"], 3)
    return res


def bench_graph_buckets(pkv, W, torch, dev, K, layers):
    """Host-paced step time of the step-graph harness against the same step
    issued eagerly, for every bucket 1..64 (live batch = the bucket size)."""
    from paged_kv_split_attn_amd.step_graphs import StepGraphs

    uni = W.make_batch(name="buckets", seed=81, B=64, Hq=32, Hkv=8, D=128, P=16,
                       lengths=lambda r: r.integers(1, 4097, size=64), poison=False, append=True)
    base = W.to_device(uni, dev)
    pools = [pkv.Pool(base["k_pool"].clone(), base["v_pool"].clone()) for _ in range(layers)]
    tmpl = pkv.Desc(max_batch=64, num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=16)
    sg = StepGraphs(tmpl, pools, uni.sm_scale, max_batch=64, max_pages=len(uni.kv_indices))
    sg.capture()
    rng = np.random.default_rng(82)
    res = []
    for B in sorted(sg.buckets):
        lens = uni.seq_lens[:B].astype(np.int32)
        idx = np.concatenate(uni.page_lists[:B]).astype(np.int32)
        q = torch.from_numpy(W.normal_bf16(rng, (layers, B, 32, 128)).view(np.int16)).to(dev)
        kn = torch.from_numpy(W.normal_bf16(rng, (layers, B, 8, 128)).view(np.int16)).to(dev)
        vn = torch.from_numpy(W.normal_bf16(rng, (layers, B, 8, 128)).view(np.int16)).to(dev)
        bk = sg.load(torch.from_numpy(lens).to(dev), torch.from_numpy(idx).to(dev), q, kn, vn)
        torch.cuda.synchronize()
        kp = max(10, K // 4)
        g_us = paced(kp, lambda i: sg.replay(bk)) * 1e3
        e_us = paced(kp, lambda i: sg.eager(bk)) * 1e3
        res.append({"batch": B, "kv_tokens": int(lens.sum()), "graph_host_paced_us": round(g_us, 1),
                    "eager_host_paced_us": round(e_us, 1),
                    "graph_speedup": round(e_us / g_us, 3)})
    return {"layers": layers, "buckets": res}


def paced(K, fn):
    """Mean wall-clock ms of fn(i) over K calls issued by the host one after
    another, the GPU idle at the start: host launch cost included."""
    import torch

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        fn(i)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / K


def timed_each(stream, K, fn):
    """Per-call ms of fn(i) for K calls, each bracketed by its own pair of HIP
    events on the stream, enqueued behind a bounded spin: returns
    (median, p10, p90, all)."""
    import torch

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(K)]
    torch.cuda.synchronize()
    torch.cuda._sleep(int(40e6))
    for i in range(K):
        ev[i][0].record(stream)
        fn(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    ms = np.array([a.elapsed_time(b) for a, b in ev])
    return float(np.median(ms)), float(np.percentile(ms, 10)), float(np.percentile(ms, 90)), ms


def timed(stream, K, fn):
    """Mean ms of fn(i) over K calls enqueued behind a bounded spin, events at the ends."""
    import torch

    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    torch.cuda._sleep(int(40e6))  # hold the GPU while the host enqueues the K calls
    start.record(stream)
    for i in range(K):
        fn(i)
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / K


def main():
    args = parse()
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}): "
              "this library has no multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import torch

    import paged_kv_split_attn_amd as pkv
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    batch = W.config(args.config, poison=False)
    if not batch.append:
        # every step appends one token per request; draw it from its own stream
        rng = np.random.default_rng(np.random.PCG64(1000 + args.config))
        batch.k_new = W.normal_bf16(rng, (batch.B, batch.Hkv, batch.D))
        batch.v_new = W.normal_bf16(rng, (batch.B, batch.Hkv, batch.D))
        batch.append = True
    print(f"[bench] workload {batch.name}: B={batch.B} Hq={batch.Hq} Hkv={batch.Hkv} D={batch.D} "
          f"P={batch.P} tokens={batch.kv_tokens} pages={batch.num_pages}", file=sys.stderr,
          flush=True)

    desc = pkv.Desc(max_batch=batch.B, num_q_heads=batch.Hq, num_kv_heads=batch.Hkv,
                    head_dim=batch.D, page_size=batch.P, num_workgroups=args.groups,
                    min_tiles_per_group=args.min_tiles)
    base = W.to_device(batch, dev)
    pool_bytes = 2 * base["k_pool"].numel() * 2
    ncopies = args.copies or max(3, math.ceil(768e6 / pool_bytes))
    if args.warm:
        ncopies = 1
    copies = [(pkv.Pool(base["k_pool"], base["v_pool"]), base["q"])]
    for _ in range(ncopies - 1):
        copies.append((pkv.Pool(base["k_pool"].clone(), base["v_pool"].clone()), base["q"].clone()))
    ws = torch.zeros(pkv.pkv_workspace_bytes(desc), dtype=torch.uint8, device=dev)
    kv_indptr = torch.zeros(batch.B + 1, dtype=torch.int32, device=dev)
    out = torch.zeros((batch.B, batch.Hq, batch.D), dtype=torch.int16, device=dev)
    seq, idx = base["seq_lens"], base["kv_indices"]
    k_new, v_new = base["k_new"], base["v_new"]
    stream = torch.cuda.current_stream()

    def step_with(i, st, plan):
        pool, q = copies[i % ncopies]
        if args.append == "fused" and plan == "launch":
            pkv.pkv_decode_plan(pool, desc, q, k_new, v_new, seq, 0, kv_indptr, idx,
                                batch.sm_scale, ws, out, st)
            return
        pkv.pkv_build_metadata(desc, seq, 0, kv_indptr, ws, st)
        if args.append == "fused":
            pkv.pkv_decode_append(pool, desc, q, k_new, v_new, kv_indptr, idx, seq,
                                  batch.sm_scale, ws, out, st)
        else:
            pkv.pkv_append_kv(pool, k_new, v_new, kv_indptr, idx, seq, st)
            pkv.pkv_decode(pool, desc, q, kv_indptr, idx, seq, batch.sm_scale, ws, out, st)

    def step_on(i, st):
        step_with(i, st, args.plan)

    def step(i):
        step_on(i, stream)

    def decode_only(i):
        pool, q = copies[i % ncopies]
        pkv.pkv_decode(pool, desc, q, kv_indptr, idx, seq, batch.sm_scale, ws, out, stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    plan = pkv.pkv_debug_validate(desc, seq, kv_indptr, idx, batch.num_pages, ws)
    if plan["status"] != pkv.PKV_OK:
        raise RuntimeError("device metadata failed validation")

    K = args.steps
    if args.graph:
        # One graph per pool copy, captured on a side stream after the eager
        # warm-up; replays run on the timing stream.
        graphs = []
        cap = torch.cuda.Stream()
        cap.wait_stream(stream)
        for i in range(ncopies):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.stream(cap):
                with torch.cuda.graph(g, stream=cap):
                    step_on(i, cap)
            graphs.append(g)
        stream.wait_stream(cap)
        torch.cuda.synchronize()

        def replay(i):
            graphs[i % ncopies].replay()
        ms_step = timed(stream, K, replay)
        # The same steps paced by the host (no spin ahead of them): each eager
        # step pays its launches' host cost, a replay one graph launch.
        graph_cmp = {"graph_device_us": round(ms_step * 1e3, 2),
                     "eager_device_us": round(timed(stream, K, step) * 1e3, 2),
                     "graph_host_paced_us": round(paced(K, replay) * 1e3, 2),
                     "eager_host_paced_us": round(paced(K, step) * 1e3, 2)}
    else:
        ms_step = timed(stream, K, step)

    call_bytes, step_bytes = algorithmic_bytes(batch)
    res = {
        "metric": METRIC,
        "value": round(step_bytes / (ms_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": batch.name, "seed": batch.seed, "B": batch.B, "Hq": batch.Hq,
                   "Hkv": batch.Hkv, "head_dim": batch.D, "page_size": batch.P,
                   "kv_tokens": batch.kv_tokens, "pool_pages": batch.num_pages,
                   "pool_copies": ncopies, "decode_grid": desc.groups(),
                   "plan_workgroups": plan["groups"], "append": args.append,
                   "plan": args.plan if args.append == "fused" else "metadata",
                   "graph": bool(args.graph),
                   "parallelism": "single-gpu"},
        "step_bytes": step_bytes,
        "call_bytes": call_bytes,
    }
    if args.append == "fused" and not args.graph:
        # The step with its plan made the other way, for comparison.
        other = "metadata" if args.plan == "launch" else "launch"
        res["step_other_plan"] = {
            "plan": other,
            "ms_per_step": round(timed(stream, K, lambda i: step_with(i, stream, other)), 5)}
    if not args.no_kernel_loop:
        # Decode-only launches (pool rotated): per-launch events, median and
        # p10/p90 of at least 100; the mean of as many back-to-back launches
        # beside it.
        # The kernel's average launch duration (the roofline figure, what a
        # kernel trace of the same loop reports) is the mean over back-to-back
        # launches; the per-launch events also count each launch's dispatch.
        KL = max(K, 100)
        ev_ms, p10_ms, p90_ms, _ = timed_each(stream, KL, decode_only)
        call_ms = timed(stream, KL, decode_only)
        achieved = call_bytes / (call_ms * 1e-3) / 1e9
        ctr = counters_for_current_kernel()
        traffic = None
        if ctr is not None:
            traffic = ctr.get("traffic_bytes_per_launch", {}).get(batch.name)
        kv_bytes = int(batch.seq_lens.astype(np.int64).sum()) * batch.Hkv * batch.D * 2 * 2
        uniq = unique_kv_bytes(batch)
        if uniq < kv_bytes:  # shared prefixes: also the rate over bytes counted once
            res["unique_call_bytes"] = call_bytes - kv_bytes + uniq
            res["unique_call_GBps"] = round(res["unique_call_bytes"] / (call_ms * 1e-3) / 1e9, 1)
        # Cache-warm: the same pool every launch (it then sits in the 256 MB
        # Infinity Cache); labelled, never the roofline figure.
        def decode_warm(i):
            pool, q = copies[0]
            pkv.pkv_decode(pool, desc, q, kv_indptr, idx, seq, batch.sm_scale, ws, out, stream)
        warm_ms, _, _, _ = timed_each(stream, KL, decode_warm)
        res.update({
            "us_per_call": round(call_ms * 1e3, 2),
            "us_per_call_event_median": round(ev_ms * 1e3, 2),
            "us_per_call_event_p10": round(p10_ms * 1e3, 2),
            "us_per_call_event_p90": round(p90_ms * 1e3, 2),
            "launches_timed": KL,
            "warm": {"us_per_call": round(warm_ms * 1e3, 2),
                     "GBps": round(call_bytes / (warm_ms * 1e-3) / 1e9, 1),
                     "note": "cache-warm: one pool copy, read again every launch"},
            "call_GBps": round(achieved, 1),
            "call_frac_of_peak": round(achieved / PEAK_HBM_GBPS, 4),
            "roofline": {"bound": "hbm", "kernel": "decode_kernel", "achieved": round(achieved, 1),
                         "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                         "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": traffic},
        })
    if args.prefill:
        res["prefill"] = bench_prefill(pkv, W, torch, dev, stream, K)
    if args.graph:
        res["graph_compare"] = graph_cmp
    if args.tokens:
        res["tokens"] = bench_tokens(pkv, W, torch, dev, stream, K)
    if not args.no_ceiling and not args.no_kernel_loop:
        res["read_ceiling"] = bench_ceiling(pkv, torch, dev, stream, K, call_bytes)
    if args.layers > 0:
        res["layered_step"] = bench_layers(pkv, torch, stream, K, batch, desc, base, args.layers,
                                           args.plan)
    if args.graph_buckets > 0:
        res["graph_buckets"] = bench_graph_buckets(pkv, W, torch, dev, K, args.graph_buckets)
    if args.mask_keep is not None:
        S = -(-int(batch.seq_lens.max()) // 4) * 4
        rng = np.random.default_rng(np.random.PCG64(2000 + args.config))
        mask = torch.from_numpy((rng.random((batch.B, S)) < args.mask_keep).astype(np.uint8)).to(dev)

        def masked_only(i):
            pool, q = copies[i % ncopies]
            pkv.pkv_decode_masked(pool, desc, q, mask, kv_indptr, idx, seq, batch.sm_scale, ws,
                                  out, stream)
        masked_ms = timed(stream, K, masked_only)
        res["masked"] = {"keep": args.mask_keep, "us_per_call": round(masked_ms * 1e3, 2),
                         "GBps": round((call_bytes + batch.B * S) / (masked_ms * 1e-3) / 1e9, 1)}
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)...", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(batch, args.cpu_seconds, cfg=args.config)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
