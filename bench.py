"""Split-KV paged decode-attention benchmark (one GPU).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 4]
                    [--block-size 16] [--v-layout plain] [--no-cpu-baseline]

A step is one pass of the whole hot path over one batch: the host planner
refreshes the plan from host-known context lengths and copies its metadata to
the device, then the partial kernel and the combine kernel run (the timed
step of aiter #5628 "tune MTP work budgets and planned reduction",
Performance: plan refresh, attention and reduction on every call). Inputs are
resident in HBM before timing starts. After W warm-up steps, K steps are
timed as a whole with no event on the stream (value, ms_per_step); a second
pass of K steps brackets each partial launch with HIP events (roofline), then
ten more steps the combine, K more with the plan left unchanged, and up to 50
steps each timed alone after a 1 GiB write has evicted the caches. Prints one
JSON line:

  value       effective TB/s = logical bytes / time per step, where logical
              bytes count Q and O, the valid K and V codes and their scales,
              the referenced page-table entries and the context lengths once
              (same page, Performance: the bandwidth note)
  roofline    the partial kernel: algorithmic bytes per launch (264 B per
              valid key per KV head for fp8 KV with two fp32 scales, i.e.
              2 D + 8) over its mean launch time from HIP events around each
              launch, against the 8 TB/s HBM peak; ``traffic`` is the HBM bytes
              per launch measured with rocprofv3 counters (FETCH_SIZE +
              WRITE_SIZE, scaled by a copy-kernel calibration) when a
              committed measurement for the current kernel source exists
  cpu_baseline  the fp64 oracle over every request of the workload, on one
              single-threaded worker process per host core (at most 16),
              as effective TB/s, with the single-core time and the CPU model
  copy_kernel  a 1 GiB device copy timed after the steps (bytes read plus
              written per second): what a plain streaming kernel reaches on
              this box, beside the published peak
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = ["skv_mfma.hip", "skv_device.h", "skv_internal.h", "skv_combine.hip"]


def logical_bytes(ctx, *, R: int, Hq: int, Hkv: int, D: int, q_bytes: int, kv_bytes: int,
                  quantized: bool, block_size: int, paged: bool = True) -> int:
    """Effective bytes of one decode call: Q and O once, valid K and V codes,
    their per-token per-KV-head fp32 scales, referenced page-table entries
    (int32, ceil(ctx / bs) per request) and the int32 context lengths."""
    B = len(ctx)
    n = sum(int(c) for c in ctx)
    qo = 2 * B * R * Hq * D * q_bytes
    kv = 2 * n * Hkv * D * kv_bytes
    sc = 2 * n * Hkv * 4 if quantized else 0
    pt = 4 * sum(-(-int(c) // block_size) for c in ctx) if paged else 0
    return qo + kv + sc + pt + 4 * B


_DT = {"f32": 4, "bf16": 2, "f16": 2, "int8": 1, "fp8": 1}


def spec_bytes(spec) -> int:
    return logical_bytes(spec.ctx, R=spec.R, Hq=spec.Hq, Hkv=spec.Hkv, D=spec.D,
                         q_bytes=_DT[spec.q_dtype], kv_bytes=_DT[spec.kv_dtype],
                         quantized=spec.kv_dtype in ("int8", "fp8"), block_size=spec.block_size)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "split_kv_flash_decode_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload_key: str):
    """HBM bytes per partial-kernel launch from a committed counter run, or None
    when there is none for this workload or the kernel source changed since."""
    path = os.path.join(PROFILES, "partial_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(workload_key)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return rec.get("hbm_bytes_per_launch")


def workload_name(spec) -> str:
    ctxs = sorted(set(spec.ctx))
    ctx_s = f"ctx {spec.ctx[0]}" if len(ctxs) == 1 else f"ctx {spec.ctx[0]}+{len(spec.ctx) - 1}x{spec.ctx[-1]}"
    return (f"B{spec.B} {ctx_s}, {'MTP' if spec.causal else 'R'}{spec.R} "
            f"{'causal' if spec.causal else ''}, Hq{spec.Hq}/Hkv{spec.Hkv}/D{spec.D}, "
            f"{spec.q_dtype} Q/O, {spec.kv_dtype} KV"
            f"{' + per-token fp32 scales' if spec.kv_dtype in ('int8', 'fp8') else ''}, "
            f"page {spec.block_size}, {spec.v_layout} V"
            + (f", {spec.partitions_per_request} partitions/request" if spec.partitions_per_request else
               ", planner partitions")
            + (f", window {spec.window}" if spec.window else "") + (", sinks" if spec.sinks else ""))


def copy_bandwidth(nbytes: int = 1 << 30, reps: int = 10) -> dict:
    """A plain device-to-device copy of ``nbytes`` on the same stream, timed
    with HIP events (median of three passes of ``reps`` copies): the box's own
    streaming rate beside the 8 TB/s peak, counting bytes read plus written."""
    import torch

    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    rates = []
    for _ in range(3):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            dst.copy_(src)
        e1.record()
        e1.synchronize()
        rates.append(2 * nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del src, dst
    torch.cuda.empty_cache()
    return {"GBps": round(sorted(rates)[1], 1), "bytes_per_copy": nbytes, "counted": "read + write",
            "frac_of_peak": round(sorted(rates)[1] / HBM_PEAK_GBS, 4)}


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


_ONE_THREAD_ENV = ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS", "BLIS_NUM_THREADS")


def _oracle_worker_init():
    """Worker set-up: one BLAS / OpenMP thread per worker process (the
    environment already says so; the limit is applied again once numpy's BLAS
    is loaded)."""
    import numpy  # noqa: F401  (loads the BLAS the limit applies to)
    import threadpoolctl

    threadpoolctl.threadpool_limits(1)
    import torch

    torch.set_num_threads(1)


def _worker_pid(_):
    time.sleep(0.05)
    return os.getpid()


def _oracle_request(task):
    """One request of the workload, built on this host core (seeded by request)
    and run through the fp64 oracle; returns (worker pid, oracle seconds,
    logical bytes). Only the oracle call is timed."""
    import oracle
    from skvgen import config_spec, make_problem

    config, spec_over, seed, b = task
    full = config_spec(config, **spec_over)
    spec = full.with_(ctx=(full.ctx[b],), B=1, name=f"{full.name}_req{b}")
    prob = make_problem(spec, seed=seed * 100003 + b, device="cpu")
    arrays = prob.host_arrays()
    t = time.perf_counter()
    oracle.decode_attention(arrays, R=spec.R, Hq=spec.Hq, Hkv=spec.Hkv, D=spec.D, causal=spec.causal,
                            window=spec.window, scale=spec.scale, q_dtype=spec.q_dtype,
                            kv_dtype=spec.kv_dtype, paged=True, block_size=spec.block_size,
                            v_layout=spec.v_layout, has_sink=spec.sinks)
    dt = time.perf_counter() - t
    return os.getpid(), dt, spec_bytes(spec)


def start_oracle_pool():
    """Worker processes for the CPU baseline, one per host core of this job's
    share (at most 16), started before this process touches the GPU (fresh
    interpreters, no GPU state inherited), each with one BLAS thread."""
    import multiprocessing as mp

    visible = len(os.sched_getaffinity(0))
    n = max(1, min(16, visible))
    saved = {k: os.environ.get(k) for k in _ONE_THREAD_ENV}
    for k in _ONE_THREAD_ENV:
        os.environ[k] = "1"
    try:
        pool = mp.get_context("spawn").Pool(n, initializer=_oracle_worker_init)
        # every worker has imported its modules before the GPU timing starts, so
        # their start-up does not compete with the timed steps for host cores
        pids = set()
        while len(pids) < n:
            pids.update(pool.map(_worker_pid, range(4 * n), chunksize=1))
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    return pool, n, visible


def cpu_baseline(pool, n_workers: int, visible: int, config: int, spec_over: dict, spec, seed: int,
                 budget_s: float = 90.0) -> dict:
    """The fp64 oracle over the requests of the workload, one request per task
    on ``n_workers`` single-threaded worker processes, until every request is
    done or ``budget_s`` of wall time has passed (the sample then says how
    many). ``value`` is the logical bytes of the requests done over the
    makespan of their oracle calls (the largest sum of oracle seconds any one
    worker spent); ``single_core_s`` is the sum over them (one core)."""
    t0 = time.perf_counter()
    res = []
    tasks = [(config, spec_over, seed, b) for b in range(spec.B)]
    for r in pool.imap_unordered(_oracle_request, tasks, chunksize=1):
        res.append(r)
        if len(res) % 16 == 0 or len(res) == spec.B:
            print(f"[bench] oracle: {len(res)} of {spec.B} requests, {time.perf_counter() - t0:.1f} s",
                  file=sys.stderr, flush=True)
        if time.perf_counter() - t0 > budget_s and len(res) < spec.B:
            pool.terminate()
            break
    wall = time.perf_counter() - t0
    per_worker = {}
    nbytes = 0
    for pid, dt, nb in res:
        per_worker[pid] = per_worker.get(pid, 0.0) + dt
        nbytes += nb
    makespan = max(per_worker.values())
    single = sum(dt for _, dt, _ in res)
    done = len(res)
    which = f"all {spec.B} requests" if done == spec.B else f"{done} of {spec.B} requests (wall-time cap)"
    return {
        "value": round(nbytes / makespan / 1e12, 6),
        "unit": "TB/s",
        "cores": n_workers,
        "kind": "oracle",
        "sample": (f"{which} of the workload, each built on the host (seeded per request) and run "
                   f"through the fp64 oracle once, on {n_workers} worker processes with one BLAS "
                   f"thread each; value = {nbytes} logical bytes / {makespan:.2f} s (largest per-worker "
                   f"oracle time)"),
        "us_per_step": round(makespan * 1e6 * spec.B / done, 1),
        "single_core_s": round(single, 3),
        "single_core_s_per_step": round(single * spec.B / done, 3),
        "wall_s_incl_input_build": round(wall, 2),
        "requests_done": done,
        "workers_used": len(per_worker),
        "host_cpus_visible": visible,
        "cpu_model": _cpu_model(),
    }


# Rows of the Performance table of aiter #5628 "tune MTP work budgets and
# planned reduction" (another implementation on the same GPU model; context,
# not the target): contexts, page size, V layout, the page's time per step in
# microseconds and its effective TB/s.
PAGE_TABLE = [
    ("B200, all 200000", 4, {}, 16, "plain", 2295.66, 4.607),
    ("B200, all 200000", 4, {}, 16, "transposed", 2332.80, 4.534),
    ("B200, all 200000", 4, {}, 128, "plain", 2325.20, 4.545),
    ("B200, all 200000", 4, {}, 128, "transposed", 2459.28, 4.297),
    ("B16, one 100000 + fifteen 1024", 5, {"ctx": (100000,) + (1024,) * 15}, 128, "transposed", 48.93, 0.633),
    ("B16, one 200000 + fifteen 1024", 5, {"ctx": (200000,) + (1024,) * 15}, 128, "transposed", 57.50, 0.998),
]


def make_step(spec, p, record_dtype: str = "f32", mode: str = "two_stage"):
    """The planned step of ``timed_steps`` on problem ``p``: returns
    (step(ev=None, refresh=True), plan, output tensor, resolved mode)."""
    import torch

    import split_kv_flash_decode_amd as skv

    dev = p.q.device
    o = torch.empty_like(p.q)
    d = skv.make_desc(p.q, p.k, p.v, paged=True, v_layout=spec.v_layout, causal=spec.causal,
                      window=spec.window, scale=spec.scale, page_table=p.page_table, has_sink=spec.sinks,
                      record_dtype=record_dtype)
    a = skv.make_args(p.q, p.k, p.v, p.ctx, o, k_scale=p.k_scale, v_scale=p.v_scale,
                      page_table=p.page_table, sinks=p.sinks, tree_mask=p.tree_mask)
    hints = skv.plan_hints_for(d, True, partitions_per_request=spec.partitions_per_request)
    host_ctx = list(spec.ctx)
    plan = skv.Plan(hints, host_ctx, dev)
    ws = skv.Workspace(d, plan.info.slots, dev)
    stream = torch.cuda.current_stream()
    counters = torch.zeros(spec.B * spec.Hkv, dtype=torch.int32, device=dev)
    if mode == "auto":
        mode = "host_plan" if plan.dev.numel() <= skv.SKV_PLAN_INLINE_MAX else "two_stage"
    host_meta = torch.empty(plan.dev.numel(), dtype=torch.int32)

    def step(ev=None, refresh=True):
        if mode == "host_plan":
            # the plan block goes to the kernels by value: no copy, one call
            if refresh:
                skv.plan_fill(plan.hints, host_ctx, plan.capacity, host_meta)
            if ev is not None:
                ev[0].record(stream)
            skv.attention_decode_paged_planned_host(d, a, host_meta, plan.capacity, ws)
            if ev is not None:
                ev[1].record(stream)
                if len(ev) > 2:
                    ev[2].record(stream)
            return
        if refresh:
            if mode == "device_plan":
                plan.refresh_device(p.ctx)
            else:
                plan.refresh(host_ctx)
        if ev is not None:
            ev[0].record(stream)
        if mode == "fused":
            skv.splitkv_fused(d, a, True, plan.capacity, ws, counters, plan_meta_dev=plan.dev)
            if ev is not None:
                ev[1].record(stream)
        else:
            skv.splitkv_partial(d, a, True, plan.capacity, ws, plan_meta_dev=plan.dev)
            if ev is not None:
                ev[1].record(stream)
            skv.splitkv_combine(d, a, plan.capacity, ws, plan_meta_dev=plan.dev)
        if ev is not None and len(ev) > 2:
            ev[2].record(stream)

    return step, plan, o, mode


def timed_steps(spec, seed: int, steps: int, warmup: int, record_dtype: str = "f32",
                mode: str = "two_stage", event_free_pass: bool = False, excl_plan_pass: bool = False,
                problem=None) -> dict:
    """Generate the workload (or take ``problem``), run the planned step (host
    plan refresh, metadata copy, partial, combine) ``warmup`` + ``steps`` times.

    ``mode`` "two_stage": host plan refresh, metadata copy, partial, combine;
    "host_plan": host plan refresh, then the planned call with the plan block
    passed to the kernels by value (no copy; its event time is reported as
    the partial time, combine 0); "auto": host_plan when the plan block fits
    the kernels' argument block, else two_stage; "fused": the single-kernel
    split + merge instead of partial + combine (its time is reported as the
    partial time, combine 0);
    "device_plan": the plan refreshed on the GPU from the device lengths
    instead of on the host. In the timed steps only the partial kernel is
    bracketed by events (each event record adds a few microseconds to the
    stream); the combine's time comes from a few extra steps afterwards.
    ``event_free_pass``: the time per step comes from a first timed pass
    without any event (on short steps even two records per step are a
    visible share), the kernel times from a second pass with events; a third
    pass times each step alone (events around the step) after a 1 GiB buffer
    write has pushed the inputs out of L2 and the 256 MB last-level cache
    (``cold_ms``, the median): the cache-cold time of workloads small enough
    to stay cache-resident between back-to-back steps.
    ``excl_plan_pass``: one more pass of ``steps`` steps with the plan left as
    it is (lengths unchanged): partial + combine only (``ms_excl_plan``).
    Returns a dict: ms (per step), part_ms, comb_ms (lists), plan, problem,
    cold_ms, ms_excl_plan (None when not measured)."""
    import torch

    from skvgen import make_problem

    dev = torch.device("cuda:0")
    p = problem if problem is not None else make_problem(spec, seed=seed, device=dev)
    torch.cuda.synchronize()
    step, plan, o, mode = make_step(spec, p, record_dtype, mode)
    stream = torch.cuda.current_stream()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    plain_ms = None
    if event_free_pass:
        t0 = time.perf_counter()
        for k in range(steps):
            step()
        torch.cuda.synchronize()
        plain_ms = (time.perf_counter() - t0) * 1e3 / steps
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        step(events[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    part_ms = [e[0].elapsed_time(e[1]) for e in events]
    extra = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(min(steps, 10))]
    for e in extra:
        step(e)
    torch.cuda.synchronize()
    comb_ms = [e[1].elapsed_time(e[2]) for e in extra]
    excl_ms = None
    if excl_plan_pass:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(steps):
            step(refresh=False)
        torch.cuda.synchronize()
        excl_ms = (time.perf_counter() - t0) * 1e3 / steps
    cold_ms = None
    if event_free_pass:
        flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        times = []
        for k in range(min(steps, 50)):
            flush.fill_(float(k))
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            step()
            e1.record(stream)
            e1.synchronize()
            times.append(e0.elapsed_time(e1))
        cold_ms = sorted(times)[len(times) // 2]
        del flush
    if mode == "host_plan":
        comb_ms = [0.0]                                  # part_ms holds the whole call
    return {"ms": plain_ms if event_free_pass else wall * 1e3 / steps, "part_ms": part_ms,
            "comb_ms": comb_ms, "plan": plan, "problem": p, "cold_ms": cold_ms, "ms_excl_plan": excl_ms,
            "output": o, "mode": mode}


def rotated_step_ms(spec, seed: int, mode: str = "auto", sets: int = 3, iters: int = 101, runs: int = 3) -> float:
    """The timing method of the planned-reduction page's Performance setup:
    ``sets`` independently allocated copies of the workload (their own inputs,
    plans and workspaces), rotated from one iteration to the next so that
    consecutive steps do not find each other's data in the caches; ``runs``
    runs of ``iters`` iterations, each timed as a whole with HIP events; the
    median of the runs' mean step times (ms)."""
    import statistics

    import torch

    from skvgen import make_problem

    dev = torch.device("cuda:0")
    probs = [make_problem(spec, seed=seed + 1000 * k, device=dev) for k in range(sets)]
    steps = [make_step(spec, p, "f32", mode)[0] for p in probs]
    torch.cuda.synchronize()
    for k in range(2 * sets):                        # warm-up of every set
        steps[k % sets]()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    res = []
    for _ in range(runs):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for k in range(iters):
            steps[k % sets]()
        e1.record(stream)
        e1.synchronize()
        res.append(e0.elapsed_time(e1) / iters)
    del probs, steps
    torch.cuda.empty_cache()
    return statistics.median(res)


def table(args) -> int:
    import torch

    from skvgen import config_spec

    for name, n, over, bs, vl, page_us, page_tbs in PAGE_TABLE:
        spec = config_spec(n, block_size=bs, v_layout=vl, **over)
        small = max(spec.ctx) * spec.B < 10_000_000
        steps, warmup = (400, 50) if small else (args.steps, args.warmup)
        r = timed_steps(spec, n, steps, warmup, event_free_pass=True, mode="auto")
        ms, part_ms, comb_ms, plan, p, cold_ms = r["ms"], r["part_ms"], r["comb_ms"], r["plan"], r["problem"], r["cold_ms"]
        tbs = spec_bytes(spec) / (ms * 1e-3) / 1e12
        step_mode, items = r["mode"], plan.info.num_items
        del p, r, plan
        torch.cuda.empty_cache()
        rot_ms = rotated_step_ms(spec, n)
        print(json.dumps({"row": f"{name}, page {bs}, {vl} V", "us_per_step": round(ms * 1e3, 2),
                          "effective_TBps": round(tbs, 3),
                          "us_per_step_cache_cold": round(cold_ms * 1e3, 2),
                          "effective_TBps_cache_cold": round(spec_bytes(spec) / (cold_ms * 1e-3) / 1e12, 3),
                          "us_per_step_page_method": round(rot_ms * 1e3, 2),
                          "effective_TBps_page_method": round(spec_bytes(spec) / (rot_ms * 1e-3) / 1e12, 3),
                          "page_us_per_step": page_us,
                          "page_TBps": page_tbs, "time_vs_page": round(ms * 1e3 / page_us, 4),
                          "time_vs_page_page_method": round(rot_ms * 1e3 / page_us, 4),
                          "partial_us_mean": round(sum(part_ms) / len(part_ms) * 1e3, 2),
                          "combine_us_mean": round(sum(comb_ms) / len(comb_ms) * 1e3, 2),
                          "plan_items": items, "step_mode": step_mode,
                          "steps": steps, "warmup": warmup}), flush=True)
    return 0


# The adjacent variants built beside the default path, each timed with the
# same step on a full-size workload and set against the same workload's
# default call: (row, config, spec overrides, record dtype, step mode).
NEXT_ROWS = [
    ("B200x200k fp8 MTP4 (default call)", 4, {}, "f32", "auto"),
    ("fp16 Q/O", 4, {"q_dtype": "f16"}, "f32", "auto"),
    ("bf16 partial records", 4, {}, "bf16", "auto"),
    ("single-kernel split + merge", 4, {}, "f32", "fused"),
    ("device-side plan refresh", 4, {}, "f32", "device_plan"),
    ("MTP4 rows under a random tree mask", 4, {"verify": "tree"}, "f32", "auto"),
    ("int8 verifier R16 (default call)", 3, {}, "f32", "auto"),
    ("int8 verifier, two-stage call with the plan copied to the device", 3, {}, "f32", "two_stage"),
    ("int8 verifier, single-kernel split + merge", 3, {}, "f32", "fused"),
    ("int8 verifier, device-side plan refresh", 3, {}, "f32", "device_plan"),
    ("int8 verifier, random tree mask", 3, {"verify": "tree"}, "f32", "auto"),
    ("int8 verifier, independent-batch mask", 3, {"verify": "independent"}, "f32", "auto"),
    ("int8 verifier, fp16 Q/O", 3, {"q_dtype": "f16"}, "f32", "auto"),
    ("mixed batch one 200000 + fifteen 1024 (default call)", 5, {}, "f32", "auto"),
    ("mixed batch, the long request at index 9 of 16", 5, {"ctx": (1024,) * 9 + (200000,) + (1024,) * 6}, "f32",
     "auto"),
    ("mixed batch, single-kernel split + merge", 5, {}, "f32", "fused"),
    ("mixed batch, device-side plan refresh", 5, {}, "f32", "device_plan"),
]


def next_rows(args) -> int:
    import torch

    from skvgen import config_spec

    base = {}
    for name, n, over, rec, mode in NEXT_ROWS:
        spec = config_spec(n, **over)
        small = max(spec.ctx) * spec.B < 10_000_000
        steps, warmup = (400, 50) if small else (args.steps, args.warmup)
        r = timed_steps(spec, n, steps, warmup, record_dtype=rec, mode=mode, event_free_pass=True)
        ms, part_ms, comb_ms, plan, p, cold_ms = r["ms"], r["part_ms"], r["comb_ms"], r["plan"], r["problem"], r["cold_ms"]
        part_us = sum(part_ms) / len(part_ms) * 1e3
        unit_bytes = 2 * spec.D * _DT[spec.kv_dtype] + (8 if spec.kv_dtype in ("int8", "fp8") else 0)
        alg = unit_bytes * sum(int(c) for c in spec.ctx) * spec.Hkv
        row = {"row": name, "workload": workload_name(spec), "us_per_step": round(ms * 1e3, 2),
               "us_per_step_cache_cold": round(cold_ms * 1e3, 2),
               "effective_TBps": round(spec_bytes(spec) / (ms * 1e-3) / 1e12, 3),
               "partial_us_mean": round(part_us, 2),
               "combine_us_mean": round(sum(comb_ms) / len(comb_ms) * 1e3, 2),
               "partial_roofline_frac": round(alg / (part_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
               "step_mode": r["mode"], "steps": steps, "warmup": warmup}
        if r["mode"] == "host_plan":
            row["note"] = "partial_us_mean is the whole planned call (partial + combine)"
        if mode == "fused":
            row["note"] = "partial_us_mean is the fused kernel (split + merge)"
        if n not in base:
            base[n] = ms
        else:
            row["time_vs_default_call"] = round(ms / base[n], 4)
        print(json.dumps(row), flush=True)
        del p
        torch.cuda.empty_cache()
    return 0


def timed_uniform(spec, S: int, seed: int, steps: int, warmup: int, problem=None) -> dict:
    """The uniform-split call (skv_attention_decode_paged_splitkv with S
    splits, or skv_attention_decode_splitkv for a problem laid out
    contiguously: partial + combine, no plan) timed like ``timed_steps``: a
    pass without events (warm), then each call alone after a 1 GiB write
    (cold)."""
    import torch

    import split_kv_flash_decode_amd as skv
    from skvgen import make_problem

    dev = torch.device("cuda:0")
    p = problem if problem is not None else make_problem(spec, seed=seed, device=dev)
    o = torch.empty_like(p.q)
    d = skv.make_desc(p.q, p.k, p.v, paged=p.paged, v_layout=spec.v_layout, causal=spec.causal,
                      window=spec.window, scale=spec.scale, page_table=p.page_table, has_sink=spec.sinks)
    a = skv.make_args(p.q, p.k, p.v, p.ctx, o, k_scale=p.k_scale, v_scale=p.v_scale,
                      page_table=p.page_table, sinks=p.sinks)
    ws = skv.Workspace(d, skv.uniform_slots(d, S), dev)
    stream = torch.cuda.current_stream()
    split_call = skv.attention_decode_paged_splitkv if p.paged else skv.attention_decode_splitkv

    def call():
        split_call(d, a, S, ws)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        call()
    torch.cuda.synchronize()
    warm = (time.perf_counter() - t0) * 1e3 / steps
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    times = []
    for k in range(min(steps, 50)):
        flush.fill_(float(k))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        call()
        e1.record(stream)
        e1.synchronize()
        times.append(e0.elapsed_time(e1))
    del flush
    return {"ms": warm, "cold_ms": sorted(times)[len(times) // 2], "problem": p}


def all_configs(args) -> int:
    """One JSON line per (workload, split mode): the five workloads with the
    planner step, plus the uniform split counts the single-request and the
    verifier workloads name. Warm: back-to-back steps without events; cold:
    each step alone after a 1 GiB write; excl_plan: partial + combine only."""
    import torch

    from skvgen import config_spec

    for n in (1, 2, 3, 4, 5):
        spec = config_spec(n)
        small = max(spec.ctx) * spec.B < 10_000_000
        steps, warmup = (400, 50) if small else (args.steps, args.warmup)
        nbytes = spec_bytes(spec)
        unit_bytes = 2 * spec.D * _DT[spec.kv_dtype] + (8 if spec.kv_dtype in ("int8", "fp8") else 0)
        alg = unit_bytes * sum(int(c) for c in spec.ctx) * spec.Hkv
        r = timed_steps(spec, n, steps, warmup, event_free_pass=True, excl_plan_pass=True, mode="auto")
        part_us = sum(r["part_ms"]) / len(r["part_ms"]) * 1e3
        row = {"config": n, "workload": workload_name(spec), "mode": f"planner ({r['mode']})",
               "plan_items": r["plan"].info.num_items, "logical_bytes": nbytes,
               "us_per_step_warm": round(r["ms"] * 1e3, 2),
               "us_per_step_cold": round(r["cold_ms"] * 1e3, 2),
               "us_per_step_excl_plan": round(r["ms_excl_plan"] * 1e3, 2),
               "TBps_warm": round(nbytes / (r["ms"] * 1e-3) / 1e12, 4),
               "TBps_cold": round(nbytes / (r["cold_ms"] * 1e-3) / 1e12, 4),
               "frac_warm": round(nbytes / (r["ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
               "frac_cold": round(nbytes / (r["cold_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
               "partial_us_mean": round(part_us, 2),
               "combine_us_mean": round(sum(r["comb_ms"]) / len(r["comb_ms"]) * 1e3, 2),
               "partial_roofline_frac": round(alg / (part_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
               "steps": steps, "warmup": warmup}
        print(json.dumps(row), flush=True)
        p = r["problem"]
        for S in (spec.splits or ()):
            u = timed_uniform(spec, S, n, steps, warmup, problem=p)
            print(json.dumps({"config": n, "workload": workload_name(spec), "mode": f"uniform S={S}",
                              "us_per_step_warm": round(u["ms"] * 1e3, 2),
                              "us_per_step_cold": round(u["cold_ms"] * 1e3, 2),
                              "TBps_warm": round(nbytes / (u["ms"] * 1e-3) / 1e12, 4),
                              "TBps_cold": round(nbytes / (u["cold_ms"] * 1e-3) / 1e12, 4),
                              "frac_warm": round(nbytes / (u["ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                              "frac_cold": round(nbytes / (u["cold_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                              "steps": steps, "warmup": warmup}), flush=True)
        if n == 1:
            # the single request also as a contiguous cache (no page table)
            from skvgen import to_contiguous
            c = to_contiguous(p)
            cbytes = logical_bytes(spec.ctx, R=spec.R, Hq=spec.Hq, Hkv=spec.Hkv, D=spec.D, q_bytes=_DT[spec.q_dtype],
                                   kv_bytes=_DT[spec.kv_dtype], quantized=spec.kv_dtype in ("int8", "fp8"),
                                   block_size=spec.block_size, paged=False)
            for S in (spec.splits or ()):
                u = timed_uniform(spec, S, n, steps, warmup, problem=c)
                print(json.dumps({"config": n, "workload": workload_name(spec).replace("page 16, ", "contiguous, "),
                                  "mode": f"uniform S={S}",
                                  "us_per_step_warm": round(u["ms"] * 1e3, 2),
                                  "us_per_step_cold": round(u["cold_ms"] * 1e3, 2),
                                  "TBps_warm": round(cbytes / (u["ms"] * 1e-3) / 1e12, 4),
                                  "TBps_cold": round(cbytes / (u["cold_ms"] * 1e-3) / 1e12, 4),
                                  "frac_warm": round(cbytes / (u["ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                  "frac_cold": round(cbytes / (u["cold_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                  "steps": steps, "warmup": warmup}), flush=True)
            del c
        del r, p
        torch.cuda.empty_cache()
    return 0


def ceiling(args) -> int:
    """The partial kernel against the read-only gather with its memory pattern
    (skv_gather_ceiling) on the same workload and plan, interleaved in one
    process: HIP events around batches of launches of each, means per launch,
    as algorithmic bytes per second and as a fraction of 8 TB/s. The gather's
    rate is what this paged layout allows the partial kernel's loads."""
    import statistics

    import torch

    import split_kv_flash_decode_amd as skv
    from skvgen import config_spec, make_problem

    over = {}
    if args.block_size:
        over["block_size"] = args.block_size
    if args.v_layout:
        over["v_layout"] = args.v_layout
    spec = config_spec(args.config, **over)
    dev = torch.device("cuda:0")
    p = make_problem(spec, seed=args.seed, device=dev)
    o = torch.empty_like(p.q)
    d = skv.make_desc(p.q, p.k, p.v, paged=True, v_layout=spec.v_layout, causal=spec.causal,
                      window=spec.window, scale=spec.scale, page_table=p.page_table, has_sink=spec.sinks)
    a = skv.make_args(p.q, p.k, p.v, p.ctx, o, k_scale=p.k_scale, v_scale=p.v_scale,
                      page_table=p.page_table, sinks=p.sinks)
    hints = skv.plan_hints_for(d, True, partitions_per_request=spec.partitions_per_request)
    plan = skv.Plan(hints, list(spec.ctx), dev)
    ws = skv.Workspace(d, plan.info.slots, dev)
    sink = torch.empty(plan.capacity * spec.Hkv, dtype=torch.int32, device=dev)

    def part():
        skv.splitkv_partial(d, a, True, plan.capacity, ws, plan_meta_dev=plan.dev)

    def gath():
        skv.gather_ceiling(d, a, plan.capacity, sink, plan_meta_dev=plan.dev)

    inner = max(1, args.steps // 10)
    for _ in range(args.warmup):
        part()
        gath()
    torch.cuda.synchronize()
    t = {"partial": [], "gather": []}
    for _ in range(10):
        for name, fn in (("partial", part), ("gather", gath)):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(inner):
                fn()
            e1.record()
            e1.synchronize()
            t[name].append(e0.elapsed_time(e1) * 1e3 / inner)
    unit_bytes = 2 * spec.D * _DT[spec.kv_dtype] + (8 if spec.kv_dtype in ("int8", "fp8") else 0)
    alg = unit_bytes * sum(int(c) for c in spec.ctx) * spec.Hkv
    row = {"workload": workload_name(spec), "algorithmic_bytes_per_launch": alg, "launches_each": 10 * inner}
    for name in ("partial", "gather"):
        us = statistics.mean(t[name])
        row[f"{name}_us_mean"] = round(us, 2)
        row[f"{name}_us_median"] = round(statistics.median(t[name]), 2)
        row[f"{name}_GBps"] = round(alg / (us * 1e-6) / 1e9, 1)
        row[f"{name}_frac_of_8TBps"] = round(alg / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
    row["partial_share_of_gather_ceiling"] = round(row["gather_us_mean"] / row["partial_us_mean"], 4)
    print(json.dumps(row), flush=True)
    return 0


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--config", type=int, default=4)
    ap.add_argument("--block-size", type=int, default=0)
    ap.add_argument("--v-layout", default="")
    ap.add_argument("--seed", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run 1 GiB device-to-device copies (counter calibration)")
    ap.add_argument("--table", action="store_true",
                    help="time the six rows of the planned-reduction page's Performance table "
                         "(one JSON line per row: back to back, cache-cold, and with the page's own "
                         "method of three rotated allocation sets; the page's time beside ours)")
    ap.add_argument("--next", action="store_true",
                    help="time the adjacent variants (fp16 Q/O, bf16 records, fused call, device "
                         "plan refresh, verify masks) against the default call on the same workloads")
    ap.add_argument("--ceiling", action="store_true",
                    help="time the partial kernel against the read-only gather with its memory pattern "
                         "(skv_gather_ceiling) on the same workload, interleaved")
    ap.add_argument("--all", action="store_true",
                    help="per-workload table: the five workloads (planner step) and the uniform split "
                         "counts they name, warm / cache-cold / plan-excluded time per step")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path needs no collectives: requests and KV heads shard without exchange)",
              file=sys.stderr)
        return 2

    side_mode = args.calibrate_copy or args.next or args.table or args.all or args.ceiling
    pool = None
    if not side_mode and not args.no_cpu_baseline:
        # the oracle's worker processes start before anything touches the GPU
        pool, n_workers, visible = start_oracle_pool()

    import torch

    from skvgen import config_spec

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.calibrate_copy:
        # A plain copy of known size: rocprofv3 FETCH_SIZE / WRITE_SIZE of these
        # dispatches give the counter-to-bytes factor used for ``traffic``.
        n = 1 << 28                                     # 2^28 fp32 = 1 GiB
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": 4 * n, "copies": 3}), flush=True)
        return 0
    if args.next:
        return next_rows(args)
    if args.table:
        return table(args)
    if args.all:
        return all_configs(args)
    if args.ceiling:
        return ceiling(args)
    overrides = {}
    if args.block_size:
        overrides["block_size"] = args.block_size
    if args.v_layout:
        overrides["v_layout"] = args.v_layout
    spec = config_spec(args.config, **overrides)
    print(f"[bench] generating {spec.name} on cuda:0 and timing ...", file=sys.stderr, flush=True)
    t = time.time()
    r = timed_steps(spec, args.seed, args.steps, args.warmup, event_free_pass=True, excl_plan_pass=True)
    ms_per_step, part_ms, comb_ms, plan = r["ms"], r["part_ms"], r["comb_ms"], r["plan"]
    ms_excl_plan, ms_cold = r["ms_excl_plan"], r["cold_ms"]
    print(f"[bench] done in {time.time() - t:.1f} s", file=sys.stderr, flush=True)
    del r
    nbytes = spec_bytes(spec)
    tbs = nbytes / (ms_per_step * 1e-3) / 1e12

    unit_bytes = 2 * spec.D * _DT[spec.kv_dtype] + (8 if spec.kv_dtype in ("int8", "fp8") else 0)
    units = sum(int(c) for c in spec.ctx) * spec.Hkv
    alg_bytes = unit_bytes * units
    part_mean = sum(part_ms) / len(part_ms)
    achieved = alg_bytes / (part_mean * 1e-3) / 1e9
    key = f"cfg{args.config}_bs{spec.block_size}_{spec.v_layout}"
    traffic = measured_traffic(key)
    fp8_scores = spec.kv_dtype == "fp8" and spec.q_dtype == "bf16"

    result = {
        "metric": "decode-attention us/step + effective KV TB/s (fraction of HBM peak)",
        "value": round(tbs, 4),
        "unit": "TB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "us_per_step": round(ms_per_step * 1e3, 2),
        "us_per_step_excl_plan": round(ms_excl_plan * 1e3, 2),
        "us_per_step_cache_cold": round(ms_cold * 1e3, 2),
        "hbm_fraction": round(tbs * 1e3 / HBM_PEAK_GBS, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(tbs / 4.607, 4) if (args.config == 4 and spec.block_size == 16
                                                 and spec.v_layout == "plain") else None,
        "dtype": "fp8+bf16" if fp8_scores else spec.q_dtype,
        "dtype_detail": ("scores Q.K^T on the fp8 matrix cores (e4m3 K codes, bf16 Q split into two "
                         "e4m3 parts with power-of-two block scales), P.V on the bf16 matrix cores, "
                         "softmax and accumulation in fp32, bf16 output"
                         if fp8_scores else f"{spec.q_dtype} Q/O, {spec.kv_dtype} KV, fp32 accumulation"),
        "data": "synthetic",
        "config": {
            "workload": workload_name(spec),
            "global_batch": spec.B,
            "seq_len": max(spec.ctx),
            "parallelism": "none (one GPU)",
            "logical_bytes_per_step": nbytes,
            "plan_items": plan.info.num_items,
            "plan_capacity": plan.capacity,
            "partial_us_mean": round(part_mean * 1e3, 2),
            "combine_us_mean": round(sum(comb_ms) / len(comb_ms) * 1e3, 2),
            "timing": ("value and ms_per_step: wall clock over the timed steps (no event on the "
                       "stream), each a host plan refresh + metadata copy + partial + combine; kernel "
                       "times: HIP events around each partial launch in a second pass of as many "
                       "steps (and around the combine in ten more); us_per_step_excl_plan: the same "
                       "number of steps with the plan left unchanged (partial + combine only); "
                       "us_per_step_cache_cold: median of steps timed alone, each after a 1 GiB "
                       "write evicts L2 and the last-level cache"),
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
        },
        "cpu_baseline": None,
    }
    result["copy_kernel"] = copy_bandwidth()
    if pool is not None:
        print("[bench] timing the fp64 oracle on host cores ...", file=sys.stderr, flush=True)
        try:
            result["cpu_baseline"] = cpu_baseline(pool, n_workers, visible, args.config, overrides, spec,
                                                  args.seed)
        finally:
            pool.close()
            pool.join()
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
