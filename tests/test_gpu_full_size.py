"""GPU parity at the workloads' full sizes, in the launch configuration that
``bench.py`` times (host plan -> metadata copy -> partial -> combine).

The fp64 oracle checks whole requests one at a time: every request where the
oracle is quick (configs 2 and 3), sampled requests otherwise (config 4: the
first, a middle and the last of 200 requests of 200,000 keys; config 5: the
200,000-key request and two 1,024-key ones). Each sampled request is copied to
the host with only the pages its table row references. Same tolerance as the
reduced-shape tests: |d| <= 5e-3 + 5e-3 |ref|, rel-L2 <= 1e-2, row cosine >=
0.9999. Scratch records start NaN-filled, so a record the combine reads but no
partial wrote shows up as NaN. The uniform split counts the workloads name
(single request 1, 2, 4, 8; verifier 2, 4, 8) run at full size too, whole
output, both kernel families. So do the adjacent variants ``bench.py --next``
times (fp16 Q/O, bf16 records, verify masks, the device plan refresh), in
that same step, on the same samples; bf16 records add the bound of their own
rounding (2^-8 times the oracle's output on |V|). The other three B200 rows
of the planned-reduction page's Performance table (page 128, transposed V),
the mixed batch with a 4096-key window and sinks, and the mixed batch with
its long request in the middle of the batch run here as well.
"""

from __future__ import annotations

import gc
import json
import os

import pytest
import torch

from skvgen import config_spec, extract_request, make_problem
from tests.gpu_run import bench_step, run, to_f64
from tests.helpers import compare, oracle_abs_value_output, oracle_output

pytestmark = pytest.mark.gpu

SAMPLES = {2: None, 3: None, 4: (0, 97, 199), 5: (0, 1, 15)}


def _samples(n, spec):
    """Requests checked: SAMPLES, except that the mixed batch always checks
    its long request (wherever it sits), the one after it and the last."""
    if n != 5:
        return SAMPLES[n] or range(spec.B)
    long_b = max(range(spec.B), key=lambda i: spec.ctx[i])
    return sorted({long_b, (long_b + 1) % spec.B, spec.B - 1})


def _record(name, b, ctx, st):
    """Append one request's error statistics to $SKV_ACCURACY_OUT (JSON lines),
    when that variable names a file: the per-workload accuracy summary."""
    path = os.environ.get("SKV_ACCURACY_OUT")
    if not path:
        return
    with open(path, "a") as f:
        f.write(json.dumps({"workload": name, "request": int(b), "ctx": int(ctx), **st}) + "\n")


@pytest.mark.parametrize("n", [2, 3, 4, 5])
def test_full_size_bench_step_matches_oracle(n):
    spec = config_spec(n)
    print(f"[full cfg{n}] {spec.name}: B {spec.B}, keys {sum(spec.ctx)}", flush=True)
    p = make_problem(spec, seed=4, device="cuda")
    o, ws, plan = bench_step(p, ws_fill=float("nan"))
    out = to_f64(o)
    reqs = _samples(n, spec)
    try:
        for b in reqs:
            sub = extract_request(p, b)
            ref = oracle_output(sub)[0]
            st = compare(out[b], ref, "lowp")
            print(f"[full cfg{n} request {b} ctx {spec.ctx[b]}] {st}", flush=True)
            _record(f"cfg{n}", b, spec.ctx[b], st)
            assert st["ok"], (n, b, st)
    finally:
        del p, o, ws, plan
        gc.collect()
        torch.cuda.empty_cache()


@pytest.mark.parametrize("n", [3, 4, 5])
def test_full_size_run_to_run_bitwise(n):
    """At full size, the single-pass call (num_splits = 1) and the planned
    step each give the same bits twice in a row, and the planned step's whole
    output matches the single pass within the workload tolerance (any split
    count equals the single pass)."""
    spec = config_spec(n)
    p = make_problem(spec, seed=5, device="cuda")
    try:
        a, _, _ = run(p, "single")
        a = a.clone()
        b, _, _ = run(p, "single")
        same = torch.equal(a, b)
        print(f"[full cfg{n}] single pass twice: bitwise {same}", flush=True)
        assert same, n
        s1, _, _ = bench_step(p, ws_fill=float("nan"))
        s1 = s1.clone()
        s2, _, _ = bench_step(p, ws_fill=float("nan"))
        same = torch.equal(s1, s2)
        print(f"[full cfg{n}] planned step twice: bitwise {same}", flush=True)
        assert same, n
        st = compare(to_f64(s1), to_f64(a), "lowp")
        print(f"[full cfg{n}] planned step vs single pass: {st}", flush=True)
        assert st["ok"], (n, st)
    finally:
        del p
        gc.collect()
        torch.cuda.empty_cache()


@pytest.mark.parametrize("n,S", [(1, 1), (1, 2), (1, 4), (1, 8), (3, 2), (3, 4), (3, 8)])
def test_full_size_uniform_split_counts(n, S):
    """The split counts the workloads name (single request: 1, 2, 4, 8;
    verifier: 2, 4, 8) at full size, both kernel families, whole output."""
    from tests.gpu_run import run
    spec = config_spec(n)
    p = make_problem(spec, seed=40 + S, device="cuda")
    ref = oracle_output(p)
    impls = ["valu"] if spec.q_dtype == "f32" else ["valu", "mfma"]
    for impl in impls:
        o, _, _ = run(p, "split", num_splits=S, impl=impl, ws_fill=float("nan"))
        st = compare(to_f64(o), ref, "f32" if spec.kv_dtype == "f32" else "lowp")
        print(f"[full cfg{n} S={S} {impl}] {st}", flush=True)
        _record(f"cfg{n}_S{S}_{impl}", 0, spec.ctx[0], st)
        assert st["ok"], (n, S, impl, st)


VARIANTS = [
    # the other three B200 rows of the planned-reduction page's Performance table
    ("cfg4_bs128_plain", 4, {"block_size": 128}, "f32", False),
    ("cfg4_bs16_transposed", 4, {"v_layout": "transposed"}, "f32", False),
    ("cfg4_bs128_transposed", 4, {"block_size": 128, "v_layout": "transposed"}, "f32", False),
    # the mixed batch with the 4096-key sliding window and per-head sinks
    ("cfg5_window4096_sinks", 5, {"window": 4096, "sinks": True}, "f32", False),
    # the mixed batch with its long request in the middle of the batch
    ("cfg5_long_at_9", 5, {"ctx": (1024,) * 9 + (200000,) + (1024,) * 6}, "f32", False),
    # sharp queries (Q x 8, |O| ~ 1): where the 5e-3 relative bound bites at full size
    ("cfg4_sharp", 4, {"q_mult": 8.0}, "f32", False),
    ("cfg3_sharp", 3, {"q_mult": 8.0}, "f32", False),
    ("cfg5_sharp_window4096_sinks", 5, {"q_mult": 8.0, "window": 4096, "sinks": True}, "f32", False),
    ("cfg4_f16", 4, {"q_dtype": "f16"}, "f32", False),
    ("cfg4_bf16_records", 4, {}, "bf16", False),
    ("cfg4_tree_mask", 4, {"verify": "tree"}, "f32", False),
    ("cfg4_device_plan", 4, {}, "f32", True),
    ("cfg3_tree_mask", 3, {"verify": "tree"}, "f32", False),
    ("cfg3_independent_mask", 3, {"verify": "independent"}, "f32", False),
    ("cfg3_f16", 3, {"q_dtype": "f16"}, "f32", False),
    ("cfg3_bf16_records_device_plan", 3, {}, "bf16", True),
]


@pytest.mark.parametrize("name,n,over,rec,dev_plan", VARIANTS, ids=[v[0] for v in VARIANTS])
def test_full_size_variant_rows_match_oracle(name, n, over, rec, dev_plan):
    spec = config_spec(n, **over)
    print(f"[full {name}] {spec.name}: B {spec.B}, keys {sum(spec.ctx)}", flush=True)
    p = make_problem(spec, seed=14, device="cuda")
    o, ws, plan = bench_step(p, ws_fill=float("nan"), record_dtype=rec, device_plan=dev_plan)
    assert o.dtype == p.q.dtype
    out = to_f64(o)
    try:
        for b in _samples(n, spec):
            sub = extract_request(p, b)
            extra = 2.0 ** -8 * oracle_abs_value_output(sub)[0] if rec == "bf16" else None
            st = compare(out[b], oracle_output(sub)[0], "lowp", extra=extra)
            print(f"[full {name} request {b} ctx {spec.ctx[b]}] {st}", flush=True)
            _record(name, b, spec.ctx[b], st)
            assert st["ok"], (name, b, st)
    finally:
        del p, o, ws, plan
        gc.collect()
        torch.cuda.empty_cache()
