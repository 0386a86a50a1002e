"""Single-kernel split + merge (skv_splitkv_fused) against the two-stage call.

The last workgroup of each (request, KV head) merges that pair's records in
increasing split order with the combine kernel's arithmetic, so the output
must be bit-identical to skv_splitkv_partial + skv_splitkv_combine whichever
workgroup arrives last. Covered: every workload family at reduced shapes,
uniform splits and the planner, both kernel families, windows and sinks,
empty requests; the arrival counters must read zero after every call; the
fused call captured in a HIP graph and replayed with new device-side lengths;
and the full-size B200 x 200k workload in the launch configuration bench.py
times.
"""

from __future__ import annotations

import pytest
import torch

import split_kv_flash_decode_amd as skv
from skvgen import config_spec, make_problem, small_spec
from tests.gpu_run import desc_args, to_f64
from tests.helpers import compare, oracle_output

pytestmark = pytest.mark.gpu


def _bits(o: torch.Tensor) -> torch.Tensor:
    return o.view(torch.int16) if o.dtype == torch.bfloat16 else o.view(torch.int32)


def _plan(spec, device, ctx=None):
    ph = skv.plan_hints(spec.B, spec.R, spec.Hkv, causal=spec.causal, window=spec.window,
                        partitions_per_request=spec.partitions_per_request)
    base = [int(c) for c in (spec.ctx if ctx is None else ctx)]
    plan = skv.Plan(ph, base, device)
    plan.refresh(base)
    torch.cuda.synchronize()
    return plan


def _run_both(p, impl, num_splits=None):
    """(two-stage output, fused output, counters after the fused call)."""
    s = p.spec
    d, a, o = desc_args(p, impl)
    if num_splits is None:
        plan = _plan(s, p.device)
        n, meta, slots = plan.capacity, plan.dev, plan.info.slots
    else:
        n, meta, slots = num_splits, None, skv.uniform_slots(d, num_splits)
    ws = skv.Workspace(d, slots, p.device, fill=float("nan"))
    o.fill_(float("nan"))
    skv.splitkv_partial(d, a, True, n, ws, plan_meta_dev=meta)
    skv.splitkv_combine(d, a, n, ws, plan_meta_dev=meta)
    torch.cuda.synchronize()
    two = o.clone()
    counters = torch.zeros(s.B * s.Hkv, dtype=torch.int32, device=p.device)
    ws2 = skv.Workspace(d, slots, p.device, fill=float("nan"))
    o.fill_(float("nan"))
    skv.splitkv_fused(d, a, True, n, ws2, counters, plan_meta_dev=meta)
    torch.cuda.synchronize()
    return two, o.clone(), counters


CASES = [
    ("cfg1", lambda: small_spec(1), "valu", 4),
    ("cfg2", lambda: small_spec(2), "auto", None),
    ("cfg2_valu", lambda: small_spec(2), "valu", 3),
    ("cfg3", lambda: small_spec(3), "auto", 8),
    ("cfg3_planned", lambda: small_spec(3), "auto", None),
    ("cfg4", lambda: small_spec(4), "auto", None),
    ("cfg4_s1", lambda: small_spec(4), "auto", 1),
    ("cfg4_s16", lambda: small_spec(4), "auto", 16),
    ("cfg4_t128", lambda: small_spec(4, block_size=128, v_layout="transposed"), "auto", None),
    ("cfg5_window_sinks", lambda: small_spec(5, window=500, sinks=True), "auto", None),
    ("cfg5_empty", lambda: small_spec(5, ctx=(6000, 0, 1, 300)), "auto", None),
    ("cfg4_bf16_valu", lambda: small_spec(4, kv_dtype="bf16"), "valu", 5),
]


@pytest.mark.parametrize("name,mk,impl,S", CASES, ids=[c[0] for c in CASES])
def test_fused_is_bit_identical_to_two_stage(name, mk, impl, S):
    spec = mk()
    p = make_problem(spec, seed=31, device="cuda")
    two, fused, counters = _run_both(p, impl, S)
    assert not torch.isnan(fused).any(), name
    assert torch.equal(_bits(fused), _bits(two)), f"{name}: fused != two-stage"
    assert int(counters.abs().sum()) == 0, f"{name}: counters not reset"
    st = compare(to_f64(fused), oracle_output(p), "f32" if spec.kv_dtype == "f32" else "lowp")
    assert st["ok"], (name, st)
    print(f"[fused {name}] bitwise equal to two-stage; {st}", flush=True)


def test_fused_repeats_and_counters_stay_zero():
    spec = small_spec(4, ctx=(3001, 1500, 71), partitions_per_request=4)
    p = make_problem(spec, seed=32, device="cuda")
    d, a, o = desc_args(p)
    plan = _plan(spec, p.device)
    ws = skv.Workspace(d, plan.info.slots, p.device)
    counters = torch.zeros(spec.B * spec.Hkv, dtype=torch.int32, device=p.device)
    outs = []
    for _ in range(4):
        o.fill_(float("nan"))
        skv.splitkv_fused(d, a, True, plan.capacity, ws, counters, plan_meta_dev=plan.dev)
        torch.cuda.synchronize()
        assert int(counters.abs().sum()) == 0
        outs.append(o.clone())
    for x in outs[1:]:
        assert torch.equal(_bits(x), _bits(outs[0]))


def test_fused_rejects_missing_counters():
    spec = small_spec(4)
    p = make_problem(spec, seed=33, device="cuda")
    d, a, o = desc_args(p)
    ws = skv.Workspace(d, skv.uniform_slots(d, 2), p.device)
    rc = skv.lib().skv_splitkv_fused(skv.ctypes.byref(d), skv.ctypes.byref(a), 1, 2, None,
                                     skv.ctypes.byref(ws.struct), None, None)
    assert rc == -1


@pytest.mark.parametrize("mode", ["uniform", "planned"])
def test_fused_graph_replay_follows_device_lengths(mode):
    spec = small_spec(4, ctx=(3001, 1500, 71), partitions_per_request=4)
    p = make_problem(spec, seed=34, device="cuda")
    d, a, o = desc_args(p)
    base = [int(c) for c in spec.ctx]
    counters = torch.zeros(spec.B * spec.Hkv, dtype=torch.int32, device=p.device)
    if mode == "uniform":
        ws = skv.Workspace(d, skv.uniform_slots(d, 3), p.device)

        def step():
            skv.splitkv_fused(d, a, True, 3, ws, counters)
    else:
        plan = _plan(spec, p.device)
        ws = skv.Workspace(d, plan.info.slots, p.device)

        def step():
            skv.splitkv_fused(d, a, True, plan.capacity, ws, counters, plan_meta_dev=plan.dev)

    torch.cuda.synchronize()
    step()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            step()
    torch.cuda.synchronize()
    for k in range(4):
        lens = [max(1, c - 41 * k) for c in base]
        p.ctx.copy_(torch.tensor(lens, dtype=torch.int32))
        o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = o.clone()
        assert int(counters.abs().sum()) == 0, f"replay {k}: counters not reset"
        o.fill_(float("nan"))
        step()
        torch.cuda.synchronize()
        assert torch.equal(_bits(got), _bits(o)), f"replay {k} != eager"
        st = compare(to_f64(got), oracle_output(p), "lowp")
        assert st["ok"], (k, st)
        print(f"[fused graph {mode}] replay {k} lengths {lens}: bitwise equal to eager", flush=True)


def test_fused_full_size_bench_workload():
    """B200 x 200k, fp8, page 16, plain V, 16 partitions per request: the
    fused call against the two-stage call, whole output, bitwise."""
    spec = config_spec(4)
    p = make_problem(spec, seed=4, device="cuda")
    two, fused, counters = _run_both(p, "auto", None)
    assert not torch.isnan(fused).any()
    assert torch.equal(_bits(fused), _bits(two))
    assert int(counters.abs().sum()) == 0
