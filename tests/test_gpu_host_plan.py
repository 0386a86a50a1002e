"""The planned call with the plan block in host memory, passed to the kernels
by value (skv_attention_decode_paged_planned_host), against the same plan
through a device copy (skv_attention_decode_paged_planned): the same kernels
read the same block, so the outputs must be bit-identical; both are held to
the oracle's bound on reduced shapes, and the bitwise identity is checked on
the full-size verifier and mixed workloads as well."""

from __future__ import annotations

import gc

import pytest
import torch

import split_kv_flash_decode_amd as skv
from skvgen import config_spec, make_problem, small_spec
from tests.gpu_run import desc_args, to_f64
from tests.helpers import compare, oracle_output

pytestmark = pytest.mark.gpu


def _both(p, impl="auto"):
    s = p.spec
    d, a, o_dev = desc_args(p, impl)
    hints = skv.plan_hints_for(d, True, partitions_per_request=s.partitions_per_request)
    plan = skv.Plan(hints, list(s.ctx), p.device)
    ws = skv.Workspace(d, plan.info.slots, p.device, fill=float("nan"))
    skv.attention_decode_paged_planned(d, a, plan.dev, plan.capacity, ws)
    o_host = torch.full_like(p.q, float("nan"))
    a2 = skv.make_args(p.q, p.k, p.v, p.ctx, o_host, k_scale=p.k_scale, v_scale=p.v_scale,
                       page_table=p.page_table, sinks=p.sinks, tree_mask=p.tree_mask)
    meta = torch.empty(plan.dev.numel(), dtype=torch.int32)
    skv.plan_fill(hints, list(s.ctx), plan.capacity, meta)
    ws2 = skv.Workspace(d, plan.info.slots, p.device, fill=float("nan"))
    skv.attention_decode_paged_planned_host(d, a2, meta, plan.capacity, ws2)
    torch.cuda.synchronize()
    return o_dev, o_host, plan


CASES = [(3, {}), (5, {}), (5, {"window": 4096, "sinks": True}), (2, {}), (1, {}), (4, {}),
         (3, {"verify": "tree"}), (5, {"q_mult": 8.0})]


@pytest.mark.parametrize("n,over", CASES, ids=[f"cfg{n}-{'-'.join(over) or 'plain'}" for n, over in CASES])
def test_host_plan_equals_device_plan_and_oracle(n, over):
    p = make_problem(small_spec(n, **over), seed=70 + n, device="cuda")
    impls = ["valu"] if p.spec.q_dtype == "f32" else ["valu", "mfma"]
    for impl in impls:
        o_dev, o_host, plan = _both(p, impl)
        assert torch.equal(o_dev, o_host), (n, over, impl)
        st = compare(to_f64(o_host), oracle_output(p), "f32" if p.spec.kv_dtype == "f32" else "lowp")
        print(f"[host plan cfg{n} {over} {impl}: {plan.info.num_items} items] {st}", flush=True)
        assert st["ok"], st


@pytest.mark.parametrize("n,over", [(3, {}), (5, {"window": 4096, "sinks": True}), (5, {})],
                         ids=["cfg3", "cfg5-window-sinks", "cfg5"])
def test_host_plan_full_size_bitwise(n, over):
    spec = config_spec(n, **over)
    print(f"[host plan full cfg{n} {over}] B {spec.B}, keys {sum(spec.ctx)}", flush=True)
    p = make_problem(spec, seed=80 + n, device="cuda")
    o_dev, o_host, plan = _both(p)
    assert plan.dev.numel() <= skv.SKV_PLAN_INLINE_MAX
    assert torch.equal(o_dev, o_host)
    del p
    gc.collect()
    torch.cuda.empty_cache()


def test_gather_ceiling_runs_on_the_bench_layouts():
    """The measurement gather (skv_gather_ceiling) over a reduced B200-shaped
    problem in each layout bench.py --ceiling uses: it completes, writes one
    value per workgroup, and the same inputs give the same values."""
    for over in ({}, {"block_size": 128}, {"v_layout": "transposed"}, {"block_size": 128, "v_layout": "transposed"}):
        p = make_problem(small_spec(4, **over), seed=90, device="cuda")
        d, a, _ = desc_args(p)
        s = p.spec
        hints = skv.plan_hints_for(d, True, partitions_per_request=s.partitions_per_request)
        plan = skv.Plan(hints, list(s.ctx), p.device)
        sink = torch.full((plan.capacity * s.Hkv,), -1, dtype=torch.int32, device="cuda")
        skv.gather_ceiling(d, a, plan.capacity, sink, plan_meta_dev=plan.dev)
        first = sink.clone()
        skv.gather_ceiling(d, a, plan.capacity, sink, plan_meta_dev=plan.dev)
        torch.cuda.synchronize()
        assert torch.equal(first, sink), over
