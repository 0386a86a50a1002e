"""Device-side plan refresh (skv_plan_refresh_device) against the host planner.

Integer work, so the bar is bit-exactness: for seeded context-length vectors
(uniform, mixed long/short, empty requests, windows, explicit counts, batches
up to the device limit, capacities below what the lengths ask for) the device
metadata block must equal skv_plan_fill's word for word. Then the planned
decode step with the device refresh captured in a HIP graph: each replay
after the lengths change in device memory must equal an eager step planned
on the host for the same lengths, bitwise, and the fp64 oracle.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import split_kv_flash_decode_amd as skv
from skvgen import make_problem, small_spec
from tests.gpu_run import desc_args, to_f64
from tests.helpers import compare, oracle_output

pytestmark = pytest.mark.gpu


def _host_meta(hints, ctx, capacity):
    meta = torch.zeros(skv.plan_meta_len(hints.batch, capacity), dtype=torch.int32)
    skv.plan_fill(hints, ctx, capacity, meta)
    return meta


def _device_meta(hints, ctx, capacity):
    ctx_dev = torch.tensor(ctx, dtype=torch.int32, device="cuda")
    meta = torch.full((skv.plan_meta_len(hints.batch, capacity),), -77, dtype=torch.int32, device="cuda")
    skv.plan_refresh_device(hints, ctx_dev, capacity, meta)
    torch.cuda.synchronize()
    return meta.cpu()


def _cases():
    rng = np.random.default_rng(606)
    out = []
    # the bench workload: 200 x 200k, MTP4, 16 per request (capacity 3200)
    out.append(("b200_mtp4_p16", dict(q_rows=4, num_kv_heads=1, partitions_per_request=16), [200000] * 200, None))
    out.append(("b200_mtp4_auto", dict(q_rows=4, num_kv_heads=1), [200000] * 200, None))
    out.append(("mixed_long_short", dict(q_rows=4, num_kv_heads=1), [200000] + [1024] * 15, None))
    out.append(("mixed_window", dict(q_rows=4, num_kv_heads=1, window=4096), [200000] + [1024] * 15, None))
    out.append(("verifier16", dict(q_rows=16, num_kv_heads=4), [20676], None))
    out.append(("batched_decode", dict(q_rows=1, num_kv_heads=8, causal=False), [4096] * 32, None))
    out.append(("with_empty", dict(q_rows=1, num_kv_heads=2, causal=False), [0, 1, 63, 64, 65, 5000, 0], None))
    out.append(("verifier16_row_groups", dict(q_rows=16, num_kv_heads=4, ctas_per_cu=1, workgroups_per_head=3),
                [20676], None))
    for i in range(12):
        B = int(rng.choice([1, 3, 17, 128, 600, 2048]))
        R = int(rng.choice([1, 4, 16]))
        ctx = [int(x) for x in rng.choice([0, 1, 37, 512, 3000, 40000, 250000], size=B)]
        kw = dict(q_rows=R, num_kv_heads=int(rng.choice([1, 2, 8])), causal=R > 1,
                  window=int(rng.choice([0, 0, 700])), max_partitions=int(rng.choice([0, 8, 64])),
                  min_tokens_per_partition=int(rng.choice([0, 128, 1024])),
                  ctas_per_cu=int(rng.choice([0, 1, 16])), workgroups_per_head=int(rng.choice([0, 1, 3])))
        if i % 4 == 3:
            kw["partitions_per_request"] = int(rng.integers(1, 40))
        out.append((f"random{i}_B{B}", kw, ctx, None))
        if i % 3 == 0:
            out.append((f"random{i}_B{B}_tight", kw, ctx, "tight"))
    return out


CASES = _cases()


@pytest.mark.parametrize("name,kw,ctx,cap", CASES, ids=[c[0] for c in CASES])
def test_device_plan_is_bit_identical_to_host_plan(name, kw, ctx, cap):
    kw = dict(kw)
    R, Hkv = kw.pop("q_rows"), kw.pop("num_kv_heads")
    hints = skv.plan_hints(len(ctx), R, Hkv, **kw)
    need = skv.plan_capacity(hints, ctx)
    capacity = need if cap is None else max(len(ctx), need // 2)   # "tight": counts must be cut
    host = _host_meta(hints, ctx, capacity)
    dev = _device_meta(hints, ctx, capacity)
    assert torch.equal(host, dev), f"{name}: first difference at word {int((host != dev).nonzero()[0])}"
    print(f"[plan {name}] B {len(ctx)} capacity {capacity} items {int(host[2])}: identical", flush=True)


def test_device_plan_rejects_oversized_batch():
    hints = skv.plan_hints(4096, 1, 1)
    ctx = torch.ones(4096, dtype=torch.int32, device="cuda")
    meta = torch.zeros(skv.plan_meta_len(4096, 4096), dtype=torch.int32, device="cuda")
    with pytest.raises(skv.SkvError) as e:
        skv.plan_refresh_device(hints, ctx, 4096, meta)
    assert e.value.status == -6


def test_graph_replay_with_device_plan_refresh():
    spec = small_spec(4, ctx=(3001, 1500, 71))
    p = make_problem(spec, seed=61, device="cuda")
    d, a, o = desc_args(p)
    base = [int(c) for c in spec.ctx]
    hints = skv.plan_hints(spec.B, spec.R, spec.Hkv, causal=spec.causal)
    plan = skv.Plan(hints, base, p.device)
    ws = skv.Workspace(d, plan.info.slots, p.device)

    def step():
        plan.refresh_device(p.ctx)
        skv.splitkv_partial(d, a, True, plan.capacity, ws, plan_meta_dev=plan.dev)
        skv.splitkv_combine(d, a, plan.capacity, ws, plan_meta_dev=plan.dev)

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
    host_plan = skv.Plan(hints, base, p.device, capacity=plan.capacity)
    for k in range(4):
        lens = [max(1, c - 613 * k) for c in base]
        p.ctx.copy_(torch.tensor(lens, dtype=torch.int32))
        o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = o.clone()
        assert torch.equal(plan.dev.cpu(), _host_meta(hints, lens, plan.capacity)), f"replay {k}: plan"
        # eager step planned on the host for the same lengths
        host_plan.refresh(lens)
        o.fill_(float("nan"))
        skv.splitkv_partial(d, a, True, host_plan.capacity, ws, plan_meta_dev=host_plan.dev)
        skv.splitkv_combine(d, a, host_plan.capacity, ws, plan_meta_dev=host_plan.dev)
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), o.view(torch.int16)), f"replay {k} != host-planned eager"
        st = compare(to_f64(got), oracle_output(p), "lowp")
        assert st["ok"], (k, st)
        print(f"[device plan graph] replay {k} lengths {lens}: bitwise equal to host-planned step", flush=True)
