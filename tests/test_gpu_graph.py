"""The split-KV calls under HIP graph capture.

The calls allocate nothing, copy nothing to the host and take their grids from
host arguments, so a captured step replays with new device-side visible
lengths. The test captures (a) a uniform 3-split decode and (b) the planned
partial + combine, replays each several times with the context lengths changed
in device memory between replays (eager work and synchronizations in between),
and checks every replay bitwise against an eager run with the same lengths and
against the fp64 oracle.
"""

from __future__ import annotations

import pytest
import torch

import split_kv_flash_decode_amd as skv
from skvgen import make_problem, small_spec
from tests.gpu_run import desc_args, to_f64
from tests.helpers import compare, oracle_output

pytestmark = pytest.mark.gpu


def _lengths(base, k):
    # shorter visible lengths, never below one key
    return [max(1, c - 37 * k) for c in base]


def _eager(fn):
    torch.cuda.synchronize()
    fn()
    torch.cuda.synchronize()


@pytest.mark.parametrize("mode", ["uniform", "planned"])
def test_graph_replay_follows_device_lengths(mode):
    spec = small_spec(4, ctx=(3001, 1500, 71), partitions_per_request=4)
    p = make_problem(spec, seed=21, device="cuda")
    d, a, o = desc_args(p)
    base = [int(c) for c in spec.ctx]
    if mode == "uniform":
        ws = skv.Workspace(d, skv.uniform_slots(d, 3), p.device)

        def step():
            skv.attention_decode_paged_splitkv(d, a, 3, ws)
    else:
        ph = skv.plan_hints(spec.B, spec.R, spec.Hkv, causal=spec.causal,
                            partitions_per_request=spec.partitions_per_request)
        plan = skv.Plan(ph, base, p.device)
        plan.refresh(base)
        torch.cuda.synchronize()
        ws = skv.Workspace(d, plan.info.slots, p.device)

        def step():
            skv.splitkv_partial(d, a, True, plan.capacity, ws, plan_meta_dev=plan.dev)
            skv.splitkv_combine(d, a, plan.capacity, ws, plan_meta_dev=plan.dev)

    _eager(step)                                        # warm up outside the capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            step()
    torch.cuda.synchronize()

    for k in range(4):
        lens = _lengths(base, k)
        p.ctx.copy_(torch.tensor(lens, dtype=torch.int32))
        o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = o.clone()
        o.fill_(float("nan"))
        _eager(step)
        eager = o.clone()
        assert torch.equal(got.view(torch.int16), eager.view(torch.int16)), f"replay {k} != eager"
        st = compare(to_f64(got), oracle_output(p), "lowp")      # the oracle reads p.ctx
        assert st["ok"], (k, st)
        print(f"[graph {mode}] replay {k} lengths {lens}: bitwise equal to eager", flush=True)
