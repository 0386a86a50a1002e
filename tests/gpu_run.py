"""Test-side driver: run a ``skvgen.Problem`` through the C ABI on the GPU."""

from __future__ import annotations

from typing import Optional

import torch

import split_kv_flash_decode_amd as skv


def desc_args(p, impl: str = "auto", o: Optional[torch.Tensor] = None, record_dtype: str = "f32"):
    s = p.spec
    o = torch.empty_like(p.q) if o is None else o
    d = skv.make_desc(p.q, p.k, p.v, paged=p.paged, v_layout=s.v_layout, causal=s.causal,
                      window=s.window, scale=s.scale, page_table=p.page_table, has_sink=s.sinks,
                      impl=impl, record_dtype=record_dtype)
    a = skv.make_args(p.q, p.k, p.v, p.ctx, o, k_scale=p.k_scale, v_scale=p.v_scale,
                      page_table=p.page_table, sinks=p.sinks, tree_mask=p.tree_mask)
    return d, a, o


def run(p, mode: str = "split", num_splits: int = 1, impl: str = "auto", ws_fill: Optional[float] = None,
        hints: Optional[dict] = None, sync: bool = True, record_dtype: str = "f32"):
    """mode: "single" (attention_decode[_paged]), "split" (uniform num_splits) or
    "planned" (planner hints ``hints``). Returns (o, workspace or None, plan or None)."""
    d, a, o = desc_args(p, impl, record_dtype=record_dtype)
    ws = plan = None
    if mode == "single":
        (skv.attention_decode_paged if p.paged else skv.attention_decode)(d, a)
    elif mode == "split":
        ws = skv.Workspace(d, skv.uniform_slots(d, num_splits), p.device, fill=ws_fill)
        (skv.attention_decode_paged_splitkv if p.paged else skv.attention_decode_splitkv)(d, a, num_splits, ws)
    elif mode == "planned":
        s = p.spec
        h = dict(causal=s.causal, window=s.window, partitions_per_request=s.partitions_per_request)
        h.update(hints or {})
        ph = skv.plan_hints(s.B, s.R, s.Hkv, **h)
        plan = skv.Plan(ph, list(s.ctx), p.device)
        ws = skv.Workspace(d, plan.info.slots, p.device, fill=ws_fill)
        skv.attention_decode_paged_planned(d, a, plan.dev, plan.capacity, ws)
    else:
        raise ValueError(mode)
    if sync:
        torch.cuda.synchronize()
    return o, ws, plan


def to_f64(o: torch.Tensor):
    return o.detach().double().cpu().numpy()


def bench_step(p, impl: str = "auto", ws_fill: Optional[float] = None, record_dtype: str = "f32",
               device_plan: bool = False):
    """The step ``bench.py`` times: plan (host) -> metadata copy -> partial -> combine,
    through splitkv_partial / splitkv_combine with the planner's capacity.
    ``device_plan``: the metadata is overwritten with -1 and re-planned on the GPU
    from the device lengths instead. Returns (o, workspace, plan)."""
    s = p.spec
    d, a, o = desc_args(p, impl, record_dtype=record_dtype)
    ph = skv.plan_hints_for(d, True, partitions_per_request=s.partitions_per_request)
    plan = skv.Plan(ph, list(s.ctx), p.device)
    ws = skv.Workspace(d, plan.info.slots, p.device, fill=ws_fill)
    plan.refresh(list(s.ctx))
    if device_plan:
        plan.dev.fill_(-1)
        skv.plan_refresh_device(ph, p.ctx, plan.capacity, plan.dev)
    skv.splitkv_partial(d, a, True, plan.capacity, ws, plan_meta_dev=plan.dev)
    skv.splitkv_combine(d, a, plan.capacity, ws, plan_meta_dev=plan.dev)
    torch.cuda.synchronize()
    return o, ws, plan
