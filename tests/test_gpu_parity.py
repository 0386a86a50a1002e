"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Reduced shapes of all five workloads (ragged contexts spanning several 64-key
tiles and partial pages), every entry point and kernel family, uniform split
counts and the planner, the "sharp" variants (Q x 8, so |O| ~ 1 and the
tolerance bites), and bitwise properties: run-to-run determinism, one split
through the combine == the single-pass kernel, paged == contiguous.
Tolerances: fp32 KV max-abs and max-rel 2e-3 (plus rel-L2 1e-4); bf16, int8 and
fp8 KV |d| <= 5e-3 + 5e-3 |ref| (plus rel-L2 1e-2 and row cosine 0.9999).
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

from skvgen import make_problem, small_spec, to_contiguous
from tests.gpu_run import run, to_f64
from tests.helpers import compare, oracle_output

pytestmark = pytest.mark.gpu

KIND = {1: "f32", 2: "lowp", 3: "lowp", 4: "lowp", 5: "lowp"}


def _problem(n, seed=0, **kw):
    return make_problem(small_spec(n, **kw), seed=seed, device="cuda")


def _check(p, o, n, label):
    ref = oracle_output(p)
    st = compare(to_f64(o), ref, KIND[n])
    print(f"[{label}] {st}", flush=True)
    assert st["ok"], (label, st)


IMPLS = {1: ["valu"], 2: ["valu", "mfma"], 3: ["valu", "mfma"], 4: ["valu", "mfma"], 5: ["valu", "mfma"]}


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("impl", ["valu", "mfma"])
def test_single_pass_matches_oracle(n, impl):
    if impl not in IMPLS[n]:
        pytest.skip("fp32 queries use the vector kernel only")
    p = _problem(n, seed=n)
    o, _, _ = run(p, "single", impl=impl)
    _check(p, o, n, f"cfg{n} single {impl}")


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("S", [1, 2, 3, 8, 16])
def test_split_matches_oracle(n, S):
    p = _problem(n, seed=10 + n)
    for impl in IMPLS[n]:
        o, _, _ = run(p, "split", num_splits=S, impl=impl, ws_fill=float("nan"))
        _check(p, o, n, f"cfg{n} S={S} {impl}")


@pytest.mark.parametrize("n", [2, 3, 4, 5])
def test_planned_matches_oracle(n):
    p = _problem(n, seed=20 + n)
    o, ws, plan = run(p, "planned", ws_fill=float("nan"))
    print("plan", plan.info.num_items, plan.info.capacity_items, plan.info.max_partitions, flush=True)
    _check(p, o, n, f"cfg{n} planned")


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
def test_planned_with_descriptor_hints_matches_oracle(n):
    """The planner with skv_plan_hints_for_desc (the kernel family's budget)."""
    from tests.gpu_run import desc_args
    import split_kv_flash_decode_amd as skv
    p = _problem(n, seed=25 + n)
    s = p.spec
    d, a, o = desc_args(p)
    h = skv.plan_hints_for(d, True, partitions_per_request=s.partitions_per_request)
    plan = skv.Plan(h, list(s.ctx), p.device)
    ws = skv.Workspace(d, plan.info.slots, p.device, fill=float("nan"))
    skv.attention_decode_paged_planned(d, a, plan.dev, plan.capacity, ws)
    torch.cuda.synchronize()
    print("plan", plan.info.num_items, plan.info.max_partitions, flush=True)
    _check(p, o, n, f"cfg{n} planned, descriptor hints")


@pytest.mark.parametrize("ctx", [(1024, 300, 6000, 1024), (300, 1024, 1024, 6000), (1024, 6000, 0, 300)],
                         ids=["long_at_2", "long_last", "long_at_1_empty_at_2"])
def test_mixed_batch_with_the_long_request_elsewhere(ctx):
    """The mixed batch with its long request moved away from index 0: the
    planner's work list, slot map and the combine must follow each request,
    not its position."""
    p = _problem(5, seed=27, ctx=ctx)
    for mode in ("planned", "split"):
        for impl in IMPLS[5]:
            if mode == "planned" and impl == "valu":
                continue
            o, _, _ = run(p, mode, num_splits=5, impl=impl, ws_fill=float("nan"))
            _check(p, o, 5, f"cfg5 ctx {ctx} {mode} {impl}")


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
def test_sharp_variant(n):
    p = _problem(n, seed=30 + n, q_mult=8.0)
    for impl in IMPLS[n]:
        for mode, S in (("single", 1), ("split", 4)):
            o, _, _ = run(p, mode, num_splits=S, impl=impl)
            _check(p, o, n, f"cfg{n} sharp {mode} S={S} {impl}")


@pytest.mark.parametrize("n", [4, 5])
def test_window_and_sinks(n):
    for window, sinks in ((0, True), (300, False), (300, True), (64, True), (1, True)):
        p = _problem(n, seed=40 + window, window=window, sinks=sinks)
        for impl in IMPLS[n]:
            for mode, S in (("single", 1), ("split", 3)):
                o, _, _ = run(p, mode, num_splits=S, impl=impl)
                _check(p, o, n, f"cfg{n} W={window} sinks={sinks} {mode} {impl}")
        o, _, _ = run(p, "planned")
        _check(p, o, n, f"cfg{n} W={window} sinks={sinks} planned")


@pytest.mark.parametrize("n", [2, 4])
@pytest.mark.parametrize("layout", ["plain", "transposed"])
@pytest.mark.parametrize("bs", [16, 32, 128])
def test_page_sizes_and_v_layouts(n, layout, bs):
    p = _problem(n, seed=50 + bs, block_size=bs, v_layout=layout)
    for impl in IMPLS[n]:
        o, _, _ = run(p, "split", num_splits=4, impl=impl)
        _check(p, o, n, f"cfg{n} bs={bs} {layout} {impl}")


@pytest.mark.parametrize("n", [1, 2, 3, 4])
def test_determinism_and_single_split_anchor(n):
    p = _problem(n, seed=60 + n)
    for impl in IMPLS[n]:
        o1, _, _ = run(p, "single", impl=impl)
        o2, _, _ = run(p, "single", impl=impl)
        assert torch.equal(o1.view(torch.int16) if o1.dtype == torch.bfloat16 else o1.view(torch.int32),
                           o2.view(torch.int16) if o2.dtype == torch.bfloat16 else o2.view(torch.int32))
        s1, _, _ = run(p, "split", num_splits=1, impl=impl)
        assert torch.equal(o1, s1), f"S=1 split != single pass ({impl})"
        a, _, _ = run(p, "split", num_splits=5, impl=impl)
        b, _, _ = run(p, "split", num_splits=5, impl=impl)
        assert torch.equal(a, b), f"S=5 not run-to-run deterministic ({impl})"


@pytest.mark.parametrize("n", [1, 2, 3, 4])
def test_paged_equals_contiguous(n):
    p = _problem(n, seed=70 + n)
    c = to_contiguous(p)
    for impl in IMPLS[n]:
        for mode, S in (("single", 1), ("split", 3)):
            a, _, _ = run(p, mode, num_splits=S, impl=impl)
            b, _, _ = run(c, mode, num_splits=S, impl=impl)
            assert torch.equal(a, b), (n, impl, mode)


@pytest.mark.parametrize("ctx", [(0,), (1,), (3,), (65,), (0, 5, 130)])
@pytest.mark.parametrize("n", [1, 4])
def test_edge_contexts(n, ctx):
    p = _problem(n, seed=80, ctx=ctx, B=len(ctx), partitions_per_request=0)
    for impl in IMPLS[n]:
        for mode, S in (("single", 1), ("split", 8)):
            o, _, _ = run(p, mode, num_splits=S, impl=impl, ws_fill=float("nan"))
            _check(p, o, n, f"cfg{n} ctx={ctx} {mode} S={S} {impl}")


@pytest.mark.parametrize("n", [1, 3, 4])
def test_maximum_split_count(n):
    """The largest uniform split count the library accepts: most splits of a
    short request are empty (chunks are rounded up to whole tiles), and the
    combine takes every request's records in batches (64 per lane). Scratch
    records start NaN-filled; the same count again gives the same bits."""
    import split_kv_flash_decode_amd as skv
    S = skv.SKV_MAX_SPLITS
    p = _problem(n, seed=150 + n)
    for impl in IMPLS[n]:
        o, _, _ = run(p, "split", num_splits=S, impl=impl, ws_fill=float("nan"))
        _check(p, o, n, f"cfg{n} S={S} {impl}")
        o2, _, _ = run(p, "split", num_splits=S, impl=impl, ws_fill=float("nan"))
        assert torch.equal(o.view(torch.int16) if o.dtype != torch.float32 else o.view(torch.int32),
                           o2.view(torch.int16) if o2.dtype != torch.float32 else o2.view(torch.int32))
    with pytest.raises(skv.SkvError):
        run(p, "split", num_splits=S + 1, impl=IMPLS[n][0])
