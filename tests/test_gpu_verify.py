"""Verify masks (args.tree_mask) against the fp64 oracle.

Tree-structured and independent-batch verification are named beside the
causal multi-row verifier route (hipfire #760 "split packed-Q8 verifier KV
scans", Summary) but not defined there; the reading here: the R query rows
are draft tokens at keys ctx - R .. ctx - 1, row j sees the committed prefix
and the drafts its mask word lets through (never one after itself). Seeded
masks: "chain" (must equal the plain causal call bitwise), "independent" (bit
j alone) and random trees (a parent per draft, the bits of its ancestors).
Both kernel families, uniform splits, the planner, the fused call, the sharp
variant, windows and sinks, 64 to 256 draft rows (one to four mask words per
row), contexts shorter than R. Bar: the low-precision tolerance
(|d| <= 5e-3 + 5e-3 |ref|, rel-L2 1e-2, row cosine 0.9999).
"""

from __future__ import annotations

import pytest
import torch

import split_kv_flash_decode_amd as skv
from skvgen import make_problem, small_spec
from tests.gpu_run import desc_args, run, to_f64
from tests.helpers import compare, oracle_output

pytestmark = pytest.mark.gpu


def _check(p, o, label):
    st = compare(to_f64(o), oracle_output(p), "lowp")
    print(f"[verify {label}] {st}", flush=True)
    assert st["ok"], (label, st)


CASES = [
    ("cfg3_tree", 3, dict(verify="tree")),
    ("cfg3_independent", 3, dict(verify="independent")),
    ("cfg4_tree", 4, dict(verify="tree")),
    ("cfg4_independent_sinks", 4, dict(verify="independent", sinks=True)),
    ("cfg5_tree_fp16", 5, dict(verify="tree", q_dtype="f16")),
    ("cfg3_tree_r64", 3, dict(verify="tree", R=64, ctx=(700,))),
    ("cfg4_tree_short_ctx", 4, dict(verify="tree", ctx=(3, 4, 2000))),
    ("cfg4_tree_sharp", 4, dict(verify="tree", q_mult=8.0)),
    ("cfg4_tree_t128", 4, dict(verify="tree", block_size=128, v_layout="transposed")),
    ("cfg4_tree_window_sinks", 4, dict(verify="tree", window=300, sinks=True)),
    ("cfg3_tree_r128", 3, dict(verify="tree", R=128, ctx=(900,))),
    ("cfg3_independent_r256", 3, dict(verify="independent", R=256, ctx=(2300,))),
    ("cfg4_tree_r200", 4, dict(verify="tree", R=200, ctx=(450, 1300, 205))),
]


@pytest.mark.parametrize("name,n,kw", CASES, ids=[c[0] for c in CASES])
def test_verify_masks_match_oracle(name, n, kw):
    p = make_problem(small_spec(n, **kw), seed=150 + n, device="cuda")
    assert p.tree_mask is not None
    for impl in ("valu", "mfma"):
        o1, _, _ = run(p, "single", impl=impl)
        _check(p, o1, f"{name} single {impl}")
        for S in (1, 4):
            o, _, _ = run(p, "split", num_splits=S, impl=impl, ws_fill=float("nan"))
            if S == 1:
                assert torch.equal(o.view(torch.int16), o1.view(torch.int16)), f"{name}: S=1 != single ({impl})"
            _check(p, o, f"{name} S={S} {impl}")
    o, _, _ = run(p, "planned", ws_fill=float("nan"))
    _check(p, o, f"{name} planned")


@pytest.mark.parametrize("n", [3, 4])
def test_chain_mask_equals_causal_call(n):
    p = make_problem(small_spec(n, verify="chain"), seed=160 + n, device="cuda")
    for impl in ("valu", "mfma"):
        masked, _, _ = run(p, "split", num_splits=3, impl=impl)
        plain_p = type(p)(**{**p.__dict__, "tree_mask": None})
        plain, _, _ = run(plain_p, "split", num_splits=3, impl=impl)
        assert torch.equal(masked.view(torch.int16), plain.view(torch.int16)), impl


def test_verify_fused_equals_two_stage():
    p = make_problem(small_spec(3, verify="tree"), seed=171, device="cuda")
    d, a, o = desc_args(p)
    ws = skv.Workspace(d, skv.uniform_slots(d, 4), p.device)
    skv.splitkv_partial(d, a, True, 4, ws)
    skv.splitkv_combine(d, a, 4, ws)
    torch.cuda.synchronize()
    two = o.clone()
    counters = torch.zeros(p.spec.B * p.spec.Hkv, dtype=torch.int32, device=p.device)
    o.fill_(float("nan"))
    skv.splitkv_fused(d, a, True, 4, ws, counters)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), two.view(torch.int16))
    _check(p, o, "fused")
