"""bf16 partial records (the descriptor's record_dtype = SKV_BF16) against the
fp64 oracle.

The planned-reduction page keeps its partial outputs in bf16 with two fp32
values per row (aiter #5628 "tune MTP work budgets and planned reduction",
Changes); here the split's un-normalised acc is rounded to bf16 while m and l
stay fp32, halving the record bytes. The combine widens the values exactly and
merges with the same arithmetic.

Bar: the low-precision tolerance (|d| <= 5e-3 + 5e-3 |ref|, rel-L2 1e-2, row
cosine 0.9999) plus the bound of the record rounding itself. Rounding acc_s to
bf16 moves it by at most 2^-8 |acc_s| (round to nearest even, 8 significant
bits), and |acc_s| <= sum over the split's keys of p_t |v_t|, so the merged
output moves by at most 2^-8 sum_t p_t |v_t| / sum_t p_t: 2^-8 times the
oracle's output on |V|. That term matters where splits cancel (the sharp
variant: a few large values of opposite signs in different splits); the
fp32-record path needs no such allowance. Covered: every workload family,
kernel family, uniform splits, the planner, the sharp variant, windows with
sinks; the fused call with bf16 records is bitwise equal to the two-stage call
with bf16 records.
"""

from __future__ import annotations

import pytest
import torch

import split_kv_flash_decode_amd as skv
from skvgen import make_problem, small_spec
from tests.gpu_run import desc_args, run, to_f64
from tests.helpers import compare, oracle_abs_value_output, oracle_output

pytestmark = pytest.mark.gpu

IMPLS = {1: ["valu"], 2: ["valu", "mfma"], 3: ["valu", "mfma"], 4: ["valu", "mfma"], 5: ["valu", "mfma"]}


def _check(p, o, label):
    st = compare(to_f64(o), oracle_output(p), "lowp", extra=2.0 ** -8 * oracle_abs_value_output(p))
    print(f"[bf16 records {label}] {st}", flush=True)
    assert st["ok"], (label, st)


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
def test_bf16_records_match_oracle(n):
    p = make_problem(small_spec(n), seed=120 + n, device="cuda")
    for impl in IMPLS[n]:
        for S in (1, 3, 16):
            o, ws, _ = run(p, "split", num_splits=S, impl=impl, ws_fill=float("nan"), record_dtype="bf16")
            assert ws.acc.dtype == torch.bfloat16
            _check(p, o, f"cfg{n} S={S} {impl}")
    if n > 1:
        o, _, _ = run(p, "planned", ws_fill=float("nan"), record_dtype="bf16")
        _check(p, o, f"cfg{n} planned")


@pytest.mark.parametrize("n", [4, 5])
def test_bf16_records_sharp_windows_sinks(n):
    for kw in (dict(q_mult=8.0), dict(window=300, sinks=True)):
        p = make_problem(small_spec(n, **kw), seed=130 + n, device="cuda")
        for impl in IMPLS[n]:
            o, _, _ = run(p, "split", num_splits=5, impl=impl, record_dtype="bf16")
            _check(p, o, f"cfg{n} {kw} {impl}")


@pytest.mark.parametrize("impl", ["valu", "auto"])
def test_bf16_records_fused_equals_two_stage(impl):
    spec = small_spec(4, ctx=(3001, 1500, 71), partitions_per_request=4)
    p = make_problem(spec, seed=141, device="cuda")
    d, a, o = desc_args(p, impl, record_dtype="bf16")
    ws = skv.Workspace(d, skv.uniform_slots(d, 6), p.device, fill=float("nan"))
    skv.splitkv_partial(d, a, True, 6, ws)
    skv.splitkv_combine(d, a, 6, ws)
    torch.cuda.synchronize()
    two = o.clone()
    counters = torch.zeros(spec.B * spec.Hkv, dtype=torch.int32, device=p.device)
    o.fill_(float("nan"))
    skv.splitkv_fused(d, a, True, 6, ws, counters)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), two.view(torch.int16))
    assert int(counters.abs().sum()) == 0
    _check(p, o, f"fused {impl}")
