"""FP16 queries and outputs against the fp64 oracle.

The validation of the planned-reduction page runs its decode tests with FP16
among the query types (aiter #5628 "tune MTP work budgets and planned
reduction", Validation). Here: fp16 Q/O over int8 and fp8 KV on both kernel
families (the matrix-core kernel multiplies Q K^T on the fp16 matrix cores,
the 8-bit codes converted to fp16 exactly), over fp32 and bf16 KV on the
vector kernel; single pass, uniform splits, the planner, the fused call and
the sharp variant, windows and sinks. Same bar as the bf16 cases
(|d| <= 5e-3 + 5e-3 |ref|, rel-L2 1e-2, row cosine 0.9999); one split
through the combine must equal the single pass bitwise.
"""

from __future__ import annotations

import pytest
import torch

import split_kv_flash_decode_amd as skv
from skvgen import make_problem, small_spec
from tests.gpu_run import desc_args, run, to_f64
from tests.helpers import compare, oracle_output

pytestmark = pytest.mark.gpu


def _problem(n, seed, **kw):
    return make_problem(small_spec(n, q_dtype="f16", **kw), seed=seed, device="cuda")


def _check(p, o, label):
    assert o.dtype == torch.float16
    st = compare(to_f64(o), oracle_output(p), "lowp")
    print(f"[f16 {label}] {st}", flush=True)
    assert st["ok"], (label, st)


# (config, KV dtype override, kernel families)
CASES = [
    ("cfg3_int8", 3, None, ["valu", "mfma"]),
    ("cfg4_fp8", 4, None, ["valu", "mfma"]),
    ("cfg5_fp8_mixed", 5, None, ["valu", "mfma"]),
    ("cfg4_int8", 4, "int8", ["valu", "mfma"]),
    ("cfg2_bf16kv", 2, None, ["valu"]),
    ("cfg1_f32kv", 1, None, ["valu"]),
]


@pytest.mark.parametrize("name,n,kv,impls", CASES, ids=[c[0] for c in CASES])
def test_f16_single_split_planned(name, n, kv, impls):
    kw = {} if kv is None else {"kv_dtype": kv}
    p = _problem(n, seed=90 + n, **kw)
    for impl in impls:
        o1, _, _ = run(p, "single", impl=impl)
        _check(p, o1, f"{name} single {impl}")
        s1, _, _ = run(p, "split", num_splits=1, impl=impl, ws_fill=float("nan"))
        assert torch.equal(o1.view(torch.int16), s1.view(torch.int16)), f"{name}: S=1 != single ({impl})"
        for S in (3, 16):
            o, _, _ = run(p, "split", num_splits=S, impl=impl, ws_fill=float("nan"))
            _check(p, o, f"{name} S={S} {impl}")
    o, _, _ = run(p, "planned", ws_fill=float("nan"))
    _check(p, o, f"{name} planned")


def test_f16_mfma_family_is_selected():
    """auto picks the matrix-core kernel for fp16 Q over 8-bit KV: its output
    equals the explicit mfma request bitwise (and differs from the vector
    kernel's rounding somewhere)."""
    p = _problem(4, seed=97)
    a, _, _ = run(p, "split", num_splits=4, impl="auto")
    m, _, _ = run(p, "split", num_splits=4, impl="mfma")
    v, _, _ = run(p, "split", num_splits=4, impl="valu")
    assert torch.equal(a.view(torch.int16), m.view(torch.int16))
    assert not torch.equal(m.view(torch.int16), v.view(torch.int16))


def test_f16_mfma_rejects_bf16_kv():
    p = _problem(2, seed=98)
    d, a, o = desc_args(p, "mfma")
    with pytest.raises(skv.SkvError):
        skv.attention_decode_paged(d, a)


@pytest.mark.parametrize("n", [3, 4, 5])
def test_f16_sharp_windows_sinks_fused(n):
    p = _problem(n, seed=99 + n, q_mult=8.0)
    for impl in ("valu", "mfma"):
        o, _, _ = run(p, "split", num_splits=4, impl=impl)
        _check(p, o, f"cfg{n} sharp S=4 {impl}")
    if n >= 4:
        p = _problem(n, seed=110 + n, window=300, sinks=True)
        for impl in ("valu", "mfma"):
            o, _, _ = run(p, "split", num_splits=3, impl=impl)
            _check(p, o, f"cfg{n} W=300 sinks {impl}")
    d, a, o = desc_args(p)
    ws = skv.Workspace(d, skv.uniform_slots(d, 5), p.device)
    two = torch.empty_like(o)
    skv.splitkv_partial(d, a, True, 5, ws)
    skv.splitkv_combine(d, a, 5, ws)
    torch.cuda.synchronize()
    two.copy_(o)
    counters = torch.zeros(p.spec.B * p.spec.Hkv, dtype=torch.int32, device=p.device)
    o.fill_(float("nan"))
    skv.splitkv_fused(d, a, True, 5, ws, counters)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), two.view(torch.int16)), "fused != two-stage"
    _check(p, o, f"cfg{n} fused")
