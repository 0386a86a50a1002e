"""The tail split of an eight-wave matrix-core launch.

When the partial kernel's eight-wave workgroups (64 query rows of a KV head,
one workgroup per CU) would leave the last round at most half full, the
launcher runs that round's items as a second launch of the four-wave kernel
with two row groups of 32 rows each. Every row's arithmetic is the same in
both kernels, so the two-stage output must be bit-identical to the
single-kernel split + merge call (which keeps one launch) and both must match
the fp64 oracle. The shapes below give grids of 300 workgroups (one or two KV
heads, uniform splits and the planner), so on a 256-CU part their last 44 run
as the second launch.
"""

from __future__ import annotations

import pytest
import torch

import split_kv_flash_decode_amd as skv
from skvgen import make_problem, small_spec
from tests.gpu_run import desc_args, to_f64
from tests.helpers import compare, oracle_output

pytestmark = pytest.mark.gpu


def _ragged(n: int, base: int) -> tuple:
    return tuple(base + (37 * i) % 400 for i in range(n))


CASES = [
    ("hkv1_planned_300", lambda: small_spec(4, B=300, ctx=_ragged(300, 600), partitions_per_request=1), None),
    ("hkv2_s1_150", lambda: small_spec(4, B=150, ctx=_ragged(150, 600), Hq=32, Hkv=2), 1),
    ("hkv2_s2_75", lambda: small_spec(4, B=75, ctx=_ragged(75, 900), Hq=32, Hkv=2), 2),
    ("hkv1_p128_vt_s3_100", lambda: small_spec(4, B=100, ctx=_ragged(100, 1200), block_size=128,
                                               v_layout="transposed"), 3),
]


def _bits(o: torch.Tensor) -> torch.Tensor:
    return o.view(torch.int16) if o.dtype == torch.bfloat16 else o.view(torch.int32)


@pytest.mark.parametrize("name,mk,S", CASES, ids=[c[0] for c in CASES])
def test_tail_split_is_bit_identical_and_matches_oracle(name, mk, S):
    spec = mk()
    p = make_problem(spec, seed=61, device="cuda")
    d, a, o = desc_args(p)
    if S is None:
        ph = skv.plan_hints(spec.B, spec.R, spec.Hkv, causal=spec.causal, window=spec.window,
                            partitions_per_request=spec.partitions_per_request)
        base = [int(c) for c in spec.ctx]
        plan = skv.Plan(ph, base, p.device)
        plan.refresh(base)
        n, meta, slots = plan.capacity, plan.dev, plan.info.slots
    else:
        n, meta, slots = S, None, skv.uniform_slots(d, S)
    rho = spec.R * spec.Hq // spec.Hkv
    print(f"[tail {name}] rows per KV head {rho}, workgroups {n * spec.Hkv if S is None else spec.B * S * spec.Hkv}",
          flush=True)
    ws = skv.Workspace(d, slots, p.device, fill=float("nan"))
    o.fill_(float("nan"))
    skv.splitkv_partial(d, a, True, n, ws, plan_meta_dev=meta)
    skv.splitkv_combine(d, a, n, ws, plan_meta_dev=meta)
    torch.cuda.synchronize()
    two = o.clone()
    counters = torch.zeros(spec.B * spec.Hkv, dtype=torch.int32, device=p.device)
    ws2 = skv.Workspace(d, slots, p.device, fill=float("nan"))
    o.fill_(float("nan"))
    skv.splitkv_fused(d, a, True, n, ws2, counters, plan_meta_dev=meta)
    torch.cuda.synchronize()
    assert not torch.isnan(two).any(), name
    assert torch.equal(_bits(two), _bits(o)), f"{name}: split launch != single launch"
    st = compare(to_f64(two), oracle_output(p), "lowp")
    print(f"[tail {name}] bitwise equal to the single launch; {st}", flush=True)
    assert st["ok"], (name, st)
