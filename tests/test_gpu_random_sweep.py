"""Seeded random sweep over the call space (``tests/sweep_cases.py``), both
kernel families against the fp64 oracle.

Every case runs on the vector kernel and, when ``skv_validate`` accepts the
descriptor for it, on the matrix-core kernel, through the uniform split call
(paged or contiguous) or the planned call, with NaN-filled partial buffers.
Bar: fp32 Q/O and KV max-abs and max-rel 2e-3 (plus rel-L2 1e-4); otherwise
|d| <= 5e-3 + 5e-3 |ref| (plus rel-L2 1e-2 and row cosine 0.9999), the
tolerances every workload test uses.
"""

from __future__ import annotations

import pytest

import split_kv_flash_decode_amd as skv
from skvgen import make_problem, to_contiguous
from tests.gpu_run import desc_args, run, to_f64
from tests.helpers import compare, oracle_output
from tests.sweep_cases import SEED, cases

pytestmark = pytest.mark.gpu

CASES = cases()


@pytest.mark.parametrize("cid,spec,cap,mode,S,hints", CASES, ids=[c[0] for c in CASES])
def test_random_case_matches_oracle(cid, spec, cap, mode, S, hints):
    p = make_problem(spec, seed=SEED + len(cid), device="cuda")
    if cap:
        p = to_contiguous(p, capacity=cap)
    ref = oracle_output(p)
    kind = "f32" if spec.kv_dtype == "f32" and spec.q_dtype == "f32" else "lowp"
    for impl in ("valu", "mfma"):
        d, _, _ = desc_args(p, impl)
        rc = skv.validate(d, p.paged, 0)          # descriptor and kernel family only
        if impl == "mfma" and rc == skv.SKV_ERR_UNSUPPORTED:
            print(f"[sweep {cid} {impl}] not taken by the matrix-core kernel", flush=True)
            continue
        assert rc == 0, (cid, impl, skv.status_str(rc))
        if mode == "planned":
            o, _, plan = run(p, "planned", impl=impl, hints=hints, ws_fill=float("nan"))
            how = f"planned items={plan.info.num_items}"
        else:
            o, _, _ = run(p, "split", num_splits=S, impl=impl, ws_fill=float("nan"))
            how = f"S={S}"
        st = compare(to_f64(o), ref, kind)
        print(f"[sweep {cid} {impl} {how}] {st}", flush=True)
        assert st["ok"], (cid, impl, st)
