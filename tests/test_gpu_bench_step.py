"""The step ``bench.py`` times (``bench.make_step``) gives, on every step, the
same bits as the step the parity tests check against the oracle
(``tests.gpu_run.bench_step``), on reduced shapes of the two long-context
workloads and in each of its modes: host plan refresh with the metadata
copied to the device block, the plan block passed by value, the device-side
plan refresh, and the single-kernel split + merge (bitwise equal to the
two-stage call by construction). Several steps run in a row, one of them
with the plan left as it is.
"""

from __future__ import annotations

import pytest
import torch

import bench
from skvgen import make_problem, small_spec
from tests.gpu_run import bench_step

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n", [4, 5])
@pytest.mark.parametrize("mode", ["two_stage", "host_plan", "device_plan", "fused"])
def test_bench_step_matches_the_checked_step(n, mode):
    spec = small_spec(n)
    p = make_problem(spec, seed=n, device="cuda")
    ref, _, _ = bench_step(p)
    torch.cuda.synchronize()
    step, plan, o, m = bench.make_step(spec, p, "f32", mode)
    assert m == mode
    for k in range(5):
        o.fill_(float("nan"))
        step(refresh=(k != 3))
        torch.cuda.synchronize()
        same = torch.equal(o, ref)
        print(f"[bench step cfg{n} {mode} step {k}] bitwise {same}", flush=True)
        assert same, (n, mode, k)
