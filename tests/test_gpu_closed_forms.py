"""A closed form on the GPU, checked without the oracle's softmax.

With every key of a KV head identical (the same codes and the same per-token
scale), all logits of a query row are equal, so its output is the plain mean
of the values it sees, whatever the split count, the page layout or the
kernel family; with an attention sink s (tiny-llm #11 split-KV design record,
Design; aiter #5628 "tune MTP work budgets and planned reduction", intro) the
mean is scaled by n / (n + e^(s - x)), x being the row's common logit
scale * <q, k>. A row that sees no key is 0. The expected values are computed
here in fp64 from the stored codes: the oracle's storage decoders, its
gather of a request's rows through the page table and its visible-range
rule, but not its softmax. Reduced shapes of every workload through the
uniform split call and the planner, and the full B200 x 200,000 workload on
sampled requests through the step bench.py times, on both kernel families
where the descriptor allows. Bar: the workload tolerance.
"""

from __future__ import annotations

import gc

import numpy as np
import pytest
import torch

import oracle
from skvgen import config_spec, make_problem, small_spec
from tests.gpu_run import bench_step, run, to_f64
from tests.helpers import compare

pytestmark = pytest.mark.gpu


def _make_keys_identical(p):
    """Every K row of the pool (and its scale) := the first key row of the
    first non-empty request, per KV head (pool pages no request references
    hold NaN codes, so the row must come from a referenced page)."""
    ctx = p.ctx.cpu().tolist()
    b = next(i for i, c in enumerate(ctx) if c > 0)
    pg = int(p.page_table[b, 0])
    row = p.k[pg:pg + 1, :, 0:1, :].clone()
    p.k[:] = row
    if p.k_scale is not None:
        p.k_scale[:] = p.k_scale[pg:pg + 1, :, 0:1].clone()
    torch.cuda.synchronize()


def _expected(p, requests):
    """[len(requests)][R][Hq][D] float64: the mean of each row's visible values
    (scaled for a sink by n / (n + e^(s - x)))."""
    s = p.spec
    arrays = p.host_arrays()
    q = oracle.decode_storage(arrays["q"], s.q_dtype)
    ctx = np.asarray(arrays["ctx"], dtype=np.int64)
    sinks = None if not s.sinks else np.asarray(arrays["sinks"], dtype=np.float64)
    G = s.Hq // s.Hkv
    out = np.zeros((len(requests), s.R, s.Hq, s.D))
    for i, b in enumerate(requests):
        n = int(ctx[b])
        if n <= 0:
            continue
        K, V = oracle.gather_request(arrays, b, n, Hkv=s.Hkv, D=s.D, kv_dtype=s.kv_dtype, paged=p.paged,
                                     block_size=s.block_size, v_layout=s.v_layout)
        for j in range(s.R):
            lo, hi = oracle.visible_range(n, s.R, j, s.causal, s.window)
            if hi <= lo:
                continue
            for h in range(s.Hq):
                g = h // G
                mean = V[g, lo:hi].mean(axis=0)
                if sinks is not None:
                    x = s.scale * float(q[b, j, h] @ K[g, 0])
                    mean = mean * ((hi - lo) / ((hi - lo) + np.exp(sinks[h] - x)))
                out[i, j, h] = mean
    return out


def _impls(n):
    return ["valu"] if n == 1 else ["valu", "mfma"]


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("sinks", [False, True])
def test_identical_keys_give_the_mean_of_the_visible_values(n, sinks):
    over = {"sinks": True, "window": 700} if sinks else {}
    spec = small_spec(n, **over)
    p = make_problem(spec, seed=90 + n, device="cuda")
    _make_keys_identical(p)
    ref = _expected(p, list(range(spec.B)))
    kind = "f32" if spec.kv_dtype == "f32" else "lowp"
    for impl in _impls(n):
        for mode, S in (("split", 1), ("split", 7), ("planned", 0)):
            o, _, _ = run(p, mode, num_splits=S, impl=impl, ws_fill=float("nan"))
            st = compare(to_f64(o), ref, kind)
            print(f"[closed form cfg{n} sinks={sinks} {impl} {mode} S={S}] {st}", flush=True)
            assert st["ok"], (n, sinks, impl, mode, S, st)


def test_identical_keys_full_size_b200():
    spec = config_spec(4)
    p = make_problem(spec, seed=91, device="cuda")
    try:
        _make_keys_identical(p)
        reqs = [0, 97, 199]
        ref = _expected(p, reqs)
        for impl in ("mfma", "valu"):
            o, _, _ = bench_step(p, impl=impl, ws_fill=float("nan"))
            out = to_f64(o)
            st = compare(out[reqs], ref, "lowp")
            print(f"[closed form B200 x 200k {impl}, requests {reqs}] {st}", flush=True)
            assert st["ok"], (impl, st)
    finally:
        del p
        gc.collect()
        torch.cuda.empty_cache()
