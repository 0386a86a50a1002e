"""The allocation-free split-KV call (partial records in the library's static
device scratch) against the call with caller-owned buffers, through the C
ABI: two calls in a row, the second on a smaller input. Same kernels, so the
outputs must be bit-identical; both are also held to the oracle's bound."""

from __future__ import annotations

import ctypes

import pytest
import torch

import split_kv_flash_decode_amd as skv
from skvgen import config_spec, make_problem, small_spec
from tests.gpu_run import desc_args, to_f64
from tests.helpers import compare, oracle_output

pytestmark = pytest.mark.gpu


def _both(p, S):
    d, a, o_ref = desc_args(p)
    ws = skv.Workspace(d, skv.uniform_slots(d, S), p.device, fill=float("nan"))
    skv.attention_decode_paged_splitkv(d, a, S, ws)
    o = torch.full_like(p.q, float("nan"))
    a2 = skv.make_args(p.q, p.k, p.v, p.ctx, o, k_scale=p.k_scale, v_scale=p.v_scale,
                       page_table=p.page_table, sinks=p.sinks)
    rc = skv.lib().skv_attention_decode_paged_splitkv_noalloc(
        ctypes.byref(d), ctypes.byref(a2), S, torch.cuda.current_stream().cuda_stream)
    assert rc == 0, skv.status_str(rc)
    torch.cuda.synchronize()
    return o_ref, o


def test_noalloc_equals_caller_buffers_twice_second_smaller():
    cases = [(config_spec(3), 8, 31), (small_spec(4, ctx=(900, 77), B=2), 3, 32)]
    for spec, S, seed in cases:
        p = make_problem(spec, seed=seed, device="cuda")
        print(f"[noalloc] {spec.name} B {spec.B} ctx {spec.ctx} S {S}", flush=True)
        o_ref, o = _both(p, S)
        assert torch.equal(o, o_ref), "allocation-free call differs from the caller-buffer call"
        st = compare(to_f64(o), oracle_output(p), "lowp")
        print(f"[noalloc {spec.name}] {st}", flush=True)
        assert st["ok"], st


def test_noalloc_refuses_records_beyond_the_scratch():
    spec = small_spec(4, ctx=(64,), B=1)
    p = make_problem(spec, seed=1, device="cuda")
    d, a, _ = desc_args(p)
    d.batch = 200                                     # 200 x 256 slots of 64 x 130 fp32 records
    rc = skv.lib().skv_attention_decode_paged_splitkv_noalloc(ctypes.byref(d), ctypes.byref(a), 256, None)
    assert rc == -10
