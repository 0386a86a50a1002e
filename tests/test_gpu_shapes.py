"""Shape matrix beyond the five workloads, both kernel families against the
fp64 oracle.

Every (KV code, head dim) pair the matrix-core kernel instantiates — bf16 at
D 64 / 128, int8 and fp8 at D 64 / 128 / 256 (bf16 D 256 runs on the vector
kernel) — with one and two row halves (2 and 80 query rows per KV head, the
latter two row groups), page sizes 16, 64 and 1024, plain and transposed V,
over three ragged requests; fp16 queries on the 8-bit codes. Same bar as the
workload tests (|d| <= 5e-3 + 5e-3 |ref|, rel-L2 1e-2, row cosine 0.9999).
"""

from __future__ import annotations

import itertools

import pytest

from skvgen import make_problem, small_spec
from tests.gpu_run import run, to_f64
from tests.helpers import compare, oracle_output

pytestmark = pytest.mark.gpu

ROWS = {"rho2": dict(R=1, Hq=4, Hkv=2), "rho80": dict(R=4, Hq=40, Hkv=2)}


def _cases():
    out = []
    for kv, D, rows, bs, vl in itertools.product(("bf16", "int8", "fp8"), (64, 128, 256), ROWS,
                                                 (16, 64, 1024), ("plain", "transposed")):
        out.append((kv, D, rows, bs, vl, "bf16"))
    for kv, D in itertools.product(("int8", "fp8"), (64, 256)):
        out.append((kv, D, "rho80", 16, "plain", "f16"))
    return out


CASES = _cases()


@pytest.mark.parametrize("kv,D,rows,bs,vl,qd", CASES, ids=["-".join(map(str, c)) for c in CASES])
def test_shape_matrix(kv, D, rows, bs, vl, qd):
    spec = small_spec(4, kv_dtype=kv, D=D, block_size=bs, v_layout=vl, q_dtype=qd,
                      ctx=(1500, 77, 1030), B=3, partitions_per_request=3, **ROWS[rows])
    p = make_problem(spec, seed=D + bs + len(kv), device="cuda")
    ref = oracle_output(p)
    impls = ["valu"] if (kv == "bf16" and D == 256) else ["valu", "mfma"]
    for impl in impls:
        o, _, _ = run(p, "split", num_splits=3, impl=impl, ws_fill=float("nan"))
        st = compare(to_f64(o), ref, "lowp")
        print(f"[shape {kv} D{D} {rows} bs{bs} {vl} q{qd} {impl}] {st}", flush=True)
        assert st["ok"], (kv, D, rows, bs, vl, qd, impl, st)
