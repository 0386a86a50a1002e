"""The random sweep's cases (``tests/sweep_cases.py``) are deterministic and
reach every option the sweep draws, so the GPU sweep covers what its header
says (host logic only, no GPU)."""

from __future__ import annotations

from tests.sweep_cases import N_CASES, cases


def test_sweep_cases_are_deterministic():
    a, b = cases(), cases()
    assert [c[0] for c in a] == [c[0] for c in b]
    assert len(a) == N_CASES and len({c[0] for c in a}) == N_CASES


def test_sweep_reaches_every_option():
    C = cases()
    specs = [c[1] for c in C]
    assert {s.kv_dtype for s in specs} == {"f32", "bf16", "int8", "fp8"}
    assert {s.q_dtype for s in specs} == {"f32", "bf16", "f16"}
    assert {s.D for s in specs} == {64, 128, 256}
    assert {s.Hkv for s in specs} == {1, 2, 4}
    assert {s.G for s in specs} >= {1, 2, 4, 8}
    assert {s.v_layout for s in specs} == {"plain", "transposed"}
    assert {s.verify for s in specs} >= {"causal", "chain", "tree"}
    assert any(s.causal and s.R > 1 for s in specs) and any(not s.causal for s in specs)
    assert any(s.window for s in specs) and any(s.sinks for s in specs)
    assert any(s.window and s.causal and s.sinks for s in specs) or \
        (any(s.window and s.causal for s in specs) and any(s.window and s.sinks for s in specs))
    paged = [s for s, c in zip(specs, C) if c[2] == 0]
    assert {s.block_size for s in paged} == {16, 32, 64, 128, 256}
    contig = [c for c in C if c[2]]
    assert contig and any(c[2] % 16 for c in contig) and any(c[2] % 16 == 0 for c in contig)
    assert all(c[2] >= max(c[1].ctx) for c in contig)
    assert {c[3] for c in C} == {"split", "planned"}
    assert {c[4] for c in C if c[3] == "split"} >= {1, 2, 3, 8, 13, 24}
    assert {c[5]["partitions_per_request"] for c in C if c[3] == "planned"} >= {0, 1, 3, 7}
    ctx = [x for s in specs for x in s.ctx]
    assert 0 in ctx and 1 in ctx and any(x % 64 and x > 64 for x in ctx)
    assert all(max(s.ctx) >= 64 for s in specs)
