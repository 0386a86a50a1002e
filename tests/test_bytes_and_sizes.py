"""Pins of the byte accounting and record-size arithmetic against printed numbers.

* ``bench.logical_bytes`` divided by the printed times reproduces every printed
  effective bandwidth of the aiter #5628 performance table to its three
  decimals; dropping or altering any term breaks at least one row.
* The partial-record sizes of our layout, and of the pages' own layouts
  computed from our slot and row counts, reproduce the scratch sizes the pages
  quote (hipfire #760 "Memory"; aiter #5628 scratch note).
"""

from __future__ import annotations

import os

import pytest

import bench

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rows():
    out = []
    with open(os.path.join(GOLD, "aiter5628_performance_table.tsv")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            ctxs, page, layout, base, pr, tbs, _ = line.rstrip("\n").split("\t")
            ctx = []
            for part in ctxs.split("+"):
                n, c = part.split("x")
                ctx += [int(c)] * int(n)
            out.append((ctx, int(page), layout, float(pr), float(tbs)))
    return out


def _bytes(ctx, page, **kw):
    args = dict(R=4, Hq=16, Hkv=1, D=128, q_bytes=2, kv_bytes=1, quantized=True, block_size=page)
    args.update(kw)
    return bench.logical_bytes(ctx, **args)


@pytest.mark.parametrize("row", _rows(), ids=lambda r: f"{len(r[0])}req-p{r[1]}-{r[2]}")
def test_effective_bandwidth_reproduces_table(row):
    ctx, page, layout, pr_us, tbs = row
    got = _bytes(ctx, page) / (pr_us * 1e-6) / 1e12
    assert round(got, 3) == tbs, (got, tbs)


def test_each_term_is_needed():
    ctx, page, _, pr_us, tbs = _rows()[0]            # B200, page 16, plain

    def tb(nbytes):
        return round(nbytes / (pr_us * 1e-6) / 1e12, 3)

    full = _bytes(ctx, page)
    assert tb(full) == tbs
    n = sum(ctx)
    assert tb(full - 4 * n // 16) != tbs                    # no page-table term
    assert tb(full + 4 * n // 16) != tbs                    # int64 table entries
    assert tb(full - 2 * 200 * 4 * 16 * 128 * 2) != tbs     # no Q / O
    assert tb(full + 2 * 200 * 4 * 16 * 128 * 2) != tbs     # fp32 Q / O
    assert tb(full - 4 * n) != tbs                           # one scale per token, not per K and V


def test_config_byte_counts():
    from skvgen import config_spec
    assert bench.spec_bytes(config_spec(1)) == 2104836
    assert bench.spec_bytes(config_spec(2)) == 537428096
    assert bench.spec_bytes(config_spec(3)) == 43404472
    assert bench.spec_bytes(config_spec(4)) == 10576554400
    assert bench.spec_bytes(config_spec(4, block_size=128)) == 10567804800
    assert bench.spec_bytes(config_spec(5)) == 57386124


def _golden_sizes():
    vals = {}
    with open(os.path.join(GOLD, "scratch_sizes.tsv")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            k, v = line.split()
            vals[k] = float(v)
    return vals


MIB = float(1 << 20)


def test_record_sizes_match_the_pages():
    import split_kv_flash_decode_amd as skv
    import torch
    g = _golden_sizes()
    # hipfire #760: 8 splits of a 16-row verifier, 24 query heads over 4 KV heads, D 256,
    # fp32 records -> our fp32 acc buffer has exactly that size
    q = torch.zeros(1, 16, 24, 256, dtype=torch.bfloat16)
    k = torch.zeros(4, 4, 16, 256, dtype=torch.int8)
    d = skv.make_desc(q, k, k.clone(), paged=True, causal=True, page_table=torch.zeros(1, 4, dtype=torch.int32))
    _, _, acc = skv.workspace_size(d, skv.uniform_slots(d, 8))
    assert round(acc / MIB, 2) == g["hipfire_s8_b16_h24_d256"]
    # aiter #5628: capacity * rows * (bf16 D + two fp32) at capacity 512 and 3200, where the
    # planner gives capacity 3200 for B200 / 200k / MTP4 and rows = MTP4 * Hq16 / Hkv1
    q = torch.zeros(200, 4, 16, 128, dtype=torch.bfloat16)
    k = torch.zeros(4, 1, 16, 128, dtype=torch.uint8)
    d = skv.make_desc(q, k, k.clone(), paged=True, causal=True, page_table=torch.zeros(200, 4, dtype=torch.int32))
    cap = skv.plan_capacity(skv.plan_hints(200, 4, 1, causal=True), [200000] * 200)
    assert cap == 3200
    m, l, acc = skv.workspace_size(d, cap)
    rows = m // 4 // cap
    assert rows == 64
    assert round(cap * rows * (2 * 128 + 8) / MIB, 2) == g["aiter_b200_planned_capacity3200"]
    assert round(2 * 256 * rows * (2 * 128 + 8) / MIB, 2) == g["aiter_b200_base_capacity512"]
    # our own fp32 records for that plan
    assert (m + l + acc) == 3200 * 64 * (128 + 2) * 4
