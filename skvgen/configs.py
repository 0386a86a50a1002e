"""Workload shapes for split-KV paged decode attention.

The five full-size workloads follow the three pages' problem statements:

* one query row over a paged fp32 cache of 2,048 visible tokens with page size
  16, 14 query heads over 2 KV heads (tiny-llm #11, "split-KV decode attention
  design record", section "Why": the profiled single-pass case);
* a batched bf16 decode with grouped-query heads;
* a 16-row causal speculative-verifier block over a 20,676-token int8 cache,
  Hq 24 / Hkv 4 / D 256 (hipfire #760 "split packed-Q8 verifier KV scans",
  Performance);
* 200 requests of 200,000 tokens with four causal MTP rows, Hq 16 / Hkv 1 /
  D 128, fp8 e4m3 KV with per-token fp32 scales, page 16 or 128, plain or
  transposed V (aiter #5628 "tune MTP work budgets and planned reduction",
  Performance table);
* the mixed batch of that table: one 200,000-token request plus fifteen of
  1,024, page 128, transposed V, optionally with a 4,096-token sliding window
  and per-head attention-sink logits (same page, intro and Changes).

``small_spec`` gives reduced shapes of each that the fp64 oracle evaluates in
seconds while still spanning several 64-token tiles and ragged tails.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence, Tuple


@dataclasses.dataclass(frozen=True)
class ProblemSpec:
    name: str
    B: int
    R: int
    Hq: int
    Hkv: int
    D: int
    ctx: Tuple[int, ...]
    causal: bool
    window: int = 0
    q_dtype: str = "bf16"          # "f32" | "bf16" | "f16"  (O has the same dtype)
    kv_dtype: str = "bf16"         # "f32" | "bf16" | "int8" | "fp8"
    block_size: int = 16
    v_layout: str = "plain"        # "plain" [bs][D] | "transposed" [D][bs]
    sinks: bool = False
    q_mult: float = 1.0            # 8.0 gives the "sharp" variant (|O| ~ 1)
    splits: Optional[Tuple[int, ...]] = None   # uniform S values exercised; None = planner
    partitions_per_request: int = 0            # explicit planner budget (0 = automatic)
    pool_factor: float = 1.25
    poison: bool = True
    verify: str = "causal"         # "causal" (no mask) | "chain" | "tree" | "independent" masks

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def rho(self) -> int:
        """Query rows that share one KV head: R * Hq / Hkv."""
        return self.R * self.G

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)

    @property
    def max_ctx(self) -> int:
        return max(self.ctx) if self.ctx else 0

    @property
    def max_pages(self) -> int:
        return max(1, -(-self.max_ctx // self.block_size))

    def with_(self, **kw) -> "ProblemSpec":
        if "ctx" in kw and not isinstance(kw["ctx"], tuple):
            kw["ctx"] = tuple(int(c) for c in kw["ctx"])
        if "B" not in kw and "ctx" in kw:
            kw["B"] = len(kw["ctx"])
        return dataclasses.replace(self, **kw)


def _uniform(B: int, c: int) -> Tuple[int, ...]:
    return tuple([c] * B)


CONFIGS = {
    1: ProblemSpec(
        name="cfg1_fp32_single_request", B=1, R=1, Hq=14, Hkv=2, D=64,
        ctx=(2048,), causal=False, q_dtype="f32", kv_dtype="f32",
        block_size=16, splits=(1, 2, 4, 8)),
    2: ProblemSpec(
        name="cfg2_bf16_batched_decode", B=32, R=1, Hq=32, Hkv=8, D=128,
        ctx=_uniform(32, 4096), causal=False, q_dtype="bf16", kv_dtype="bf16",
        block_size=16),
    3: ProblemSpec(
        name="cfg3_int8_verifier16", B=1, R=16, Hq=24, Hkv=4, D=256,
        ctx=(20676,), causal=True, q_dtype="bf16", kv_dtype="int8",
        block_size=16, splits=(2, 4, 8)),
    4: ProblemSpec(
        name="cfg4_fp8_b200_mtp4", B=200, R=4, Hq=16, Hkv=1, D=128,
        ctx=_uniform(200, 200000), causal=True, q_dtype="bf16", kv_dtype="fp8",
        block_size=16, v_layout="plain", partitions_per_request=16),
    5: ProblemSpec(
        name="cfg5_fp8_mixed_mtp4", B=16, R=4, Hq=16, Hkv=1, D=128,
        ctx=(200000,) + _uniform(15, 1024), causal=True, q_dtype="bf16",
        kv_dtype="fp8", block_size=128, v_layout="transposed"),
}


def config_spec(n: int, **overrides) -> ProblemSpec:
    return CONFIGS[n].with_(**overrides) if overrides else CONFIGS[n]


def small_spec(n: int, **overrides) -> ProblemSpec:
    """Reduced shapes of config ``n`` with the same heads, dtypes and layouts.

    Contexts are ragged (not multiples of the page size nor of 64) and span
    several tiles, so tails, partial pages and split boundaries are exercised.
    """
    base = CONFIGS[n]
    if n == 1:
        s = base.with_(ctx=(2048,))                       # full size is already small
    elif n == 2:
        s = base.with_(ctx=(1000, 4096, 33, 517), B=4)
    elif n == 3:
        s = base.with_(ctx=(2077,))
    elif n == 4:
        s = base.with_(ctx=(3001, 1500, 64 + 7), B=3, partitions_per_request=4)
    elif n == 5:
        s = base.with_(ctx=(6000, 1024, 1024, 300), B=4)
    else:
        raise KeyError(n)
    return s.with_(**overrides) if overrides else s


def logical_pages(ctx: Sequence[int], block_size: int) -> int:
    return sum(-(-int(c) // block_size) for c in ctx)
