"""Seeded random cases over the call space, shared by the GPU sweep and its
CPU-side coverage check.

Each case draws every option on its own: KV codes (fp32, bf16, int8, fp8),
query dtype, head dim 64 / 128 / 256, KV heads and group size, query tokens
per request, causal masking (with chain, tree or independent verify masks on
some causal cases), a sliding window, attention sinks, page size 16-256 or a
contiguous cache, plain or transposed V, two to five requests whose visible
lengths include 0 and 1 and lengths off the page and 64-key tile grids, and a
uniform split count (1-24) or the planner (automatic or an explicit count per
request). Sizes stay small enough for the fp64 oracle to finish each case in
about a second.
"""

from __future__ import annotations

import random

from skvgen.configs import ProblemSpec

N_CASES = 64
SEED = 20261202


def _ctx(rng: random.Random, B: int):
    out = []
    for _ in range(B):
        kind = rng.random()
        if kind < 0.12:
            out.append(0)
        elif kind < 0.2:
            out.append(1)
        elif kind < 0.35:
            out.append(rng.randint(2, 70))
        else:
            out.append(rng.randint(71, 2600))
    if max(out) < 64:                      # at least one request spans several tiles
        out[rng.randrange(B)] = rng.randint(300, 2600)
    return tuple(out)


def cases():
    """List of (case id, ProblemSpec, contiguous capacity (0: paged), mode,
    num_splits, planner hints)."""
    rng = random.Random(SEED)
    out = []
    for i in range(N_CASES):
        kv = rng.choice(("f32", "bf16", "int8", "fp8", "int8", "fp8"))
        qd = "f32" if kv == "f32" and rng.random() < 0.6 else rng.choice(("bf16", "f16"))
        D = rng.choice((64, 128, 256))
        Hkv = rng.choice((1, 2, 4))
        G = rng.choice((1, 2, 4, 6, 8))
        R = rng.choice((1, 1, 2, 4, 5, 8))
        causal = R > 1 and rng.random() < 0.7
        B = rng.randint(2, 5)
        ctx = _ctx(rng, B)
        window = rng.randint(1, max(ctx) + 16) if rng.random() < 0.3 else 0
        sinks = rng.random() < 0.3
        paged = rng.random() < 0.8
        bs = rng.choice((16, 32, 64, 128, 256)) if paged else 16
        # contiguous cache: capacity past the longest request, a multiple of 16
        # (matrix-core loads) or not (vector kernel only)
        cap = 0 if paged else max(ctx) + rng.choice((16 - max(ctx) % 16 if max(ctx) % 16 else 0, 37, 100))
        vl = rng.choice(("plain", "transposed"))
        verify = rng.choice(("chain", "tree", "independent")) if causal and rng.random() < 0.25 else "causal"
        if paged and rng.random() < 0.4:
            mode, S = "planned", 0
            hints = {"partitions_per_request": rng.choice((0, 0, 1, 3, 7))}
        else:
            mode, S, hints = "split", rng.choice((1, 2, 3, 5, 8, 13, 24)), None
        spec = ProblemSpec(
            name=f"sweep{i}", B=B, R=R, Hq=Hkv * G, Hkv=Hkv, D=D, ctx=ctx, causal=causal,
            window=window, q_dtype=qd, kv_dtype=kv, block_size=bs, v_layout=vl, sinks=sinks,
            verify=verify)
        cid = (f"{i}-{kv}-q{qd}-D{D}-h{Hkv}x{G}-R{R}{'c' if causal else ''}"
               f"{'-w' + str(window) if window else ''}{'-sink' if sinks else ''}"
               f"-{'bs' + str(bs) if paged else 'contig' + str(cap)}-{vl}"
               f"-{'nomask' if verify == 'causal' else verify}-"
               f"{'plan' + str(hints['partitions_per_request']) if mode == 'planned' else 'S' + str(S)}")
        out.append((cid, spec, cap, mode, S, hints))
    return out
