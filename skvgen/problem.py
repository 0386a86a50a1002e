"""Seeded problem construction: values, storage encodings, page pools, poison.

Recipe (every draw from one ``torch.Generator`` seeded with ``seed``, on the
device the problem is built on, in this order):

1. Q ~ N(0, 1) * q_mult, shape [B][R][Hq][D], then stored as fp32, bf16 or
   fp16 (round-to-nearest-even cast).
2. K pool values ~ N(0, 1), shape [P][Hkv][bs][D], drawn page chunk by page
   chunk; V pool values likewise.
3. Storage encoding of K and V per (page, head, slot) row of D values:
   fp32 as is; bf16 by RNE cast; int8 symmetric: s = max|x| / 127,
   code = clip(round_half_even(x / s), -127, 127); fp8 e4m3fn: s = max|x| / 448,
   code = e4m3(clip(x / s, -448, 448)) with RNE (torch's cast). Scales are fp32
   [P][Hkv][bs], one per token per KV head for K and one for V.
4. Transposed V stores each (page, head) block as [D][bs] instead of [bs][D];
   it holds exactly the same codes as the plain layout for the same seed.
5. Sink logits ~ N(0, 1), shape [Hq], when requested.
6. A random permutation of the P pool pages; request b takes the next
   ceil(ctx_b / bs) of them as its logical pages 0, 1, ...  P is
   max(N + 1, ceil(1.25 N)) for N referenced pages, so spare pages exist.
7. Verify masks (``spec.verify`` other than "causal"), int64 [B][R][W] with
   W = ceil(R / 64) words per row (bit i % 64 of word i / 64 = draft i):
   "chain" sets bits 0..j of row j; "independent" bit j alone; "tree" draws,
   per request, a parent for each draft i (uniform over the prefix root and
   the drafts 0..i-1, one torch.randint per draft) and sets the bits of i
   and its ancestors.

Poison (``spec.poison``): every spare pool page, and every slot of a request's
last page at or beyond its context length, is filled with NaN (fp32/bf16),
with the e4m3 NaN code 0x7F (fp8), and its K and V scales are NaN (int8 and
fp8). Page-table entries past a request's last page all point at one spare,
poisoned page. A correct kernel never lets any of that reach an output.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

from .configs import ProblemSpec

_TORCH_STORAGE = {
    "f32": torch.float32,
    "bf16": torch.bfloat16,
    "int8": torch.int8,
    "fp8": torch.uint8,      # e4m3fn codes kept as raw bytes
}


@dataclasses.dataclass
class Problem:
    spec: ProblemSpec
    paged: bool
    q: torch.Tensor                    # [B][R][Hq][D] fp32, bf16 or fp16
    k: torch.Tensor                    # paged [P][Hkv][bs][D]; contiguous [B][Hkv][cap][D]
    v: torch.Tensor                    # plain as k; transposed [..][Hkv][D][bs or cap]
    k_scale: Optional[torch.Tensor]    # fp32 [P][Hkv][bs] or [B][Hkv][cap]
    v_scale: Optional[torch.Tensor]
    page_table: Optional[torch.Tensor]  # int32 [B][max_pages]
    ctx: torch.Tensor                  # int32 [B]
    sinks: Optional[torch.Tensor]      # fp32 [Hq]
    kv_capacity: int                   # contiguous tokens per (request, KV head)
    tree_mask: Optional[torch.Tensor] = None   # int64 [B][R][ceil(R / 64)] verify masks

    @property
    def device(self) -> torch.device:
        return self.q.device

    @property
    def num_pages(self) -> int:
        return int(self.k.shape[0]) if self.paged else 0

    def to(self, device) -> "Problem":
        def mv(t):
            return None if t is None else t.to(device)
        return dataclasses.replace(
            self, q=mv(self.q), k=mv(self.k), v=mv(self.v), k_scale=mv(self.k_scale),
            v_scale=mv(self.v_scale), page_table=mv(self.page_table), ctx=mv(self.ctx),
            sinks=mv(self.sinks), tree_mask=mv(self.tree_mask))

    def host_arrays(self) -> dict:
        """Storage as numpy arrays: bf16 and fp16 as uint16 bit patterns, fp8 as uint8 codes."""
        def np_store(t):
            if t is None:
                return None
            t = t.detach().cpu().contiguous()
            if t.dtype in (torch.bfloat16, torch.float16):
                return t.view(torch.int16).numpy().view(np.uint16)
            return t.numpy()
        return {name: np_store(getattr(self, name))
                for name in ("q", "k", "v", "k_scale", "v_scale", "page_table", "ctx", "sinks",
                             "tree_mask")}


def _encode_rows(x: torch.Tensor, kv_dtype: str):
    """Encode fp32 rows (last dim = D) into storage; returns (codes, scale or None)."""
    if kv_dtype == "f32":
        return x.contiguous(), None
    if kv_dtype == "bf16":
        return x.to(torch.bfloat16), None
    amax = x.abs().amax(dim=-1)
    if kv_dtype == "int8":
        s = amax / 127.0
        s = torch.where(s > 0, s, torch.ones_like(s))
        codes = torch.round(x / s.unsqueeze(-1)).clamp_(-127, 127).to(torch.int8)
        return codes, s.to(torch.float32)
    if kv_dtype == "fp8":
        s = amax / 448.0
        s = torch.where(s > 0, s, torch.ones_like(s))
        y = (x / s.unsqueeze(-1)).clamp_(-448.0, 448.0)
        codes = y.to(torch.float8_e4m3fn).view(torch.uint8)
        return codes, s.to(torch.float32)
    raise ValueError(kv_dtype)


def _poison_value(kv_dtype: str):
    if kv_dtype in ("f32", "bf16"):
        return float("nan")
    if kv_dtype == "fp8":
        return 0x7F
    return None   # int8: codes stay, scales carry the poison


def make_problem(spec: ProblemSpec, seed: int, device="cpu", paged: bool = True,
                 chunk_pages: int = 1 << 16) -> Problem:
    """Build a seeded paged problem for ``spec`` on ``device``."""
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(int(seed))
    B, R, Hq, Hkv, D, bs = spec.B, spec.R, spec.Hq, spec.Hkv, spec.D, spec.block_size
    assert len(spec.ctx) == B and Hq % Hkv == 0

    q = torch.randn((B, R, Hq, D), generator=g, device=dev, dtype=torch.float32)
    if spec.q_mult != 1.0:
        q.mul_(spec.q_mult)
    if spec.q_dtype in ("bf16", "f16"):
        q = q.to(torch.bfloat16 if spec.q_dtype == "bf16" else torch.float16)

    pages_per_req = [-(-int(c) // bs) for c in spec.ctx]
    n_ref = sum(pages_per_req)
    P = max(n_ref + 1, int(math.ceil(n_ref * spec.pool_factor)))
    st = _TORCH_STORAGE[spec.kv_dtype]
    quant = spec.kv_dtype in ("int8", "fp8")

    def draw_pool():
        codes = torch.empty((P, Hkv, bs, D), dtype=st, device=dev)
        scales = torch.empty((P, Hkv, bs), dtype=torch.float32, device=dev) if quant else None
        for p0 in range(0, P, chunk_pages):
            p1 = min(P, p0 + chunk_pages)
            x = torch.randn((p1 - p0, Hkv, bs, D), generator=g, device=dev, dtype=torch.float32)
            c, s = _encode_rows(x, spec.kv_dtype)
            codes[p0:p1] = c
            if quant:
                scales[p0:p1] = s
            del x, c, s
        return codes, scales

    k, ks = draw_pool()
    v, vs = draw_pool()
    sinks = torch.randn((Hq,), generator=g, device=dev, dtype=torch.float32) if spec.sinks else None
    perm = torch.randperm(P, generator=g, device=dev).to(torch.int32)

    max_pages = spec.max_pages
    spare = perm[n_ref]
    table = torch.empty((B, max_pages), dtype=torch.int32, device=dev)
    table[:] = spare
    off = 0
    for b, n in enumerate(pages_per_req):
        table[b, :n] = perm[off:off + n]
        off += n

    if spec.poison:
        pv = _poison_value(spec.kv_dtype)
        spare_pages = perm[n_ref:].long()
        tails = []   # (page, first poisoned slot)
        for b, c in enumerate(spec.ctx):
            c = int(c)
            if c % bs:
                tails.append((int(table[b, c // bs]), c % bs))
        for codes in (k, v):
            if pv is not None:
                codes[spare_pages] = pv
                for page, s0 in tails:
                    codes[page, :, s0:, :] = pv
        if quant:
            for sc in (ks, vs):
                sc[spare_pages] = float("nan")
                for page, s0 in tails:
                    sc[page, :, s0:] = float("nan")

    if spec.v_layout == "transposed":
        v = v.transpose(-1, -2).contiguous()

    ctx = torch.tensor(spec.ctx, dtype=torch.int32, device=dev)
    tree = verify_masks(spec, g) if spec.verify != "causal" else None
    return Problem(spec=spec, paged=True, q=q, k=k, v=v, k_scale=ks, v_scale=vs,
                   page_table=table, ctx=ctx, sinks=sinks, kv_capacity=max_pages * bs,
                   tree_mask=None if tree is None else tree.to(dev))


def verify_masks(spec: ProblemSpec, g: torch.Generator) -> torch.Tensor:
    """int64 [B][R][W] verify masks of ``spec.verify`` (recipe step 7); bit i
    of row j: draft i is visible to row j."""
    B, R = spec.B, spec.R
    W = (R + 63) // 64
    assert R <= 256
    rows = []
    for _ in range(B):
        m = []
        for i in range(R):
            if spec.verify == "chain":
                w = (1 << (i + 1)) - 1
            elif spec.verify == "independent":
                w = 1 << i
            elif spec.verify == "tree":
                par = int(torch.randint(-1, i, (1,), generator=g, device=g.device)) if i > 0 else -1
                w = (m[par] if par >= 0 else 0) | (1 << i)
            else:
                raise ValueError(spec.verify)
            m.append(w)
        words = []
        for w in m:
            ws = [(w >> (64 * k)) & ((1 << 64) - 1) for k in range(W)]
            words.append([x - (1 << 64) if x >= 1 << 63 else x for x in ws])   # as int64 bits
        rows.append(words)
    return torch.tensor(rows, dtype=torch.int64)


def to_contiguous(p: Problem, capacity: Optional[int] = None) -> Problem:
    """Re-lay a paged problem out as contiguous [B][Hkv][cap][D] rows (same values).

    Slots at or beyond a request's context are filled with the poison pattern.
    """
    assert p.paged
    spec = p.spec
    B, Hkv, D, bs = spec.B, spec.Hkv, spec.D, spec.block_size
    cap = capacity or p.kv_capacity
    assert cap >= spec.max_ctx
    dev = p.device
    quant = spec.kv_dtype in ("int8", "fp8")
    v_plain = p.v if spec.v_layout == "plain" else p.v.transpose(-1, -2)
    pv = _poison_value(spec.kv_dtype)
    kc = torch.zeros((B, Hkv, cap, D), dtype=p.k.dtype, device=dev)
    vc = torch.zeros((B, Hkv, cap, D), dtype=p.v.dtype, device=dev)
    if pv is not None and spec.poison:
        kc[:] = pv
        vc[:] = pv
    ksc = vsc = None
    if quant:
        ksc = torch.full((B, Hkv, cap), float("nan"), dtype=torch.float32, device=dev)
        vsc = torch.full((B, Hkv, cap), float("nan"), dtype=torch.float32, device=dev)
    for b in range(B):
        c = int(spec.ctx[b])
        if c == 0:
            continue
        t = torch.arange(c, device=dev)
        pages = p.page_table[b, (t // bs)].long()
        slots = t % bs
        kc[b, :, :c, :] = p.k[pages, :, slots, :].transpose(0, 1)
        vc[b, :, :c, :] = v_plain[pages, :, slots, :].transpose(0, 1)
        if quant:
            ksc[b, :, :c] = p.k_scale[pages, :, slots].transpose(0, 1)
            vsc[b, :, :c] = p.v_scale[pages, :, slots].transpose(0, 1)
    if spec.v_layout == "transposed":
        vc = vc.transpose(-1, -2).contiguous()
    return dataclasses.replace(p, paged=False, k=kc, v=vc, k_scale=ksc, v_scale=vsc,
                               page_table=None, kv_capacity=cap)


def extract_request(p: Problem, b: int) -> Problem:
    """A one-request paged problem holding only the pages request ``b`` references.

    Pages are copied to the host in the order of the request's page-table row and
    the new table is 0..n-1; values, scales and the poisoned tail are unchanged.
    """
    assert p.paged
    spec = p.spec
    c = int(spec.ctx[b])
    n = max(1, -(-c // spec.block_size))
    rows = p.page_table[b, :n].long()
    sub = spec.with_(ctx=(c,), B=1, name=spec.name + f"_req{b}")
    return Problem(
        spec=sub, paged=True,
        q=p.q[b:b + 1].cpu(), k=p.k[rows].cpu(), v=p.v[rows].cpu(),
        k_scale=None if p.k_scale is None else p.k_scale[rows].cpu(),
        v_scale=None if p.v_scale is None else p.v_scale[rows].cpu(),
        page_table=torch.arange(n, dtype=torch.int32).view(1, n),
        ctx=torch.tensor([c], dtype=torch.int32),
        sinks=None if p.sinks is None else p.sinks.cpu(),
        kv_capacity=n * spec.block_size,
        tree_mask=None if p.tree_mask is None else p.tree_mask[b:b + 1].cpu())
