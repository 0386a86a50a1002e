"""fp64 decode attention and an fp64 model of split-KV, written from the pages.

Test infrastructure only (see the package docstring).

Sources (page titles and sections; no code is printed on any of them):

* tiny-llm #11, "split-KV decode attention design record", section "Design":
  one workgroup per (head, split) computes its own token range from the device
  visible length with chunk = ceil(visible / splits) and emits the local online-
  softmax statistics (m_i, l_i, acc_i); a combine step merges them "by the
  flash-decoding formula". Section "points for reviewer decision" (Q3): the
  single-split result is normalized by 1/(l + 1e-9) and exp(0) = 1.
* hipfire #760, "split packed-Q8 verifier KV scans", Summary: the live causal
  prefix of a multi-row verifier is partitioned across 2/4/8 workgroups, each
  emitting a normalized output plus its log-sum-exp, merged by a stable
  max-LSE reduction.
* aiter #5628, "tune MTP work budgets and planned reduction": MTP rows with
  causal masking (intro, Performance), sliding windows and attention sinks
  ("sink normalization", "masked fallback", Changes), windowed work capped by
  the causal-window union and tile alignment (Changes), BF16 Q/O with FP8 KV
  and per-token FP32 scales (Performance).

Readings taken where the pages are silent:

* a request's context length counts its R query tokens; causal row j sits at
  position p_j = ctx - R + j and sees keys t <= p_j; a non-causal row sees all
  ctx keys (p_j = ctx - 1);
* a window W keeps the last W keys up to and including p_j: t > p_j - W;
* query head h reads KV head h // (Hq / Hkv);
* a sink is one extra logit per query head in the softmax denominator, with no
  value vector, taken in natural-log units and not multiplied by the scale;
* a row that sees no key outputs 0, with or without a sink;
* split boundaries are aligned to ``SPLIT_ALIGN`` tokens and cover only the
  union of the rows' visible ranges (window start aligned down);
* verify masks (hipfire #760, Summary, names tree-structured and
  independent-batch verification without defining them): the R query tokens
  are drafts at keys ctx - R .. ctx - 1, ancestors before descendants; row j
  sees the prefix t < ctx - R and draft key ctx - R + i only when bit i of its
  mask word is set, and never a key after its own position.

The plain attention below uses exact division (no 1e-9 term: its relative
effect is below 1e-9 whenever the denominator is at least 1, which holds since
the maximal term is e^0 = 1).
"""

from __future__ import annotations

from typing import List, Optional, Tuple

import numpy as np

from .codecs import decode_storage

SPLIT_ALIGN = 64


def row_positions(ctx: int, R: int, causal: bool) -> List[int]:
    """Absolute position of each of the R query rows of a request."""
    if causal:
        return [ctx - R + j for j in range(R)]
    return [ctx - 1] * R


def visible_range(ctx: int, R: int, j: int, causal: bool, window: int) -> Tuple[int, int]:
    """Half-open key range [lo, hi) that query row j sees; empty when lo >= hi."""
    p = row_positions(ctx, R, causal)[j]
    hi = min(p + 1, ctx)
    lo = 0 if window <= 0 else max(0, p - window + 1)
    return max(lo, 0), max(hi, 0)


def verify_keys(ctx: int, R: int, j: int, mask_word: int, lo: int, hi: int) -> np.ndarray:
    """Keys of [lo, hi) that causal row j sees under its verify mask word:
    every prefix key t < ctx - R, and draft key ctx - R + i when bit i is set."""
    base = ctx - R
    keys = [t for t in range(lo, hi) if t < base or (mask_word >> (t - base)) & 1]
    return np.array(keys, dtype=np.int64)


def _dequant(codes, scales, dtype):
    x = decode_storage(codes, dtype)
    if scales is not None and dtype in ("int8", "fp8"):
        x = x * np.asarray(scales, dtype=np.float32).astype(np.float64)[..., None]
    return x


def gather_request(arrays: dict, b: int, n: int, *, Hkv: int, D: int, kv_dtype: str,
                   paged: bool, block_size: int, v_layout: str) -> Tuple[np.ndarray, np.ndarray]:
    """Logical, dequantized K and V rows of request b: two float64 [Hkv][n][D].

    Paged layout: K pool [page][Hkv][bs][D]; V pool the same ("plain") or
    [page][Hkv][D][bs] ("transposed"); scales [page][Hkv][bs]. Logical token t
    lives in page page_table[b][t // bs] at slot t % bs.
    Contiguous layout: K [B][Hkv][cap][D]; V [B][Hkv][cap][D] or [B][Hkv][D][cap];
    scales [B][Hkv][cap].
    """
    k, v = arrays["k"], arrays["v"]
    ks, vs = arrays.get("k_scale"), arrays.get("v_scale")
    if paged:
        npg = -(-n // block_size)
        pages = np.asarray(arrays["page_table"][b, :npg], dtype=np.int64)
        kp = k[pages]                                   # [npg][Hkv][bs][D]
        vp = v[pages]
        if v_layout == "transposed":
            vp = np.swapaxes(vp, -1, -2)                # -> [npg][Hkv][bs][D]
        kp = np.swapaxes(kp, 0, 1).reshape(Hkv, npg * block_size, D)[:, :n]
        vp = np.swapaxes(vp, 0, 1).reshape(Hkv, npg * block_size, D)[:, :n]
        ksc = vsc = None
        if ks is not None:
            ksc = np.swapaxes(ks[pages], 0, 1).reshape(Hkv, npg * block_size)[:, :n]
            vsc = np.swapaxes(vs[pages], 0, 1).reshape(Hkv, npg * block_size)[:, :n]
    else:
        kp = k[b][:, :n]
        vb = v[b]
        if v_layout == "transposed":
            vb = np.swapaxes(vb, -1, -2)
        vp = vb[:, :n]
        ksc = None if ks is None else ks[b][:, :n]
        vsc = None if vs is None else vs[b][:, :n]
    return _dequant(kp, ksc, kv_dtype), _dequant(vp, vsc, kv_dtype)


def decode_attention(arrays: dict, *, R: int, Hq: int, Hkv: int, D: int, causal: bool,
                     window: int, scale: float, q_dtype: str, kv_dtype: str, paged: bool,
                     block_size: int, v_layout: str, has_sink: bool,
                     requests: Optional[List[int]] = None) -> np.ndarray:
    """O[b][j][h][:] = softmax over visible t of scale * <q, k_t> (with sink) applied to V.

    Two-pass softmax in float64 over the gathered, dequantized cache. Returns a
    float64 array [len(requests)][R][Hq][D] (all requests by default). With
    ``arrays["tree_mask"]`` (int64 [B][R] or [B][R][W] bit patterns, word k
    holding drafts 64k .. 64k + 63) the visible keys of a causal row are
    further restricted by its verify mask (``verify_keys``).
    """
    q = decode_storage(arrays["q"], q_dtype)
    ctx = np.asarray(arrays["ctx"], dtype=np.int64)
    sinks = None
    if has_sink:
        sinks = np.asarray(arrays["sinks"], dtype=np.float32).astype(np.float64)
    G = Hq // Hkv
    tree = arrays.get("tree_mask")
    reqs = list(range(q.shape[0])) if requests is None else list(requests)
    out = np.zeros((len(reqs), R, Hq, D), dtype=np.float64)
    for i, b in enumerate(reqs):
        n = int(ctx[b])
        if n <= 0:
            continue
        K, V = gather_request(arrays, b, n, Hkv=Hkv, D=D, kv_dtype=kv_dtype, paged=paged,
                              block_size=block_size, v_layout=v_layout)
        for j in range(R):
            lo, hi = visible_range(n, R, j, causal, window)
            keys = np.arange(lo, hi)
            if tree is not None:
                words = np.asarray(tree[b, j]).reshape(-1)          # [W] 64-bit words, word k = drafts 64k..
                mask = sum((int(w) & ((1 << 64) - 1)) << (64 * k) for k, w in enumerate(words))
                keys = verify_keys(n, R, j, mask, lo, hi)
            if keys.size == 0:
                continue                                   # no visible key: O = 0
            for g in range(Hkv):
                heads = slice(g * G, (g + 1) * G)
                x = scale * (q[b, j, heads] @ K[g, keys].T)      # [G][n_vis]
                M = x.max(axis=1)
                if sinks is not None:
                    M = np.maximum(M, sinks[heads])
                e = np.exp(x - M[:, None])
                L = e.sum(axis=1)
                if sinks is not None:
                    L = L + np.exp(sinks[heads] - M)
                out[i, j, heads] = (e @ V[g, keys]) / L[:, None]
    return out


def split_bounds(ctx: int, R: int, causal: bool, window: int, num_splits: int,
                 align: int = SPLIT_ALIGN) -> List[Tuple[int, int]]:
    """Token range [lo, hi) of each split s of one request (possibly empty).

    The split range is the union of the rows' visible ranges, [u_lo, ctx), with
    u_lo the earliest row's window start aligned down to ``align`` (0 without a
    window). chunk = ceil((ctx - u_lo) / S) rounded up to ``align``; split s
    covers [u_lo + s * chunk, min(u_lo + (s + 1) * chunk, ctx)).
    """
    if ctx <= 0:
        return [(0, 0)] * num_splits
    u_lo = 0
    if window > 0:
        p_min = min(row_positions(ctx, R, causal))
        u_lo = max(0, p_min - window + 1)
        u_lo = (u_lo // align) * align
    span = ctx - u_lo
    chunk = -(-span // num_splits)
    chunk = -(-chunk // align) * align
    out = []
    for s in range(num_splits):
        lo = u_lo + s * chunk
        hi = min(u_lo + (s + 1) * chunk, ctx)
        out.append((lo, hi) if lo < hi else (lo, lo))
    return out


def split_partials(x: np.ndarray, v: np.ndarray, bounds: List[Tuple[int, int]],
                   vis: Tuple[int, int]):
    """Per-split statistics of one query row.

    ``x`` holds the row's logits for every key position [0, n), ``v`` the value
    rows [n][D], ``vis`` the row's visible range. For split s with key set
    T_s = [lo_s, hi_s) intersected with ``vis``:
    m_s = max x_t, l_s = sum e^(x_t - m_s), acc_s = sum e^(x_t - m_s) v_t, and an
    empty T_s gives (m, l, acc) = (-inf, 0, 0).
    Returns arrays m [S], l [S], acc [S][D].
    """
    S = len(bounds)
    D = v.shape[1]
    m = np.full(S, -np.inf)
    l = np.zeros(S)
    acc = np.zeros((S, D))
    for s, (lo, hi) in enumerate(bounds):
        a, b = max(lo, vis[0]), min(hi, vis[1])
        if a >= b:
            continue
        xs = x[a:b]
        m[s] = xs.max()
        e = np.exp(xs - m[s])
        l[s] = e.sum()
        acc[s] = e @ v[a:b]
    return m, l, acc


def combine_flash(m: np.ndarray, l: np.ndarray, acc: np.ndarray,
                  sink: Optional[float] = None) -> np.ndarray:
    """Merge raw split statistics: M = max_s m_s (and the sink),
    L = sum_s e^(m_s - M) l_s (+ e^(sink - M)), O = sum_s e^(m_s - M) acc_s / L.
    Empty splits (l = 0) are skipped; if every split is empty, O = 0."""
    live = l > 0
    if not live.any():
        return np.zeros(acc.shape[1])
    M = m[live].max()
    if sink is not None:
        M = max(M, sink)
    w = np.exp(m[live] - M)
    L = (w * l[live]).sum()
    if sink is not None:
        L += np.exp(sink - M)
    return (w[:, None] * acc[live]).sum(axis=0) / L


def combine_lse(o: np.ndarray, lse: np.ndarray, sink: Optional[float] = None) -> np.ndarray:
    """Merge normalized split outputs O_s with their log-sum-exp LSE_s:
    M' = max_s LSE_s (and the sink), O = sum_s e^(LSE_s - M') O_s /
    (sum_s e^(LSE_s - M') + e^(sink - M')). Splits with LSE = -inf are skipped."""
    live = np.isfinite(lse)
    if not live.any():
        return np.zeros(o.shape[1])
    M = lse[live].max()
    if sink is not None:
        M = max(M, sink)
    w = np.exp(lse[live] - M)
    den = w.sum()
    if sink is not None:
        den += np.exp(sink - M)
    return (w[:, None] * o[live]).sum(axis=0) / den
