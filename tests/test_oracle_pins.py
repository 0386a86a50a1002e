"""Pins of the fp64 oracle against things other than itself.

* brute force: dense softmax(scale * Q K^T + mask) V with an explicit mask
  matrix, scipy's softmax, and torch's own bf16 / fp8 decoders, on logical
  (un-paged) arrays that the test scatters into a paged pool itself;
* closed forms: identical keys give the mean of the visible values (and the
  position-coded value pins every causal / window bound to the token), the
  sink variant of that, one-hot logits select one value row exactly;
* split algebra: per-split statistics merged by either rule equal the plain
  result, for any number of splits, including empty splits;
* layout invariance: page size, page permutation and V layout leave the
  result bitwise unchanged.
"""

from __future__ import annotations

import itertools
import math

import numpy as np
import pytest
import scipy.special
import torch

import oracle


# ---------------------------------------------------------------------------
# tiny problems built from logical codes, scattered into a pool by the test

def _random_codes(rng, shape, kv_dtype):
    if kv_dtype == "f32":
        return rng.standard_normal(shape).astype(np.float32)
    if kv_dtype == "bf16":
        x = torch.from_numpy(rng.standard_normal(shape).astype(np.float32)).to(torch.bfloat16)
        return x.view(torch.int16).numpy().view(np.uint16)
    if kv_dtype == "int8":
        return rng.integers(-127, 128, size=shape).astype(np.int8)
    if kv_dtype == "fp8":
        c = rng.integers(0, 256, size=shape).astype(np.uint8)
        c[(c & 0x7F) == 0x7F] = 0x38        # replace the two NaN codes by 1.0
        return c
    raise ValueError(kv_dtype)


def _torch_decode(codes, kv_dtype):
    """Library decoders (torch), independent of the oracle's codecs."""
    if kv_dtype == "f32":
        return codes.astype(np.float64)
    if kv_dtype == "bf16":
        return torch.from_numpy(codes.view(np.int16)).view(torch.bfloat16).double().numpy()
    if kv_dtype == "int8":
        return codes.astype(np.float64)
    if kv_dtype == "fp8":
        return torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    if kv_dtype == "f16":
        return torch.from_numpy(codes.view(np.int16)).view(torch.float16).double().numpy()
    raise ValueError(kv_dtype)


def _build_tiny(rng, *, B, R, Hq, Hkv, D, ctx, bs, kv_dtype, q_dtype, v_layout, sinks):
    Tmax = max(max(ctx), 1)
    Kc = _random_codes(rng, (B, Hkv, Tmax, D), kv_dtype)
    Vc = _random_codes(rng, (B, Hkv, Tmax, D), kv_dtype)
    quant = kv_dtype in ("int8", "fp8")
    Ks = (rng.uniform(0.01, 0.05, size=(B, Hkv, Tmax)).astype(np.float32) if quant else None)
    Vs = (rng.uniform(0.01, 0.05, size=(B, Hkv, Tmax)).astype(np.float32) if quant else None)
    qv = rng.standard_normal((B, R, Hq, D)).astype(np.float32)
    if q_dtype in ("bf16", "f16"):
        qt = torch.bfloat16 if q_dtype == "bf16" else torch.float16
        q = torch.from_numpy(qv).to(qt).view(torch.int16).numpy().view(np.uint16)
    else:
        q = qv
    sk = rng.standard_normal(Hq).astype(np.float32) if sinks else None
    # scatter into a shuffled page pool
    npg = [-(-c // bs) for c in ctx]
    P = sum(npg) + 3
    perm = rng.permutation(P)
    maxp = max(max(npg), 1)
    table = np.full((B, maxp), perm[-1], dtype=np.int32)
    kpool = np.zeros((P, Hkv, bs, D), dtype=Kc.dtype)
    vpool = np.zeros((P, Hkv, bs, D), dtype=Vc.dtype)
    kspool = np.full((P, Hkv, bs), np.nan, dtype=np.float32) if quant else None
    vspool = np.full((P, Hkv, bs), np.nan, dtype=np.float32) if quant else None
    off = 0
    for b in range(B):
        for i in range(npg[b]):
            page = perm[off]
            off += 1
            table[b, i] = page
            for s in range(bs):
                t = i * bs + s
                if t < ctx[b]:
                    kpool[page, :, s] = Kc[b, :, t]
                    vpool[page, :, s] = Vc[b, :, t]
                    if quant:
                        kspool[page, :, s] = Ks[b, :, t]
                        vspool[page, :, s] = Vs[b, :, t]
    if v_layout == "transposed":
        vpool = np.ascontiguousarray(np.swapaxes(vpool, -1, -2))
    arrays = dict(q=q, k=kpool, v=vpool, k_scale=kspool, v_scale=vspool, page_table=table,
                  ctx=np.array(ctx, dtype=np.int32), sinks=sk)
    logical = dict(Kc=Kc, Vc=Vc, Ks=Ks, Vs=Vs, q=q, sinks=sk)
    return arrays, logical


def _brute_force(logical, *, B, R, Hq, Hkv, D, ctx, causal, window, scale, kv_dtype, q_dtype):
    K = _torch_decode(logical["Kc"], kv_dtype)
    V = _torch_decode(logical["Vc"], kv_dtype)
    if logical["Ks"] is not None:
        K = K * logical["Ks"].astype(np.float64)[..., None]
        V = V * logical["Vs"].astype(np.float64)[..., None]
    q = _torch_decode(logical["q"], q_dtype) if q_dtype in ("bf16", "f16") else logical["q"].astype(np.float64)
    G = Hq // Hkv
    Tmax = K.shape[2]
    out = np.zeros((B, R, Hq, D))
    t = np.arange(Tmax)
    for b in range(B):
        for j in range(R):
            p = ctx[b] - R + j if causal else ctx[b] - 1
            mask = (t < ctx[b]) & (t <= p)
            if window > 0:
                mask &= t > p - window
            if not mask.any():
                continue
            for h in range(Hq):
                g = h // G
                logits = scale * (K[b, g] @ q[b, j, h])
                logits = np.where(mask, logits, -np.inf)
                if logical["sinks"] is not None:
                    logits = np.append(logits, float(logical["sinks"][h]))
                pr = scipy.special.softmax(logits)
                out[b, j, h] = pr[:Tmax] @ V[b, g]
    return out


CASES = [
    # B, R, Hq, Hkv, D, ctx, bs, kv, q, causal, window, sinks, v_layout
    (1, 1, 2, 1, 4, (1,), 16, "f32", "f32", False, 0, False, "plain"),
    (2, 1, 4, 2, 8, (37, 5), 16, "f32", "f32", False, 0, False, "plain"),
    (3, 3, 6, 2, 4, (40, 16, 2), 3, "bf16", "bf16", True, 0, False, "transposed"),
    (2, 3, 3, 3, 8, (17, 0), 1, "int8", "bf16", True, 5, False, "plain"),
    (2, 3, 4, 1, 8, (33, 9), 2, "fp8", "bf16", True, 4, True, "transposed"),
    (1, 3, 2, 1, 4, (2,), 16, "fp8", "bf16", True, 0, True, "plain"),      # ctx < R
    (2, 1, 4, 4, 4, (23, 31), 16, "int8", "f32", False, 7, True, "plain"),
    (1, 3, 4, 2, 8, (40,), 3, "bf16", "f32", False, 0, True, "transposed"),  # non-causal MTP
    (2, 4, 4, 1, 8, (29, 7), 4, "fp8", "f16", True, 0, False, "plain"),      # fp16 queries
    (1, 2, 4, 2, 8, (25,), 16, "int8", "f16", True, 6, True, "transposed"),
]


@pytest.mark.parametrize("case", CASES, ids=[f"case{i}" for i in range(len(CASES))])
def test_oracle_matches_brute_force(case):
    B, R, Hq, Hkv, D, ctx, bs, kv, qd, causal, window, sinks, vl = case
    rng = np.random.default_rng(1234 + sum(ctx))
    arrays, logical = _build_tiny(rng, B=B, R=R, Hq=Hq, Hkv=Hkv, D=D, ctx=ctx, bs=bs,
                                  kv_dtype=kv, q_dtype=qd, v_layout=vl, sinks=sinks)
    scale = 1.0 / math.sqrt(D)
    ref = _brute_force(logical, B=B, R=R, Hq=Hq, Hkv=Hkv, D=D, ctx=ctx, causal=causal,
                       window=window, scale=scale, kv_dtype=kv, q_dtype=qd)
    got = oracle.decode_attention(arrays, R=R, Hq=Hq, Hkv=Hkv, D=D, causal=causal, window=window,
                                  scale=scale, q_dtype=qd, kv_dtype=kv, paged=True, block_size=bs,
                                  v_layout=vl, has_sink=sinks)
    assert np.isfinite(got).all()
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# closed forms

def _const_key_problem(ctx, R, D=4, Hq=2, Hkv=1, bs=5, sinks=None, v_layout="plain"):
    """All keys equal (so every logit is equal); V[t][0] = t, V[t][1] = 1."""
    n = max(ctx, 1)
    npg = -(-n // bs)
    k = np.zeros((npg, Hkv, bs, D), dtype=np.float32)
    k[...] = np.array([0.5, -1.0, 0.25, 2.0][:D], dtype=np.float32)
    v = np.zeros((npg, Hkv, bs, D), dtype=np.float32)
    for t in range(npg * bs):
        v[t // bs, :, t % bs, 0] = t
        v[t // bs, :, t % bs, 1] = 1.0
    if v_layout == "transposed":
        v = np.ascontiguousarray(np.swapaxes(v, -1, -2))
    q = np.ones((1, R, Hq, D), dtype=np.float32)
    table = np.arange(npg, dtype=np.int32)[::-1].copy().reshape(1, npg)
    # reverse the table and the values consistently: logical page i is pool page npg-1-i
    k = k[::-1].copy()
    v = v[::-1].copy()
    arrays = dict(q=q, k=k, v=v, page_table=table, ctx=np.array([ctx], dtype=np.int32),
                  sinks=None if sinks is None else np.full(Hq, sinks, dtype=np.float32))
    return arrays


@pytest.mark.parametrize("ctx,R,causal,window", [
    (1, 1, False, 0), (23, 1, False, 0), (23, 4, True, 0), (23, 4, True, 3), (23, 4, True, 1),
    (23, 4, False, 6), (3, 4, True, 0), (64, 16, True, 0), (64, 16, True, 50), (100, 4, True, 100),
])
@pytest.mark.parametrize("v_layout", ["plain", "transposed"])
def test_identical_keys_give_mean_of_visible_values(ctx, R, causal, window, v_layout):
    arrays = _const_key_problem(ctx, R, v_layout=v_layout)
    out = oracle.decode_attention(arrays, R=R, Hq=2, Hkv=1, D=4, causal=causal, window=window,
                                  scale=0.5, q_dtype="f32", kv_dtype="f32", paged=True,
                                  block_size=5, v_layout=v_layout, has_sink=False)
    for j in range(R):
        p = ctx - R + j if causal else ctx - 1
        lo = max(0, p - window + 1) if window else 0
        hi = min(p, ctx - 1)
        if hi < lo:
            assert np.all(out[0, j] == 0)
            continue
        # mean of t over [lo, hi] is (lo + hi) / 2; the constant column averages to 1
        np.testing.assert_allclose(out[0, j, :, 0], (lo + hi) / 2.0, rtol=0, atol=1e-12)
        np.testing.assert_allclose(out[0, j, :, 1], 1.0, rtol=0, atol=1e-14)


def _as_int64_bits(words):
    """Masks (Python ints, one per row) -> int64 [B][R][W] words, W = ceil(R / 64)."""
    W = max(1, -(-len(words[0]) // 64))
    def split(w):
        ws = [(w >> (64 * k)) & ((1 << 64) - 1) for k in range(W)]
        return [x - (1 << 64) if x >= 1 << 63 else x for x in ws]
    return np.array([[split(w) for w in row] for row in words], dtype=np.int64)


@pytest.mark.parametrize("ctx,R,kind,window", [
    (23, 4, "independent", 0), (23, 4, "tree", 0), (64, 16, "tree", 0), (64, 16, "independent", 0),
    (3, 4, "tree", 0), (4, 4, "independent", 0), (70, 64, "tree", 0), (70, 64, "high_bits", 0),
    (300, 130, "tree", 0), (300, 130, "independent", 0), (260, 256, "high_bits", 0), (100, 200, "tree", 0),
    (64, 16, "tree", 9), (300, 130, "tree", 40), (70, 64, "independent", 100),
])
def test_identical_keys_under_verify_masks_give_mean_of_visible_values(ctx, R, kind, window):
    """Equal logits: each row averages exactly the keys its mask lets through,
    so the position-coded column pins the visible set (prefix keys below
    ctx - R, the masked drafts, none after the row's own position)."""
    rng = np.random.default_rng(ctx + R)
    words = []
    for i in range(R):
        if kind == "independent":
            w = 1 << i
        elif kind == "high_bits":                  # bits after the row: no effect
            w = ((1 << R) - 1) ^ ((1 << i) - 1)
        else:
            par = int(rng.integers(-1, i)) if i > 0 else -1
            w = (words[par] if par >= 0 else 0) | (1 << i)
        words.append(w)
    arrays = _const_key_problem(ctx, R)
    arrays["tree_mask"] = _as_int64_bits([words])
    out = oracle.decode_attention(arrays, R=R, Hq=2, Hkv=1, D=4, causal=True, window=window,
                                  scale=0.5, q_dtype="f32", kv_dtype="f32", paged=True,
                                  block_size=5, v_layout="plain", has_sink=False)
    base = ctx - R
    for j in range(R):
        lo = max(0, base + j - window + 1) if window else 0      # the window, on top of the mask
        vis = [t for t in range(lo, max(base, 0))]
        vis += [base + i for i in range(j + 1) if base + i >= max(lo, 0) and (words[j] >> i) & 1]
        if not vis:
            assert np.all(out[0, j] == 0)
            continue
        np.testing.assert_allclose(out[0, j, :, 0], float(np.mean(vis)), rtol=0, atol=1e-12)
        np.testing.assert_allclose(out[0, j, :, 1], 1.0, rtol=0, atol=1e-14)


def test_chain_mask_equals_causal():
    rng = np.random.default_rng(77)
    arrays, _ = _build_tiny(rng, B=2, R=5, Hq=4, Hkv=2, D=8, ctx=(40, 6), bs=4, kv_dtype="fp8",
                            q_dtype="bf16", v_layout="plain", sinks=True)
    kw = dict(R=5, Hq=4, Hkv=2, D=8, causal=True, window=0, scale=0.3, q_dtype="bf16", kv_dtype="fp8",
              paged=True, block_size=4, v_layout="plain", has_sink=True)
    plain = oracle.decode_attention(arrays, **kw)
    arrays["tree_mask"] = _as_int64_bits([[(1 << (j + 1)) - 1 for j in range(5)]] * 2)
    chain = oracle.decode_attention(arrays, **kw)
    np.testing.assert_array_equal(chain, plain)


def test_independent_rows_equal_single_row_problems():
    """Independent-batch verify: row j equals a one-row, non-causal problem over
    the prefix and draft j alone (the cache rebuilt without the other drafts)."""
    rng = np.random.default_rng(78)
    R, ctx, D = 4, 29, 8
    arrays, logical = _build_tiny(rng, B=1, R=R, Hq=2, Hkv=1, D=D, ctx=(ctx,), bs=4, kv_dtype="int8",
                                  q_dtype="f32", v_layout="plain", sinks=False)
    arrays["tree_mask"] = _as_int64_bits([[1 << j for j in range(R)]])
    out = oracle.decode_attention(arrays, R=R, Hq=2, Hkv=1, D=D, causal=True, window=0, scale=0.4,
                                  q_dtype="f32", kv_dtype="int8", paged=True, block_size=4,
                                  v_layout="plain", has_sink=False)
    base = ctx - R
    for j in range(R):
        keep = list(range(base)) + [base + j]
        n = len(keep)
        # pool pages of one token each: [n][Hkv][1][D]
        k = np.ascontiguousarray(logical["Kc"][0][:, keep].transpose(1, 0, 2)[:, :, None, :])
        v = np.ascontiguousarray(logical["Vc"][0][:, keep].transpose(1, 0, 2)[:, :, None, :])
        one = dict(q=logical["q"][:, j:j + 1], k=k, v=v,
                   k_scale=np.ascontiguousarray(logical["Ks"][0][:, keep].T[:, :, None]),
                   v_scale=np.ascontiguousarray(logical["Vs"][0][:, keep].T[:, :, None]),
                   page_table=np.arange(n, dtype=np.int32).reshape(1, n),
                   ctx=np.array([n], dtype=np.int32), sinks=None)
        ref = oracle.decode_attention(one, R=1, Hq=2, Hkv=1, D=D, causal=False, window=0, scale=0.4,
                                      q_dtype="f32", kv_dtype="int8", paged=True, block_size=1,
                                      v_layout="plain", has_sink=False)
        np.testing.assert_allclose(out[0, j], ref[0, 0], rtol=0, atol=1e-13)


@pytest.mark.parametrize("sink", [-3.0, 0.0, 0.7, 5.0])
def test_identical_keys_with_sink_closed_form(sink):
    ctx, R = 19, 2
    arrays = _const_key_problem(ctx, R, sinks=sink)
    scale = 0.5
    c = scale * float(np.dot(np.ones(4), [0.5, -1.0, 0.25, 2.0]))   # the common logit
    out = oracle.decode_attention(arrays, R=R, Hq=2, Hkv=1, D=4, causal=True, window=0,
                                  scale=scale, q_dtype="f32", kv_dtype="f32", paged=True,
                                  block_size=5, v_layout="plain", has_sink=True)
    for j in range(R):
        n = ctx - R + j + 1
        mean_t = (n - 1) / 2.0
        sk = float(np.float32(sink))                  # sinks are stored as fp32
        w = n * math.exp(c) / (n * math.exp(c) + math.exp(sk))
        np.testing.assert_allclose(out[0, j, :, 0], w * mean_t, rtol=1e-13, atol=0)
        np.testing.assert_allclose(out[0, j, :, 1], w, rtol=1e-13, atol=0)


def test_sink_does_not_revive_an_empty_row():
    arrays = _const_key_problem(2, 4, sinks=1.0)
    out = oracle.decode_attention(arrays, R=4, Hq=2, Hkv=1, D=4, causal=True, window=0, scale=0.5,
                                  q_dtype="f32", kv_dtype="f32", paged=True, block_size=5,
                                  v_layout="plain", has_sink=True)
    assert np.all(out[0, 0] == 0) and np.all(out[0, 1] == 0)   # rows at positions -2, -1
    assert np.all(out[0, 2, :, 1] > 0)


@pytest.mark.parametrize("j_hot", [0, 7, 22])
def test_one_hot_logit_selects_one_value_row(j_hot):
    rng = np.random.default_rng(j_hot)
    n, D, bs = 23, 8, 4
    npg = -(-n // bs)
    k = np.zeros((npg, 1, bs, D), dtype=np.float32)
    k[..., 0] = -400.0
    k[j_hot // bs, 0, j_hot % bs, 0] = 400.0       # logit gap 800 after scale 1
    v = rng.standard_normal((npg, 1, bs, D)).astype(np.float32)
    q = np.zeros((1, 1, 1, D), dtype=np.float32)
    q[..., 0] = 1.0
    arrays = dict(q=q, k=k, v=v, page_table=np.arange(npg, dtype=np.int32).reshape(1, -1),
                  ctx=np.array([n], dtype=np.int32), sinks=None)
    out = oracle.decode_attention(arrays, R=1, Hq=1, Hkv=1, D=D, causal=False, window=0, scale=1.0,
                                  q_dtype="f32", kv_dtype="f32", paged=True, block_size=bs,
                                  v_layout="plain", has_sink=False)
    assert np.array_equal(out[0, 0, 0], v[j_hot // bs, 0, j_hot % bs].astype(np.float64))


# ---------------------------------------------------------------------------
# split algebra

@pytest.mark.parametrize("S", [1, 2, 3, 4, 5, 6, 7, 8, 16, 256])
@pytest.mark.parametrize("sink", [None, 0.3])
def test_split_statistics_merge_to_the_plain_result(S, sink):
    rng = np.random.default_rng(S)
    n, D, R = 1000, 8, 4
    x_all = rng.standard_normal((R, n)) * 3.0
    v = rng.standard_normal((n, D))
    for causal, window in [(True, 0), (True, 300), (False, 0)]:
        bounds = oracle.split_bounds(n, R, causal, window, S)
        for j in range(R):
            lo, hi = oracle.visible_range(n, R, j, causal, window)
            x = x_all[j]
            ref_e = np.exp(x[lo:hi] - max(x[lo:hi].max(), sink if sink is not None else -np.inf))
            den = ref_e.sum() + (np.exp(sink - max(x[lo:hi].max(), sink)) if sink is not None else 0)
            ref = ref_e @ v[lo:hi] / den
            m, l, acc = oracle.split_partials(x, v, bounds, (lo, hi))
            got = oracle.combine_flash(m, l, acc, sink)
            np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-15)
            live = l > 0
            o_s = np.zeros_like(acc)
            o_s[live] = acc[live] / l[live, None]
            lse = np.full(S, -np.inf)
            lse[live] = m[live] + np.log(l[live])
            got2 = oracle.combine_lse(o_s, lse, sink)
            np.testing.assert_allclose(got2, ref, rtol=1e-12, atol=1e-15)


def test_single_split_weight_is_exactly_one():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(50)
    v = rng.standard_normal((50, 3))
    m, l, acc = oracle.split_partials(x, v, [(0, 50)], (0, 50))
    got = oracle.combine_flash(m, l, acc)
    assert np.exp(m[0] - m[0]) == 1.0
    np.testing.assert_array_equal(got, acc[0] / l[0])


@pytest.mark.parametrize("ctx", [0, 1, 63, 64, 65, 2048, 20676, 200000])
@pytest.mark.parametrize("S", [1, 2, 3, 8, 16, 256])
@pytest.mark.parametrize("R,causal,window", [(1, False, 0), (4, True, 0), (4, True, 4096), (16, True, 0)])
def test_split_bounds_partition_the_visible_union(ctx, S, R, causal, window):
    b = oracle.split_bounds(ctx, R, causal, window, S)
    assert len(b) == S
    covered = []
    for lo, hi in b:
        assert lo <= hi
        if hi > lo:
            assert lo % oracle.SPLIT_ALIGN == 0
            covered.append((lo, hi))
    for (a0, a1), (b0, b1) in zip(covered, covered[1:]):
        assert a1 == b0                                  # contiguous, disjoint, in order
    union_lo = min((oracle.visible_range(ctx, R, j, causal, window)[0] for j in range(R)), default=0)
    if ctx > 0 and covered:
        assert covered[0][0] <= union_lo and covered[-1][1] == ctx
        # chunk = ceil(span / S) rounded up to the alignment (design record's chunk rule)
        span = ctx - covered[0][0]
        chunk = -(-(-(-span // S)) // oracle.SPLIT_ALIGN) * oracle.SPLIT_ALIGN
        assert covered[0][1] - covered[0][0] == min(chunk, span)
    if ctx == 2048 and S == 8 and window == 0:
        assert [hi - lo for lo, hi in b] == [256] * 8


# ---------------------------------------------------------------------------
# layout invariance (through skvgen problems)

def test_layout_and_page_size_invariance():
    import dataclasses
    from skvgen import make_problem, small_spec
    spec = small_spec(4, ctx=(300, 77), B=2)
    p = make_problem(spec, seed=11)
    base = p.host_arrays()
    kw = dict(R=spec.R, Hq=spec.Hq, Hkv=spec.Hkv, D=spec.D, causal=True, window=0,
              scale=spec.scale, q_dtype="bf16", kv_dtype="fp8", has_sink=False)
    ref = oracle.decode_attention(base, paged=True, block_size=16, v_layout="plain", **kw)
    # transposed V: same codes, other layout
    tv = dict(base)
    tv["v"] = np.ascontiguousarray(np.swapaxes(base["v"], -1, -2))
    out = oracle.decode_attention(tv, paged=True, block_size=16, v_layout="transposed", **kw)
    assert np.array_equal(out, ref)
    # re-page with page size 4 and a new permutation
    rng = np.random.default_rng(5)
    for new_bs in (4, 32, 1):
        arr = _repage(base, spec, new_bs, rng)
        out = oracle.decode_attention(arr, paged=True, block_size=new_bs, v_layout="plain", **kw)
        assert np.array_equal(out, ref), new_bs
    # contiguous
    from skvgen import to_contiguous
    c = to_contiguous(p).host_arrays()
    out = oracle.decode_attention(c, paged=False, block_size=16, v_layout="plain", **kw)
    assert np.array_equal(out, ref)


def _repage(arrays, spec, new_bs, rng):
    bs = spec.block_size
    ctx = arrays["ctx"]
    B = len(ctx)
    k, v, ks, vs, tab = (arrays[n] for n in ("k", "v", "k_scale", "v_scale", "page_table"))
    npg = [-(-int(c) // new_bs) for c in ctx]
    P = sum(npg) + 1
    perm = rng.permutation(P)
    nk = np.zeros((P, spec.Hkv, new_bs, spec.D), dtype=k.dtype)
    nv = np.zeros_like(nk)
    nks = np.zeros((P, spec.Hkv, new_bs), dtype=np.float32)
    nvs = np.zeros_like(nks)
    table = np.full((B, max(npg)), perm[-1], dtype=np.int32)
    off = 0
    for b in range(B):
        for i in range(npg[b]):
            page = perm[off]
            off += 1
            table[b, i] = page
            for s in range(new_bs):
                t = i * new_bs + s
                if t >= ctx[b]:
                    continue
                src = tab[b, t // bs]
                nk[page, :, s] = k[src, :, t % bs]
                nv[page, :, s] = v[src, :, t % bs]
                nks[page, :, s] = ks[src, :, t % bs]
                nvs[page, :, s] = vs[src, :, t % bs]
    out = dict(arrays)
    out.update(k=nk, v=nv, k_scale=nks, v_scale=nvs, page_table=table)
    return out
