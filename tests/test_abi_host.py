"""Host-side checks of the C ABI (no GPU needed): the library loads and exports
every function include/skv.h declares, arguments are validated before any
launch, record sizes follow the documented layout, and the split planner
reproduces the pages' example and its own invariants."""

from __future__ import annotations

import ctypes
import os
import re

import pytest
import torch

import split_kv_flash_decode_amd as skv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    if not os.path.exists(skv.LIB_PATH):
        from split_kv_flash_decode_amd import build
        build.build()
    return skv.lib()


def test_library_exports_every_declared_function():
    L = _lib()
    with open(os.path.join(ROOT, "include", "skv.h")) as f:
        text = f.read()
    names = sorted(set(re.findall(r"^\s*(?:int|int64_t|const char\*)\s+(skv_\w+)\(", text, re.M)))
    assert len(names) >= 15, names
    for n in names:
        assert hasattr(L, n), f"{n} missing from libskv.so"
    assert set(names) == set(skv.EXPORTS), "binding and header disagree"
    assert skv.abi_version() == 4


def test_binding_constants_match_the_header():
    with open(os.path.join(ROOT, "include", "skv.h")) as f:
        text = f.read()
    defs = {m.group(1): int(m.group(2)) for m in re.finditer(r"^#define (SKV_\w+) \(?(-?\d+)\)?", text, re.M)}
    codes = [n for n in defs if n == "SKV_OK" or n.startswith("SKV_ERR_")]
    assert len(codes) >= 11, codes
    for n in codes + ["SKV_MAX_SPLITS", "SKV_SPLIT_ALIGN"]:
        assert getattr(skv, n) == defs[n], n
    for n in codes:
        if n != "SKV_OK":
            assert skv.status_str(defs[n]) != "unknown status", n


def _desc(**kw):
    _lib()
    q = torch.zeros(kw.pop("B", 2), kw.pop("R", 4), kw.pop("Hq", 16), kw.pop("D", 128),
                    dtype=kw.pop("qdt", torch.bfloat16))
    kdt = kw.pop("kdt", torch.uint8)
    bs = kw.pop("bs", 16)
    k = torch.zeros(8, kw.pop("Hkv", 1), bs, q.shape[-1], dtype=kdt)
    d = skv.make_desc(q, k, k.clone(), paged=True, causal=True,
                      page_table=torch.zeros(q.shape[0], 4, dtype=torch.int32), **kw)
    return d


def test_validation_codes():
    d = _desc()
    assert skv.validate(d, True, 0) == 0
    assert skv.validate(d, True, 4) == -1                 # partials missing
    bad = _desc()
    bad.head_dim = 96
    assert skv.validate(bad, True, 0) == -2
    bad = _desc(Hkv=2)
    bad.num_q_heads = 15
    assert skv.validate(bad, True, 0) == -2
    bad = _desc()
    bad.block_size = 24
    assert skv.validate(bad, True, 0) == -2
    bad = _desc()
    bad.kv_dtype = 7
    assert skv.validate(bad, True, 0) == -3
    bad = _desc()
    bad.q_dtype = 2
    assert skv.validate(bad, True, 0) == -3
    assert skv.validate(_desc(qdt=torch.float16), True, 0) == 0
    bad = _desc()
    bad.record_dtype = 3                                   # records are fp32 or bf16
    assert skv.validate(bad, True, 0) == -3
    assert skv.validate(_desc(), True, 257) == -4
    assert skv.validate(_desc(), True, -1) == -4
    f32 = _desc(qdt=torch.float32, kdt=torch.float32, impl="mfma")
    assert skv.validate(f32, True, 0) == -6                # matrix-core path needs bf16 Q
    small_page = _desc(bs=8, impl="mfma")
    assert skv.validate(small_page, True, 0) == -6
    assert skv.validate(_desc(bs=8), True, 0) == 0         # auto falls back to the vector kernel


def test_partial_capacity_is_checked():
    d = _desc()
    need = skv.uniform_slots(d, 4)
    assert need == 2 * 4 * 1
    p = skv.Partials(16, 16, 16, need - 1)
    assert skv.lib().skv_validate(ctypes.byref(d), 1, 4, ctypes.byref(p)) == -5
    p = skv.Partials(16, 16, 16, need)
    assert skv.lib().skv_validate(ctypes.byref(d), 1, 4, ctypes.byref(p)) == 0


def test_partial_accumulators_must_be_16_byte_aligned():
    d = _desc()
    need = skv.uniform_slots(d, 4)
    for off in (4, 8, 12):
        p = skv.Partials(16, 16, 4096 + off, need)
        assert skv.lib().skv_validate(ctypes.byref(d), 1, 4, ctypes.byref(p)) == -9
    p = skv.Partials(16, 16, 4096, need)
    assert skv.lib().skv_validate(ctypes.byref(d), 1, 4, ctypes.byref(p)) == 0
    assert "aligned" in skv.status_str(-9)


def test_compute_calls_fail_closed_without_launching():
    d = _desc()
    a = skv.Args()                                        # all NULL
    L = skv.lib()
    assert L.skv_attention_decode_paged(ctypes.byref(d), ctypes.byref(a), None) == -1
    assert L.skv_attention_decode_paged_splitkv(ctypes.byref(d), ctypes.byref(a), 4, None, None) == -1
    assert L.skv_attention_decode_paged(None, ctypes.byref(a), None) == -1
    d.head_dim = 100
    assert L.skv_attention_decode(ctypes.byref(d), ctypes.byref(a), None) == -2
    for s in (0, -3, 1, -4, -8, -9, 99):
        assert isinstance(skv.status_str(s), str) and skv.status_str(s)


def test_verify_masks_need_causal_rows_up_to_the_maximum():
    L = skv.lib()
    fake = 1 << 20                                        # never dereferenced: the call fails first
    for kw, setup in ((dict(), lambda d: setattr(d, "causal", 0)),
                      (dict(R=257, Hq=4), lambda d: None)):
        d = _desc(**kw)
        setup(d)
        a = skv.Args(fake, fake, fake, fake, fake, fake, fake, None, fake, fake)
        assert L.skv_attention_decode_paged(ctypes.byref(d), ctypes.byref(a), None) == -6
        a.tree_mask = None
        assert L.skv_validate(ctypes.byref(d), 1, 0, None) == 0


def test_workspace_sizes():
    d = _desc(B=3, R=4, Hq=16, Hkv=2, D=256)
    m, l, acc = skv.workspace_size(d, 10)
    rho = 4 * 8
    assert m == l == 10 * rho * 4
    assert acc == 10 * rho * 256 * 4
    d16 = _desc(B=3, R=4, Hq=16, Hkv=2, D=256, record_dtype="bf16")
    assert skv.workspace_size(d16, 10) == (m, l, 10 * rho * 256 * 2)


# ---------------------------------------------------------------------------
# planner

def _plan(ctx, R=4, Hkv=1, capacity=None, **kw):
    _lib()
    h = skv.plan_hints(len(ctx), R, Hkv, **kw)
    cap = capacity or skv.plan_capacity(h, ctx)
    meta = torch.zeros(skv.plan_meta_len(len(ctx), cap), dtype=torch.int32)
    info = skv.plan_fill(h, ctx, cap, meta)
    return meta, info, cap


def _decode(meta):
    B, C, n, pmax = (int(x) for x in meta[:4])
    P = meta[4:4 + B].tolist()
    slot0 = meta[4 + B:4 + 2 * B].tolist()
    work = meta[4 + 2 * B:4 + 2 * B + C].tolist()
    return B, C, n, pmax, P, slot0, work


def test_planner_reproduces_the_b200_example():
    # aiter #5628, Changes: B200 / C200k / MTP4 selects 16 partitions per request, capacity 3200
    meta, info, cap = _plan([200000] * 200)
    B, C, n, pmax, P, slot0, work = _decode(meta)
    assert cap == C == 3200 and n == 3200 and set(P) == {16}
    assert info.slots == 3200 and info.max_partitions == 16 == info.min_partitions


def test_planner_budget_floor_for_small_batches():
    # intro of the same page: the base budget is two workgroups per CU (512 on 256 CUs)
    meta, info, cap = _plan([200000] + [1024] * 15)
    B, C, n, pmax, P, slot0, work = _decode(meta)
    assert P[0] == 160                                    # the long request takes the budget, capped
    meta, info, cap = _plan([200000] + [1024] * 15, max_partitions=256)
    assert _decode(meta)[4][0] == 256                     # an explicit cap up to the maximum of 256
    assert all(2 <= p <= 4 for p in P[1:])
    assert n == sum(P) <= C


def test_planner_invariants_and_work_list():
    import random
    rng = random.Random(3)
    for trial in range(30):
        B = rng.randint(1, 40)
        ctx = [rng.choice([0, 1, 63, 64, 65, 1000, 20676, 200000, rng.randint(0, 300000)]) for _ in range(B)]
        R = rng.choice([1, 4, 16])
        window = rng.choice([0, 0, 4096, 100])
        meta, info, cap = _plan(ctx, R=R, Hkv=rng.choice([1, 2, 8]), window=window,
                                partitions_per_request=rng.choice([0, 0, 3, 16]),
                                max_partitions=rng.choice([0, 0, 7]))
        B_, C, n, pmax, P, slot0, work = _decode(meta)
        assert B_ == B and n == sum(P) and C == cap and pmax == max(P)
        assert all(1 <= p <= 256 for p in P)
        acc = 0
        for b in range(B):
            assert slot0[b] == acc
            acc += P[b]
            # never more partitions than 64-key tiles of the window-capped span
            span = ctx[b] if window == 0 else min(ctx[b], window + R - 1 + 63)
            assert P[b] <= max(1, -(-span // 64))
        items = [w for w in work if w >= 0]
        assert len(items) == n and all(w == -1 for w in work[n:])
        assert sorted(items) == sorted(b * 256 + s for b in range(B) for s in range(P[b]))


def test_explicit_partitions_and_caps_take_precedence():
    meta, _, _ = _plan([200000] * 4, partitions_per_request=7)
    assert _decode(meta)[4] == [7] * 4
    meta, _, _ = _plan([200000] * 4, max_partitions=5)
    assert _decode(meta)[4] == [5] * 4
    meta, _, _ = _plan([100] * 4, partitions_per_request=7)
    assert _decode(meta)[4] == [2] * 4                    # only two 64-key tiles


def test_window_caps_planned_work():
    meta, _, _ = _plan([200000], window=4096, min_tokens_per_partition=256)
    P = _decode(meta)[4]
    assert P[0] <= -(-(4096 + 3 + 63) // 256)


def test_refresh_keeps_capacity():
    _lib()
    h = skv.plan_hints(8, 4, 1)
    cap = skv.plan_capacity(h, [1000] * 8)
    meta = torch.zeros(skv.plan_meta_len(8, cap), dtype=torch.int32)
    info = skv.plan_fill(h, [200000] * 8, cap, meta)          # much longer contexts, same capacity
    B, C, n, pmax, P, slot0, work = _decode(meta)
    assert C == cap and n <= cap and info.num_items == n
    with pytest.raises(skv.SkvError):
        skv.plan_fill(h, [1000] * 8, 7, torch.zeros(skv.plan_meta_len(8, 7), dtype=torch.int32))


def test_device_plan_refresh_fails_closed_on_the_host():
    """Host checks of skv_plan_refresh_device run before any HIP call."""
    L = skv.lib()
    h = skv.plan_hints(4, 1, 1)
    fake = ctypes.c_void_p(4096)
    n = skv.plan_meta_len(4, 8)
    assert L.skv_plan_refresh_device(ctypes.byref(h), None, 8, fake, n, None) == -1
    assert L.skv_plan_refresh_device(ctypes.byref(h), fake, 8, None, n, None) == -1
    assert L.skv_plan_refresh_device(ctypes.byref(h), fake, 3, fake, n, None) == -5   # capacity < B
    assert L.skv_plan_refresh_device(ctypes.byref(h), fake, 8, fake, n - 1, None) == -8
    big = skv.plan_hints(4097, 1, 1)
    assert L.skv_plan_refresh_device(ctypes.byref(big), fake, 8192, fake,
                                     skv.plan_meta_len(4097, 8192), None) == -6
    bad = skv.plan_hints(4, 0, 1)
    assert L.skv_plan_refresh_device(ctypes.byref(bad), fake, 8, fake, n, None) == -8


def test_plan_hints_for_desc_follow_the_kernel_family():
    # matrix-core kernel: one workgroup per CU, one per group of 64 (32 at D 256) rows
    h = skv.plan_hints_for(_desc(B=2, R=4, Hq=16, Hkv=1, D=128))            # bf16 Q, fp8 KV, rho 64
    assert (h.batch, h.q_rows, h.num_kv_heads, h.causal) == (2, 4, 1, 1)
    assert (h.ctas_per_cu, h.workgroups_per_head, h.min_tokens_per_partition) == (1, 1, 0)
    h = skv.plan_hints_for(_desc(B=1, R=16, Hq=24, Hkv=4, D=256, kdt=torch.int8))   # rho 96 at D 256
    assert (h.ctas_per_cu, h.workgroups_per_head) == (1, 3)
    h = skv.plan_hints_for(_desc(B=1, R=4, Hq=40, Hkv=2, D=128, kdt=torch.int8))    # rho 80
    assert h.workgroups_per_head == 2
    # vector kernel (fp32 Q): one-wave workgroups of 8 rows, tile-sized partitions
    h = skv.plan_hints_for(_desc(B=1, R=1, Hq=14, Hkv=2, D=64, qdt=torch.float32, kdt=torch.float32))
    assert (h.ctas_per_cu, h.workgroups_per_head, h.min_tokens_per_partition) == (16, 1, 64)
    h = skv.plan_hints_for(_desc(R=4, Hq=16, Hkv=1, bs=8))                  # page 8: vector kernel
    assert (h.ctas_per_cu, h.workgroups_per_head) == (16, 8)
    bad = _desc()
    bad.head_dim = 96
    assert skv.lib().skv_plan_hints_for_desc(ctypes.byref(bad), 1, ctypes.byref(skv.PlanHints())) == -2


def test_planner_budget_counts_workgroups_per_head():
    # int8 verifier: B1, R16, Hkv 4, three row groups -> 256 / (4 * 3) = 21 partitions
    _, info, _ = _plan([20676], R=16, Hkv=4, ctas_per_cu=1, workgroups_per_head=3)
    assert info.num_items == 21
    # the same without row groups: 256 / 4 = 64, then 20676 / 256 = 80 keys-limited -> 64
    _, info, _ = _plan([20676], R=16, Hkv=4, ctas_per_cu=1)
    assert info.num_items == 64
    # the page's example is unchanged: B200 x 200k MTP4 -> 16 per request
    _, info, cap = _plan([200000] * 200, R=4, Hkv=1, ctas_per_cu=1, workgroups_per_head=1)
    assert info.num_items == 3200 and info.max_partitions == 16 and cap == 3200
    with pytest.raises(skv.SkvError):
        _plan([100], workgroups_per_head=-1)


# ---------------------------------------------------------------------------
# the boundary's names against the contract that lists them

# Every export the split-KV contract names, and the call that provides it here.
# Where the shipped name differs, the mapping says how (the documented reading).
CONTRACT = {
    "skv_attention_decode": "skv_attention_decode",
    "skv_attention_decode_paged": "skv_attention_decode_paged",
    "skv_attention_decode_splitkv": "skv_attention_decode_splitkv",
    "skv_attention_decode_paged_splitkv": "skv_attention_decode_paged_splitkv",
    "skv_splitkv_workspace_size": "skv_splitkv_workspace_size",   # also as skv_workspace_size
    "skv_plan_make": "skv_plan_make",                             # capacity/fill are its parts
    "skv_plan_refresh": "skv_plan_refresh",
    "skv_validate": "skv_validate",                               # with an added `paged` argument
    "skv_status_str": "skv_status_str",
    "skv_abi_version": "skv_abi_version",
}


def test_contract_names_are_exported():
    L = _lib()
    for want, have in CONTRACT.items():
        assert hasattr(L, have), f"{want} -> {have} missing"


def test_splitkv_workspace_size_is_workspace_size():
    for kw in (dict(), dict(B=3, R=16, Hq=24, Hkv=4, D=256), dict(record_dtype="bf16")):
        d = _desc(**kw)
        for slots in (0, 1, 3200):
            assert skv.splitkv_workspace_size(d, slots) == skv.workspace_size(d, slots)


def test_plan_make_and_refresh_equal_capacity_and_fill():
    _lib()
    for ctx, kw in (([200000] * 200, dict()), ([200000] + [1024] * 15, dict(window=4096)),
                    ([20676], dict(ctas_per_cu=1, workgroups_per_head=3))):
        R = 16 if len(ctx) == 1 else 4
        h = skv.plan_hints(len(ctx), R, 4 if len(ctx) == 1 else 1, **kw)
        cap = skv.plan_capacity(h, ctx)
        meta_ref = torch.zeros(skv.plan_meta_len(len(ctx), cap), dtype=torch.int32)
        info_ref = skv.plan_fill(h, ctx, cap, meta_ref)
        plan = skv.plan_make(h, cap)                      # explicit capacity
        assert plan.capacity_items == cap and plan.meta_len == meta_ref.numel()
        meta = torch.full((plan.meta_len,), -7, dtype=torch.int32)
        info = skv.plan_refresh(plan, ctx, meta)
        assert torch.equal(meta, meta_ref)
        assert (info.num_items, info.capacity_items, info.max_partitions, info.slots) == \
            (info_ref.num_items, info_ref.capacity_items, info_ref.max_partitions, info_ref.slots)
        # refresh with other lengths keeps the capacity
        info2 = skv.plan_refresh(plan, [max(1, c // 3) for c in ctx], meta)
        assert info2.capacity_items == cap and int(meta[1]) == cap
    # capacity from the work hint alone: B200 x 200k (total 40M keys) -> 3200
    h = skv.plan_hints(200, 4, 1, total_context_length=200 * 200000)
    assert skv.plan_make(h).capacity_items == 3200
    with pytest.raises(skv.SkvError):
        skv.plan_make(skv.plan_hints(4, 4, 1))            # neither a capacity nor a work hint
    plan = skv.plan_make(skv.plan_hints(4, 4, 1), 8)
    assert skv.lib().skv_plan_refresh(ctypes.byref(plan), None) == -1   # no lengths
    assert skv.lib().skv_plan_refresh(None, None) == -1


def test_validate_takes_paged_or_contiguous():
    """skv_validate(d, paged, num_splits, p): the contract's three-argument form
    plus `paged`, since a descriptor carries both layouts' fields and only the
    caller knows which entry point it will call."""
    d = _desc()
    d.kv_capacity = 0                                     # fine for a paged call
    assert skv.validate(d, True, 0) == 0
    assert skv.validate(d, False, 0) == -2                # a contiguous call needs kv_capacity
    d.kv_capacity = 4096
    d.max_pages = 0
    assert skv.validate(d, False, 0) == 0
    assert skv.validate(d, True, 0) == -2


def test_matrix_core_kernel_refuses_32_bit_offset_overflow():
    """Contiguous transposed V: the matrix-core kernel's per-lane byte offset
    (D - 1) * kv_capacity * bytes must fit in 31 bits; larger caches go to the
    vector kernel (auto) or are refused (explicit matrix-core)."""
    _lib()
    q = torch.zeros(1, 4, 16, 256, dtype=torch.bfloat16)
    k = torch.zeros(1, 1, 16, 256, dtype=torch.uint8)

    def desc(cap, impl, vl="transposed"):
        d = skv.make_desc(q, k, k.clone().view(1, 1, 256, 16) if vl == "transposed" else k.clone(),
                          paged=False, causal=True, impl=impl, v_layout=vl)
        d.kv_capacity = cap
        return d

    fits = (1 << 31) // 256 - 16                          # 8,388,592 keys: 256 * cap < 2^31
    assert skv.validate(desc(fits, "mfma"), False, 0) == 0
    too_big = (1 << 31) // 256                            # 256 * cap == 2^31
    assert skv.validate(desc(too_big, "mfma"), False, 0) == -6
    assert skv.validate(desc(too_big, "auto"), False, 0) == 0
    assert skv.validate(desc(too_big, "mfma", "plain"), False, 0) == 0   # plain V: 64-bit rows


def test_noalloc_call_refuses_records_beyond_the_static_scratch():
    """The allocation-free call checks its record bytes against the static
    scratch before any HIP call: too many records -> SKV_ERR_SCRATCH, and the
    usual argument errors first."""
    L = _lib()
    fake = 1 << 20                                        # never dereferenced: the call fails first
    a = skv.Args(fake, fake, fake, fake, fake, fake, fake, None, fake, None)
    d = _desc(B=200, R=4, Hq=16, Hkv=1, D=128)
    # 200 * 256 * 1 slots x 64 rows x (128 + 2) x 4 B = 1.7 GB > 128 MiB
    assert L.skv_attention_decode_paged_splitkv_noalloc(ctypes.byref(d), ctypes.byref(a), 256, None) == -10
    assert "static scratch" in skv.status_str(-10)
    assert L.skv_attention_decode_paged_splitkv_noalloc(ctypes.byref(d), ctypes.byref(skv.Args()), 16,
                                                        None) == -1
    assert L.skv_attention_decode_paged_splitkv_noalloc(ctypes.byref(d), ctypes.byref(a), 0, None) == -4
    assert L.skv_attention_decode_paged_splitkv_noalloc(ctypes.byref(d), ctypes.byref(a), 257, None) == -4


def test_host_plan_call_checks_size_and_header_before_launching():
    """skv_attention_decode_paged_planned_host: plans above SKV_PLAN_INLINE_MAX
    int32 are refused (the B200 x 200k plan is 4 + 400 + 3200), and a block
    whose header does not say (B, C) is refused; nothing is launched."""
    L = _lib()
    fake = 1 << 20
    a = skv.Args(fake, fake, fake, fake, fake, fake, fake, None, fake, None)
    p = skv.Partials(4096, 4096, 4096, 1 << 30)
    d = _desc(B=200, R=4, Hq=16, Hkv=1, D=128)
    big = torch.zeros(skv.plan_meta_len(200, 3200), dtype=torch.int32)
    big[0], big[1] = 200, 3200
    ptr = ctypes.cast(big.data_ptr(), ctypes.POINTER(ctypes.c_int32))
    assert L.skv_attention_decode_paged_planned_host(ctypes.byref(d), ctypes.byref(a), ptr, 3200,
                                                     ctypes.byref(p), None) == -6
    d = _desc(B=16, R=4, Hq=16, Hkv=1, D=128)
    h = skv.plan_hints(16, 4, 1)
    ctx = [200000] + [1024] * 15
    cap = skv.plan_capacity(h, ctx)
    meta = torch.zeros(skv.plan_meta_len(16, cap), dtype=torch.int32)
    skv.plan_fill(h, ctx, cap, meta)
    assert meta.numel() <= 480
    bad = meta.clone()
    bad[1] = cap + 1                                      # header says another capacity
    ptr = ctypes.cast(bad.data_ptr(), ctypes.POINTER(ctypes.c_int32))
    assert L.skv_attention_decode_paged_planned_host(ctypes.byref(d), ctypes.byref(a), ptr, cap,
                                                     ctypes.byref(p), None) == -8
    assert L.skv_attention_decode_paged_planned_host(ctypes.byref(d), ctypes.byref(a), None, cap,
                                                     ctypes.byref(p), None) == -1


def test_gather_ceiling_checks_arguments_before_launching():
    """skv_gather_ceiling (measurement only) validates like the partial stage:
    a NULL sink, a short sink and unsupported layouts fail before any launch."""
    L = _lib()
    fake = 1 << 20
    a = skv.Args(fake, fake, fake, fake, fake, fake, fake, None, fake, None)
    d = _desc(B=2, R=4, Hq=16, Hkv=1, D=128)
    assert L.skv_gather_ceiling(ctypes.byref(d), ctypes.byref(a), 4, None, None, 8, None) == -1
    assert L.skv_gather_ceiling(ctypes.byref(d), ctypes.byref(a), 4, None, fake, 7, None) == -5   # 2*4*1 > 7
    assert L.skv_gather_ceiling(ctypes.byref(d), ctypes.byref(a), 0, None, fake, 8, None) == -4
    small = _desc(B=2, R=4, Hq=16, Hkv=1, D=128, bs=8)
    assert L.skv_gather_ceiling(ctypes.byref(small), ctypes.byref(a), 4, None, fake, 8, None) == -6
