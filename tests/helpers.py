"""Test-side glue: run the oracle on a generated problem, compare results."""

from __future__ import annotations

import numpy as np

import oracle


def oracle_output(problem, requests=None) -> np.ndarray:
    """fp64 oracle output [B'][R][Hq][D] for a ``skvgen.Problem``."""
    s = problem.spec
    return oracle.decode_attention(
        problem.host_arrays(), R=s.R, Hq=s.Hq, Hkv=s.Hkv, D=s.D, causal=s.causal,
        window=s.window, scale=s.scale, q_dtype=s.q_dtype, kv_dtype=s.kv_dtype,
        paged=problem.paged, block_size=s.block_size, v_layout=s.v_layout,
        has_sink=s.sinks, requests=requests)


def oracle_abs_value_output(problem) -> np.ndarray:
    """The oracle's output with every value vector replaced by its elementwise
    magnitude: sum_t p_t |v_t| / sum_t p_t (times the merge's 1 / (L + 1e-9)),
    the weight an output element gives to errors relative to each value.
    Magnitudes are taken on the stored codes (sign bit cleared; int8 codes are
    within +-127), so the scales, the poison and the probabilities are
    untouched."""
    s = problem.spec
    arrays = dict(problem.host_arrays())
    v = arrays["v"]
    if s.kv_dtype == "f32":
        v = np.abs(v)
    elif s.kv_dtype == "bf16":
        v = v & np.uint16(0x7FFF)
    elif s.kv_dtype == "fp8":
        v = v & np.uint8(0x7F)
    elif s.kv_dtype == "int8":
        v = np.abs(v.astype(np.int16)).astype(np.int8)
    arrays["v"] = v
    return oracle.decode_attention(
        arrays, R=s.R, Hq=s.Hq, Hkv=s.Hkv, D=s.D, causal=s.causal,
        window=s.window, scale=s.scale, q_dtype=s.q_dtype, kv_dtype=s.kv_dtype,
        paged=problem.paged, block_size=s.block_size, v_layout=s.v_layout,
        has_sink=s.sinks)


def compare(out: np.ndarray, ref: np.ndarray, kind: str, extra=None) -> dict:
    """Error statistics of ``out`` vs the fp64 ``ref`` (same shape, last dim = D).

    kind "f32": max-abs <= 2e-3 and max-rel <= 2e-3 over |ref| >= 2e-3, rel-L2 <= 1e-4.
    kind "lowp": |out - ref| <= 5e-3 + 5e-3 |ref| elementwise, rel-L2 <= 1e-2 and
    min row cosine >= 0.9999 over rows with a nonzero reference.
    ``extra`` (same shape as ref): a further elementwise allowance added to the
    "lowp" bound, for a stage whose rounding is bounded separately.
    """
    out = np.asarray(out, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert out.shape == ref.shape, (out.shape, ref.shape)
    d = np.abs(out - ref)
    nrm = np.linalg.norm(ref)
    rel_l2 = float(np.linalg.norm(out - ref) / nrm) if nrm > 0 else float(np.linalg.norm(out))
    o2 = out.reshape(-1, out.shape[-1])
    r2 = ref.reshape(-1, ref.shape[-1])
    rn = np.linalg.norm(r2, axis=1)
    on = np.linalg.norm(o2, axis=1)
    live = rn > 0
    cos = (o2[live] * r2[live]).sum(axis=1) / np.maximum(on[live] * rn[live], 1e-300)
    big = np.abs(ref) >= 2e-3
    stats = {
        "max_abs": float(d.max()) if d.size else 0.0,
        "max_rel": float((d[big] / np.abs(ref[big])).max()) if big.any() else 0.0,
        "rel_l2": rel_l2,
        "min_cos": float(cos.min()) if cos.size else 1.0,
        "finite": bool(np.isfinite(out).all()),
        "zero_rows_ok": bool(np.all(on[~live] == 0)),
    }
    if kind == "f32":
        stats["ok"] = (stats["finite"] and stats["max_abs"] <= 2e-3 and stats["max_rel"] <= 2e-3
                       and stats["rel_l2"] <= 1e-4 and stats["zero_rows_ok"])
    elif kind == "lowp":
        bound = 5e-3 + 5e-3 * np.abs(ref) + (0.0 if extra is None else np.asarray(extra, dtype=np.float64))
        elem = bool(np.all(d <= bound))
        stats["worst_margin"] = float((d - bound).max()) if d.size else 0.0
        stats["elementwise"] = elem
        stats["ok"] = (stats["finite"] and elem and stats["rel_l2"] <= 1e-2
                       and stats["min_cos"] >= 0.9999 and stats["zero_rows_ok"])
    else:
        raise ValueError(kind)
    return stats
