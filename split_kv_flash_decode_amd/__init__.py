"""Python binding of libskv.so, the split-KV paged decode-attention library.

Argument marshalling only: every function here checks tensor shapes, dtypes and
devices, fills the C structs of ``include/skv.h`` and calls the function of the
same name in the HIP library on the current torch stream. No attention
arithmetic runs in Python, and nothing falls back to a CPU path: if the
library is missing, ``lib()`` raises.

Storage conventions (the C header documents them in full):
  q, o        [B][R][Hq][D] torch.float32, torch.bfloat16 or torch.float16 (o has q's dtype)
  paged k     [pages][Hkv][block_size][D]; v the same ("plain") or
              [pages][Hkv][D][block_size] ("transposed")
  contiguous  k [B][Hkv][cap][D]; v [B][Hkv][cap][D] or [B][Hkv][D][cap]
  KV dtypes   float32, bfloat16, int8 (codes), uint8 or float8_e4m3fn (e4m3 codes)
  scales      float32 [pages][Hkv][block_size] or [B][Hkv][cap] (int8 / fp8 only)
  page_table  int32 [B][max_pages]; ctx_lens int32 [B]; sinks float32 [Hq]
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libskv.so")

SKV_F32, SKV_BF16, SKV_INT8, SKV_FP8_E4M3, SKV_F16 = 0, 1, 2, 3, 4
SKV_V_PLAIN, SKV_V_TRANSPOSED = 0, 1
SKV_IMPL_AUTO, SKV_IMPL_VALU, SKV_IMPL_MFMA = 0, 1, 2
SKV_SPLIT_ALIGN = 64
SKV_MAX_SPLITS = 256
SKV_PLAN_INLINE_MAX = 480
(SKV_OK, SKV_ERR_NULL, SKV_ERR_SHAPE, SKV_ERR_DTYPE, SKV_ERR_SPLITS, SKV_ERR_CAPACITY, SKV_ERR_UNSUPPORTED,
 SKV_ERR_LAUNCH, SKV_ERR_PLAN, SKV_ERR_ALIGN, SKV_ERR_SCRATCH) = range(0, -11, -1)

_c_i32 = ctypes.c_int32
_c_ptr = ctypes.c_void_p


class Desc(ctypes.Structure):
    _fields_ = [("batch", _c_i32), ("q_rows", _c_i32), ("num_q_heads", _c_i32),
                ("num_kv_heads", _c_i32), ("head_dim", _c_i32), ("causal", _c_i32),
                ("window", _c_i32), ("scale", ctypes.c_float), ("q_dtype", _c_i32),
                ("kv_dtype", _c_i32), ("block_size", _c_i32), ("max_pages", _c_i32),
                ("kv_capacity", _c_i32), ("v_layout", _c_i32), ("has_sink", _c_i32),
                ("impl", _c_i32), ("record_dtype", _c_i32)]


class Args(ctypes.Structure):
    _fields_ = [("q", _c_ptr), ("k", _c_ptr), ("v", _c_ptr), ("k_scale", _c_ptr),
                ("v_scale", _c_ptr), ("page_table", _c_ptr), ("ctx_lens", _c_ptr),
                ("sinks", _c_ptr), ("o", _c_ptr), ("tree_mask", _c_ptr)]


class Partials(ctypes.Structure):
    _fields_ = [("m", _c_ptr), ("l", _c_ptr), ("acc", _c_ptr), ("capacity_slots", ctypes.c_int64)]


class PlanHints(ctypes.Structure):
    _fields_ = [("batch", _c_i32), ("q_rows", _c_i32), ("num_kv_heads", _c_i32),
                ("causal", _c_i32), ("window", _c_i32), ("num_cus", _c_i32),
                ("ctas_per_cu", _c_i32), ("partitions_per_request", _c_i32),
                ("max_partitions", _c_i32), ("work_per_partition", _c_i32),
                ("min_tokens_per_partition", _c_i32), ("workgroups_per_head", _c_i32),
                ("total_context_length", ctypes.c_int64)]


class PlanInfo(ctypes.Structure):
    _fields_ = [("num_items", _c_i32), ("capacity_items", _c_i32), ("max_partitions", _c_i32),
                ("min_partitions", _c_i32), ("slots", ctypes.c_int64)]


class SkvPlan(ctypes.Structure):
    _fields_ = [("hints", PlanHints), ("capacity_items", _c_i32), ("meta_len", ctypes.c_int64),
                ("meta", ctypes.POINTER(_c_i32)), ("info", PlanInfo)]


EXPORTS = {
    "skv_abi_version": (_c_i32, []),
    "skv_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "skv_validate": (ctypes.c_int, [ctypes.POINTER(Desc), _c_i32, _c_i32, ctypes.POINTER(Partials)]),
    "skv_workspace_size": (ctypes.c_int, [ctypes.POINTER(Desc), ctypes.c_int64, ctypes.POINTER(ctypes.c_size_t),
                                          ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_size_t)]),
    "skv_splitkv_workspace_size": (ctypes.c_int, [ctypes.POINTER(Desc), ctypes.c_int64,
                                                  ctypes.POINTER(ctypes.c_size_t),
                                                  ctypes.POINTER(ctypes.c_size_t),
                                                  ctypes.POINTER(ctypes.c_size_t)]),
    "skv_uniform_slots": (ctypes.c_int64, [ctypes.POINTER(Desc), _c_i32]),
    "skv_attention_decode": (ctypes.c_int, [ctypes.POINTER(Desc), ctypes.POINTER(Args), _c_ptr]),
    "skv_attention_decode_paged": (ctypes.c_int, [ctypes.POINTER(Desc), ctypes.POINTER(Args), _c_ptr]),
    "skv_attention_decode_splitkv": (ctypes.c_int, [ctypes.POINTER(Desc), ctypes.POINTER(Args), _c_i32,
                                                    ctypes.POINTER(Partials), _c_ptr]),
    "skv_attention_decode_paged_splitkv": (ctypes.c_int, [ctypes.POINTER(Desc), ctypes.POINTER(Args), _c_i32,
                                                          ctypes.POINTER(Partials), _c_ptr]),
    "skv_attention_decode_paged_splitkv_noalloc": (ctypes.c_int, [ctypes.POINTER(Desc), ctypes.POINTER(Args),
                                                                  _c_i32, _c_ptr]),
    "skv_plan_meta_len": (ctypes.c_int64, [_c_i32, _c_i32]),
    "skv_plan_capacity": (ctypes.c_int, [ctypes.POINTER(PlanHints), ctypes.POINTER(_c_i32),
                                         ctypes.POINTER(_c_i32)]),
    "skv_plan_fill": (ctypes.c_int, [ctypes.POINTER(PlanHints), ctypes.POINTER(_c_i32), _c_i32,
                                     ctypes.POINTER(_c_i32), ctypes.c_int64, ctypes.POINTER(PlanInfo)]),
    "skv_plan_make": (ctypes.c_int, [ctypes.POINTER(PlanHints), ctypes.POINTER(SkvPlan)]),
    "skv_plan_refresh": (ctypes.c_int, [ctypes.POINTER(SkvPlan), ctypes.POINTER(_c_i32)]),
    "skv_attention_decode_paged_planned": (ctypes.c_int, [ctypes.POINTER(Desc), ctypes.POINTER(Args),
                                                          _c_ptr, _c_i32, ctypes.POINTER(Partials), _c_ptr]),
    "skv_attention_decode_paged_planned_host": (ctypes.c_int, [ctypes.POINTER(Desc), ctypes.POINTER(Args),
                                                               ctypes.POINTER(_c_i32), _c_i32,
                                                               ctypes.POINTER(Partials), _c_ptr]),
    "skv_splitkv_partial": (ctypes.c_int, [ctypes.POINTER(Desc), ctypes.POINTER(Args), _c_i32, _c_i32,
                                           _c_ptr, ctypes.POINTER(Partials), _c_ptr]),
    "skv_splitkv_combine": (ctypes.c_int, [ctypes.POINTER(Desc), ctypes.POINTER(Args), _c_i32,
                                           _c_ptr, ctypes.POINTER(Partials), _c_ptr]),
    "skv_splitkv_fused": (ctypes.c_int, [ctypes.POINTER(Desc), ctypes.POINTER(Args), _c_i32, _c_i32,
                                         _c_ptr, ctypes.POINTER(Partials), _c_ptr, _c_ptr]),
    "skv_gather_ceiling": (ctypes.c_int, [ctypes.POINTER(Desc), ctypes.POINTER(Args), _c_i32, _c_ptr, _c_ptr,
                                          ctypes.c_int64, _c_ptr]),
    "skv_plan_refresh_device": (ctypes.c_int, [ctypes.POINTER(PlanHints), _c_ptr, _c_i32, _c_ptr,
                                               ctypes.c_int64, _c_ptr]),
    "skv_plan_hints_for_desc": (ctypes.c_int, [ctypes.POINTER(Desc), _c_i32, ctypes.POINTER(PlanHints)]),
}

_LIB = None


class SkvError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = lib().skv_status_str(status).decode() if _LIB is not None else str(status)
        super().__init__(f"{where}: status {status} ({msg})")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded HIP library; raises if it has not been built."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m split_kv_flash_decode_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, argt) in EXPORTS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = argt
        _LIB = L
    return _LIB


def _check(rc: int, where: str):
    if rc != 0:
        raise SkvError(rc, where)


# ---------------------------------------------------------------------------
# descriptor / argument marshalling

_KV_CODES = {torch.float32: SKV_F32, torch.bfloat16: SKV_BF16, torch.int8: SKV_INT8,
             torch.uint8: SKV_FP8_E4M3, torch.float8_e4m3fn: SKV_FP8_E4M3}
_Q_CODES = {torch.float32: SKV_F32, torch.bfloat16: SKV_BF16, torch.float16: SKV_F16}


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _need(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def make_desc(q, k, v, *, paged: bool, v_layout: str = "plain", causal: bool = False,
              window: int = 0, scale: Optional[float] = None, page_table=None,
              has_sink: bool = False, impl: str = "auto", record_dtype: str = "f32") -> Desc:
    """Build the descriptor of a call from its tensors (shapes, dtypes, layout)."""
    _need(q.dim() == 4 and q.is_contiguous(), "q must be a contiguous [B][R][Hq][D] tensor")
    _need(q.dtype in _Q_CODES, f"q dtype {q.dtype} unsupported")
    _need(k.dtype in _KV_CODES and v.dtype == k.dtype, "k and v must share a supported dtype")
    _need(k.dim() == 4 and v.dim() == 4 and k.is_contiguous() and v.is_contiguous(),
          "k and v must be contiguous 4-d tensors")
    B, R, Hq, D = q.shape
    Hkv = k.shape[1]
    vl = {"plain": SKV_V_PLAIN, "transposed": SKV_V_TRANSPOSED}[v_layout]
    d = Desc()
    d.batch, d.q_rows, d.num_q_heads, d.num_kv_heads, d.head_dim = B, R, Hq, Hkv, D
    d.causal = int(bool(causal))
    d.window = int(window)
    d.scale = float(scale) if scale is not None else 1.0 / math.sqrt(D)
    d.q_dtype = _Q_CODES[q.dtype]
    d.kv_dtype = _KV_CODES[k.dtype]
    d.v_layout = vl
    d.has_sink = int(bool(has_sink))
    d.impl = {"auto": SKV_IMPL_AUTO, "valu": SKV_IMPL_VALU, "mfma": SKV_IMPL_MFMA}[impl]
    d.record_dtype = {"f32": SKV_F32, "bf16": SKV_BF16}[record_dtype]
    _need(k.shape[3] == D, "k's last dim must be D")
    if paged:
        _need(page_table is not None and page_table.dtype == torch.int32 and page_table.dim() == 2,
              "paged calls need an int32 [B][max_pages] page table")
        d.block_size = k.shape[2]
        d.max_pages = page_table.shape[1]
        exp_v = (k.shape[0], Hkv, D, d.block_size) if vl == SKV_V_TRANSPOSED else tuple(k.shape)
    else:
        d.kv_capacity = k.shape[2]
        _need(k.shape[0] == B, "contiguous k must be [B][Hkv][cap][D]")
        exp_v = (B, Hkv, D, d.kv_capacity) if vl == SKV_V_TRANSPOSED else tuple(k.shape)
    _need(tuple(v.shape) == exp_v, f"v shape {tuple(v.shape)} != expected {exp_v}")
    return d


def make_args(q, k, v, ctx_lens, o, *, k_scale=None, v_scale=None, page_table=None,
              sinks=None, tree_mask=None) -> Args:
    dev = q.device
    for name, t in (("k", k), ("v", v), ("ctx_lens", ctx_lens), ("o", o), ("k_scale", k_scale),
                    ("v_scale", v_scale), ("page_table", page_table), ("sinks", sinks),
                    ("tree_mask", tree_mask)):
        if t is not None:
            _need(t.device == dev, f"{name} is on {t.device}, q on {dev}")
            _need(t.is_contiguous(), f"{name} must be contiguous")
    _need(dev.type == "cuda", "tensors must be on a HIP device")
    _need(ctx_lens.dtype == torch.int32, "ctx_lens must be int32")
    _need(o.shape == q.shape and o.dtype == q.dtype, "o must match q's shape and dtype")
    for name, t in (("k_scale", k_scale), ("v_scale", v_scale), ("sinks", sinks)):
        if t is not None:
            _need(t.dtype == torch.float32, f"{name} must be float32")
    a = Args()
    a.q, a.k, a.v, a.o = _ptr(q), _ptr(k), _ptr(v), _ptr(o)
    a.k_scale, a.v_scale = _ptr(k_scale), _ptr(v_scale)
    a.page_table, a.ctx_lens, a.sinks = _ptr(page_table), _ptr(ctx_lens), _ptr(sinks)
    if tree_mask is not None:
        B, R = q.shape[:2]
        W = (R + 63) // 64
        ok = tuple(tree_mask.shape) == (B, R, W) or (W == 1 and tuple(tree_mask.shape) == (B, R))
        _need(tree_mask.dtype in (torch.int64, torch.uint64) and ok,
              "tree_mask must be a 64-bit integer [B][R][ceil(R/64)] tensor ([B][R] when R <= 64)")
        a.tree_mask = _ptr(tree_mask)
    return a


class Workspace:
    """Caller-owned partial-record buffers for ``slots`` records: fp32 m and l,
    acc in the descriptor's record dtype (fp32 or bf16)."""

    def __init__(self, desc: Desc, slots: int, device, fill: Optional[float] = None):
        mb, lb, ab = workspace_size(desc, slots)
        kw = dict(dtype=torch.float32, device=device)
        self.m = torch.empty(mb // 4, **kw)
        self.l = torch.empty(lb // 4, **kw)
        if desc.record_dtype == SKV_BF16:
            self.acc = torch.empty(ab // 2, dtype=torch.bfloat16, device=device)
        else:
            self.acc = torch.empty(ab // 4, **kw)
        if fill is not None:
            for t in (self.m, self.l, self.acc):
                t.fill_(fill)
        self.slots = slots
        self.struct = Partials(self.m.data_ptr(), self.l.data_ptr(), self.acc.data_ptr(), slots)


# ---------------------------------------------------------------------------
# the C ABI, one Python function per entry point

def abi_version() -> int:
    return lib().skv_abi_version()


def status_str(status: int) -> str:
    return lib().skv_status_str(status).decode()


def validate(desc: Desc, paged: bool, num_splits: int, ws: Optional[Workspace] = None) -> int:
    return lib().skv_validate(ctypes.byref(desc), int(paged), int(num_splits),
                              ctypes.byref(ws.struct) if ws is not None else None)


def workspace_size(desc: Desc, slots: int):
    m, l, a = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().skv_workspace_size(ctypes.byref(desc), int(slots), ctypes.byref(m), ctypes.byref(l),
                                    ctypes.byref(a)), "skv_workspace_size")
    return m.value, l.value, a.value


def splitkv_workspace_size(desc: Desc, slots: int):
    m, l, a = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib().skv_splitkv_workspace_size(ctypes.byref(desc), int(slots), ctypes.byref(m), ctypes.byref(l),
                                            ctypes.byref(a)), "skv_splitkv_workspace_size")
    return m.value, l.value, a.value


def uniform_slots(desc: Desc, num_splits: int) -> int:
    return lib().skv_uniform_slots(ctypes.byref(desc), int(num_splits))


def attention_decode(desc: Desc, args: Args, stream=None):
    _check(lib().skv_attention_decode(ctypes.byref(desc), ctypes.byref(args), _stream(stream)),
           "skv_attention_decode")


def attention_decode_paged(desc: Desc, args: Args, stream=None):
    _check(lib().skv_attention_decode_paged(ctypes.byref(desc), ctypes.byref(args), _stream(stream)),
           "skv_attention_decode_paged")


def attention_decode_splitkv(desc: Desc, args: Args, num_splits: int, ws: Workspace, stream=None):
    _check(lib().skv_attention_decode_splitkv(ctypes.byref(desc), ctypes.byref(args), int(num_splits),
                                              ctypes.byref(ws.struct), _stream(stream)),
           "skv_attention_decode_splitkv")


def attention_decode_paged_splitkv(desc: Desc, args: Args, num_splits: int, ws: Workspace, stream=None):
    _check(lib().skv_attention_decode_paged_splitkv(ctypes.byref(desc), ctypes.byref(args), int(num_splits),
                                                    ctypes.byref(ws.struct), _stream(stream)),
           "skv_attention_decode_paged_splitkv")


def attention_decode_paged_splitkv_noalloc(desc: Desc, args: Args, num_splits: int, stream=None):
    """The split-KV call with its partial records in the library's static
    device scratch (no caller buffers, nothing allocated)."""
    _check(lib().skv_attention_decode_paged_splitkv_noalloc(ctypes.byref(desc), ctypes.byref(args),
                                                            int(num_splits), _stream(stream)),
           "skv_attention_decode_paged_splitkv_noalloc")


def attention_decode_paged_planned(desc: Desc, args: Args, plan_meta_dev: torch.Tensor, capacity: int,
                                   ws: Workspace, stream=None):
    _check(lib().skv_attention_decode_paged_planned(ctypes.byref(desc), ctypes.byref(args),
                                                    plan_meta_dev.data_ptr(), int(capacity),
                                                    ctypes.byref(ws.struct), _stream(stream)),
           "skv_attention_decode_paged_planned")


def attention_decode_paged_planned_host(desc: Desc, args: Args, plan_meta_host: torch.Tensor, capacity: int,
                                        ws: Workspace, stream=None):
    """The planned call with the plan block in host memory (a CPU int32
    tensor as plan_fill wrote it), passed to the kernels by value."""
    _need(plan_meta_host.device.type == "cpu" and plan_meta_host.dtype == torch.int32
          and plan_meta_host.is_contiguous(), "plan_meta_host must be a contiguous CPU int32 tensor")
    _check(lib().skv_attention_decode_paged_planned_host(
        ctypes.byref(desc), ctypes.byref(args), ctypes.cast(plan_meta_host.data_ptr(), ctypes.POINTER(_c_i32)),
        int(capacity), ctypes.byref(ws.struct), _stream(stream)), "skv_attention_decode_paged_planned_host")


def splitkv_partial(desc: Desc, args: Args, paged: bool, num_splits: int, ws: Workspace,
                    plan_meta_dev: Optional[torch.Tensor] = None, stream=None):
    _check(lib().skv_splitkv_partial(ctypes.byref(desc), ctypes.byref(args), int(paged), int(num_splits),
                                     _ptr(plan_meta_dev), ctypes.byref(ws.struct), _stream(stream)),
           "skv_splitkv_partial")


def splitkv_combine(desc: Desc, args: Args, num_splits: int, ws: Workspace,
                    plan_meta_dev: Optional[torch.Tensor] = None, stream=None):
    _check(lib().skv_splitkv_combine(ctypes.byref(desc), ctypes.byref(args), int(num_splits),
                                     _ptr(plan_meta_dev), ctypes.byref(ws.struct), _stream(stream)),
           "skv_splitkv_combine")


def splitkv_fused(desc: Desc, args: Args, paged: bool, num_splits: int, ws: Workspace,
                  counters: torch.Tensor, plan_meta_dev: Optional[torch.Tensor] = None, stream=None):
    """Single-kernel split + merge: ``counters`` is a zeroed int32 device tensor
    of at least B * Hkv entries (left zero after the call)."""
    if counters.dtype != torch.int32 or not counters.is_cuda or counters.numel() < desc.batch * desc.num_kv_heads:
        raise ValueError("counters: int32 device tensor of B * Hkv entries expected")
    _check(lib().skv_splitkv_fused(ctypes.byref(desc), ctypes.byref(args), int(paged), int(num_splits),
                                   _ptr(plan_meta_dev), ctypes.byref(ws.struct), _ptr(counters),
                                   _stream(stream)),
           "skv_splitkv_fused")


def gather_ceiling(desc: Desc, args: Args, num_splits: int, sink: torch.Tensor,
                   plan_meta_dev: Optional[torch.Tensor] = None, stream=None):
    """Measurement only: the read-only gather with the partial kernel's memory
    pattern (sink: int32/uint32 device tensor of at least items * Hkv)."""
    _need(sink.is_cuda and sink.dtype in (torch.int32, torch.uint32) and sink.is_contiguous(),
          "sink must be a contiguous 32-bit device tensor")
    _check(lib().skv_gather_ceiling(ctypes.byref(desc), ctypes.byref(args), int(num_splits), _ptr(plan_meta_dev),
                                    _ptr(sink), int(sink.numel()), _stream(stream)), "skv_gather_ceiling")


def plan_meta_len(batch: int, capacity: int) -> int:
    return lib().skv_plan_meta_len(int(batch), int(capacity))


def _ctx_array(host_ctx):
    arr = (_c_i32 * len(host_ctx))(*[int(c) for c in host_ctx])
    return arr


def plan_hints(batch: int, q_rows: int, num_kv_heads: int, *, causal: bool = True, window: int = 0,
               num_cus: int = 0, ctas_per_cu: int = 0, partitions_per_request: int = 0,
               max_partitions: int = 0, work_per_partition: int = 0,
               min_tokens_per_partition: int = 0, workgroups_per_head: int = 0,
               total_context_length: int = 0) -> PlanHints:
    h = PlanHints()
    h.batch, h.q_rows, h.num_kv_heads = batch, q_rows, num_kv_heads
    h.causal, h.window, h.num_cus, h.ctas_per_cu = int(causal), window, num_cus, ctas_per_cu
    h.partitions_per_request, h.max_partitions = partitions_per_request, max_partitions
    h.work_per_partition, h.min_tokens_per_partition = work_per_partition, min_tokens_per_partition
    h.workgroups_per_head = workgroups_per_head
    h.total_context_length = total_context_length
    return h


def plan_hints_for(desc: Desc, paged: bool = True, **overrides) -> PlanHints:
    """skv_plan_hints_for_desc, then any field given in ``overrides``."""
    h = PlanHints()
    _check(lib().skv_plan_hints_for_desc(ctypes.byref(desc), int(paged), ctypes.byref(h)),
           "skv_plan_hints_for_desc")
    for k, v in overrides.items():
        _need(hasattr(h, k), f"no planner hint {k}")
        setattr(h, k, int(v))
    return h


def plan_capacity(hints: PlanHints, host_ctx=None) -> int:
    cap = _c_i32()
    arr = _ctx_array(host_ctx) if host_ctx is not None else None
    _check(lib().skv_plan_capacity(ctypes.byref(hints), arr, ctypes.byref(cap)), "skv_plan_capacity")
    return cap.value


def plan_fill(hints: PlanHints, host_ctx, capacity: int, meta: torch.Tensor) -> PlanInfo:
    """Fill the host int32 tensor ``meta`` (CPU, contiguous) with a plan."""
    _need(meta.device.type == "cpu" and meta.dtype == torch.int32 and meta.is_contiguous(),
          "meta must be a contiguous CPU int32 tensor")
    info = PlanInfo()
    arr = _ctx_array(host_ctx)
    _check(lib().skv_plan_fill(ctypes.byref(hints), arr, int(capacity),
                               ctypes.cast(meta.data_ptr(), ctypes.POINTER(_c_i32)), meta.numel(),
                               ctypes.byref(info)), "skv_plan_fill")
    return info


def plan_make(hints: PlanHints, capacity: int = 0) -> SkvPlan:
    """skv_plan_make: a plan object with fixed capacity (``capacity`` > 0, or
    sized from ``hints.total_context_length``); its ``meta`` is still unset."""
    plan = SkvPlan()
    plan.capacity_items = int(capacity)
    _check(lib().skv_plan_make(ctypes.byref(hints), ctypes.byref(plan)), "skv_plan_make")
    return plan


def plan_refresh(plan: SkvPlan, host_ctx, meta: torch.Tensor) -> PlanInfo:
    """skv_plan_refresh into the host int32 tensor ``meta`` (CPU, contiguous,
    at least ``plan.meta_len`` entries)."""
    _need(meta.device.type == "cpu" and meta.dtype == torch.int32 and meta.is_contiguous()
          and meta.numel() >= plan.meta_len, "meta must be a contiguous CPU int32 tensor of meta_len entries")
    plan.meta = ctypes.cast(meta.data_ptr(), ctypes.POINTER(_c_i32))
    _check(lib().skv_plan_refresh(ctypes.byref(plan), _ctx_array(host_ctx)), "skv_plan_refresh")
    return plan.info


def plan_refresh_device(hints: PlanHints, ctx_dev: torch.Tensor, capacity: int, meta_dev: torch.Tensor,
                        stream=None) -> None:
    """Re-plan on the GPU from device context lengths into the device block
    ``meta_dev`` (bit-identical to plan_fill for the same lengths)."""
    if ctx_dev.dtype != torch.int32 or meta_dev.dtype != torch.int32 or not (ctx_dev.is_cuda and meta_dev.is_cuda):
        raise ValueError("ctx_dev and meta_dev: int32 device tensors expected")
    _check(lib().skv_plan_refresh_device(ctypes.byref(hints), _ptr(ctx_dev), int(capacity), _ptr(meta_dev),
                                         int(meta_dev.numel()), _stream(stream)),
           "skv_plan_refresh_device")


class Plan:
    """A plan's fixed-capacity metadata: pinned host copies and one device copy.

    ``refresh(host_ctx)`` re-plans on the host and enqueues the host-to-device
    copy on the current stream (two pinned host buffers alternate, each
    reused only after its previous copy has completed).
    """

    def __init__(self, hints: PlanHints, host_ctx, device, capacity: Optional[int] = None):
        self.hints = hints
        self.capacity = capacity if capacity is not None else plan_capacity(hints, host_ctx)
        n = plan_meta_len(hints.batch, self.capacity)
        self.host = [torch.empty(n, dtype=torch.int32).pin_memory() for _ in range(2)]
        self.events = [torch.cuda.Event(), torch.cuda.Event()]
        self.used = [False, False]
        self.dev = torch.empty(n, dtype=torch.int32, device=device)
        self.turn = 0
        self.info = None
        self.refresh(host_ctx)

    def refresh(self, host_ctx, stream=None):
        i = self.turn
        self.turn ^= 1
        if self.used[i]:
            self.events[i].synchronize()           # its previous copy has completed
        self.info = plan_fill(self.hints, host_ctx, self.capacity, self.host[i])
        s = torch.cuda.current_stream() if stream is None else stream
        if stream is None:
            self.dev.copy_(self.host[i], non_blocking=True)
        else:
            with torch.cuda.stream(s):
                self.dev.copy_(self.host[i], non_blocking=True)
        self.events[i].record(s)
        self.used[i] = True
        return self.info

    def refresh_device(self, ctx_dev: torch.Tensor, stream=None) -> None:
        """Re-plan on the GPU from the device lengths (capturable; ``info``
        keeps the last host-side values)."""
        plan_refresh_device(self.hints, ctx_dev, self.capacity, self.dev, stream)
