"""Python binding of libhisparse.so (MI355X / gfx950 HiSparse sparse-decode path).

Argument marshalling only: every function takes torch tensors, checks their dtype,
device and contiguity, and forwards raw pointers, sizes and the current HIP stream to
the C ABI declared in include/hisparse.h.  All computation runs in the library's HIP
kernels.  Importing this module fails loudly when the library has not been built.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhisparse.so")

HS_OK, HS_ERR_INVALID_ARG, HS_ERR_CAPACITY, HS_ERR_UNSUPPORTED, HS_ERR_HIP = 0, -1, -2, -3, -4
HS_ERR_SCRATCH = -5
NOALLOC_SCRATCH_BYTES = 32 << 20
HS_BF16, HS_F32 = 0, 1

EXPORTED = ("hs_resolve_topk", "hs_swap_in", "hs_sparse_decode_attn", "hs_sparse_decode_attn_paged",
            "hs_sparse_decode_attn_mixed", "hs_sparse_decode_attn_cus",
            "hs_sparse_decode_attn_mixed_cus",
            "hs_attn_workspace_bytes", "hs_attn_plan_info", "hs_attn_plan_info_cus", "hs_finalize_accepted", "hs_backup_rows", "hs_apply_plan",
            "hs_append_accepted", "hs_host_read", "hs_sparse_decode_attn_noalloc",
            "hs_greedy_argmax",
            "hs_status_string", "hs_version")


class HsError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed: {msg} ({status})")
        self.status = status


class HsHotState(ctypes.Structure):
    _fields_ = [("num_reqs", ctypes.c_int32), ("capacity", ctypes.c_int32),
                ("slot_loc", ctypes.c_void_p), ("slot_stamp", ctypes.c_void_p),
                ("loc_to_hot", ctypes.c_void_p), ("host_rows", ctypes.c_int64),
                ("row_elems", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("hot_kv", ctypes.c_void_p), ("host_pool", ctypes.c_void_p)]


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it first "
                          "(python sparse_attention_kv_amd/build.py)")
    lib = ctypes.CDLL(LIB_PATH)
    i32, i64, vp, f32, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_float, ctypes.c_size_t
    lib.hs_resolve_topk.argtypes = [vp, i32, i32, vp, vp, i32, vp, i32, i32, i32, vp, vp, vp]
    lib.hs_resolve_topk.restype = i32
    lib.hs_swap_in.argtypes = [ctypes.POINTER(HsHotState), vp, i32, i32, vp, vp, vp, vp]
    lib.hs_swap_in.restype = i32
    lib.hs_sparse_decode_attn.argtypes = [vp, vp, i64, vp, i32, i32, i32, i32, i32, f32, i32,
                                          vp, vp, vp, sz, vp]
    lib.hs_sparse_decode_attn.restype = i32
    lib.hs_sparse_decode_attn_cus.argtypes = [vp, vp, i64, vp, i32, i32, i32, i32, i32, f32, i32,
                                              vp, vp, vp, sz, i32, vp]
    lib.hs_sparse_decode_attn_cus.restype = i32
    lib.hs_sparse_decode_attn_paged.argtypes = [vp, vp, i64, vp, vp, vp, i32, vp, i32, i32, i32,
                                                i32, i32, i32, i32, i32, f32, i32, vp, vp, vp, sz,
                                                vp]
    lib.hs_sparse_decode_attn_paged.restype = i32
    lib.hs_sparse_decode_attn_mixed.argtypes = [vp, vp, i64, vp, vp, i64, vp, vp, i32, i32, i32,
                                                i32, i32, f32, i32, vp, vp, vp, sz, vp]
    lib.hs_sparse_decode_attn_mixed.restype = i32
    lib.hs_sparse_decode_attn_mixed_cus.argtypes = [vp, vp, i64, vp, vp, i64, vp, vp, i32, i32,
                                                    i32, i32, i32, f32, i32, vp, vp, vp, sz, i32,
                                                    vp]
    lib.hs_sparse_decode_attn_mixed_cus.restype = i32
    lib.hs_attn_workspace_bytes.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.hs_attn_plan_info.argtypes = [i32, i32, i32, i32, i32, i32, vp, vp]
    lib.hs_attn_plan_info.restype = i32
    lib.hs_attn_plan_info_cus.argtypes = [i32, i32, i32, i32, i32, i32, i32, vp, vp]
    lib.hs_attn_plan_info_cus.restype = i32
    lib.hs_attn_workspace_bytes.restype = sz
    lib.hs_finalize_accepted.argtypes = [ctypes.POINTER(HsHotState), vp, i32, vp, vp, i32, vp, vp,
                                         i32, i32, i32, vp, vp, vp, vp]
    lib.hs_finalize_accepted.restype = i32
    lib.hs_backup_rows.argtypes = [vp, i64, vp, i64, i32, i32, vp, i32, vp, i32, i32, i32, vp]
    lib.hs_backup_rows.restype = i32
    lib.hs_apply_plan.argtypes = [vp, vp, i64, i32, i32, i32, i32, vp, i32, vp, vp, vp, vp]
    lib.hs_apply_plan.restype = i32
    lib.hs_append_accepted.argtypes = [vp, i64, i32, vp, i32, i32, i32, vp, vp, vp, i32, i32, vp]
    lib.hs_append_accepted.restype = i32
    lib.hs_sparse_decode_attn_noalloc.argtypes = [vp, vp, i64, vp, i32, i32, i32, i32, i32, f32,
                                                  i32, vp, vp, vp]
    lib.hs_sparse_decode_attn_noalloc.restype = i32
    lib.hs_greedy_argmax.argtypes = [vp, i32, i32, vp, vp]
    lib.hs_greedy_argmax.restype = i32
    lib.hs_host_read.argtypes = [vp, vp, i64, vp]
    lib.hs_host_read.restype = i32
    lib.hs_status_string.argtypes = [i32]
    lib.hs_status_string.restype = ctypes.c_char_p
    lib.hs_version.argtypes = []
    lib.hs_version.restype = ctypes.c_char_p
    return lib


_lib = _load()


def version() -> str:
    return _lib.hs_version().decode()


def status_string(status: int) -> str:
    return _lib.hs_status_string(status).decode()


def _check(fn: str, status: int):
    if status != HS_OK:
        raise HsError(fn, status, status_string(status))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _shape(ok: bool, what: str):
    """Shape agreement between arguments, checked before any device or dtype check: a
    mis-sized buffer would otherwise become an out-of-bounds device access."""
    if not ok:
        raise ValueError(f"shape mismatch: {what}")


def _dev(t: torch.Tensor, name: str, dtype=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return HS_BF16
    if dt == torch.float32:
        return HS_F32
    raise ValueError(f"unsupported dtype {dt}")


# ------------------------------------------------------------------------------------
def hs_resolve_topk(topk_pos: torch.Tensor, req_id: torch.Tensor, causal_limit: torch.Tensor,
                    block_table: torch.Tensor, block_size: int, physical_block_stride: int,
                    out_slots: torch.Tensor, out_valid: Optional[torch.Tensor] = None,
                    stream=None):
    """Top-k token positions [rows, topk] -> physical KV rows (see include/hisparse.h)."""
    i32 = torch.int32
    _shape(topk_pos.dim() == 2 and block_table.dim() == 2, "topk_pos and block_table must be 2-D")
    rows, topk = topk_pos.shape
    _shape(tuple(req_id.shape) == (rows,) and tuple(causal_limit.shape) == (rows,),
           "req_id and causal_limit must be [rows]")
    _shape(out_slots.shape == topk_pos.shape, "out_slots must be [rows, topk]")
    _shape(out_valid is None or tuple(out_valid.shape) == (rows,), "out_valid must be [rows]")
    _dev(topk_pos, "topk_pos", i32); _dev(req_id, "req_id", i32)
    _dev(causal_limit, "causal_limit", i32); _dev(block_table, "block_table", i32)
    _dev(out_slots, "out_slots", i32)
    if out_valid is not None:
        _dev(out_valid, "out_valid", i32)
    num_reqs, bt_stride = block_table.shape
    _check("hs_resolve_topk", _lib.hs_resolve_topk(
        _ptr(topk_pos), rows, topk, _ptr(req_id), _ptr(causal_limit), num_reqs,
        _ptr(block_table), bt_stride, block_size, physical_block_stride, _ptr(out_slots),
        _ptr(out_valid), _stream(stream)))


@dataclass
class HotState:
    """Device tensors of one hot buffer plus the pinned host pool (hs_hot_state)."""
    slot_loc: torch.Tensor     # int32 [num_reqs, capacity]
    slot_stamp: torch.Tensor   # int32 [num_reqs, capacity]
    loc_to_hot: torch.Tensor   # int32 [host_rows]
    hot_kv: torch.Tensor       # [num_reqs * capacity, row_elems]
    host_pool: torch.Tensor    # pinned host [host_rows, row_elems] (or device)
    # Host-side record of the newest tick stamped into this state through the wrappers
    # (None: unknown).  DecodeStep overlaps wave r+1's swap with wave r's attention only
    # when its first tick is above it (victims are then never slots wave r uses).
    max_stamp: Optional[int] = None

    def note_tick(self, tick: int):
        self.max_stamp = tick if self.max_stamp is None else max(self.max_stamp, tick)

    def check_shapes(self):
        _shape(self.slot_loc.dim() == 2 and self.slot_stamp.shape == self.slot_loc.shape,
               "slot_loc and slot_stamp must be [num_reqs, capacity]")
        num_reqs, cap = self.slot_loc.shape
        _shape(self.loc_to_hot.dim() == 1 and self.host_pool.dim() == 2 and
               self.loc_to_hot.shape[0] == self.host_pool.shape[0],
               "loc_to_hot must be [host_rows] with host_pool [host_rows, row_elems]")
        _shape(self.hot_kv.dim() == 2 and self.hot_kv.shape[0] == num_reqs * cap and
               self.hot_kv.shape[1] == self.host_pool.shape[1],
               "hot_kv must be [num_reqs * capacity, row_elems]")

    def as_struct(self) -> HsHotState:
        self.check_shapes()
        for name in ("slot_loc", "slot_stamp", "loc_to_hot", "hot_kv"):
            _dev(getattr(self, name), name)
        for name in ("slot_loc", "slot_stamp", "loc_to_hot"):
            _dev(getattr(self, name), name, torch.int32)
        if not self.host_pool.is_contiguous():
            raise ValueError("host_pool must be contiguous")
        if self.host_pool.dtype != self.hot_kv.dtype:
            raise ValueError("host_pool and hot_kv dtypes differ")
        num_reqs, cap = self.slot_loc.shape
        return HsHotState(num_reqs, cap, self.slot_loc.data_ptr(), self.slot_stamp.data_ptr(),
                          self.loc_to_hot.data_ptr(), self.host_pool.shape[0],
                          self.hot_kv.shape[1], _dtype_code(self.hot_kv.dtype),
                          self.hot_kv.data_ptr(), self.host_pool.data_ptr())


def hs_swap_in(state: HotState, wave_rows: torch.Tensor, tick: int, out_hot_idx: torch.Tensor,
               out_miss_count: torch.Tensor, out_miss_pos: Optional[torch.Tensor] = None,
               stream=None):
    """One wave of swap-in: wave_rows [num_reqs, topk] host rows (see include/hisparse.h)."""
    i32 = torch.int32
    state.check_shapes()
    num_reqs = state.slot_loc.shape[0]
    _shape(wave_rows.dim() == 2 and wave_rows.shape[0] == num_reqs,
           "wave_rows must be [num_reqs, topk]")
    _shape(out_hot_idx.shape == wave_rows.shape, "out_hot_idx must be [num_reqs, topk]")
    _shape(tuple(out_miss_count.shape) == (num_reqs,), "out_miss_count must be [num_reqs]")
    _shape(out_miss_pos is None or out_miss_pos.shape == wave_rows.shape,
           "out_miss_pos must be [num_reqs, topk]")
    _dev(wave_rows, "wave_rows", i32); _dev(out_hot_idx, "out_hot_idx", i32)
    _dev(out_miss_count, "out_miss_count", i32)
    if out_miss_pos is not None:
        _dev(out_miss_pos, "out_miss_pos", i32)
    st = state.as_struct()
    _check("hs_swap_in", _lib.hs_swap_in(ctypes.byref(st), _ptr(wave_rows), wave_rows.shape[1],
                                         tick, _ptr(out_hot_idx), _ptr(out_miss_count),
                                         _ptr(out_miss_pos), _stream(stream)))
    state.note_tick(tick)


def hs_attn_workspace_bytes(num_rows: int, num_heads: int, d_qk: int, d_v: int, topk: int,
                            dtype: torch.dtype) -> int:
    return int(_lib.hs_attn_workspace_bytes(num_rows, num_heads, d_qk, d_v, topk, _dtype_code(dtype)))


def hs_attn_plan_info(num_rows: int, num_heads: int, d_qk: int, d_v: int, topk: int,
                      dtype: torch.dtype):
    """(heads per workgroup, key splits) of the attention launch for these sizes: 32, 64 or
    128 for the bf16 kernels, 1 for the fp32 path (see include/hisparse.h)."""
    hpw, spl = ctypes.c_int32(0), ctypes.c_int32(0)
    _check("hs_attn_plan_info", _lib.hs_attn_plan_info(num_rows, num_heads, d_qk, d_v, topk,
                                                       _dtype_code(dtype), ctypes.byref(hpw),
                                                       ctypes.byref(spl)))
    return hpw.value, spl.value


def hs_attn_plan_info_cus(num_rows: int, num_heads: int, d_qk: int, d_v: int, topk: int,
                          dtype: torch.dtype, max_cus: int):
    """hs_attn_plan_info for hs_sparse_decode_attn_cus with ``max_cus`` compute units."""
    hpw, spl = ctypes.c_int32(0), ctypes.c_int32(0)
    _check("hs_attn_plan_info_cus", _lib.hs_attn_plan_info_cus(
        num_rows, num_heads, d_qk, d_v, topk, _dtype_code(dtype), max_cus, ctypes.byref(hpw),
        ctypes.byref(spl)))
    return hpw.value, spl.value


def hs_sparse_decode_attn_cus(q: torch.Tensor, kv: torch.Tensor, indices: torch.Tensor,
                              scale: float, d_v: int, out: torch.Tensor,
                              lse: Optional[torch.Tensor] = None,
                              workspace: Optional[torch.Tensor] = None, max_cus: int = 256,
                              stream=None):
    """hs_sparse_decode_attn sized for ``max_cus`` compute units, leaving the rest of the GPU
    to a kernel running beside it (see include/hisparse.h)."""
    _attn_shapes(q, kv, indices, d_v, out, lse)
    _dev(q, "q"); _dev(kv, "kv"); _dev(indices, "indices", torch.int32); _dev(out, "out", q.dtype)
    if kv.dtype != q.dtype:
        raise ValueError("q and kv dtypes differ")
    if lse is not None:
        _dev(lse, "lse", torch.float32)
    if workspace is not None:
        _dev(workspace, "workspace")
    rows, heads, d_qk = q.shape
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("hs_sparse_decode_attn_cus", _lib.hs_sparse_decode_attn_cus(
        _ptr(q), _ptr(kv), kv.shape[0], _ptr(indices), rows, heads, d_qk, d_v, indices.shape[1],
        float(scale), _dtype_code(q.dtype), _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes,
        int(max_cus), _stream(stream)))


def hs_sparse_decode_attn(q: torch.Tensor, kv: torch.Tensor, indices: torch.Tensor, scale: float,
                          d_v: int, out: torch.Tensor, lse: Optional[torch.Tensor] = None,
                          workspace: Optional[torch.Tensor] = None, stream=None):
    """Sparse attention of q [rows, H, d_qk] over kv[indices] (see include/hisparse.h)."""
    _attn_shapes(q, kv, indices, d_v, out, lse)
    _dev(q, "q"); _dev(kv, "kv"); _dev(indices, "indices", torch.int32); _dev(out, "out", q.dtype)
    if kv.dtype != q.dtype:
        raise ValueError("q and kv dtypes differ")
    if lse is not None:
        _dev(lse, "lse", torch.float32)
    if workspace is not None:
        _dev(workspace, "workspace")
    rows, heads, d_qk = q.shape
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check("hs_sparse_decode_attn", _lib.hs_sparse_decode_attn(
        _ptr(q), _ptr(kv), kv.shape[0], _ptr(indices), rows, heads, d_qk, d_v, indices.shape[1],
        float(scale), _dtype_code(q.dtype), _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes,
        _stream(stream)))


def hs_sparse_decode_attn_noalloc(q: torch.Tensor, kv: torch.Tensor, indices: torch.Tensor,
                                  scale: float, d_v: int, out: torch.Tensor,
                                  lse: Optional[torch.Tensor] = None, stream=None):
    """hs_sparse_decode_attn with the key-split workspace in the library's fixed per-GPU
    scratch: for callers that cannot allocate (see include/hisparse.h)."""
    _attn_shapes(q, kv, indices, d_v, out, lse)
    _dev(q, "q"); _dev(kv, "kv"); _dev(indices, "indices", torch.int32); _dev(out, "out", q.dtype)
    if kv.dtype != q.dtype:
        raise ValueError("q and kv dtypes differ")
    if lse is not None:
        _dev(lse, "lse", torch.float32)
    rows, heads, d_qk = q.shape
    _check("hs_sparse_decode_attn_noalloc", _lib.hs_sparse_decode_attn_noalloc(
        _ptr(q), _ptr(kv), kv.shape[0], _ptr(indices), rows, heads, d_qk, d_v, indices.shape[1],
        float(scale), _dtype_code(q.dtype), _ptr(out), _ptr(lse), _stream(stream)))


def _attn_shapes(q, kv, indices, d_v, out, lse):
    _shape(q.dim() == 3 and kv.dim() == 2 and indices.dim() == 2, "q [rows, H, d_qk], kv "
           "[kv_rows, d_qk] and indices [rows, topk] expected")
    rows, heads, d_qk = q.shape
    _shape(kv.shape[1] == d_qk, "kv rows must be d_qk wide")
    _shape(indices.shape[0] == rows, "indices must have one row per query row")
    _shape(tuple(out.shape) == (rows, heads, d_v), "out must be [rows, H, d_v]")
    _shape(lse is None or tuple(lse.shape) == (rows, heads), "lse must be [rows, H]")


def _paged_args(q, kv_pool, topk_pos, req_id, causal_limit, block_table, block_size,
                physical_block_stride, scale, d_v, out, lse, workspace):
    """Checks and converts the arguments of hs_sparse_decode_attn_paged (all but the stream)."""
    i32 = torch.int32
    _attn_shapes(q, kv_pool, topk_pos, d_v, out, lse)
    rows = q.shape[0]
    _shape(tuple(req_id.shape) == (rows,) and tuple(causal_limit.shape) == (rows,),
           "req_id and causal_limit must be [rows]")
    _shape(block_table.dim() == 2, "block_table must be [num_reqs, bt_stride]")
    _dev(q, "q"); _dev(kv_pool, "kv_pool"); _dev(out, "out", q.dtype)
    _dev(topk_pos, "topk_pos", i32); _dev(req_id, "req_id", i32)
    _dev(causal_limit, "causal_limit", i32); _dev(block_table, "block_table", i32)
    if kv_pool.dtype != q.dtype:
        raise ValueError("q and kv_pool dtypes differ")
    if lse is not None:
        _dev(lse, "lse", torch.float32)
    if workspace is not None:
        _dev(workspace, "workspace")
    rows, heads, d_qk = q.shape
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return (_ptr(q), _ptr(kv_pool), kv_pool.shape[0], _ptr(topk_pos), _ptr(req_id),
            _ptr(causal_limit), block_table.shape[0], _ptr(block_table), block_table.shape[1],
            block_size, physical_block_stride, rows, heads, d_qk, d_v, topk_pos.shape[1],
            float(scale), _dtype_code(q.dtype), _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes)


def hs_sparse_decode_attn_paged(q: torch.Tensor, kv_pool: torch.Tensor, topk_pos: torch.Tensor,
                                req_id: torch.Tensor, causal_limit: torch.Tensor,
                                block_table: torch.Tensor, block_size: int,
                                physical_block_stride: int, scale: float, d_v: int,
                                out: torch.Tensor, lse: Optional[torch.Tensor] = None,
                                workspace: Optional[torch.Tensor] = None, stream=None):
    """Resolve + attention of a fully resident batch in one call (see include/hisparse.h)."""
    args = _paged_args(q, kv_pool, topk_pos, req_id, causal_limit, block_table, block_size,
                       physical_block_stride, scale, d_v, out, lse, workspace)
    _check("hs_sparse_decode_attn_paged", _lib.hs_sparse_decode_attn_paged(*args, _stream(stream)))


class PagedAttnCall:
    """hs_sparse_decode_attn_paged with its arguments checked and marshalled once.

    For callers whose decode buffers stay at fixed addresses from step to step: each call
    passes the stored pointers and sizes, plus the current (or given) stream, to the same C
    entry point.  The tensors are referenced here, so the stored pointers stay valid; their
    contents may change between calls.
    """

    def __init__(self, q, kv_pool, topk_pos, req_id, causal_limit, block_table, block_size,
                 physical_block_stride, scale, d_v, out, lse=None, workspace=None):
        args = _paged_args(q, kv_pool, topk_pos, req_id, causal_limit, block_table, block_size,
                           physical_block_stride, scale, d_v, out, lse, workspace)
        types = _lib.hs_sparse_decode_attn_paged.argtypes
        self._args = tuple(a if isinstance(a, ctypes.c_void_p) or a is None else t(a)
                           for a, t in zip(args, types))
        self._keep = (q, kv_pool, topk_pos, req_id, causal_limit, block_table, out, lse, workspace)
        self._fn = _lib.hs_sparse_decode_attn_paged

    def __call__(self, stream=None):
        status = self._fn(*self._args, _stream(stream))
        if status != HS_OK:
            raise HsError("hs_sparse_decode_attn_paged", status, status_string(status))


def hs_greedy_argmax(logits: torch.Tensor, out_argmax: torch.Tensor, stream=None):
    """Lowest index of each bf16 logit row's maximum (see include/hisparse.h)."""
    _shape(logits.dim() == 2 and tuple(out_argmax.shape) == (logits.shape[0],),
           "logits [rows, vocab] and out_argmax [rows] expected")
    _dev(logits, "logits", torch.bfloat16); _dev(out_argmax, "out_argmax", torch.int32)
    _check("hs_greedy_argmax", _lib.hs_greedy_argmax(_ptr(logits), logits.shape[0],
                                                     logits.shape[1], _ptr(out_argmax),
                                                     _stream(stream)))


def hs_finalize_accepted(state: HotState, logits: Optional[torch.Tensor], draft_ids: torch.Tensor,
                         new_kv: torch.Tensor, rows_per_req: int, seq_len: torch.Tensor,
                         block_table: torch.Tensor, block_size: int, tick: int,
                         out_argmax: torch.Tensor, out_accept_len: torch.Tensor,
                         out_next_token: torch.Tensor, stream=None):
    """Greedy accept + accepted-prefix KV keep (see include/hisparse.h).  ``logits=None``:
    ``out_argmax`` already holds the rows' argmax (hs_greedy_argmax) and is read."""
    i32 = torch.int32
    state.check_shapes()
    num_reqs = state.slot_loc.shape[0]
    rows = num_reqs * rows_per_req
    _shape(logits is None or (logits.dim() == 2 and logits.shape[0] == rows),
           "logits must be [num_reqs * rows_per_req, vocab]")
    _shape(tuple(draft_ids.shape) == (rows,) and tuple(out_argmax.shape) == (rows,),
           "draft_ids and out_argmax must be [num_reqs * rows_per_req]")
    _shape(tuple(new_kv.shape) == (rows, state.hot_kv.shape[1]),
           "new_kv must be [num_reqs * rows_per_req, row_elems]")
    _shape(tuple(seq_len.shape) == (num_reqs,) and tuple(out_accept_len.shape) == (num_reqs,) and
           tuple(out_next_token.shape) == (num_reqs,),
           "seq_len, out_accept_len and out_next_token must be [num_reqs]")
    _shape(block_table.dim() == 2 and block_table.shape[0] == num_reqs,
           "block_table must be [num_reqs, bt_stride]")
    if logits is not None:
        _dev(logits, "logits", torch.bfloat16)
    _dev(draft_ids, "draft_ids", i32)
    _dev(new_kv, "new_kv", state.hot_kv.dtype); _dev(seq_len, "seq_len", i32)
    _dev(block_table, "block_table", i32); _dev(out_argmax, "out_argmax", i32)
    _dev(out_accept_len, "out_accept_len", i32); _dev(out_next_token, "out_next_token", i32)
    st = state.as_struct()
    _check("hs_finalize_accepted", _lib.hs_finalize_accepted(
        ctypes.byref(st), _ptr(logits), 0 if logits is None else logits.shape[1], _ptr(draft_ids),
        _ptr(new_kv),
        rows_per_req, _ptr(seq_len), _ptr(block_table), block_table.shape[1], block_size, tick,
        _ptr(out_argmax), _ptr(out_accept_len), _ptr(out_next_token), _stream(stream)))
    state.note_tick(tick)


def hs_backup_rows(dev_cache: torch.Tensor, host_cache: torch.Tensor, src_slots: torch.Tensor,
                   dst_rows: torch.Tensor, src_block_size: int = 1, src_block_stride: int = 1,
                   stream=None):
    """Device -> host backup of KV rows (see include/hisparse.h).

    ``dev_cache`` [layers, rows, elems] (or [rows, elems] for one layer) on the device;
    ``host_cache`` pinned CPU tensor of the same dtype and layer count; ``src_slots``
    int32 [layers, n] (one list per layer) or [n] (shared); ``dst_rows`` int32 [n].
    """
    _dev(dev_cache, "dev_cache"); _dev(src_slots, "src_slots", torch.int32)
    _dev(dst_rows, "dst_rows", torch.int32)
    if host_cache.is_cuda or not host_cache.is_pinned() or not host_cache.is_contiguous():
        raise ValueError("host_cache must be a contiguous pinned host tensor")
    if host_cache.dtype != dev_cache.dtype or host_cache.dim() != dev_cache.dim():
        raise ValueError("host_cache must match dev_cache in dtype and rank")
    if dev_cache.dim() == 2:
        layers, dev_rows, elems = 1, dev_cache.shape[0], dev_cache.shape[1]
        host_rows, host_elems = host_cache.shape
    elif dev_cache.dim() == 3:
        layers, dev_rows, elems = dev_cache.shape
        host_layers, host_rows, host_elems = host_cache.shape
        if host_layers != layers:
            raise ValueError("host_cache and dev_cache differ in layer count")
    else:
        raise ValueError("dev_cache must be [rows, elems] or [layers, rows, elems]")
    if host_elems != elems:
        raise ValueError("host_cache and dev_cache rows differ in size")
    n = dst_rows.shape[0]
    if src_slots.dim() == 2:
        if src_slots.shape != (layers, n):
            raise ValueError("src_slots must be [layers, n] or [n]")
        per_layer = 1
    elif src_slots.dim() == 1 and src_slots.shape[0] == n:
        per_layer = 0
    else:
        raise ValueError("src_slots must be [layers, n] or [n]")
    _check("hs_backup_rows", _lib.hs_backup_rows(
        _ptr(dev_cache), dev_rows, ctypes.c_void_p(host_cache.data_ptr()), host_rows, layers,
        elems * dev_cache.element_size(), _ptr(src_slots), per_layer, _ptr(dst_rows), n,
        src_block_size, src_block_stride, _stream(stream)))



def hs_apply_plan(hot_kv: torch.Tensor, host_pool: torch.Tensor, wave_rows: torch.Tensor,
                  hot_idx: torch.Tensor, miss_count: torch.Tensor, miss_pos: torch.Tensor,
                  capacity: int, stream=None):
    """Fill follower caches from the leader's swap plan (see include/hisparse.h).

    ``hot_kv`` [caches, num_reqs*capacity, elems] (or [num_reqs*capacity, elems]) on the
    device; ``host_pool`` pinned [caches, host_rows, elems] (or 2-D) of the same dtype;
    ``wave_rows``, ``hot_idx``, ``miss_pos`` int32 [num_reqs, topk] and ``miss_count``
    int32 [num_reqs]: the leader's hs_swap_in input and outputs.
    """
    i32 = torch.int32
    _dev(hot_kv, "hot_kv"); _dev(wave_rows, "wave_rows", i32); _dev(hot_idx, "hot_idx", i32)
    _dev(miss_count, "miss_count", i32); _dev(miss_pos, "miss_pos", i32)
    if host_pool.is_cuda or not host_pool.is_pinned() or not host_pool.is_contiguous():
        raise ValueError("host_pool must be a contiguous pinned host tensor")
    if host_pool.dtype != hot_kv.dtype or host_pool.dim() != hot_kv.dim():
        raise ValueError("host_pool must match hot_kv in dtype and rank")
    if hot_kv.dim() == 2:
        caches, elems, host_rows = 1, hot_kv.shape[1], host_pool.shape[0]
        host_elems = host_pool.shape[1]
    elif hot_kv.dim() == 3:
        caches, elems = hot_kv.shape[0], hot_kv.shape[2]
        if host_pool.shape[0] != caches:
            raise ValueError("host_pool and hot_kv differ in cache count")
        host_rows, host_elems = host_pool.shape[1], host_pool.shape[2]
    else:
        raise ValueError("hot_kv must be [rows, elems] or [caches, rows, elems]")
    if host_elems != elems:
        raise ValueError("host_pool and hot_kv rows differ in size")
    num_reqs, topk = wave_rows.shape
    if hot_kv.shape[-2] != num_reqs * capacity:
        raise ValueError("hot_kv must hold num_reqs * capacity rows per cache")
    if hot_idx.shape != wave_rows.shape or miss_pos.shape != wave_rows.shape or \
            miss_count.shape != (num_reqs,):
        raise ValueError("plan tensors must be [num_reqs, topk] (miss_count [num_reqs])")
    _check("hs_apply_plan", _lib.hs_apply_plan(
        _ptr(hot_kv), ctypes.c_void_p(host_pool.data_ptr()), host_rows, caches, num_reqs,
        capacity, elems * hot_kv.element_size(), _ptr(wave_rows), topk, _ptr(hot_idx),
        _ptr(miss_count), _ptr(miss_pos), _stream(stream)))


def hs_sparse_decode_attn_mixed(q: torch.Tensor, kv_a: torch.Tensor, indices_a: torch.Tensor,
                                kv_b: torch.Tensor, indices_b: torch.Tensor,
                                row_sel: torch.Tensor, scale: float, d_v: int, out: torch.Tensor,
                                lse: Optional[torch.Tensor] = None,
                                workspace: Optional[torch.Tensor] = None, stream=None,
                                max_cus: Optional[int] = None):
    """Attention whose rows read one of two caches (see include/hisparse.h); with
    ``max_cus``, hs_sparse_decode_attn_mixed_cus (planned for that many compute units)."""
    i32 = torch.int32
    _attn_shapes(q, kv_a, indices_a, d_v, out, lse)
    _shape(kv_b.dim() == 2 and kv_b.shape[1] == q.shape[2], "kv_b rows must be d_qk wide")
    _dev(q, "q"); _dev(kv_a, "kv_a", q.dtype); _dev(kv_b, "kv_b", q.dtype)
    _dev(indices_a, "indices_a", i32); _dev(indices_b, "indices_b", i32)
    _dev(row_sel, "row_sel", i32); _dev(out, "out", q.dtype)
    if lse is not None:
        _dev(lse, "lse", torch.float32)
    if workspace is not None:
        _dev(workspace, "workspace")
    rows, heads, d_qk = q.shape
    if indices_a.shape != indices_b.shape or indices_a.shape[0] != rows or row_sel.shape != (rows,):
        raise ValueError("indices_a, indices_b must be [rows, topk] and row_sel [rows]")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    args = (_ptr(q), _ptr(kv_a), kv_a.shape[0], _ptr(indices_a), _ptr(kv_b), kv_b.shape[0],
            _ptr(indices_b), _ptr(row_sel), rows, heads, d_qk, d_v, indices_a.shape[1],
            float(scale), _dtype_code(q.dtype), _ptr(out), _ptr(lse), _ptr(workspace), ws_bytes)
    if max_cus is None:
        _check("hs_sparse_decode_attn_mixed", _lib.hs_sparse_decode_attn_mixed(*args,
                                                                               _stream(stream)))
    else:
        _check("hs_sparse_decode_attn_mixed_cus", _lib.hs_sparse_decode_attn_mixed_cus(
            *args, int(max_cus), _stream(stream)))



def hs_append_accepted(ctx_cache: torch.Tensor, ctx_block_table: torch.Tensor,
                       ctx_len: torch.Tensor, new_rows: torch.Tensor, accept_len: torch.Tensor,
                       block_size: int, physical_block_stride: int, rows_per_req: int,
                       stream=None):
    """Append each request's accepted prefix to the draft model's context cache and advance
    ctx_len in place (see include/hisparse.h)."""
    i32 = torch.int32
    _dev(ctx_cache, "ctx_cache"); _dev(ctx_block_table, "ctx_block_table", i32)
    _dev(ctx_len, "ctx_len", i32); _dev(new_rows, "new_rows", ctx_cache.dtype)
    _dev(accept_len, "accept_len", i32)
    num_reqs = ctx_len.shape[0]
    if ctx_cache.dim() != 2 or new_rows.dim() != 2 or new_rows.shape[1] != ctx_cache.shape[1]:
        raise ValueError("ctx_cache and new_rows must be [rows, elems] of the same width")
    if new_rows.shape[0] != num_reqs * rows_per_req or accept_len.shape != (num_reqs,) or \
            ctx_block_table.shape[0] != num_reqs:
        raise ValueError("new_rows must hold num_reqs * rows_per_req rows")
    _check("hs_append_accepted", _lib.hs_append_accepted(
        _ptr(ctx_cache), ctx_cache.shape[0], ctx_cache.shape[1] * ctx_cache.element_size(),
        _ptr(ctx_block_table), ctx_block_table.shape[1], block_size, physical_block_stride,
        _ptr(ctx_len), _ptr(new_rows), _ptr(accept_len), num_reqs, rows_per_req, _stream(stream)))


def hs_host_read(host_src: torch.Tensor, dst: torch.Tensor, stream=None):
    """Streaming zero-copy read of a pinned host tensor into a device tensor of the same byte
    size: the host link's reference read rate (see include/hisparse.h)."""
    if host_src.is_cuda or not host_src.is_pinned() or not host_src.is_contiguous():
        raise ValueError("host_src must be a contiguous pinned host tensor")
    nbytes = host_src.numel() * host_src.element_size()
    _shape(dst.numel() * dst.element_size() == nbytes, "dst must hold as many bytes as host_src")
    _dev(dst, "dst")
    _check("hs_host_read", _lib.hs_host_read(ctypes.c_void_p(host_src.data_ptr()), _ptr(dst),
                                             nbytes, _stream(stream)))
