"""ctypes binding of libcacheblend.so (argument marshalling only).

Every step of the blend runs in the library's HIP kernels; torch supplies
device memory and the current stream.  There is no fallback: if the library
is not built, loading it raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np
import torch

# The in-tree build; CB_LIBRARY may name another build of the same library.
LIB_PATH = os.environ.get("CB_LIBRARY") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libcacheblend.so")

CB_OK, CB_ERR_INVALID_ARG, CB_ERR_UNSUPPORTED, CB_ERR_HIP = 0, 1, 2, 3
CB_DTYPE_F32, CB_DTYPE_BF16 = 0, 1
ROPE_HALF, ROPE_INTERLEAVED = 0, 1
CB_DEV_V, CB_DEV_K, CB_DEV_KV = 0, 1, 2
CB_ATTN_COUNTERS_ZERO = 1
CB_LAYER_WORKSPACE_ZEROED = 1
CB_SELECT_COUNTER_BYTES = 4096
CB_CHECK_CAND_RANGE, CB_CHECK_CAND_ORDER, CB_CHECK_SEL_RANGE = 1, 2, 4
CB_CHECK_SEL_ORDER, CB_CHECK_LOCAL_RANGE, CB_CHECK_LOCAL_MISMATCH = 8, 16, 32
CB_ORDER_AUTO, CB_ORDER_ROTATE_FIRST, CB_ORDER_SELECT_FIRST = 0, 1, 2
ORDERS = {"auto": CB_ORDER_AUTO, "rotate-first": CB_ORDER_ROTATE_FIRST,
          "select-first": CB_ORDER_SELECT_FIRST}
DEV_SOURCES = {"v": CB_DEV_V, "k": CB_DEV_K, "kv": CB_DEV_KV}

_i32p = ctypes.POINTER(ctypes.c_int32)


class Geom(ctypes.Structure):
    _fields_ = [("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class Ragged(ctypes.Structure):
    _fields_ = [("n_req", ctypes.c_int32),
                ("tok_off", ctypes.c_void_p), ("cand_off", ctypes.c_void_p),
                ("sel_off", ctypes.c_void_p),
                ("h_tok_off", _i32p), ("h_cand_off", _i32p), ("h_sel_off", _i32p)]


class LayerArgs(ctypes.Structure):
    _fields_ = [("geom", Geom), ("rg", Ragged),
                ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("k_new_c", ctypes.c_void_p), ("v_new_c", ctypes.c_void_p),
                ("q_c", ctypes.c_void_p), ("delta", ctypes.c_void_p),
                ("cand_idx", ctypes.c_void_p), ("rope_theta", ctypes.c_double),
                ("rope_style", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
                ("dev", ctypes.c_void_p), ("sel_local", ctypes.c_void_p),
                ("sel_global", ctypes.c_void_p), ("out", ctypes.c_void_p),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
                ("dev_source", ctypes.c_int32), ("order", ctypes.c_int32),
                ("flags", ctypes.c_uint32)]


class AttnPlan(ctypes.Structure):
    _fields_ = [("mfma", ctypes.c_int32), ("key_split", ctypes.c_int32),
                ("rows_per_tile", ctypes.c_int32), ("key_chunk", ctypes.c_int32),
                ("tiles", ctypes.c_int64), ("workgroups", ctypes.c_int64),
                ("workspace_bytes", ctypes.c_size_t), ("stream_spans", ctypes.c_int32)]


class CbError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


_STATUS = {0: "CB_OK", 1: "CB_ERR_INVALID_ARG", 2: "CB_ERR_UNSUPPORTED", 3: "CB_ERR_HIP"}
_LIB = None

_SIGNATURES = {
    "cb_rerotate": [ctypes.POINTER(Geom), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                    ctypes.c_int64, ctypes.c_int32, ctypes.c_double, ctypes.c_int32, ctypes.c_void_p],
    "cb_deviation_topk": [ctypes.POINTER(Geom), ctypes.POINTER(Ragged), ctypes.c_void_p,
                          ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                          ctypes.c_void_p, ctypes.c_void_p],
    "cb_kv_deviation_topk": [ctypes.POINTER(Geom), ctypes.POINTER(Ragged), ctypes.c_int32,
                             ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                             ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                             ctypes.c_void_p],
    "cb_topk": [ctypes.POINTER(Ragged), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                ctypes.c_void_p, ctypes.c_void_p],
    "cb_fuse_scatter": [ctypes.POINTER(Geom), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                        ctypes.c_void_p],
    "cb_check_indices": [ctypes.POINTER(Ragged), ctypes.c_void_p, ctypes.c_void_p,
                         ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p],
    "cb_rerotate_fuse": [ctypes.POINTER(Geom), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                         ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                         ctypes.c_int64, ctypes.c_int64, ctypes.c_double, ctypes.c_int32,
                         ctypes.c_void_p],
    "cb_partial_attn": [ctypes.POINTER(Geom), ctypes.POINTER(Ragged), ctypes.c_void_p,
                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                        ctypes.c_void_p, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t,
                        ctypes.c_void_p],
    "cb_partial_attn_workspace_size": [ctypes.POINTER(Geom), ctypes.POINTER(Ragged),
                                       ctypes.POINTER(ctypes.c_size_t)],
    "cb_partial_attn_plan": [ctypes.POINTER(Geom), ctypes.POINTER(Ragged), ctypes.c_size_t,
                             ctypes.POINTER(AttnPlan)],
    "cb_partial_attn_describe_plan": [ctypes.POINTER(Geom), ctypes.POINTER(Ragged),
                                      ctypes.POINTER(AttnPlan)],
    "cb_partial_attn_with_plan": [ctypes.POINTER(Geom), ctypes.POINTER(Ragged),
                                  ctypes.POINTER(AttnPlan), ctypes.c_void_p, ctypes.c_void_p,
                                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                  ctypes.c_void_p, ctypes.c_float, ctypes.c_void_p,
                                  ctypes.c_size_t, ctypes.c_uint32, ctypes.c_void_p],
    "cb_blend_layer": [ctypes.POINTER(LayerArgs), ctypes.c_void_p],
    "cb_blend_layer_noalloc": [ctypes.POINTER(LayerArgs), ctypes.c_void_p],
    "cb_blend_layer_order": [ctypes.POINTER(LayerArgs), ctypes.POINTER(ctypes.c_int32)],
}


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m selective_recompute_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.argtypes = args
            fn.restype = ctypes.c_int
        handle.cb_status_str.argtypes = [ctypes.c_int]
        handle.cb_status_str.restype = ctypes.c_char_p
        handle.cb_last_error.argtypes = []
        handle.cb_last_error.restype = ctypes.c_char_p
        handle.cb_abi_version.argtypes = []
        handle.cb_abi_version.restype = ctypes.c_int32
        _LIB = handle
    return _LIB


def check(status: int):
    if status != CB_OK:
        raise CbError(status, lib().cb_last_error().decode())


def dtype_code(t: torch.dtype) -> int:
    if t == torch.float32:
        return CB_DTYPE_F32
    if t == torch.bfloat16:
        return CB_DTYPE_BF16
    raise TypeError(f"unsupported dtype {t}")


def geom(n_q_heads: int, n_kv_heads: int, head_dim: int, dtype: torch.dtype) -> Geom:
    return Geom(n_q_heads, n_kv_heads, head_dim, dtype_code(dtype))


def _dev(t: Optional[torch.Tensor], dtype=None) -> Optional[int]:
    """Device address of a contiguous GPU tensor (None stays NULL)."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"expected {dtype}, got {t.dtype}")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


class RaggedBatch:
    """Device offsets and their host mirrors for one ragged call."""

    def __init__(self, tok_off: Sequence[int], cand_off: Sequence[int], sel_off: Sequence[int],
                 device="cuda"):
        self.h_tok = np.ascontiguousarray(tok_off, dtype=np.int32)
        self.h_cand = np.ascontiguousarray(cand_off, dtype=np.int32)
        self.h_sel = np.ascontiguousarray(sel_off, dtype=np.int32)
        self.tok = torch.from_numpy(self.h_tok).to(device)
        self.cand = torch.from_numpy(self.h_cand).to(device)
        self.sel = torch.from_numpy(self.h_sel).to(device)
        self.n_req = len(self.h_tok) - 1

    @property
    def n_tokens(self) -> int:
        return int(self.h_tok[-1])

    @property
    def n_cand(self) -> int:
        return int(self.h_cand[-1])

    @property
    def n_sel(self) -> int:
        return int(self.h_sel[-1])

    def struct(self) -> Ragged:
        return Ragged(self.n_req, _dev(self.tok, torch.int32), _dev(self.cand, torch.int32),
                      _dev(self.sel, torch.int32),
                      self.h_tok.ctypes.data_as(_i32p), self.h_cand.ctypes.data_as(_i32p),
                      self.h_sel.ctypes.data_as(_i32p))


def rerotate(g: Geom, k_out: torch.Tensor, k_in: torch.Tensor, delta: torch.Tensor,
             n_tok: int, n_layers: int, rope_theta: float, rope_style: int = ROPE_HALF,
             stream=None):
    check(lib().cb_rerotate(ctypes.byref(g), _dev(k_out), _dev(k_in), _dev(delta, torch.int32),
                            n_tok, n_layers, rope_theta, rope_style, _stream(stream)))


def deviation_topk(g: Geom, rb: RaggedBatch, v_new_c, v_old, cand_idx, dev, sel_local,
                   sel_global, stream=None):
    rg = rb.struct()
    check(lib().cb_deviation_topk(ctypes.byref(g), ctypes.byref(rg), _dev(v_new_c), _dev(v_old),
                                  _dev(cand_idx, torch.int32), _dev(dev, torch.float32),
                                  _dev(sel_local, torch.int32), _dev(sel_global, torch.int32),
                                  _stream(stream)))


def kv_deviation_topk(g: Geom, rb: RaggedBatch, source: int, k_new_c, k_cached, v_new_c, v_old,
                      cand_idx, dev, sel_local, sel_global, stream=None):
    rg = rb.struct()
    check(lib().cb_kv_deviation_topk(ctypes.byref(g), ctypes.byref(rg), source, _dev(k_new_c),
                                     _dev(k_cached), _dev(v_new_c), _dev(v_old),
                                     _dev(cand_idx, torch.int32), _dev(dev, torch.float32),
                                     _dev(sel_local, torch.int32), _dev(sel_global, torch.int32),
                                     _stream(stream)))


def topk(rb: RaggedBatch, dev, cand_idx, sel_local, sel_global, stream=None):
    rg = rb.struct()
    check(lib().cb_topk(ctypes.byref(rg), _dev(dev, torch.float32), _dev(cand_idx, torch.int32),
                        _dev(sel_local, torch.int32), _dev(sel_global, torch.int32),
                        _stream(stream)))


def fuse_scatter(g: Geom, k_fused, v_fused, k_new_c, v_new_c, sel_local, sel_global,
                 k_total: int, stream=None):
    check(lib().cb_fuse_scatter(ctypes.byref(g), _dev(k_fused), _dev(v_fused), _dev(k_new_c),
                                _dev(v_new_c), _dev(sel_local, torch.int32),
                                _dev(sel_global, torch.int32), k_total, _stream(stream)))


def check_indices(rb: RaggedBatch, cand_idx=None, sel_local=None, sel_global=None,
                  stream=None) -> torch.Tensor:
    """cb_check_indices: a device int32 tensor with the OR of the violated
    preconditions (0: all hold); the caller reads it when it wants to."""
    flags = torch.empty(1, dtype=torch.int32, device=rb.tok.device)
    check(lib().cb_check_indices(ctypes.byref(rb.struct()), _dev(cand_idx, torch.int32),
                                 _dev(sel_local, torch.int32), _dev(sel_global, torch.int32),
                                 _dev(flags, torch.int32), _stream(stream)))
    return flags


def rerotate_fuse(g: Geom, k, v, k_new_c, v_new_c, delta, sel_local, sel_global, k_total: int,
                  n_tok: int, rope_theta: float, rope_style: int = ROPE_HALF, stream=None):
    check(lib().cb_rerotate_fuse(ctypes.byref(g), _dev(k), _dev(v), _dev(k_new_c), _dev(v_new_c),
                                 _dev(delta, torch.int32), _dev(sel_local, torch.int32),
                                 _dev(sel_global, torch.int32), k_total, n_tok, rope_theta,
                                 rope_style, _stream(stream)))


def attn_workspace_bytes(g: Geom, rb: RaggedBatch) -> int:
    """Workspace with which cb_partial_attn may split long rows (0 = none)."""
    n = ctypes.c_size_t(0)
    rg = rb.struct()
    check(lib().cb_partial_attn_workspace_size(ctypes.byref(g), ctypes.byref(rg), ctypes.byref(n)))
    return int(n.value)


def attn_plan(g: Geom, rb: RaggedBatch, workspace_bytes: Optional[int] = None) -> dict:
    """The decomposition cb_partial_attn uses (cb_attn_plan as a dict);
    workspace_bytes None = as much as the plan can use."""
    plan = AttnPlan()
    rg = rb.struct()
    ws = ctypes.c_size_t(-1).value if workspace_bytes is None else workspace_bytes
    check(lib().cb_partial_attn_plan(ctypes.byref(g), ctypes.byref(rg), ws, ctypes.byref(plan)))
    return {name: getattr(plan, name) for name, _ in AttnPlan._fields_}


def describe_plan(g: Geom, rb: RaggedBatch, mfma: int = 1, key_split: int = 1,
                  key_chunk: int = 0, stream_spans: int = 0) -> dict:
    """A pinned plan with its derived fields (cb_partial_attn_describe_plan)."""
    plan = AttnPlan(mfma, key_split, 0, key_chunk, 0, 0, 0, stream_spans)
    rg = rb.struct()
    check(lib().cb_partial_attn_describe_plan(ctypes.byref(g), ctypes.byref(rg),
                                              ctypes.byref(plan)))
    return {name: getattr(plan, name) for name, _ in AttnPlan._fields_}


def workspace_tensor(nbytes: int, device="cuda") -> Optional[torch.Tensor]:
    """A device buffer of at least nbytes (16-byte aligned), zero-filled, or
    None for 0.  Zero-filled, it may be passed to cb_blend_layer with
    CB_LAYER_WORKSPACE_ZEROED."""
    if nbytes <= 0:
        return None
    return torch.zeros(nbytes, dtype=torch.uint8, device=device)


def _ws(ws: Optional[torch.Tensor]):
    return (None, 0) if ws is None else (_dev(ws), ws.numel() * ws.element_size())


def partial_attn(g: Geom, rb: RaggedBatch, out, q_c, sel_local, sel_global, k_fused, v_fused,
                 softmax_scale: float, workspace: Optional[torch.Tensor] = None, stream=None):
    rg = rb.struct()
    ws_ptr, ws_bytes = _ws(workspace)
    check(lib().cb_partial_attn(ctypes.byref(g), ctypes.byref(rg), _dev(out), _dev(q_c),
                                _dev(sel_local, torch.int32), _dev(sel_global, torch.int32),
                                _dev(k_fused), _dev(v_fused), softmax_scale, ws_ptr, ws_bytes,
                                _stream(stream)))


def partial_attn_with_plan(g: Geom, rb: RaggedBatch, plan: dict, out, q_c, sel_local,
                           sel_global, k_fused, v_fused, softmax_scale: float,
                           workspace: Optional[torch.Tensor] = None, stream=None,
                           counters_zero: bool = False):
    """cb_partial_attn with a pinned plan (a dict with mfma, key_split, key_chunk).
    counters_zero: pass CB_ATTN_COUNTERS_ZERO (the workspace was zero-filled and
    has since been used only with this plan)."""
    p = AttnPlan(plan["mfma"], plan.get("key_split", 1), 0, plan.get("key_chunk", 0), 0, 0, 0,
                 plan.get("stream_spans", 0))
    rg = rb.struct()
    ws_ptr, ws_bytes = _ws(workspace)
    flags = CB_ATTN_COUNTERS_ZERO if counters_zero else 0
    check(lib().cb_partial_attn_with_plan(ctypes.byref(g), ctypes.byref(rg), ctypes.byref(p),
                                          _dev(out), _dev(q_c), _dev(sel_local, torch.int32),
                                          _dev(sel_global, torch.int32), _dev(k_fused),
                                          _dev(v_fused), softmax_scale, ws_ptr, ws_bytes,
                                          flags, _stream(stream)))


def blend_layer(g: Geom, rb: RaggedBatch, *, k, v, k_new_c, v_new_c, q_c, delta, cand_idx,
                rope_theta: float, rope_style: int, softmax_scale: float, dev, sel_local,
                sel_global, out, workspace: Optional[torch.Tensor] = None,
                dev_source: int = CB_DEV_V, order: int = CB_ORDER_AUTO, flags: int = 0,
                stream=None):
    """cb_blend_layer.  flags: CB_LAYER_WORKSPACE_ZEROED when the workspace was
    zero-filled (workspace_tensor) and used since only by cb_blend_layer."""
    args = LayerArgs(g, rb.struct(), _dev(k), _dev(v), _dev(k_new_c), _dev(v_new_c), _dev(q_c),
                     _dev(delta, torch.int32), _dev(cand_idx, torch.int32), rope_theta,
                     rope_style, softmax_scale, _dev(dev, torch.float32),
                     _dev(sel_local, torch.int32), _dev(sel_global, torch.int32), _dev(out),
                     *_ws(workspace), dev_source, order, flags)
    check(lib().cb_blend_layer(ctypes.byref(args), _stream(stream)))


def blend_layer_noalloc(g: Geom, rb: RaggedBatch, *, k, v, k_new_c, v_new_c, q_c, delta,
                        cand_idx, rope_theta: float, rope_style: int, softmax_scale: float, dev,
                        sel_local, sel_global, out, dev_source: int = CB_DEV_V,
                        order: int = CB_ORDER_AUTO, stream=None):
    """cb_blend_layer_noalloc: the attention workspace is the library's static
    device scratch (no workspace argument)."""
    args = LayerArgs(g, rb.struct(), _dev(k), _dev(v), _dev(k_new_c), _dev(v_new_c), _dev(q_c),
                     _dev(delta, torch.int32), _dev(cand_idx, torch.int32), rope_theta,
                     rope_style, softmax_scale, _dev(dev, torch.float32),
                     _dev(sel_local, torch.int32), _dev(sel_global, torch.int32), _dev(out),
                     None, 0, dev_source, order, 0)
    check(lib().cb_blend_layer_noalloc(ctypes.byref(args), _stream(stream)))


class PreparedLayer:
    """A cb_layer_args struct built ahead of time (keeps its inputs alive), so a
    timed loop only pays for the C call."""

    def __init__(self, g: Geom, rb: RaggedBatch, *, k, v, k_new_c, v_new_c, q_c, delta,
                 cand_idx, rope_theta, rope_style, softmax_scale, dev, sel_local, sel_global,
                 out, workspace: Optional[torch.Tensor] = None, dev_source: int = CB_DEV_V,
                 order: int = CB_ORDER_AUTO, flags: int = 0):
        self._keep = (rb, k, v, k_new_c, v_new_c, q_c, delta, cand_idx, dev, sel_local,
                      sel_global, out, workspace)
        self.args = LayerArgs(g, rb.struct(), _dev(k), _dev(v), _dev(k_new_c), _dev(v_new_c),
                              _dev(q_c), _dev(delta, torch.int32), _dev(cand_idx, torch.int32),
                              rope_theta, rope_style, softmax_scale, _dev(dev, torch.float32),
                              _dev(sel_local, torch.int32), _dev(sel_global, torch.int32),
                              _dev(out), *_ws(workspace), dev_source, order, flags)
        self.ref = ctypes.byref(self.args)

    def resolved_order(self) -> int:
        """CB_ORDER_ROTATE_FIRST or CB_ORDER_SELECT_FIRST, as cb_blend_layer runs it."""
        o = ctypes.c_int32(-1)
        check(lib().cb_blend_layer_order(self.ref, ctypes.byref(o)))
        return o.value

    def launch(self, stream_handle: int):
        st = lib().cb_blend_layer(self.ref, stream_handle)
        if st != CB_OK:
            check(st)
