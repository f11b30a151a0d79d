"""Python binding of libmoe_mxfp4.so: the routed-expert MXFP4 MoE layer on
AMD MI355X (gfx950).

Argument marshalling only: every step of the layer runs in the HIP library.
torch provides device memory and the current stream.  If the library has not
been built, importing the low-level entry points raises at once; there is no
other execution path.

Names follow the C ABI in include/moe_mxfp4.h:
  query_sizes(cfg)                      -> (repacked_bytes, workspace_bytes)
  Plan(cfg, w13_codes, w13_scales, w2_codes, w2_scales)     (moe_mxfp4_plan)
  Plan.forward(hidden, topk_ids, topk_weights, out=None, acc=None)
  Plan.forward_noalloc(...)             the same, scratch in the library (moe_mxfp4_forward_noalloc)
  Plan.route(topk_ids)                  -> (counts, offsets, perm, rowpos)
  Plan.workspace_region(region)         -> the workspace bytes of an intermediate (MXFP8 h)
  mxfp8_quantize(x_bf16)                -> (codes, scales)
  router_topk(logits, k)                -> (topk_ids, topk_weights)  (moe_router_topk)
  probe_memory(kind, src, dst, sink)    peak micro-benchmarks (moe_probe_memory / moe_probe_mfma)
  probe_mfma(kind, iters, sink)         -> flops of the launch
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_mxfp4.so")

MOE_ACT_BF16 = 0
MOE_ACT_MXFP8 = 1
STATUS_NAMES = {0: "MOE_OK", 1: "MOE_ERR_ARG", 2: "MOE_ERR_SHAPE", 3: "MOE_ERR_ALIGN", 4: "MOE_ERR_CAPACITY",
                5: "MOE_ERR_SCALE_BYTE", 6: "MOE_ERR_WORKSPACE", 7: "MOE_ERR_UNSUPPORTED", 8: "MOE_ERR_HIP",
                9: "MOE_ERR_TIMEOUT"}
MOE_WS_H_CODES = 0
MOE_WS_H_SCALES = 1
EXPORTS = ("moe_mxfp4_query_sizes", "moe_mxfp4_plan", "moe_mxfp4_forward", "moe_mxfp4_forward_noalloc",
           "moe_mxfp4_forward_fused",
           "moe_mxfp4_fused_status", "moe_mxfp4_route", "moe_mxfp4_workspace_region", "moe_mxfp8_quantize",
           "moe_router_topk", "moe_probe_memory", "moe_probe_mfma", "moe_probe_mfma_f8f4_blocks",
           "moe_mxfp4_set_stage_events",
           "moe_mxfp4_destroy", "moe_mxfp4_last_error")
_STATUS_FNS = tuple(n for n in EXPORTS if n not in ("moe_mxfp4_destroy", "moe_mxfp4_last_error"))


class MoeError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status
        self.message = message


class _Config(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("intermediate", ctypes.c_int32), ("num_experts", ctypes.c_int32),
                ("top_k", ctypes.c_int32), ("max_tokens", ctypes.c_int32), ("act", ctypes.c_int32)]


@dataclasses.dataclass(frozen=True)
class Config:
    hidden: int
    intermediate: int
    num_experts: int
    top_k: int
    max_tokens: int
    act: int = MOE_ACT_BF16

    def c(self) -> _Config:
        return _Config(self.hidden, self.intermediate, self.num_experts, self.top_k, self.max_tokens, self.act)


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"libmoe_mxfp4.so not found at {path}; build it with "
                          f"`python -m mxfp4_routed_expert_topk_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    cfgp = ctypes.POINTER(_Config)
    lib.moe_mxfp4_query_sizes.argtypes = [cfgp, ctypes.POINTER(sz), ctypes.POINTER(sz)]
    lib.moe_mxfp4_plan.argtypes = [cfgp, vp, vp, vp, vp, vp, sz, vp, ctypes.POINTER(vp)]
    lib.moe_mxfp4_forward.argtypes = [vp, vp, vp, vp, i32, vp, vp, vp, sz, vp]
    lib.moe_mxfp4_forward_fused.argtypes = [vp, vp, vp, vp, i32, vp, vp, vp, sz, vp]
    lib.moe_mxfp4_forward_noalloc.argtypes = [vp, vp, vp, vp, i32, vp, vp, vp]
    lib.moe_mxfp4_fused_status.argtypes = [vp, vp, sz, vp]
    lib.moe_mxfp4_route.argtypes = [vp, vp, i32, vp, vp, vp, vp, vp, sz, vp]
    lib.moe_mxfp4_workspace_region.argtypes = [vp, i32, ctypes.POINTER(sz), ctypes.POINTER(sz)]
    lib.moe_mxfp8_quantize.argtypes = [vp, i32, i32, vp, vp, vp]
    lib.moe_router_topk.argtypes = [vp, i32, i32, i32, vp, vp, vp]
    lib.moe_probe_memory.argtypes = [i32, vp, vp, sz, vp, i32, vp]
    lib.moe_probe_mfma.argtypes = [i32, i32, vp, i32, ctypes.POINTER(ctypes.c_double), vp]
    lib.moe_probe_mfma_f8f4_blocks.argtypes = [vp, vp, vp, vp, vp, vp, i32, vp]
    lib.moe_mxfp4_set_stage_events.argtypes = [vp, ctypes.POINTER(vp), i32]
    lib.moe_mxfp4_destroy.argtypes = [vp]
    lib.moe_mxfp4_destroy.restype = None
    lib.moe_mxfp4_last_error.argtypes = []
    lib.moe_mxfp4_last_error.restype = ctypes.c_char_p
    for name in _STATUS_FNS:
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != 0:
        raise MoeError(status, load_library().moe_mxfp4_last_error().decode())


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


MOE_ERR_ARG = 1


def _arg_error(msg: str):
    return MoeError(MOE_ERR_ARG, msg)


def _need(t, name: str, dtype, rows_min: int, cols: Optional[int], device, ndim: int = 2):
    """Raise MoeError(MOE_ERR_ARG) unless `t` is a contiguous tensor of `dtype`
    on `device`, shaped [>= rows_min, cols] (cols None: any)."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise _arg_error(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if t.dtype != dtype:
        raise _arg_error(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise _arg_error(f"{name} must have {ndim} dimensions, got shape {tuple(t.shape)}")
    if device is not None and t.device != device:
        raise _arg_error(f"{name} must be on {device}, got {t.device}")
    if not t.is_contiguous():
        raise _arg_error(f"{name} must be contiguous")
    if ndim == 2:
        if t.shape[0] < rows_min:
            raise _arg_error(f"{name} must have at least {rows_min} rows, got shape {tuple(t.shape)}")
        if cols is not None and t.shape[1] != cols:
            raise _arg_error(f"{name} must have {cols} columns, got shape {tuple(t.shape)}")
    elif t.numel() < rows_min:
        raise _arg_error(f"{name} must hold at least {rows_min} elements, got {t.numel()}")


def _stream(stream=None) -> int:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def query_sizes(cfg: Config):
    lib = load_library()
    rb, wb = ctypes.c_size_t(), ctypes.c_size_t()
    _check(lib.moe_mxfp4_query_sizes(ctypes.byref(cfg.c()), ctypes.byref(rb), ctypes.byref(wb)))
    return rb.value, wb.value


class Plan:
    """A plan over repacked weights.  Holds the repacked buffer and the
    forward workspace as torch uint8 tensors on the current device."""

    def __init__(self, cfg: Config, w13_codes, w13_scales, w2_codes, w2_scales, stream=None):
        import torch
        lib = load_library()
        self.cfg = cfg
        self.repacked_bytes, self.workspace_bytes = query_sizes(cfg)
        dev = w13_codes.device
        self.repacked = torch.empty(self.repacked_bytes, dtype=torch.uint8, device=dev)
        # zero-filled: the fused forward keeps its counters here and starts from zeros
        self.workspace = torch.zeros(self.workspace_bytes, dtype=torch.uint8, device=dev)
        h = ctypes.c_void_p()
        _check(lib.moe_mxfp4_plan(ctypes.byref(cfg.c()), _ptr(w13_codes), _ptr(w13_scales), _ptr(w2_codes),
                                  _ptr(w2_scales), _ptr(self.repacked), self.repacked_bytes, _stream(stream),
                                  ctypes.byref(h)))
        self._h = h
        self._events = None

    def close(self):
        if getattr(self, "_h", None) and self._h.value:
            load_library().moe_mxfp4_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _forward_args(self, hidden, topk_ids, topk_weights, out, acc, num_tokens, workspace):
        """Check the tensors of a forward against the plan (dtype, shape, device,
        contiguity; MoeError(MOE_ERR_ARG) otherwise) and allocate `out` if None."""
        import torch
        c = self.cfg
        dev = self.workspace.device
        if not isinstance(hidden, torch.Tensor) or hidden.dim() != 2:
            raise _arg_error("hidden must be a 2-D torch.Tensor [T, hidden]")
        T = hidden.shape[0] if num_tokens is None else int(num_tokens)
        if T < 0 or T > hidden.shape[0]:
            raise _arg_error(f"num_tokens must be in [0, {hidden.shape[0]}] (rows of hidden), got {T}")
        _need(hidden, "hidden", torch.bfloat16, T, c.hidden, dev)
        _need(topk_ids, "topk_ids", torch.int32, T, c.top_k, dev)
        _need(topk_weights, "topk_weights", torch.float32, T, c.top_k, dev)
        if out is None:
            out = torch.empty((hidden.shape[0], c.hidden), dtype=torch.bfloat16, device=dev)
        _need(out, "out", torch.bfloat16, T, c.hidden, dev)
        if acc is not None:
            _need(acc, "acc", torch.float32, T, c.hidden, dev)
        ws = self.workspace if workspace is None else workspace
        _need(ws, "workspace", torch.uint8, 0, None, dev, ndim=1)
        return T, out, ws

    def forward(self, hidden, topk_ids, topk_weights, out=None, acc=None, num_tokens=None, stream=None,
                workspace=None):
        T, out, ws = self._forward_args(hidden, topk_ids, topk_weights, out, acc, num_tokens, workspace)
        _check(load_library().moe_mxfp4_forward(self._h, _ptr(hidden), _ptr(topk_ids), _ptr(topk_weights), T,
                                                _ptr(acc), _ptr(out), _ptr(ws), ws.numel(), _stream(stream)))
        return out

    def forward_noalloc(self, hidden, topk_ids, topk_weights, out=None, acc=None, num_tokens=None, stream=None):
        """The same forward with the library's fixed scratch instead of a
        workspace (moe_mxfp4_forward_noalloc); pass `out` to allocate nothing."""
        T, out, _ = self._forward_args(hidden, topk_ids, topk_weights, out, acc, num_tokens, None)
        _check(load_library().moe_mxfp4_forward_noalloc(self._h, _ptr(hidden), _ptr(topk_ids), _ptr(topk_weights), T,
                                                        _ptr(acc), _ptr(out), _stream(stream)))
        return out

    def forward_fused(self, hidden, topk_ids, topk_weights, out=None, acc=None, num_tokens=None, stream=None,
                      workspace=None):
        """The same forward in one kernel launch (bf16 plans, at most 256 routes)."""
        T, out, ws = self._forward_args(hidden, topk_ids, topk_weights, out, acc, num_tokens, workspace)
        _check(load_library().moe_mxfp4_forward_fused(self._h, _ptr(hidden), _ptr(topk_ids), _ptr(topk_weights),
                                                      T, _ptr(acc), _ptr(out), _ptr(ws), ws.numel(),
                                                      _stream(stream)))
        return out

    def fused_status(self, stream=None, workspace=None):
        """Raise MoeError(MOE_ERR_TIMEOUT) if the last fused forward's waits timed out (synchronises)."""
        ws = self.workspace if workspace is None else workspace
        _check(load_library().moe_mxfp4_fused_status(self._h, _ptr(ws), ws.numel(), _stream(stream)))

    def route(self, topk_ids, num_tokens=None, stream=None):
        import torch
        dev = self.workspace.device
        if not isinstance(topk_ids, torch.Tensor) or topk_ids.dim() != 2:
            raise _arg_error("topk_ids must be a 2-D torch.Tensor [T, top_k]")
        T = topk_ids.shape[0] if num_tokens is None else int(num_tokens)
        if T < 0 or T > topk_ids.shape[0]:
            raise _arg_error(f"num_tokens must be in [0, {topk_ids.shape[0]}] (rows of topk_ids), got {T}")
        _need(topk_ids, "topk_ids", torch.int32, T, self.cfg.top_k, dev)
        E, n = self.cfg.num_experts, max(1, T * self.cfg.top_k)
        counts = torch.empty(E, dtype=torch.int32, device=dev)
        offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
        perm = torch.full((n,), -7, dtype=torch.int32, device=dev)
        rowpos = torch.empty(n, dtype=torch.int32, device=dev)
        _check(load_library().moe_mxfp4_route(self._h, _ptr(topk_ids), T, _ptr(counts), _ptr(offsets), _ptr(perm),
                                              _ptr(rowpos), _ptr(self.workspace), self.workspace.numel(),
                                              _stream(stream)))
        return counts, offsets, perm, rowpos

    def workspace_region(self, region, workspace=None):
        """The uint8 view of `workspace` (default: the plan's) holding an
        intermediate of the last forward on it (MOE_WS_H_CODES: MXFP8 h codes
        [T_max*k, I]; MOE_WS_H_SCALES: their E8M0 bytes [T_max*k, I/32])."""
        off, nb = ctypes.c_size_t(), ctypes.c_size_t()
        _check(load_library().moe_mxfp4_workspace_region(self._h, int(region), ctypes.byref(off), ctypes.byref(nb)))
        ws = self.workspace if workspace is None else workspace
        return ws[off.value: off.value + nb.value]

    def set_stage_events(self, events):
        """events: list of 5 torch.cuda.Event(enable_timing=True) or None to stop."""
        lib = load_library()
        if not events:
            _check(lib.moe_mxfp4_set_stage_events(self._h, None, 0))
            self._events = None
            return
        for ev in events:
            if not ev.cuda_event:      # torch creates the HIP event on its first record
                ev.record()
        arr = (ctypes.c_void_p * len(events))(*[ev.cuda_event for ev in events])
        self._events = (events, arr)   # keep alive while set
        _check(lib.moe_mxfp4_set_stage_events(self._h, arr, len(events)))


def router_topk(logits, top_k, ids=None, weights=None, stream=None):
    """topk_ids int32 [T, k] and topk_weights fp32 [T, k] from fp32 logits [T, E]
    (moe_router_topk)."""
    import torch
    if not isinstance(logits, torch.Tensor) or logits.dim() != 2:
        raise _arg_error("logits must be a 2-D torch.Tensor [T, num_experts]")
    T, E = logits.shape
    _need(logits, "logits", torch.float32, T, E, logits.device)
    ids = torch.empty((T, top_k), dtype=torch.int32, device=logits.device) if ids is None else ids
    weights = torch.empty((T, top_k), dtype=torch.float32, device=logits.device) if weights is None else weights
    _need(ids, "topk_ids", torch.int32, T, top_k, logits.device)
    _need(weights, "topk_weights", torch.float32, T, top_k, logits.device)
    _check(load_library().moe_router_topk(_ptr(logits), T, E, top_k, _ptr(ids), _ptr(weights), _stream(stream)))
    return ids, weights


def mxfp8_quantize(x_bf16, stream=None):
    import torch
    if not isinstance(x_bf16, torch.Tensor) or x_bf16.dim() != 2:
        raise _arg_error("x must be a 2-D torch.Tensor [rows, cols]")
    rows, cols = x_bf16.shape
    _need(x_bf16, "x", torch.bfloat16, rows, cols, x_bf16.device)
    codes = torch.empty((rows, cols), dtype=torch.uint8, device=x_bf16.device)
    scales = torch.empty((rows, max(cols // 32, 0)), dtype=torch.uint8, device=x_bf16.device)
    _check(load_library().moe_mxfp8_quantize(_ptr(x_bf16), rows, cols, _ptr(codes), _ptr(scales), _stream(stream)))
    return codes, scales


MOE_PROBE_READ, MOE_PROBE_READ_NT, MOE_PROBE_COPY = 0, 1, 2
MOE_PROBE_MFMA_BF16, MOE_PROBE_MFMA_F8F4 = 0, 1


def probe_memory(kind, src, dst, sink, grid, stream=None):
    """One launch of a memory probe over src (and dst): moe_probe_memory."""
    nbytes = src.numel() * src.element_size()
    _check(load_library().moe_probe_memory(int(kind), _ptr(src), _ptr(dst), nbytes, _ptr(sink), int(grid),
                                           _stream(stream)))


def probe_mfma(kind, iters, sink, grid, stream=None):
    """One launch of an MFMA probe: moe_probe_mfma; returns its flops."""
    fl = ctypes.c_double()
    _check(load_library().moe_probe_mfma(int(kind), int(iters), _ptr(sink), int(grid), ctypes.byref(fl),
                                         _stream(stream)))
    return fl.value


def probe_mfma_f8f4_blocks(a_lanes, b_lanes, a_scales, b_scales, c, stream=None):
    """d = one scaled MFMA per problem (moe_probe_mfma_f8f4_blocks); tensors in lane order."""
    import torch
    n = a_lanes.shape[0]
    dev = a_lanes.device
    _need(a_lanes, "a_lanes", torch.uint8, n, None, dev, ndim=3)
    _need(b_lanes, "b_lanes", torch.uint8, n, None, dev, ndim=3)
    _need(a_scales, "a_scales", torch.uint8, n, 64, dev)
    _need(b_scales, "b_scales", torch.uint8, n, 64, dev)
    _need(c, "c", torch.float32, n, None, dev, ndim=3)
    if a_lanes.shape[1:] != (64, 32) or b_lanes.shape[1:] != (64, 16) or c.shape[1:] != (64, 4):
        raise _arg_error("operands must be a [n,64,32], b [n,64,16], c [n,64,4]")
    d = torch.empty_like(c)
    _check(load_library().moe_probe_mfma_f8f4_blocks(_ptr(a_lanes), _ptr(b_lanes), _ptr(a_scales), _ptr(b_scales),
                                                     _ptr(c), _ptr(d), n, _stream(stream)))
    return d
