"""Python binding of the cco_moe C ABI (argument marshalling only).

Every step of the path runs in the library's HIP kernels; torch supplies
device memory (tensors' data pointers) and the stream (torch's current
stream unless one is given).  Method names follow the C entry points:

    heap = SymHeap(nslots, per_slot_bytes)          # cco_sym_heap_create
    moe = MoE(heap, max_tokens, hidden, topk, num_experts, inter)  # cco_moe_create
    moe.plan(idx)                                   # cco_moe_plan
    moe.dispatch(x, w)                              # cco_moe_dispatch
    # (or moe.dispatch_fp8(x8, scales, w)           # cco_moe_dispatch_fp8)
    moe.expert(w13, w2)                             # cco_moe_expert
    out, code = moe.combine(w)                      # cco_moe_combine
    code, slot_total, counts = moe.status()         # cco_moe_status
"""
from __future__ import annotations

import ctypes

import numpy as np
import torch

from . import _capi
from ._capi import CcoError, check, lib

_hip = None


def _hip_lib() -> ctypes.CDLL:
    global _hip
    if _hip is None:
        for name in ("libamdhip64.so", "/opt/rocm/lib/libamdhip64.so"):
            try:
                _hip = ctypes.CDLL(name)
                break
            except OSError:
                continue
        if _hip is None:
            raise ImportError("libamdhip64.so not found")
        _hip.hipMemcpy.restype = ctypes.c_int
        _hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
    return _hip


def device_to_host(ptr: int, nbytes: int, dtype=np.uint8) -> np.ndarray:
    """Synchronous copy of nbytes at device address ptr into a new host array
    (all queued device work is finished first)."""
    torch.cuda.synchronize()
    buf = np.empty(nbytes, np.uint8)
    if nbytes:
        rc = _hip_lib().hipMemcpy(buf.ctypes.data, ctypes.c_void_p(ptr), nbytes, 2)  # D2H
        if rc != 0:
            raise RuntimeError("hipMemcpy D2H failed (%d)" % rc)
    return buf.view(dtype)


def host_to_device(ptr: int, data: np.ndarray) -> None:
    torch.cuda.synchronize()
    data = np.ascontiguousarray(data)
    if data.nbytes:
        rc = _hip_lib().hipMemcpy(ctypes.c_void_p(ptr), data.ctypes.data, data.nbytes, 1)  # H2D
        if rc != 0:
            raise RuntimeError("hipMemcpy H2D failed (%d)" % rc)


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _ptr(t: torch.Tensor | None, dtype: torch.dtype | None = None, name: str = "tensor"):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s must be %s, got %s" % (name, dtype, t.dtype))
    return ctypes.c_void_p(t.data_ptr())


class SymHeap:
    """One flat device buffer of `nslots` slots (cco_sym_heap_create)."""

    def __init__(self, nslots: int, per_slot_bytes: int, device: int | None = None):
        if device is None:
            device = torch.cuda.current_device()
        h = ctypes.c_void_p()
        check(lib.cco_sym_heap_create(int(device), int(nslots), int(per_slot_bytes),
                                      ctypes.byref(h)), "cco_sym_heap_create")
        self._h = h
        self.device = device
        self.nslots = nslots
        base, stride = ctypes.c_void_p(), ctypes.c_uint64()
        check(lib.cco_sym_heap_info(h, ctypes.byref(base), ctypes.byref(stride), None, None),
              "cco_sym_heap_info")
        self.base = base.value
        self.stride = stride.value
        self._objs: list[MoE] = []

    @property
    def handle(self) -> ctypes.c_void_p:
        if self._h is None:
            raise RuntimeError("heap already destroyed")
        return self._h

    def slot_ptr(self, slot: int, offset: int = 0) -> int | None:
        """cco_sym_heap_slot_ptr: base + slot * stride + offset."""
        return lib.cco_sym_heap_slot_ptr(self.handle, int(slot), int(offset))

    def used(self) -> int:
        u = ctypes.c_uint64()
        check(lib.cco_sym_heap_info(self.handle, None, None, None, ctypes.byref(u)),
              "cco_sym_heap_info")
        return u.value

    def destroy(self) -> None:
        if self._h is not None:
            check(lib.cco_sym_heap_destroy(self._h), "cco_sym_heap_destroy")
            self._h = None
            for m in self._objs:
                m._m = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.destroy()

    def __del__(self):
        try:
            self.destroy()
        except Exception:
            pass


def shape_struct(max_tokens, hidden, topk, num_experts, inter) -> _capi.cco_moe_shape:
    return _capi.cco_moe_shape(int(max_tokens), int(hidden), int(topk), int(num_experts),
                               int(inter))


def required_slot_bytes(max_tokens, hidden, topk, num_experts, inter, nslots) -> int:
    """cco_moe_required_slot_bytes (0 for an invalid shape)."""
    s = shape_struct(max_tokens, hidden, topk, num_experts, inter)
    return int(lib.cco_moe_required_slot_bytes(ctypes.byref(s), int(nslots)))


class MoE:
    """Windows and routing state of one MoE layer on a SymHeap (cco_moe_create)."""

    def __init__(self, heap: SymHeap, max_tokens: int, hidden: int, topk: int,
                 num_experts: int, inter: int):
        self.heap = heap
        self.shape = shape_struct(max_tokens, hidden, topk, num_experts, inter)
        m = ctypes.c_void_p()
        check(lib.cco_moe_create(heap.handle, ctypes.byref(self.shape), ctypes.byref(m)),
              "cco_moe_create")
        self._m = m
        heap._objs.append(self)
        self.T_max, self.H, self.K, self.E, self.I = max_tokens, hidden, topk, num_experts, inter
        self.S = heap.nslots
        self.eps = num_experts // heap.nslots
        lay = _capi.cco_moe_layout()
        check(lib.cco_moe_get_layout(m, ctypes.byref(lay)), "cco_moe_get_layout")
        self.layout = lay
        self.cap = lay.cap
        r = _capi.cco_moe_routing()
        check(lib.cco_moe_get_routing(m, ctypes.byref(r)), "cco_moe_get_routing")
        self.routing_ptrs = r
        self.T = None

    @property
    def handle(self) -> ctypes.c_void_p:
        if self._m is None:
            raise RuntimeError("the heap of this MoE was destroyed")
        return self._m

    # ------------------------------------------------------------ stages --
    def plan(self, idx: torch.Tensor, stream=None) -> None:
        """cco_moe_plan; idx int32 [T, K] on the device."""
        if idx.dim() != 2 or idx.shape[1] != self.K:
            raise ValueError("idx must be [T, %d]" % self.K)
        T = idx.shape[0]
        check(lib.cco_moe_plan(self.handle, _ptr(idx, torch.int32, "idx"), T, _stream(stream)),
              "cco_moe_plan")
        self.T = T

    def dispatch(self, x: torch.Tensor, w: torch.Tensor, stream=None) -> None:
        """cco_moe_dispatch; x bf16 [T, H], w fp32 [T, K]."""
        T = x.shape[0]
        if tuple(x.shape) != (T, self.H) or tuple(w.shape) != (T, self.K):
            raise ValueError("x must be [T, H] and w [T, K]")
        check(lib.cco_moe_dispatch(self.handle, _ptr(x, torch.bfloat16, "x"),
                                   _ptr(w, torch.float32, "w"), T, _stream(stream)),
              "cco_moe_dispatch")

    def dispatch_fp8(self, x8: torch.Tensor, scales: torch.Tensor | None, w: torch.Tensor,
                     stream=None) -> None:
        """cco_moe_dispatch_fp8; x8 [T, H] of any 1-byte dtype (moved as raw
        bytes), scales fp32 [T, ns] or None, w fp32 [T, K]."""
        T = x8.shape[0]
        if x8.dim() != 2 or x8.shape[1] != self.H or x8.element_size() != 1:
            raise ValueError("x8 must be [T, H] of a 1-byte dtype")
        if tuple(w.shape) != (T, self.K):
            raise ValueError("w must be [T, K]")
        ns = 0
        if scales is not None:
            if scales.dim() != 2 or scales.shape[0] != T:
                raise ValueError("scales must be [T, ns]")
            ns = scales.shape[1]
        check(lib.cco_moe_dispatch_fp8(self.handle, _ptr(x8, None, "x8"),
                                       _ptr(scales, torch.float32, "scales"), ns,
                                       _ptr(w, torch.float32, "w"), T, _stream(stream)),
              "cco_moe_dispatch_fp8")

    def expert(self, w13: torch.Tensor | None, w2: torch.Tensor | None, stream=None) -> None:
        """cco_moe_expert; w13 bf16 [E, 2I, H], w2 bf16 [E, H, I]."""
        if self.I > 0:
            if tuple(w13.shape) != (self.E, 2 * self.I, self.H) or \
               tuple(w2.shape) != (self.E, self.H, self.I):
                raise ValueError("w13 must be [E, 2I, H] and w2 [E, H, I]")
        check(lib.cco_moe_expert(self.handle, _ptr(w13, torch.bfloat16, "w13"),
                                 _ptr(w2, torch.bfloat16, "w2"), _stream(stream)),
              "cco_moe_expert")

    def combine(self, w: torch.Tensor, out: torch.Tensor | None = None,
                expert_out: list[int | torch.Tensor | None] | None = None, stream=None):
        """cco_moe_combine -> (out bf16 [T, H], status code: CCO_OK or
        CCO_INFO_COPIED).  expert_out: per-slot device pointers (or tensors)
        of the expert output; None uses the staging views (zero copy)."""
        T = w.shape[0]
        if tuple(w.shape) != (T, self.K):
            raise ValueError("w must be [T, K]")
        if out is None:
            out = torch.empty((T, self.H), dtype=torch.bfloat16, device=w.device)
        arr = None
        if expert_out is not None:
            if len(expert_out) != self.S:
                raise ValueError("expert_out needs one entry per slot")
            vals = []
            for v in expert_out:
                if v is None:
                    vals.append(None)
                elif isinstance(v, torch.Tensor):
                    vals.append(v.data_ptr())
                else:
                    vals.append(int(v))
            arr = (ctypes.c_void_p * self.S)(*vals)
        code = lib.cco_moe_combine(self.handle, arr, _ptr(w, torch.float32, "w"),
                                   _ptr(out, torch.bfloat16, "out"), T, _stream(stream))
        check(code, "cco_moe_combine", allow=(_capi.CCO_OK, _capi.CCO_INFO_COPIED))
        return out, code

    def fused(self, idx: torch.Tensor, x: torch.Tensor, w: torch.Tensor,
              w13: torch.Tensor | None, w2: torch.Tensor | None,
              out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
        """cco_moe_fused: the whole path in one launch; returns out bf16 [T, H]."""
        T = idx.shape[0]
        if idx.dim() != 2 or idx.shape[1] != self.K or tuple(x.shape) != (T, self.H) or \
           tuple(w.shape) != (T, self.K):
            raise ValueError("idx [T, K], x [T, H] and w [T, K] expected")
        if self.I > 0 and (tuple(w13.shape) != (self.E, 2 * self.I, self.H) or
                           tuple(w2.shape) != (self.E, self.H, self.I)):
            raise ValueError("w13 must be [E, 2I, H] and w2 [E, H, I]")
        if out is None:
            out = torch.empty((T, self.H), dtype=torch.bfloat16, device=x.device)
        check(lib.cco_moe_fused(self.handle, _ptr(idx, torch.int32, "idx"),
                                _ptr(x, torch.bfloat16, "x"), _ptr(w, torch.float32, "w"),
                                _ptr(w13, torch.bfloat16, "w13"), _ptr(w2, torch.bfloat16, "w2"),
                                _ptr(out, torch.bfloat16, "out"), T, _stream(stream)),
              "cco_moe_fused")
        self.T = T
        return out

    def stage_in_sdma(self, slot: int, src: torch.Tensor | int, rows: int, stream=None) -> None:
        """cco_moe_stage_in_sdma: rows of `src` (bf16 [rows, H] tensor or a
        device address) into slot's staging window on the copy engines."""
        if isinstance(src, torch.Tensor):
            if src.dtype != torch.bfloat16 or src.dim() != 2 or src.shape[1] != self.H or \
               src.shape[0] < rows or not src.is_contiguous():
                raise ValueError("src must be a contiguous bf16 [>= rows, H] tensor")
            src = src.data_ptr()
        check(lib.cco_moe_stage_in_sdma(self.handle, int(slot), ctypes.c_void_p(int(src)),
                                        int(rows), _stream(stream)), "cco_moe_stage_in_sdma")

    def status(self, stream=None):
        """cco_moe_status -> (code, slot_total [S], counts [E]) (synchronises)."""
        st = np.zeros(self.S, np.int32)
        cnt = np.zeros(self.E, np.int32)
        code = lib.cco_moe_status(self.handle, _stream(stream), st.ctypes.data_as(ctypes.c_void_p),
                                  cnt.ctypes.data_as(ctypes.c_void_p))
        if code == _capi.CCO_ERR_HIP or code == _capi.CCO_ERR_INVALID_ARG:
            raise CcoError(code, "cco_moe_status")
        return code, st, cnt

    # ------------------------------------------------------------- views --
    def dispatch_view(self, slot: int) -> int:
        """Device address of slot's receive window (cco_moe_dispatch_view)."""
        return lib.cco_moe_dispatch_view(self.handle, int(slot))

    def combine_in_view(self, slot: int) -> int:
        """Device address of slot's combine staging window."""
        return lib.cco_moe_combine_in_view(self.handle, int(slot))

    # ----------------------------------------------------- host readback --
    def read_routing(self):
        """Host copies of (pos [T, K], counts [E], expert_off [E], slot_total [S])."""
        T = self.T or 0
        r = self.routing_ptrs
        pos = device_to_host(r.pos, T * self.K * 4, np.int32).reshape(T, self.K)
        counts = device_to_host(r.counts, self.E * 4, np.int32)
        off = device_to_host(r.expert_off, self.E * 4, np.int32)
        tot = device_to_host(r.slot_total, self.S * 4, np.int32)
        return pos, counts, off, tot

    def read_window(self, slot: int, offset: int, nbytes: int, dtype=np.uint8) -> np.ndarray:
        """Host copy of nbytes at `offset` of slot `slot` (offsets from the layout)."""
        return device_to_host(self.heap.slot_ptr(slot, 0) + offset, nbytes, dtype)

    def read_rows(self, which: str, slot: int, row0: int, nrows: int) -> np.ndarray:
        """Host copy of rows [row0, row0 + nrows) of a window:
        'disp_x' / 'out_tok' (uint16 [n, H]), 'hbuf' (uint16 [n, I]),
        'meta' (structured {src, w, e})."""
        lay = self.layout
        if which == "disp_x":
            off, width, dt = lay.disp_x, self.H * 2, np.uint16
        elif which == "out_tok":
            off, width, dt = lay.out_tok, self.H * 2, np.uint16
        elif which == "hbuf":
            off, width, dt = lay.hbuf, self.I * 2, np.uint16
        elif which == "meta":
            dt = np.dtype([("src", np.int32), ("w", np.float32), ("e", np.int32)])
            b = self.read_window(slot, lay.disp_meta + row0 * 12, nrows * 12)
            return b.view(dt)
        else:
            raise ValueError(which)
        b = self.read_window(slot, off + row0 * width, nrows * width)
        return b.view(dt).reshape(nrows, width // 2)

    # ------------------------------------------------------------ timing --
    def set_timing(self, enable: bool) -> None:
        check(lib.cco_moe_set_timing(self.handle, int(bool(enable))), "cco_moe_set_timing")

    def timing_summary(self) -> dict:
        """{kernel kind: (timed launches, total ms)}; resets the counters."""
        n = np.zeros(_capi.CCO_NUM_KERNEL_KINDS, np.int32)
        ms = np.zeros(_capi.CCO_NUM_KERNEL_KINDS, np.float64)
        check(lib.cco_moe_timing_summary(self.handle, n.ctypes.data_as(ctypes.c_void_p),
                                         ms.ctypes.data_as(ctypes.c_void_p)),
              "cco_moe_timing_summary")
        return {k: (int(n[i]), float(ms[i])) for i, k in enumerate(_capi.KERNEL_KINDS)}
