"""Python binding of libqmoe.so (ctypes): argument marshalling only.

Every step of the routed-MoE call runs in the library's HIP kernels; torch is
used for device memory and the current stream. The names follow the C ABI in
include/qmoe.h. Importing this module does not load the library; the first
use does, and fails loudly when it has not been built.
"""

from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "_lib", "libqmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_DEVICE, MOE_ERR_HIP = range(6)
MID_E4M3, MID_MXFP4 = 0, 1  # moe_mid_format
LAYOUT_W13_PACKED, LAYOUT_W2_PACKED = 1, 2  # moe_weight_layout flags


def layout_for(mid_format: int) -> int:
    """The weight layout calls with this mid format read: gate/up packed, and
    down packed with the MXFP4 mid."""
    return LAYOUT_W13_PACKED | (LAYOUT_W2_PACKED if mid_format == MID_MXFP4 else 0)
NOALLOC_SCRATCH_BYTES = 64 << 20  # MOE_NOALLOC_SCRATCH_BYTES of include/qmoe.h


class moe_shape(ctypes.Structure):
    _fields_ = [("M", ctypes.c_int64), ("H", ctypes.c_int64), ("E", ctypes.c_int64), ("I", ctypes.c_int64),
                ("top_k", ctypes.c_int64), ("routed_scaling", ctypes.c_float), ("shared_I", ctypes.c_int64)]


LAYOUT_FIELDS = ["total_bytes", "topk_ids", "topk_w", "count", "offset", "sorted_entry", "xq", "xs", "midq",
                 "mids", "y", "sh_xq", "sh_xs", "sh_hq", "sh_hs", "sh_y"]


class moe_ws_layout(ctypes.Structure):
    _fields_ = [(f, ctypes.c_size_t) for f in LAYOUT_FIELDS]


TP_MAX = 8  # MOE_TP_MAX


class moe_tp_exchange(ctypes.Structure):
    _fields_ = [("tp", ctypes.c_int32), ("rank", ctypes.c_int32), ("epoch", ctypes.c_uint32),
                ("spin_limit", ctypes.c_int32), ("inbox", ctypes.c_void_p), ("inbox_tags", ctypes.c_void_p),
                ("push", ctypes.c_void_p * TP_MAX), ("push_tags", ctypes.c_void_p * TP_MAX),
                ("status", ctypes.c_void_p)]


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_str(status)} (status {status})")


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (built in-tree by quantized_moe_expert_route_amd.build)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m quantized_moe_expert_route_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, st = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    L.moe_status_str.restype = ctypes.c_char_p
    L.moe_status_str.argtypes = [st]
    L.moe_stage_count.restype = ctypes.c_int
    L.moe_stage_count.argtypes = []
    L.moe_stage_name.restype = ctypes.c_char_p
    L.moe_stage_name.argtypes = [ctypes.c_int]
    L.moe_shape_workspace_bytes.restype = st
    L.moe_shape_workspace_bytes.argtypes = [ctypes.POINTER(moe_shape), ctypes.POINTER(ctypes.c_size_t)]
    L.moe_plan_create.restype = st
    L.moe_plan_create.argtypes = [ctypes.POINTER(moe_shape), ctypes.POINTER(vp)]
    L.moe_plan_destroy.restype = None
    L.moe_plan_destroy.argtypes = [vp]
    L.moe_plan_workspace_bytes.restype = ctypes.c_size_t
    L.moe_plan_workspace_bytes.argtypes = [vp]
    L.moe_plan_layout.restype = st
    L.moe_plan_layout.argtypes = [vp, ctypes.POINTER(moe_ws_layout)]
    L.moe_plan_set_workspace.restype = st
    L.moe_plan_set_workspace.argtypes = [vp, vp, ctypes.c_size_t, vp]
    L.moe_plan_set_shared.restype = st
    L.moe_plan_set_shared.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    L.moe_plan_shared_pack_bytes.restype = ctypes.c_size_t
    L.moe_plan_shared_pack_bytes.argtypes = [vp]
    L.moe_plan_set_stage_events.restype = st
    L.moe_plan_set_stage_events.argtypes = [vp, ctypes.POINTER(vp), ctypes.c_int]
    L.moe_plan_set_call_events.restype = st
    L.moe_plan_set_call_events.argtypes = [vp, vp, vp]
    L.moe_plan_stage_launches.restype = ctypes.c_int
    L.moe_plan_stage_launches.argtypes = [vp, i64, ctypes.c_int]
    L.moe_forward.restype = st
    L.moe_forward.argtypes = [vp, i64, vp, vp, vp, vp, vp, vp, vp, vp]
    L.moe_forward_noalloc.restype = st
    L.moe_forward_noalloc.argtypes = [vp, i64, vp, vp, vp, vp, vp, vp, vp, vp]
    L.moe_pack_w13.restype = st
    L.moe_pack_w13.argtypes = [vp, vp, i64, i64, i64, vp, vp, vp]
    L.moe_pack_w2.restype = st
    L.moe_pack_w2.argtypes = [vp, vp, i64, i64, i64, vp, vp, vp]
    L.moe_plan_set_shared_slot.restype = st
    L.moe_plan_set_shared_slot.argtypes = [vp, ctypes.c_int]
    L.moe_plan_set_mid_format.restype = st
    L.moe_plan_set_mid_format.argtypes = [vp, ctypes.c_int]
    L.moe_plan_set_weight_layout.restype = st
    L.moe_plan_set_weight_layout.argtypes = [vp, ctypes.c_uint]
    L.moe_plan_set_tp_exchange.restype = st
    L.moe_plan_set_tp_exchange.argtypes = [vp, ctypes.POINTER(moe_tp_exchange)]
    _lib = L
    return L


def status_str(status: int) -> str:
    return lib().moe_status_str(status).decode()


def stage_names():
    L = lib()
    return [L.moe_stage_name(i).decode() for i in range(L.moe_stage_count())]


def shape_workspace_bytes(M, H, E, I, top_k, routed_scaling=2.5, shared_I=0) -> int:
    s = moe_shape(M, H, E, I, top_k, routed_scaling, shared_I)
    out = ctypes.c_size_t(0)
    st = lib().moe_shape_workspace_bytes(ctypes.byref(s), ctypes.byref(out))
    if st != MOE_OK:
        raise MoeError(st, "moe_shape_workspace_bytes")
    return out.value


def _ptr(t) -> int:
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    import torch

    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def pack_w13(w13, s13, out=None, stream=None):
    """Gate/up weights and scales (row-major MXFP4 [E, 2I, H/2] and E8M0
    [E, 2I, H/32], uint8 device tensors) -> (w13_packed, s13_packed) in the
    layout moe_forward reads (moe_pack_w13). Enqueued on `stream`; `out`
    may give the two destination tensors, else they are allocated here."""
    import torch

    E, R, Hh = w13.shape
    if R % 2 or tuple(s13.shape) != (E, R, Hh // 16):
        raise ValueError("w13 must be [E, 2I, H/2] and s13 [E, 2I, H/32]")
    if out is None:
        out = (torch.empty_like(w13), torch.empty_like(s13))
    wp, sp = out
    st = lib().moe_pack_w13(_ptr(w13), _ptr(s13), E, R // 2, 2 * Hh, _ptr(wp), _ptr(sp), _stream(stream))
    if st != MOE_OK:
        raise MoeError(st, "moe_pack_w13")
    return wp, sp


def pack_w2(w2, s2, out=None, stream=None):
    """Down weights and scales (row-major MXFP4 [E, H, I/2] and E8M0
    [E, H, I/32], uint8 device tensors) -> (w2_packed, s2_packed) in the
    layout the MXFP4-mid down reads (moe_pack_w2); s2_packed is [E, H, 16]."""
    import torch

    E, H, Ih = w2.shape
    if tuple(s2.shape) != (E, H, Ih // 16):
        raise ValueError("w2 must be [E, H, I/2] and s2 [E, H, I/32]")
    if out is None:
        out = (torch.empty_like(w2), torch.empty((E, H, 16), dtype=torch.uint8, device=w2.device))
    wp, sp = out
    st = lib().moe_pack_w2(_ptr(w2), _ptr(s2), E, 2 * Ih, H, _ptr(wp), _ptr(sp), _stream(stream))
    if st != MOE_OK:
        raise MoeError(st, "moe_pack_w2")
    return wp, sp


class Plan:
    """A plan for one shape, owning a device workspace allocated through torch."""

    def __init__(self, M: int, H: int, E: int, I: int, top_k: int, routed_scaling: float = 2.5,
                 shared_I: int = 0, device=None, weight_layout: int = LAYOUT_W13_PACKED):
        import torch

        self.shape = moe_shape(M, H, E, I, top_k, routed_scaling, shared_I)
        self._h = ctypes.c_void_p()
        st = lib().moe_plan_create(ctypes.byref(self.shape), ctypes.byref(self._h))
        if st != MOE_OK:
            raise MoeError(st, "moe_plan_create")
        self.device = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
        nbytes = lib().moe_plan_workspace_bytes(self._h)
        self.workspace = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=self.device)
        st = lib().moe_plan_set_workspace(self._h, _ptr(self.workspace), self.workspace.numel(), _stream(None))
        if st != MOE_OK:
            raise MoeError(st, "moe_plan_set_workspace")
        self._shared = None
        self._events = None
        self._layout = LAYOUT_W13_PACKED
        self.set_weight_layout(weight_layout)

    def set_weight_layout(self, layout: int):
        """Declare the layout of the weights later calls pass (LAYOUT_W13_PACKED:
        w13/s13 from pack_w13, the only gate/up layout served; | LAYOUT_W2_PACKED:
        w2/s2 from pack_w2, required by and only by the MXFP4 mid)."""
        st = lib().moe_plan_set_weight_layout(self._h, int(layout))
        if st != MOE_OK:
            raise MoeError(st, "moe_plan_set_weight_layout")
        self._layout = int(layout)

    def _tensor(self, name, t, dtypes, numel=None, rows=None, cols=None, min_numel=None):
        """The library sees bare pointers: a tensor on another device, of
        another element type, strided, or smaller than the plan's shape would
        be read or written out of bounds, so each is checked here."""
        import torch

        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch tensor")
        if t.device != self.device:
            raise ValueError(f"{name} is on {t.device}, the plan on {self.device}")
        if t.dtype not in dtypes:
            raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if numel is not None and t.numel() != numel:
            raise ValueError(f"{name} holds {t.numel()} elements, the plan's shape needs {numel}")
        if min_numel is not None and t.numel() < min_numel:
            raise ValueError(f"{name} holds {t.numel()} elements, at least {min_numel} are needed")
        if cols is not None and (t.dim() != 2 or t.shape[1] != cols or t.shape[0] < rows):
            raise ValueError(f"{name} is {tuple(t.shape)}, expected at least [{rows}, {cols}]")

    def _check_call(self, M, x, logits, w13, s13, w2, s2, out):
        import torch

        s = self.shape
        if not 0 <= int(M) <= s.M:
            raise ValueError(f"M = {M} outside [0, {s.M}] (the plan's shape)")
        H, E, I = s.H, s.E, s.I
        bf16 = (torch.int16, torch.bfloat16)
        self._tensor("x", x, bf16, rows=M, cols=H)
        self._tensor("logits", logits, (torch.float32,), rows=M, cols=E)
        self._tensor("out", out, bf16, rows=M, cols=H)
        u8 = (torch.uint8,)
        self._tensor("w13", w13, u8, numel=E * 2 * I * H // 2)
        self._tensor("s13", s13, u8, numel=E * 2 * I * H // 32)
        self._tensor("w2", w2, u8, numel=E * H * I // 2)
        self._tensor("s2", s2, u8, numel=E * H * (16 if self._layout & LAYOUT_W2_PACKED else I // 32))

    def layout(self) -> Dict[str, int]:
        L = moe_ws_layout()
        st = lib().moe_plan_layout(self._h, ctypes.byref(L))
        if st != MOE_OK:
            raise MoeError(st, "moe_plan_layout")
        return {f: getattr(L, f) for f in LAYOUT_FIELDS}

    def set_shared(self, ws13, ss13, ws2, ss2, stream=None):
        """Bind the block-FP8 shared expert: row-major E4M3 ws13 [2 Is, H] and
        ws2 [H, Is] (uint8), fp32 block scales ss13 [2 Is/128, H/128] and ss2
        [H/128, Is/128]. The library packs the weights into a buffer this
        object allocates and keeps (with the scales)."""
        import torch

        H, Is = self.shape.H, self.shape.shared_I
        self._tensor("ws13", ws13, (torch.uint8,), numel=2 * Is * H)
        self._tensor("ss13", ss13, (torch.float32,), numel=(2 * Is // 128) * (H // 128))
        self._tensor("ws2", ws2, (torch.uint8,), numel=H * Is)
        self._tensor("ss2", ss2, (torch.float32,), numel=(H // 128) * (Is // 128))
        nbytes = lib().moe_plan_shared_pack_bytes(self._h)
        packed = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=self.device)
        st = lib().moe_plan_set_shared(self._h, _ptr(ws13), _ptr(ss13), _ptr(ws2), _ptr(ss2), _ptr(packed),
                                       packed.numel(), _stream(stream))
        if st != MOE_OK:
            raise MoeError(st, "moe_plan_set_shared")
        self._shared = (ss13, ss2, packed)  # kept alive while the plan uses them

    def set_shared_slot(self, on: bool):
        """Expert E-1 as the shared expert, fused as the last slot of every token."""
        st = lib().moe_plan_set_shared_slot(self._h, int(bool(on)))
        if st != MOE_OK:
            raise MoeError(st, "moe_plan_set_shared_slot")

    def set_tp_exchange(self, tp=None, rank=0, epoch=1, inbox=None, inbox_tags=None, push=(), push_tags=(),
                        status=None, spin_limit=1 << 20):
        """Tensor-parallel exchange epilogue (moe_plan_set_tp_exchange); tp=None
        turns it off. inbox: float64 [tp, M, H], inbox_tags: int32 [tp, M, H/512],
        push / push_tags: per rank (None at this rank), status: int32 [1]."""
        if tp is None:
            st = lib().moe_plan_set_tp_exchange(self._h, None)
            self._tpx = None
        else:
            import torch

            M, H = self.shape.M, self.shape.H
            tags = (torch.int32, torch.uint32)
            self._tensor("inbox", inbox, (torch.float64,), numel=tp * M * H)
            self._tensor("inbox_tags", inbox_tags, tags, numel=tp * M * (H // 512))
            self._tensor("status", status, tags, min_numel=1)
            for p in range(tp):
                if p != rank:
                    self._tensor(f"push[{p}]", push[p], (torch.float64,), min_numel=M * H)
                    self._tensor(f"push_tags[{p}]", push_tags[p], tags, min_numel=M * (H // 512))
            x = moe_tp_exchange()
            x.tp, x.rank, x.epoch, x.spin_limit = tp, rank, epoch, spin_limit
            x.inbox, x.inbox_tags, x.status = _ptr(inbox), _ptr(inbox_tags), _ptr(status)
            for p in range(tp):
                if p != rank:
                    x.push[p] = _ptr(push[p])
                    x.push_tags[p] = _ptr(push_tags[p])
            st = lib().moe_plan_set_tp_exchange(self._h, ctypes.byref(x))
            self._tpx = (inbox, inbox_tags, tuple(push), tuple(push_tags), status)  # kept alive
        if st != MOE_OK:
            raise MoeError(st, "moe_plan_set_tp_exchange")

    def set_mid_format(self, fmt: int):
        """MID_E4M3 (default) or MID_MXFP4 for the plan's later calls (the
        MXFP4 mid reads packed down weights: declare them with
        set_weight_layout(LAYOUT_W13_PACKED | LAYOUT_W2_PACKED))."""
        st = lib().moe_plan_set_mid_format(self._h, int(fmt))
        if st != MOE_OK:
            raise MoeError(st, "moe_plan_set_mid_format")

    def set_stage_events(self, events):
        """events: raw hipEvent_t handles (ints), [start0, stop0, start1, stop1, ...]
        for every stage; None clears."""
        if events is None:
            st = lib().moe_plan_set_stage_events(self._h, None, 0)
            self._events = None
        else:
            arr = (ctypes.c_void_p * len(events))(*events)
            st = lib().moe_plan_set_stage_events(self._h, arr, len(events))
            self._events = arr
        if st != MOE_OK:
            raise MoeError(st, "moe_plan_set_stage_events")

    def set_call_events(self, start, stop):
        """start/stop: raw hipEvent_t handles (ints) recorded at the first
        kernel's start and the last kernel's end of every call; None clears."""
        st = lib().moe_plan_set_call_events(self._h, start, stop)
        if st != MOE_OK:
            raise MoeError(st, "moe_plan_set_call_events")
        if start is not None:
            self._events = None

    def forward(self, x, logits, w13, s13, w2, s2, out, M: Optional[int] = None, stream=None):
        """Enqueue the call on `stream` (default: torch's current stream)."""
        if M is None:
            M = x.shape[0]
        self._check_call(M, x, logits, w13, s13, w2, s2, out)
        st = lib().moe_forward(self._h, int(M), _ptr(x), _ptr(logits), _ptr(w13), _ptr(s13), _ptr(w2),
                               _ptr(s2), _ptr(out), _stream(stream))
        if st != MOE_OK:
            raise MoeError(st, "moe_forward")
        return out

    def forward_noalloc(self, x, logits, w13, s13, w2, s2, out, M: Optional[int] = None, stream=None):
        """moe_forward_noalloc: the same call on the library's static device
        scratch instead of this plan's workspace (nothing is allocated)."""
        if M is None:
            M = x.shape[0]
        self._check_call(M, x, logits, w13, s13, w2, s2, out)
        st = lib().moe_forward_noalloc(self._h, int(M), _ptr(x), _ptr(logits), _ptr(w13), _ptr(s13), _ptr(w2),
                                       _ptr(s2), _ptr(out), _stream(stream))
        if st != MOE_OK:
            raise MoeError(st, "moe_forward_noalloc")
        return out

    def stage_launches(self, M: int):
        """Kernels each stage launches for a call of M tokens."""
        return [lib().moe_plan_stage_launches(self._h, int(M), i) for i in range(lib().moe_stage_count())]

    def view(self, name: str, dtype, shape):
        """A torch view of an intermediate inside the workspace (see moe_ws_layout)."""
        import math

        import torch

        off = self.layout()[name]
        itemsize = torch.empty(0, dtype=dtype).element_size()
        n = math.prod(shape)
        return self.workspace[off:off + n * itemsize].view(dtype).view(*shape)

    def close(self):
        if self._h:
            lib().moe_plan_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class HipEvents:
    """A few raw hipEvent_t handles from libamdhip64 (for per-stage timing)."""

    def __init__(self, n: int):
        self._hip = ctypes.CDLL("libamdhip64.so")
        self._hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self._hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self._hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self._hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self._hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.handles = []
        for _ in range(n):
            h = ctypes.c_void_p()
            if self._hip.hipEventCreate(ctypes.byref(h)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.handles.append(h.value)

    def record(self, i: int, stream) -> None:
        """Record event i on a torch stream (or a raw hipStream_t)."""
        h = stream.cuda_stream if hasattr(stream, "cuda_stream") else stream
        if self._hip.hipEventRecord(self.handles[i], h) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, i: int, j: int) -> float:
        self._hip.hipEventSynchronize(self.handles[j])
        ms = ctypes.c_float(0)
        if self._hip.hipEventElapsedTime(ctypes.byref(ms), self.handles[i], self.handles[j]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def close(self):
        for h in self.handles:
            self._hip.hipEventDestroy(h)
        self.handles = []
