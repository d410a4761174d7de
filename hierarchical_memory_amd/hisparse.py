"""Python binding of the HiSparse swap-in C ABI (``include/hisparse.h``).

Argument marshalling only: every step of the path runs in the HIP library.
PyTorch supplies device memory and streams. The binding raises if the built
library is missing; there is no fallback.
"""
from __future__ import annotations

import ctypes
import json
import os
from typing import Any, Dict, Optional, Sequence, Tuple, Union

import numpy as np

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libhisparse.so")
_lib = None

HS_OK, HS_E_INVALID, HS_E_NOMEM, HS_E_HIP, HS_E_STATE = 0, -1, -2, -3, -4
HS_STATUS_BAD_ID, HS_STATUS_DUP_ID, HS_STATUS_BAD_STATE, HS_STATUS_STALE = 1, 2, 4, 8
HS_EVICT_LRU, HS_EVICT_FIFO = 0, 1
HS_PLAN_ROW_SOURCES = 1
HS_STATE_TABLES, HS_STATE_ROWS = 1, 2

EXPORTED = ("hs_required_sizes", "hs_create", "hs_host_pool", "hs_bind_device", "hs_reset", "hs_resolve",
            "hs_plan", "hs_copy", "hs_trial", "hs_commit", "hs_offload", "hs_advance_tail", "hs_gather",
            "hs_rebuild_order", "hs_step_static", "hs_export_state", "hs_import_state", "hs_destroy", "hs_last_error")
HS_STATIC_PLAN_BYTES = 8 << 20


class HiSparseError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[{code}] {msg}")
        self.code = code


class HsConfig(ctypes.Structure):
    _fields_ = [("num_requests", ctypes.c_int32), ("top_k", ctypes.c_int32), ("device_buffer_size", ctypes.c_int32),
                ("host_to_device_ratio", ctypes.c_float), ("row_bytes", ctypes.c_int32),
                ("max_context", ctypes.c_int32), ("tail_tokens", ctypes.c_int32), ("eviction_policy", ctypes.c_int32)]


class HsDeviceViews(ctypes.Structure):
    _fields_ = [(n, t) for name in ("hot", "tail", "slot_tok", "stamp", "lru_order", "page", "step", "epoch")
                for n, t in ((name, ctypes.c_void_p), (name + "_bytes", ctypes.c_uint64))]


class HsSizes(ctypes.Structure):
    _fields_ = [("host_rows", ctypes.c_int32), ("host_pool_bytes", ctypes.c_uint64), ("hot_bytes", ctypes.c_uint64),
                ("tail_bytes", ctypes.c_uint64), ("slot_tok_bytes", ctypes.c_uint64), ("stamp_bytes", ctypes.c_uint64),
                ("lru_order_bytes", ctypes.c_uint64), ("page_bytes", ctypes.c_uint64), ("step_bytes", ctypes.c_uint64),
                ("topk_bytes", ctypes.c_uint64), ("out_bytes", ctypes.c_uint64), ("gather_bytes", ctypes.c_uint64),
                ("plan_bytes", ctypes.c_uint64), ("trial_bytes", ctypes.c_uint64), ("lds_bytes", ctypes.c_uint32),
                ("lds_bytes_launch", ctypes.c_uint32), ("lds_bytes_launch_gather", ctypes.c_uint32),
                ("token_slot_table", ctypes.c_uint32), ("lds_bytes_rank", ctypes.c_uint32),
                ("sparse_rank", ctypes.c_uint32), ("epoch_bytes", ctypes.c_uint64), ("state_tables_bytes", ctypes.c_uint64),
                ("state_rows_bytes", ctypes.c_uint64)]


def library_path() -> str:
    return _LIB_PATH


def lib():
    """The loaded HIP library. Raises ImportError when it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(f"libhisparse.so is not built ({_LIB_PATH}); run __graft_entry__.build() or "
                              "python hierarchical_memory_amd/build.py")
        # torch ships its own HIP runtime with the same soname; loading torch first makes the library bind
        # to that one runtime instead of bringing a second one into the process
        import torch  # noqa: F401
        L = ctypes.CDLL(_LIB_PATH)
        vp, i32 = ctypes.c_void_p, ctypes.c_int32
        L.hs_required_sizes.argtypes = [ctypes.POINTER(HsConfig), ctypes.POINTER(HsSizes)]
        L.hs_create.argtypes = [ctypes.POINTER(HsConfig), ctypes.POINTER(vp)]
        L.hs_host_pool.argtypes = [vp, ctypes.POINTER(vp), ctypes.POINTER(ctypes.c_uint64), ctypes.POINTER(i32)]
        L.hs_bind_device.argtypes = [vp, ctypes.POINTER(HsDeviceViews)]
        L.hs_reset.argtypes = [vp, vp, i32, vp]
        L.hs_resolve.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp]
        L.hs_plan.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, vp]
        L.hs_copy.argtypes = [vp, vp, vp, vp, vp]
        L.hs_step_static.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp]
        L.hs_export_state.argtypes = [vp, vp, ctypes.c_uint64, ctypes.c_uint32, vp]
        L.hs_import_state.argtypes = [vp, vp, ctypes.c_uint64, ctypes.c_uint32, vp]
        L.hs_trial.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp]
        L.hs_commit.argtypes = [vp, vp, vp, vp, vp, vp]
        L.hs_offload.argtypes = [vp, vp, vp, i32, vp, vp]
        L.hs_advance_tail.argtypes = [vp, vp, vp, vp, vp]
        L.hs_gather.argtypes = [vp, vp, vp, vp]
        L.hs_rebuild_order.argtypes = [vp, vp]
        L.hs_destroy.argtypes = [vp]
        L.hs_destroy.restype = None
        L.hs_last_error.argtypes = []
        L.hs_last_error.restype = ctypes.c_char_p
        for name in ("hs_required_sizes", "hs_create", "hs_host_pool", "hs_bind_device", "hs_reset", "hs_resolve",
                     "hs_plan", "hs_copy", "hs_trial", "hs_commit", "hs_offload", "hs_advance_tail", "hs_gather",
                     "hs_rebuild_order", "hs_step_static", "hs_export_state", "hs_import_state"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def hs_last_error() -> str:
    return lib().hs_last_error().decode()


def _check(rc: int) -> None:
    if rc != HS_OK:
        raise HiSparseError(rc, hs_last_error())


def config(num_requests: int, top_k: int, device_buffer_size: int, host_to_device_ratio: float = 0.0,
           row_bytes: int = 1152, max_context: int = 0, tail_tokens: int = 0,
           eviction_policy: int = HS_EVICT_LRU) -> HsConfig:
    return HsConfig(num_requests, top_k, device_buffer_size, host_to_device_ratio, row_bytes, max_context, tail_tokens,
                    eviction_policy)


def config_from_hisparse_json(spec: Union[str, Dict[str, Any]], num_requests: int, row_bytes: int = 1152,
                              max_context: int = 0, tail_tokens: int = 0) -> HsConfig:
    """Config from the pages' launch option ``--hisparse-config '{"top_k": .., "device_buffer_size": ..,
    "host_to_device_ratio": ..}'``."""
    d = json.loads(spec) if isinstance(spec, str) else dict(spec)
    unknown = set(d) - {"top_k", "device_buffer_size", "host_to_device_ratio"}
    if unknown:
        raise ValueError(f"unknown hisparse-config keys: {sorted(unknown)}")
    return config(num_requests, int(d["top_k"]), int(d["device_buffer_size"]),
                  float(d.get("host_to_device_ratio", 0.0)), row_bytes, max_context, tail_tokens)


def hs_required_sizes(cfg: HsConfig) -> HsSizes:
    s = HsSizes()
    _check(lib().hs_required_sizes(ctypes.byref(cfg), ctypes.byref(s)))
    return s


class _Limits:
    """What a context's calls need of their tensor arguments, computed once at hs_create: element counts of
    the int32 arrays and byte counts of the row buffers."""
    __slots__ = ("R", "RK", "plan", "gather", "trial", "row_bytes")

    def __init__(self, cfg: HsConfig, s: HsSizes):
        self.R, self.RK = cfg.num_requests, cfg.num_requests * cfg.top_k
        self.plan, self.gather, self.trial = s.plan_bytes // 4, s.gather_bytes, s.trial_bytes
        self.row_bytes = cfg.row_bytes


# Limits of every live context, by its address: the calls below check each tensor against them (dtype and
# element count, from tensor metadata only) before a pointer reaches the library, whose C calls take raw
# pointers and cannot.
_CTX_SIZES: Dict[int, _Limits] = {}


def _ctx_key(ctx) -> int:
    if ctx is None:
        return 0
    return int(ctx.value or 0) if isinstance(ctx, ctypes.c_void_p) else int(ctx)


def _register(ctx, cfg: HsConfig, sizes: HsSizes) -> None:
    _CTX_SIZES[_ctx_key(ctx)] = _Limits(cfg, sizes)


def hs_create(cfg: HsConfig) -> ctypes.c_void_p:
    ctx = ctypes.c_void_p()
    _check(lib().hs_create(ctypes.byref(cfg), ctypes.byref(ctx)))
    _register(ctx, cfg, hs_required_sizes(cfg))
    return ctx


def hs_host_pool(ctx) -> Tuple[int, int, int]:
    base, stride, rows = ctypes.c_void_p(), ctypes.c_uint64(), ctypes.c_int32()
    _check(lib().hs_host_pool(ctx, ctypes.byref(base), ctypes.byref(stride), ctypes.byref(rows)))
    return base.value, stride.value, rows.value


_INT32 = None


def _arg(name: str, t, lim: Optional[_Limits], count: int = 0, nbytes: int = 0, int32: bool = True,
         nullable: bool = False):
    """Checks one tensor argument from its metadata and returns it (None when absent): int32 index arrays must
    be torch.int32 with at least count elements; row buffers may have any dtype but must hold nbytes. Without a
    known context (lim None) only the dtype is checked (the library then refuses the context)."""
    if t is None:
        if nullable:
            return None
        raise ValueError(f"{name} must not be None")
    if int32 and t.dtype is not _INT32:
        raise ValueError(f"{name} must be a torch.int32 tensor, got {t.dtype}")
    if lim is not None:
        if count and t.numel() < count:
            raise ValueError(f"{name} has {t.numel()} elements, the context needs at least {count}")
        if nbytes and t.numel() * t.element_size() < nbytes:
            raise ValueError(f"{name} has {t.numel() * t.element_size()} bytes, the context needs at least {nbytes}")
    return t


def _lim(ctx) -> Optional[_Limits]:
    global _INT32
    if _INT32 is None:
        import torch
        _INT32 = torch.int32
    return _CTX_SIZES.get(_ctx_key(ctx))


def _ptr(t) -> Optional[int]:
    """Device address of a tensor argument. Every tensor the calls take is device memory read or written by a
    kernel, so a tensor on the CPU (or with gaps) is refused here rather than handed to the GPU."""
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"expected a GPU tensor, got one on {t.device}")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return t.data_ptr()


def _bytes(t) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def hs_bind_device(ctx, hot, tail, slot_tok, stamp, lru_order, page, step, epoch) -> None:
    v = HsDeviceViews()
    for name, t in (("hot", hot), ("tail", tail), ("slot_tok", slot_tok), ("stamp", stamp),
                    ("lru_order", lru_order), ("page", page), ("step", step), ("epoch", epoch)):
        if t is not None and not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        setattr(v, name, None if t is None else t.data_ptr())  # the library checks these itself
        setattr(v, name + "_bytes", _bytes(t))
    _check(lib().hs_bind_device(ctx, ctypes.byref(v)))


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def _ptrs(*tensors):
    """Device addresses of already checked tensor arguments (None stays None)."""
    return [_ptr(t) for t in tensors]


def hs_reset(ctx, request_ids=None, stream=None) -> None:
    n = -1 if request_ids is None else request_ids.numel()
    (ids,) = _ptrs(_arg("request_ids", request_ids, _lim(ctx), nullable=True))
    _check(lib().hs_reset(ctx, ids, n, _stream(stream)))


def _step_args(lim, topk, tail0, out, miss, status, gather, gather_required=False):
    R, RK = (lim.R, lim.RK) if lim is not None else (0, 0)
    return (_arg("topk", topk, lim, RK), _arg("tail0", tail0, lim, R, nullable=True), _arg("out", out, lim, RK),
            _arg("miss", miss, lim, R), _arg("status", status, lim, R),
            _arg("gather", gather, lim, nbytes=lim.gather if lim is not None else 0, int32=False,
                 nullable=not gather_required))


def hs_resolve(ctx, topk, tail0, out, miss, status, gather=None, stream=None) -> None:
    _check(lib().hs_resolve(ctx, *_ptrs(*_step_args(_lim(ctx), topk, tail0, out, miss, status, gather)),
                            _stream(stream)))


def hs_plan(ctx, topk, tail0, out, miss, status, plan, stream=None, row_sources: bool = False) -> None:
    """row_sources: also record each position's row source, which a gathering hs_copy of this plan needs."""
    lim = _lim(ctx)
    a = _ptrs(*_step_args(lim, topk, tail0, out, miss, status, None)[:5],
              _arg("plan", plan, lim, lim.plan if lim is not None else 0))
    _check(lib().hs_plan(ctx, *a, HS_PLAN_ROW_SOURCES if row_sources else 0, _stream(stream)))


def hs_copy(ctx, plan, miss, gather=None, stream=None) -> None:
    lim = _lim(ctx)
    a = _ptrs(_arg("plan", plan, lim, lim.plan if lim is not None else 0),
              _arg("miss", miss, lim, lim.R if lim is not None else 0),
              _arg("gather", gather, lim, nbytes=lim.gather if lim is not None else 0, int32=False, nullable=True))
    _check(lib().hs_copy(ctx, *a, _stream(stream)))


def hs_step_static(ctx, topk, tail0, out, miss, status, gather=None, stream=None) -> None:
    """hs_plan + hs_copy in one call with the plan in the library's static device array (allocates nothing)."""
    _check(lib().hs_step_static(ctx, *_ptrs(*_step_args(_lim(ctx), topk, tail0, out, miss, status, gather)),
                                _stream(stream)))


def hs_trial(ctx, topk, tail0, out, miss, status, gather, trial, stream=None) -> None:
    lim = _lim(ctx)
    a = _ptrs(*_step_args(lim, topk, tail0, out, miss, status, gather, gather_required=True),
              _arg("trial", trial, lim, nbytes=lim.trial if lim is not None else 0))
    _check(lib().hs_trial(ctx, *a, _stream(stream)))


def hs_commit(ctx, trial, gather, accept=None, status=None, stream=None) -> None:
    lim = _lim(ctx)
    R = lim.R if lim is not None else 0
    a = _ptrs(_arg("trial", trial, lim, nbytes=lim.trial if lim is not None else 0),
              _arg("gather", gather, lim, nbytes=lim.gather if lim is not None else 0, int32=False),
              _arg("accept", accept, lim, R, nullable=True), _arg("status", status, lim, R, nullable=True))
    _check(lib().hs_commit(ctx, *a, _stream(stream)))


def hs_offload(ctx, rows, pos, status=None, stream=None) -> None:
    """rows: device [R, n, row_bytes] (uint8, or any dtype whose last dimension spans row_bytes); pos: device
    int32 [R]."""
    if rows is None:
        raise ValueError("rows must not be None")
    lim = _lim(ctx)
    if rows.dim() != 3:
        raise ValueError(f"rows must be [requests, n, row] (3 dimensions), got shape {tuple(rows.shape)}")
    if lim is not None and (rows.shape[0] != lim.R or rows.shape[2] * rows.element_size() != lim.row_bytes):
        raise ValueError(f"rows must be [{lim.R}, n, {lim.row_bytes} bytes], got shape {tuple(rows.shape)} of "
                         f"{rows.dtype}")
    R = lim.R if lim is not None else 0
    a = _ptrs(_arg("rows", rows, lim, int32=False), _arg("pos", pos, lim, R),
              _arg("status", status, lim, R, nullable=True))
    _check(lib().hs_offload(ctx, a[0], a[1], int(rows.shape[1]), a[2], _stream(stream)))


def hs_advance_tail(ctx, tail0, n, status=None, stream=None) -> None:
    """tail0: device int32 [R], advanced in place; n: device int32 [R]."""
    lim = _lim(ctx)
    R = lim.R if lim is not None else 0
    a = _ptrs(_arg("tail0", tail0, lim, R), _arg("n", n, lim, R), _arg("status", status, lim, R, nullable=True))
    _check(lib().hs_advance_tail(ctx, *a, _stream(stream)))


def hs_gather(ctx, out, gather, stream=None) -> None:
    lim = _lim(ctx)
    a = _ptrs(_arg("out", out, lim, lim.RK if lim is not None else 0),
              _arg("gather", gather, lim, nbytes=lim.gather if lim is not None else 0, int32=False))
    _check(lib().hs_gather(ctx, *a, _stream(stream)))


def hs_export_state(ctx, dst, what: int = 3, stream=None) -> None:
    """dst: a device tensor of at least state_tables_bytes / state_rows_bytes (as what selects); the library
    checks its byte size."""
    (p,) = _ptrs(_arg("dst", dst, _lim(ctx), int32=False))
    _check(lib().hs_export_state(ctx, p, _bytes(dst), what, _stream(stream)))


def hs_import_state(ctx, src, what: int = 3, stream=None) -> None:
    (p,) = _ptrs(_arg("src", src, _lim(ctx), int32=False))
    _check(lib().hs_import_state(ctx, p, _bytes(src), what, _stream(stream)))


def hs_rebuild_order(ctx, stream=None) -> None:
    _check(lib().hs_rebuild_order(ctx, _stream(stream)))


def hs_destroy(ctx) -> None:
    if ctx:
        _CTX_SIZES.pop(_ctx_key(ctx), None)
        lib().hs_destroy(ctx)


class SwapIn:
    """A context plus the torch device tensors it works on (plumbing around the C ABI).

    ``host_pool()`` is a numpy view of the pinned pool, [R, H, row_bytes] uint8, for the caller to fill.
    """

    def __init__(self, cfg: HsConfig, device: str = "cuda"):
        import torch
        self.cfg = cfg
        self.sizes = hs_required_sizes(cfg)
        self.R, self.k, self.B = cfg.num_requests, cfg.top_k, cfg.device_buffer_size
        self.H, self.T, self.rb = self.sizes.host_rows, cfg.tail_tokens, cfg.row_bytes
        self.device = torch.device(device)
        self.ctx = hs_create(cfg)
        dev = self.device
        self.hot = torch.zeros((self.R, self.B, self.rb), dtype=torch.uint8, device=dev)
        self.tail = torch.zeros((self.R, self.T, self.rb), dtype=torch.uint8, device=dev) if self.T else None
        self.slot_tok = torch.empty((self.R, self.B), dtype=torch.int32, device=dev)
        self.stamp = torch.empty((self.R, self.B), dtype=torch.int32, device=dev)
        self.lru_order = torch.empty((self.R, self.B), dtype=torch.int16, device=dev)
        self.page = torch.empty((self.R, self.H), dtype=torch.int32, device=dev)
        self.step = torch.empty((self.R,), dtype=torch.int32, device=dev)
        self.epoch = torch.zeros((self.R,), dtype=torch.int32, device=dev)
        hs_bind_device(self.ctx, self.hot, self.tail, self.slot_tok, self.stamp, self.lru_order, self.page, self.step,
                       self.epoch)
        hs_reset(self.ctx)

    def host_pool(self) -> np.ndarray:
        base, stride, rows = hs_host_pool(self.ctx)
        buf = (ctypes.c_uint8 * (self.R * stride)).from_address(base)
        return np.frombuffer(buf, dtype=np.uint8).reshape(self.R, rows, self.rb)

    def host_pool_address(self) -> int:
        return hs_host_pool(self.ctx)[0]

    def reset(self, request_ids=None, stream=None) -> None:
        hs_reset(self.ctx, request_ids, stream)

    def outputs(self, gather: bool = False):
        import torch
        out = torch.empty((self.R, self.k), dtype=torch.int32, device=self.device)
        miss = torch.empty((self.R,), dtype=torch.int32, device=self.device)
        status = torch.empty((self.R,), dtype=torch.int32, device=self.device)
        g = torch.empty((self.R, self.k, self.rb), dtype=torch.uint8, device=self.device) if gather else None
        return out, miss, status, g

    def resolve(self, topk, tail0=None, gather: bool = False, outputs=None, stream=None):
        out, miss, status, g = outputs if outputs is not None else self.outputs(gather)
        hs_resolve(self.ctx, topk, tail0, out, miss, status, g, stream)
        return out, miss, status, g

    def trial_buffer(self):
        import torch
        return torch.empty((self.sizes.trial_bytes // 4,), dtype=torch.int32, device=self.device)

    def state_buffer(self, what: int = 3):
        """A device buffer for hs_export_state / hs_import_state of what (HS_STATE_TABLES | HS_STATE_ROWS), zeroed
        so that the alignment padding between sections (never written) compares equal across snapshots."""
        import torch
        n = (self.sizes.state_tables_bytes if what & HS_STATE_TABLES else 0) + \
            (self.sizes.state_rows_bytes if what & HS_STATE_ROWS else 0)
        return torch.zeros((n,), dtype=torch.uint8, device=self.device)

    def plan_buffer(self):
        import torch
        return torch.empty((self.R, 4, self.k), dtype=torch.int32, device=self.device)

    def close(self) -> None:
        if self.ctx:
            hs_destroy(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
