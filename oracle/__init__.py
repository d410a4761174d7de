"""ORACLE — test infrastructure, not product code.

Python handle on the plain single-threaded CPU model of the HiSparse swap-in
step in ``hs_oracle.c``. Only the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import it. It shares no code with the
HIP library and imports nothing from it: its inputs come from the ``workload``
generator, never from the GPU path.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "hs_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

BAD_ID = 1
DUP_ID = 2
LRU = 0
FIFO = 1


def build(force: bool = True, src: str = _SRC, dst: str = _LIB_PATH) -> str:
    """Compile the oracle with gcc (no HIP)."""
    if force or not os.path.exists(dst):
        tmp = dst + ".tmp"
        subprocess.run(["gcc", "-O2", "-std=c11", "-shared", "-fPIC", "-o", tmp, src], check=True)
        os.replace(tmp, dst)
    return dst


class Dims(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("k", ctypes.c_int32), ("H", ctypes.c_int32), ("T", ctypes.c_int32),
                ("row_bytes", ctypes.c_int64), ("policy", ctypes.c_int32)]


def load(path: Optional[str] = None):
    """Load the oracle library (``path`` lets tests load a deliberately broken copy)."""
    global _lib
    if path is None and _lib is not None:
        return _lib
    p = path or _LIB_PATH
    if path is None and not os.path.exists(p):
        build(force=True)
    lib = ctypes.CDLL(p)
    vp = ctypes.c_void_p
    lib.oracle_reset.argtypes = [ctypes.POINTER(Dims), vp, vp, vp, vp]
    lib.oracle_reset.restype = None
    lib.oracle_resolve_batch.argtypes = [ctypes.POINTER(Dims), ctypes.c_int32] + [vp] * 13
    lib.oracle_resolve_batch.restype = ctypes.c_int
    lib.oracle_offload.argtypes = [ctypes.POINTER(Dims), vp, vp, vp, vp, ctypes.c_int32, ctypes.c_int32]
    lib.oracle_offload.restype = ctypes.c_int
    lib.oracle_advance_tail.argtypes = [ctypes.POINTER(Dims), vp, vp, vp, vp, vp, ctypes.c_int32]
    lib.oracle_advance_tail.restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


class Oracle:
    """State of ``n`` requests and one-step transitions, all on the CPU.

    ``host`` is uint8 [n, H, row_bytes] (the caller fills it from the workload generator);
    ``tail`` (optional) is uint8 [n, T, row_bytes].
    """

    def __init__(self, n: int, B: int, k: int, H: int, row_bytes: int, T: int = 0,
                 host: Optional[np.ndarray] = None, tail: Optional[np.ndarray] = None, lib_path: Optional[str] = None,
                 policy: int = LRU):
        self.n, self.B, self.k, self.H, self.T, self.rb = n, B, k, H, T, row_bytes
        self.policy = policy
        self.dims = Dims(B, k, H, T, row_bytes, policy)
        self.lib = load(lib_path)
        self.slot_tok = np.full((n, B), -1, np.int32)
        self.stamp = np.full((n, B), -1, np.int32)
        self.page = np.full((n, H), -1, np.int32)
        self.t = np.zeros(n, np.int32)
        self.hot = np.zeros((n, B, row_bytes), np.uint8)
        self.host = host if host is not None else np.zeros((n, H, row_bytes), np.uint8)
        assert self.host.shape == (n, H, row_bytes) and self.host.dtype == np.uint8 and self.host.flags.c_contiguous
        self.tail = tail
        if tail is not None:
            assert tail.shape == (n, T, row_bytes) and tail.dtype == np.uint8 and tail.flags.c_contiguous

    def reset(self, requests: Optional[Sequence[int]] = None) -> None:
        for r in (range(self.n) if requests is None else requests):
            self.lib.oracle_reset(ctypes.byref(self.dims), _p(self.slot_tok[r]), _p(self.stamp[r]),
                                  _p(self.page[r]), ctypes.c_void_p(self.t.ctypes.data + 4 * int(r)))

    def step(self, ids: np.ndarray, tail0: Optional[np.ndarray] = None, gather: bool = False
             ) -> Tuple[np.ndarray, np.ndarray, np.ndarray, Optional[np.ndarray]]:
        """One resolve of every request. ids: int32 [n, k]. Returns (out, miss, status, gathered rows)."""
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        assert ids.shape == (self.n, self.k)
        out = np.empty((self.n, self.k), np.int32)
        miss = np.empty(self.n, np.int32)
        status = np.empty(self.n, np.int32)
        g = np.empty((self.n, self.k, self.rb), np.uint8) if gather else None
        t0 = None if tail0 is None else np.ascontiguousarray(tail0, dtype=np.int32)
        rc = self.lib.oracle_resolve_batch(ctypes.byref(self.dims), self.n, _p(self.slot_tok), _p(self.stamp),
                                           _p(self.page), _p(self.t), _p(self.hot), _p(self.host), _p(self.tail),
                                           _p(ids), _p(t0), _p(out), _p(miss), _p(status), _p(g))
        if rc != 0:
            raise RuntimeError(f"oracle step failed ({rc}): more misses than free slots")
        return out, miss, status, g

    def offload(self, rows: np.ndarray, pos: np.ndarray) -> np.ndarray:
        """rows: uint8 [n_req, n, row_bytes] written as host rows pos[r] .. pos[r] + n - 1 (and into the hot slot
        of a token that has one). Returns the per-request status."""
        rows = np.ascontiguousarray(rows, dtype=np.uint8)
        n = rows.shape[1]
        st = np.zeros(self.n, np.int32)
        for r in range(self.n):
            st[r] = self.lib.oracle_offload(ctypes.byref(self.dims), _p(self.host[r]), _p(self.hot[r]),
                                            _p(self.page[r]), _p(rows[r]), int(pos[r]), n)
        return st

    def advance_tail(self, tail0: np.ndarray, n: np.ndarray) -> np.ndarray:
        """Move each request's tail window forward by n[r] tokens (tail0 updated in place, int32 [n_req]);
        the leaving rows go to the host rows (and hot slots). Returns the per-request status."""
        assert self.tail is not None and tail0.dtype == np.int32 and tail0.flags.c_contiguous
        st = np.zeros(self.n, np.int32)
        for r in range(self.n):
            st[r] = self.lib.oracle_advance_tail(ctypes.byref(self.dims), _p(self.host[r]), _p(self.tail[r]),
                                                 _p(self.hot[r]), _p(self.page[r]),
                                                 ctypes.c_void_p(tail0.ctypes.data + 4 * r), int(n[r]))
        return st
