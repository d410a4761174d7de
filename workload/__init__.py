"""Seeded synthetic inputs for the HiSparse swap-in path.

This package only draws inputs: per-step top-k token-id streams and the bf16
rows of the host KV pool. It holds none of the swap-in method's arithmetic,
so both the CPU oracle (under ``oracle/``) and the HIP path consume it without
sharing any of the method's code.

The workloads mirror the settings the pages describe for HiSparse: top-k 2048
per decode step, a hot device buffer of 2x or 3x top-k slots, a host pool that
holds the whole context ("HiSparse: Turbocharging Sparse Attention with
Hierarchical Memory", section 2, and the launch configuration in section 3),
and the device-resident tail of Mixed residency ("vLLM GLM 5.3 最適化: Hybrid
HiSparse オフローディング", section 2 Mixed Residency). The pages measure on
LongBenchV2 and on serving traces; these seeded streams stand in for them.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import subprocess
from typing import List, Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "streams.c")
_LIB_PATH = os.path.join(_HERE, "libworkload.so")
_lib = None

MASK64 = (1 << 64) - 1
GOLDEN = 0x9E3779B97F4A7C15


def build(force: bool = True) -> str:
    """Compile the C generator (gcc, OpenMP) next to its source."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.run(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11", "-o", tmp, _SRC, "-lm"],
                       check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _Spec(ctypes.Structure):
    _fields_ = [("k", ctypes.c_int32), ("L0", ctypes.c_int32), ("grow", ctypes.c_int32),
                ("keep_permille", ctypes.c_int32), ("window", ctypes.c_int32), ("tail", ctypes.c_int32),
                ("partB_permille", ctypes.c_int32)]


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        lib.ws_streams.argtypes = [ctypes.POINTER(_Spec), ctypes.c_uint64, ctypes.c_int32, ctypes.c_int32,
                                   ctypes.c_void_p]
        lib.ws_streams.restype = ctypes.c_int
        lib.ws_fill_rows.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int32,
                                     ctypes.c_uint64]
        lib.ws_fill_rows.restype = ctypes.c_int
        _lib = lib
    return _lib


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: sizes of the path plus the stream recipe."""
    name: str
    num_requests: int          # R
    top_k: int                 # k
    buffer_slots: int          # B, hot slots per request
    host_rows: int             # host pool rows per request
    L0: int                    # context length at step 0
    grow: bool                 # context grows by one token per step; the new token is always selected
    keep_permille: int         # share of the previous step kept, in 1/1000
    window: int                # recent window of the refill's second half
    partB_permille: int        # share of the refill from the window (or the device tail), in 1/1000
    steps: int
    tail_tokens: int = 0       # T device-resident tail tokens per request (hybrid residency)
    fused_gather: bool = False
    row_elems: int = 576       # bf16 elements per KV row (1152 B)
    stream_seed: int = 1000
    row_seed: int = 2000

    @property
    def row_bytes(self) -> int:
        return 2 * self.row_elems

    @property
    def tail0(self) -> Optional[int]:
        """First device-resident token (hybrid residency), else None."""
        return self.L0 - self.tail_tokens if self.tail_tokens else None

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    def spec(self) -> _Spec:
        return _Spec(self.top_k, self.L0, int(self.grow), self.keep_permille, self.window, self.tail_tokens,
                     self.partB_permille)


# The five workloads. Sizes: top-k 2048, hot buffer 2x top-k (4096) or swept over
# 2048/4096/6144, host pool = whole context; rows of 576 bf16.
SINGLE_4K = Workload("single_request_L4096_B512_k256", 1, 256, 512, 4096, 4096, False, 800, 512, 500, 64,
                     stream_seed=1000, row_seed=2000)
GROW_32 = Workload("grow_32req_L32768_B4096_k2048", 32, 2048, 4096, 33024, 32768, True, 800, 4096, 500, 256,
                   stream_seed=1001, row_seed=2001)
SWEEP_BASE = Workload("sweep_64req_L65536_k2048", 64, 2048, 4096, 65536, 65536, False, 800, 4096, 500, 512,
                      stream_seed=1002, row_seed=2002)
CONC_256 = Workload("concurrency_256req_L32768_B4096_k2048", 256, 2048, 4096, 40960, 32768, True, 800, 8192, 500,
                    1024, stream_seed=1003, row_seed=2003)
HYBRID_64 = Workload("hybrid_tail_64req_L131072_T8192_B4096_k2048", 64, 2048, 4096, 131072, 131072, False, 800, 0,
                     300, 256, tail_tokens=8192, fused_gather=True, stream_seed=1004, row_seed=2004)


def sweep_workloads() -> List[Workload]:
    """Buffer-size sweep: B in {2048, 4096, 6144} x keep in {0.6, 0.8, 0.95}; one stream seed per keep
    share, so the three buffer sizes see identical streams."""
    out = []
    for j, keep in enumerate((600, 800, 950)):
        for B in (2048, 4096, 6144):
            out.append(SWEEP_BASE.with_(name=f"sweep_64req_L65536_B{B}_keep{keep}_k2048", buffer_slots=B,
                                        keep_permille=keep, stream_seed=1002 + 10 * j))
    return out


ALL = [SINGLE_4K, GROW_32, *sweep_workloads(), CONC_256, HYBRID_64]


def streams(w: Workload, n_steps: Optional[int] = None, requests: Optional[int] = None) -> np.ndarray:
    """Top-k ids [R, steps, k] int32 from the C generator."""
    n_steps = w.steps if n_steps is None else n_steps
    R = w.num_requests if requests is None else requests
    out = np.empty((R, n_steps, w.top_k), dtype=np.int32)
    sp = w.spec()
    rc = _load().ws_streams(ctypes.byref(sp), ctypes.c_uint64(w.stream_seed), R, n_steps, out.ctypes.data)
    if rc != 0:
        raise ValueError(f"stream generator failed for {w.name}")
    return out


def fill_rows(dst: np.ndarray, row0: int, n_rows: int, row_elems: int, seed: int) -> None:
    """Fill ``dst`` (uint16 [n_rows, row_elems], C-contiguous) with the rows named row0 .. row0+n_rows-1."""
    assert dst.dtype == np.uint16 and dst.flags.c_contiguous and dst.size == n_rows * row_elems
    rc = _load().ws_fill_rows(dst.ctypes.data, row0, n_rows, row_elems, ctypes.c_uint64(seed))
    if rc != 0:
        raise ValueError("row filler failed")


def fill_rows_ptr(ptr: int, row0: int, n_rows: int, row_elems: int, seed: int) -> None:
    """Same as fill_rows for raw host memory (e.g. the library's pinned pool)."""
    rc = _load().ws_fill_rows(ctypes.c_void_p(ptr), row0, n_rows, row_elems, ctypes.c_uint64(seed))
    if rc != 0:
        raise ValueError("row filler failed")


# ---------------------------------------------------------------------------
# Slow pure-Python twin of the stream generator, used to check the C one.
# ---------------------------------------------------------------------------

def _mix(z: int) -> int:
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
    return z ^ (z >> 31)


class _PyRng:
    def __init__(self, seed: int, r: int, t: int):
        self.s = _mix(seed ^ _mix(((r << 32) | t) & MASK64))

    def below(self, n: int) -> int:
        self.s = (self.s + GOLDEN) & MASK64
        return (((_mix(self.s) >> 32) * n) >> 32)


def streams_py(w: Workload, n_steps: int, requests: int) -> np.ndarray:
    k = w.top_k
    out = np.empty((requests, n_steps, k), dtype=np.int32)
    for r in range(requests):
        prev: List[int] = []
        for t in range(n_steps):
            g = _PyRng(w.stream_seed, r, t)
            L = w.L0 + (t if w.grow else 0)
            cur: List[int] = []
            seen = set()

            def draw(lo: int, hi: int, n: int) -> None:
                while n > 0:
                    x = lo + g.below(hi - lo)
                    if x in seen:
                        continue
                    seen.add(x)
                    cur.append(x)
                    n -= 1

            if t == 0:
                if w.grow:
                    cur.append(L - 1)
                    seen.add(L - 1)
                draw(0, L, k - len(cur))
            else:
                keep = (w.keep_permille * k) // 1000
                tmp = list(prev)
                for i in range(keep):
                    j = i + g.below(k - i)
                    tmp[i], tmp[j] = tmp[j], tmp[i]
                    cur.append(tmp[i])
                    seen.add(tmp[i])
                if w.grow:
                    cur.append(L - 1)
                    seen.add(L - 1)
                n_new = k - len(cur)
                nB = (w.partB_permille * n_new) // 1000
                nA = n_new - nB
                if w.tail_tokens:
                    draw(0, L - w.tail_tokens, nA)
                    draw(L - w.tail_tokens, L, nB)
                else:
                    draw(0, L, nA)
                    draw(max(0, L - w.window), L, nB)
            for i in range(k - 1, 0, -1):
                j = g.below(i + 1)
                cur[i], cur[j] = cur[j], cur[i]
            out[r, t] = cur
            prev = cur
    return out
