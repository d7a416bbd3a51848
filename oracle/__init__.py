"""Python face of the CPU oracle (``xq_oracle.c``).

TEST INFRASTRUCTURE. Only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. It never imports
the HIP library's package and the HIP library never loads it.

All functions take and return host numpy arrays. The module-level functions
use the default build; ``Oracle(path)`` wraps another build of the same
source (the tests build copies with one planted mistake each and check that
the pins catch it).
"""

from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "xq_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
CFLAGS = ["-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared",
          "-Wall", "-Wextra"]
_lock = threading.Lock()
_default = None

Q8K_BYTES = 320
Q4K_BYTES = 144


def compile_oracle(out_path: str, defines=()) -> str:
    """Compile ``xq_oracle.c`` with gcc into ``out_path``."""
    tmp = out_path + ".tmp%d" % os.getpid()
    cmd = ["gcc", *CFLAGS, *("-D" + d for d in defines), SOURCE, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out_path)
    return out_path


def build(force: bool = True) -> str:
    """Compile the default oracle into ``oracle/liboracle.so``."""
    if force or not os.path.exists(_LIB):
        compile_oracle(_LIB)
    return _LIB


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _u8(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    return a.reshape(-1).view(np.uint8)


def _rows_arg(rows):
    if rows is None:
        return None, None, 0
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
    return r, _ptr(r), r.size


class Oracle:
    """One loaded build of the oracle library."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        I = ctypes.c_int64
        lib.xqo_f16_to_f64.argtypes = [ctypes.c_uint16]
        lib.xqo_f16_to_f64.restype = ctypes.c_double
        lib.xqo_quantize_q8k.argtypes = [P, I, I, P]
        lib.xqo_dequant_q8k.argtypes = [P, I, I, P]
        lib.xqo_q4k_scale_min.argtypes = [P, ctypes.c_int, P, P]
        lib.xqo_q4k_code.argtypes = [P, ctypes.c_int]
        lib.xqo_q4k_code.restype = ctypes.c_int
        lib.xqo_dequant_q4k.argtypes = [P, I, I, P]
        lib.xqo_q4k_partials.argtypes = [P, P, I, I, P, I, P, P]
        lib.xqo_gemv_q4k.argtypes = [P, P, I, I, P, I, P, P, P]
        lib.xqo_gemm_q4k.argtypes = [P, P, I, I, I, P, P, I, P, P, P]
        lib.xqo_iq4nl_codebook.argtypes = [ctypes.c_int]
        lib.xqo_iq4nl_codebook.restype = ctypes.c_int
        lib.xqo_dequant_iq4nl.argtypes = [P, I, I, P]
        lib.xqo_iq4nl_partials.argtypes = [P, P, I, I, P, I, P]
        lib.xqo_gemv_iq4nl.argtypes = [P, P, I, I, P, I, P, P, P]
        lib.xqo_dequant_q4_0.argtypes = [P, I, I, P]
        lib.xqo_q4_0_partials.argtypes = [P, P, I, I, P, I, P]
        lib.xqo_gemv_q4_0.argtypes = [P, P, I, I, P, I, P, P, P]
        self.lib = lib
        self.path = path

    # ---- f16 -------------------------------------------------------------
    def f16_to_f64(self, bits: int) -> float:
        return self.lib.xqo_f16_to_f64(int(bits) & 0xFFFF)

    # ---- q8_K ------------------------------------------------------------
    def quantize_q8k(self, x: np.ndarray) -> np.ndarray:
        """f32 [rows, K] -> uint8 [rows, K/256, 320]."""
        x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
        if x.ndim == 1:
            x = x.reshape(1, -1)
        rows, K = x.shape
        assert K % 256 == 0
        out = np.empty((rows, K // 256, Q8K_BYTES), dtype=np.uint8)
        self.lib.xqo_quantize_q8k(_ptr(x), rows, K, _ptr(out))
        return out

    def dequant_q8k(self, xq: np.ndarray, rows: int, K: int) -> np.ndarray:
        xq = _u8(xq)
        out = np.empty((rows, K), dtype=np.float64)
        self.lib.xqo_dequant_q8k(_ptr(xq), rows, K, _ptr(out))
        return out

    # ---- Q4_K ------------------------------------------------------------
    def q4k_scale_min(self, block: np.ndarray, j: int):
        blk = _u8(block)
        sc = ctypes.c_int()
        m = ctypes.c_int()
        self.lib.xqo_q4k_scale_min(_ptr(blk), j, ctypes.byref(sc), ctypes.byref(m))
        return sc.value, m.value

    def q4k_code(self, block: np.ndarray, i: int) -> int:
        return self.lib.xqo_q4k_code(_ptr(_u8(block)), i)

    def dequant_q4k(self, w, N: int, K: int) -> np.ndarray:
        w = _u8(w)
        out = np.empty((N, K), dtype=np.float64)
        self.lib.xqo_dequant_q4k(_ptr(w), N, K, _ptr(out))
        return out

    def q4k_partials(self, w, xq, N: int, K: int, rows=None):
        """Exact per-block partials (S, M), int32 [nrows, K/256]."""
        w = _u8(w)
        xq = _u8(xq)
        r, rp, n = _rows_arg(rows)
        nrows = N if r is None else n
        S = np.empty((nrows, K // 256), dtype=np.int32)
        M = np.empty((nrows, K // 256), dtype=np.int32)
        self.lib.xqo_q4k_partials(_ptr(w), _ptr(xq), N, K, rp, n, _ptr(S), _ptr(M))
        return S, M

    def gemv_q4k(self, w, xq, N: int, K: int, rows=None, elem=False):
        """(y, T), double [nrows]: y by the plain definition; T the sum of
        |terms| of the f32 bar: over the row's blocks, |d*xs*S| + |dmin*xs*M|.
        With elem=True: (y, T, Te), Te the sum over elements of
        |d*sc*q*xhat| + |dmin*m*xhat| (Te >= T >= |y|)."""
        w = _u8(w)
        xq = _u8(xq)
        r, rp, n = _rows_arg(rows)
        nrows = N if r is None else n
        y, T, Te = (np.empty(nrows, dtype=np.float64) for _ in range(3))
        self.lib.xqo_gemv_q4k(_ptr(w), _ptr(xq), N, K, rp, n, _ptr(y), _ptr(T), _ptr(Te))
        return (y, T, Te) if elem else (y, T)

    def gemm_q4k(self, w, xq, M: int, N: int, K: int, ms=None, ns=None, elem=False):
        """(Y, T) as gemv_q4k per (token, row): full [M, N] arrays, or values at
        the listed (m, n) pairs; (Y, T, Te) with elem=True."""
        w = _u8(w)
        xq = _u8(xq)
        if ms is None:
            Y, T, Te = (np.empty(M * N, dtype=np.float64) for _ in range(3))
            self.lib.xqo_gemm_q4k(_ptr(w), _ptr(xq), M, N, K, None, None, 0, _ptr(Y), _ptr(T),
                                  _ptr(Te))
            out = (Y.reshape(M, N), T.reshape(M, N), Te.reshape(M, N))
            return out if elem else out[:2]
        ms = np.ascontiguousarray(np.asarray(ms, dtype=np.int64))
        ns = np.ascontiguousarray(np.asarray(ns, dtype=np.int64))
        assert ms.shape == ns.shape
        Y, T, Te = (np.empty(ms.size, dtype=np.float64) for _ in range(3))
        self.lib.xqo_gemm_q4k(_ptr(w), _ptr(xq), M, N, K, _ptr(ms), _ptr(ns), ms.size,
                              _ptr(Y), _ptr(T), _ptr(Te))
        return (Y, T, Te) if elem else (Y, T)

    # ---- IQ4_NL ----------------------------------------------------------
    def iq4nl_codebook(self, nibble: int) -> int:
        return self.lib.xqo_iq4nl_codebook(nibble)

    def dequant_iq4nl(self, w, N: int, K: int) -> np.ndarray:
        w = _u8(w)
        out = np.empty((N, K), dtype=np.float64)
        self.lib.xqo_dequant_iq4nl(_ptr(w), N, K, _ptr(out))
        return out

    def iq4nl_partials(self, w, xq, N: int, K: int, rows=None):
        """Exact per-block partials D, int32 [nrows, K/32]."""
        w = _u8(w)
        xq = _u8(xq)
        r, rp, n = _rows_arg(rows)
        nrows = N if r is None else n
        D = np.empty((nrows, K // 32), dtype=np.int32)
        self.lib.xqo_iq4nl_partials(_ptr(w), _ptr(xq), N, K, rp, n, _ptr(D))
        return D

    def gemv_iq4nl(self, w, xq, N: int, K: int, rows=None, elem=False):
        """(y, T): T the sum over 32-blocks of |d_c*xs*D_c|; with elem=True
        (y, T, Te), Te the sum over elements of |d_c*kv*xhat|."""
        w = _u8(w)
        xq = _u8(xq)
        r, rp, n = _rows_arg(rows)
        nrows = N if r is None else n
        y, T, Te = (np.empty(nrows, dtype=np.float64) for _ in range(3))
        self.lib.xqo_gemv_iq4nl(_ptr(w), _ptr(xq), N, K, rp, n, _ptr(y), _ptr(T), _ptr(Te))
        return (y, T, Te) if elem else (y, T)

    def dequant_q4_0(self, w, N: int, K: int) -> np.ndarray:
        """Q4_0 resident rows (the IQ4_NL row shape) -> f64 weights d*(nibble-8)."""
        w = _u8(w)
        out = np.empty((N, K), dtype=np.float64)
        self.lib.xqo_dequant_q4_0(_ptr(w), N, K, _ptr(out))
        return out

    def q4_0_partials(self, w, xq, N: int, K: int, rows=None):
        """Exact per-block partials D = sum (nibble-8)*code, int32 [nrows, K/32]."""
        w = _u8(w)
        xq = _u8(xq)
        r, rp, n = _rows_arg(rows)
        nrows = N if r is None else n
        D = np.empty((nrows, K // 32), dtype=np.int32)
        self.lib.xqo_q4_0_partials(_ptr(w), _ptr(xq), N, K, rp, n, _ptr(D))
        return D

    def gemv_q4_0(self, w, xq, N: int, K: int, rows=None, elem=False):
        """(y, T) as gemv_iq4nl, weights d_c*(nibble-8)."""
        w = _u8(w)
        xq = _u8(xq)
        r, rp, n = _rows_arg(rows)
        nrows = N if r is None else n
        y, T, Te = (np.empty(nrows, dtype=np.float64) for _ in range(3))
        self.lib.xqo_gemv_q4_0(_ptr(w), _ptr(xq), N, K, rp, n, _ptr(y), _ptr(T), _ptr(Te))
        return (y, T, Te) if elem else (y, T)


def repack_iq4nl(file_blocks, n_blocks: int, block_base: int, bpr: int, resident=None):
    """IQ4_NL file blocks -> resident rows, by the layouts' definitions
    ("25 — Writing XPU Kernels", section 25.4: a resident row is the row's f16
    block scales, zero-padded to a multiple of 4 bytes, then its 16-byte
    payloads; a file block is the f16 scale followed by its 16 payload bytes).
    Blocks block_base .. block_base + n_blocks - 1 (block g is block g % bpr of
    row g // bpr) are written into `resident` (uint8[rows, row_bytes]; a new
    zero-filled array when None), with a row's pad bytes when the chunk holds
    the row's last block. Plain numpy, one block at a time."""
    blocks = np.asarray(file_blocks, dtype=np.uint8).reshape(n_blocks, 18)
    prefix = ((2 * bpr + 3) // 4) * 4
    row_bytes = prefix + 16 * bpr
    rows = (block_base + n_blocks + bpr - 1) // bpr
    if resident is None:
        resident = np.zeros((rows, row_bytes), dtype=np.uint8)
    for b in range(n_blocks):
        g = block_base + b
        r, j = divmod(g, bpr)
        resident[r, 2 * j:2 * j + 2] = blocks[b, 0:2]
        resident[r, prefix + 16 * j:prefix + 16 * j + 16] = blocks[b, 2:18]
        if j == bpr - 1:
            resident[r, 2 * bpr:prefix] = 0
    return resident


def default() -> Oracle:
    """The default build, compiled on first use when it is missing."""
    global _default
    with _lock:
        if _default is None:
            if not os.path.exists(_LIB):
                build(force=True)
            _default = Oracle(_LIB)
    return _default


def __getattr__(name):
    # Module-level aliases of the default build's methods.
    if not name.startswith("_") and hasattr(Oracle, name):
        return getattr(default(), name)
    raise AttributeError(name)
