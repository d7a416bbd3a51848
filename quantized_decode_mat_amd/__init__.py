"""Python binding of libxq (the C ABI in include/xq.h).

The functions carry the C names and only marshal arguments: tensors become
device pointers, ``stream=None`` becomes torch's current HIP stream, and a
refused call raises ``XQError`` with the library's own sentence. Before the
call, the binding checks that every tensor is a device tensor large enough for
the layout the C function will read or write, so a wrong-sized buffer is
refused on the host instead of being read out of bounds. Every step of the
computation runs in the library's HIP kernels; there is no host path.

Three calls take a caller-owned device workspace (``workspace=``, a device
tensor of at least the bytes the matching ``*_workspace_bytes`` query gives,
zeroed before its first use); the binding passes it through and allocates
nothing.
"""

from __future__ import annotations

import ctypes
import os
import threading

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libxq.so")
_lock = threading.Lock()
_lib = None

XQ_OK, XQ_E_NULL, XQ_E_SHAPE, XQ_E_ALIGN, XQ_E_DEVICE, XQ_E_LAUNCH = range(6)
XQ_MAX_K = 1048576
EXPORTS = (
    "xq_quantize_q8k", "xq_gemv_q4k", "xq_gemv_iq4nl", "xq_gemm_q4k_small_m",
    "xq_q8k_bytes", "xq_q4k_bytes", "xq_iq4nl_bytes", "xq_status_name", "xq_last_error",
    "xq_bench_stream_read", "xq_bench_sink_words", "xq_gemv_q4k_id", "xq_gemv_iq4nl_id",
    "xq_repack_iq4nl", "xq_repack_dword_prefix_launches", "xq_gemv_q4_0", "xq_gemm_q4k_id",
    "xq_gemv_q4k_q8k", "xq_gemm_q4k_small_m_workspace_bytes", "xq_gemv_q4k_q8k_workspace_bytes",
    "xq_gemm_q4k_id_workspace_bytes", "xq_gemm_q4k_small_m_noalloc",
)
XQ_NOALLOC_SCRATCH_BYTES = 8 * 1024 * 1024


class XQError(RuntimeError):
    def __init__(self, status: int, func: str, text: str):
        self.status = status
        super().__init__("%s: %s (%s)" % (func, text, _name(status)))


def lib() -> ctypes.CDLL:
    """The loaded libxq.so (built in-tree first if it is not there)."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                from . import build as _build
                _build.build()
            L = ctypes.CDLL(LIB_PATH)
            P, I, S = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
            L.xq_quantize_q8k.argtypes = [P, P, I, I, P]
            L.xq_gemv_q4k.argtypes = [P, P, P, I, I, P]
            L.xq_gemv_iq4nl.argtypes = [P, P, P, I, I, P]
            L.xq_gemv_q4_0.argtypes = [P, P, P, I, I, P]
            Z = ctypes.c_size_t
            L.xq_gemm_q4k_small_m.argtypes = [P, P, P, I, I, I, P, Z, P]
            L.xq_gemm_q4k_small_m_noalloc.argtypes = [P, P, P, I, I, I, P]
            L.xq_bench_stream_read.argtypes = [P, I, P, P]
            L.xq_gemv_q4k_id.argtypes = [P, P, P, P, I, I, I, I, I, P]
            L.xq_gemv_iq4nl_id.argtypes = [P, P, P, P, I, I, I, I, I, P]
            L.xq_repack_iq4nl.argtypes = [P, P, I, I, I, P]
            L.xq_gemm_q4k_id.argtypes = [P, P, P, P, I, I, I, I, I, I, P, Z, P]
            L.xq_gemv_q4k_q8k.argtypes = [P, P, P, P, I, I, P, Z, P]
            L.xq_gemm_q4k_small_m_workspace_bytes.argtypes = [I, I, I]
            L.xq_gemm_q4k_small_m_workspace_bytes.restype = Z
            L.xq_gemv_q4k_q8k_workspace_bytes.argtypes = [I]
            L.xq_gemv_q4k_q8k_workspace_bytes.restype = Z
            L.xq_gemm_q4k_id_workspace_bytes.argtypes = [I, I, I]
            L.xq_gemm_q4k_id_workspace_bytes.restype = Z
            L.xq_repack_dword_prefix_launches.argtypes = []
            L.xq_repack_dword_prefix_launches.restype = I
            for f in ("xq_quantize_q8k", "xq_gemv_q4k", "xq_gemv_iq4nl", "xq_gemm_q4k_small_m",
                      "xq_bench_stream_read", "xq_gemv_q4k_id", "xq_gemv_iq4nl_id", "xq_repack_iq4nl",
                      "xq_gemv_q4_0", "xq_gemm_q4k_id", "xq_gemv_q4k_q8k",
                      "xq_gemm_q4k_small_m_noalloc"):
                getattr(L, f).restype = S
            for f in ("xq_q8k_bytes", "xq_q4k_bytes", "xq_iq4nl_bytes"):
                getattr(L, f).argtypes = [I, I]
                getattr(L, f).restype = ctypes.c_size_t
            L.xq_bench_sink_words.argtypes = [I]
            L.xq_bench_sink_words.restype = I
            L.xq_status_name.argtypes = [S]
            L.xq_status_name.restype = ctypes.c_char_p
            L.xq_last_error.argtypes = []
            L.xq_last_error.restype = ctypes.c_char_p
            _lib = L
    return _lib


def _name(status: int) -> str:
    return lib().xq_status_name(status).decode()


def _ptr(a, need_bytes: int, what: str):
    """Device pointer of a tensor (checked to hold need_bytes), or a raw int."""
    if a is None:
        return None
    if isinstance(a, int):
        return a
    if not isinstance(a, torch.Tensor):
        raise TypeError("%s: expected a torch.Tensor or an int pointer" % what)
    if not a.is_cuda:
        raise ValueError("%s: must be a device tensor" % what)
    if not a.is_contiguous():
        raise ValueError("%s: must be contiguous" % what)
    have = a.numel() * a.element_size()
    if have < need_bytes:
        raise ValueError("%s: holds %d bytes, the layout needs %d" % (what, have, need_bytes))
    return a.data_ptr()


def _workspace(ws, need: int):
    """(pointer, bytes) of a workspace tensor checked to hold `need` bytes;
    (None, 0) for None (the library refuses it when the call needs one)."""
    if ws is None:
        return None, 0
    p = _ptr(ws, need, "workspace")
    return p, (ws.numel() * ws.element_size() if isinstance(ws, torch.Tensor) else need)


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, func: str):
    if status != XQ_OK:
        raise XQError(status, func, lib().xq_last_error().decode())


def xq_q8k_bytes(rows: int, K: int) -> int:
    return lib().xq_q8k_bytes(rows, K)


def xq_q4k_bytes(N: int, K: int) -> int:
    return lib().xq_q4k_bytes(N, K)


def xq_iq4nl_bytes(N: int, K: int) -> int:
    return lib().xq_iq4nl_bytes(N, K)


def xq_status_name(status: int) -> str:
    return _name(status)


def xq_last_error() -> str:
    return lib().xq_last_error().decode()


def xq_quantize_q8k(xq, x, rows: int, K: int, stream=None) -> None:
    _check(lib().xq_quantize_q8k(_ptr(xq, xq_q8k_bytes(rows, K), "xq"),
                                 _ptr(x, 4 * rows * K, "x"), rows, K, _stream(stream)),
           "xq_quantize_q8k")


def xq_gemv_q4k(y, w, xq, N: int, K: int, stream=None) -> None:
    _check(lib().xq_gemv_q4k(_ptr(y, 4 * N, "y"), _ptr(w, xq_q4k_bytes(N, K), "w"),
                             _ptr(xq, xq_q8k_bytes(1, K), "xq"), N, K, _stream(stream)),
           "xq_gemv_q4k")


def xq_gemv_iq4nl(y, w, xq, N: int, K: int, stream=None) -> None:
    _check(lib().xq_gemv_iq4nl(_ptr(y, 4 * N, "y"), _ptr(w, xq_iq4nl_bytes(N, K), "w"),
                               _ptr(xq, xq_q8k_bytes(1, K), "xq"), N, K, _stream(stream)),
           "xq_gemv_iq4nl")


def xq_gemv_q4k_q8k_workspace_bytes(N: int) -> int:
    return lib().xq_gemv_q4k_q8k_workspace_bytes(N)


def xq_gemv_q4k_q8k(y, yq, w, xq, N: int, K: int, workspace=None, stream=None) -> None:
    wp, wb = _workspace(workspace, xq_gemv_q4k_q8k_workspace_bytes(N))
    _check(lib().xq_gemv_q4k_q8k(_ptr(y, 4 * N, "y"), _ptr(yq, xq_q8k_bytes(1, N), "yq"),
                                 _ptr(w, xq_q4k_bytes(N, K), "w"), _ptr(xq, xq_q8k_bytes(1, K), "xq"),
                                 N, K, wp, wb, _stream(stream)),
           "xq_gemv_q4k_q8k")


def xq_gemv_q4_0(y, w, xq, N: int, K: int, stream=None) -> None:
    _check(lib().xq_gemv_q4_0(_ptr(y, 4 * N, "y"), _ptr(w, xq_iq4nl_bytes(N, K), "w"),
                              _ptr(xq, xq_q8k_bytes(1, K), "xq"), N, K, _stream(stream)),
           "xq_gemv_q4_0")


def xq_gemv_q4k_id(y, slab, xq, sel, n_experts: int, used: int, rows: int, K: int,
                   x_stride_blocks: int = 0, stream=None) -> None:
    xrows = used if x_stride_blocks else 1
    _check(lib().xq_gemv_q4k_id(_ptr(y, 4 * used * rows, "y"),
                                _ptr(slab, xq_q4k_bytes(n_experts * rows, K), "slab"),
                                _ptr(xq, xq_q8k_bytes(xrows, K), "xq"), _ptr(sel, 4 * used, "sel"),
                                n_experts, used, rows, K, x_stride_blocks, _stream(stream)),
           "xq_gemv_q4k_id")


def xq_gemv_iq4nl_id(y, slab, xq, sel, n_experts: int, used: int, rows: int, K: int,
                     x_stride_blocks: int = 0, stream=None) -> None:
    xrows = used if x_stride_blocks else 1
    _check(lib().xq_gemv_iq4nl_id(_ptr(y, 4 * used * rows, "y"),
                                  _ptr(slab, xq_iq4nl_bytes(n_experts * rows, K), "slab"),
                                  _ptr(xq, xq_q8k_bytes(xrows, K), "xq"),
                                  _ptr(sel, 4 * used, "sel"), n_experts, used, rows, K,
                                  x_stride_blocks, _stream(stream)),
           "xq_gemv_iq4nl_id")


def xq_repack_iq4nl(resident, file_blocks, n_blocks: int, block_base: int, bpr: int,
                    stream=None) -> None:
    rows = (block_base + n_blocks + bpr - 1) // bpr
    _check(lib().xq_repack_iq4nl(_ptr(resident, rows * iq4nl_row_bytes(bpr), "resident"),
                                 _ptr(file_blocks, 18 * n_blocks, "file_blocks"), n_blocks,
                                 block_base, bpr, _stream(stream)),
           "xq_repack_iq4nl")


def xq_repack_dword_prefix_launches() -> int:
    return lib().xq_repack_dword_prefix_launches()


def iq4nl_row_bytes(bpr: int) -> int:
    """Bytes of one resident IQ4_NL row of bpr blocks (any bpr >= 1)."""
    return ((2 * bpr + 3) // 4) * 4 + 16 * bpr


def xq_gemm_q4k_small_m_workspace_bytes(M: int, N: int, K: int) -> int:
    return lib().xq_gemm_q4k_small_m_workspace_bytes(M, N, K)


def xq_gemm_q4k_small_m(y, w, xq, M: int, N: int, K: int, workspace=None, stream=None) -> None:
    wp, wb = _workspace(workspace, xq_gemm_q4k_small_m_workspace_bytes(M, N, K))
    _check(lib().xq_gemm_q4k_small_m(_ptr(y, 4 * M * N, "y"), _ptr(w, xq_q4k_bytes(N, K), "w"),
                                     _ptr(xq, xq_q8k_bytes(M, K), "xq"), M, N, K, wp, wb,
                                     _stream(stream)),
           "xq_gemm_q4k_small_m")


def xq_gemm_q4k_small_m_noalloc(y, w, xq, M: int, N: int, K: int, stream=None) -> None:
    _check(lib().xq_gemm_q4k_small_m_noalloc(_ptr(y, 4 * M * N, "y"),
                                             _ptr(w, xq_q4k_bytes(N, K), "w"),
                                             _ptr(xq, xq_q8k_bytes(M, K), "xq"), M, N, K,
                                             _stream(stream)),
           "xq_gemm_q4k_small_m_noalloc")


def xq_gemm_q4k_id_workspace_bytes(n_tokens: int, n_used: int, n_experts: int) -> int:
    return lib().xq_gemm_q4k_id_workspace_bytes(n_tokens, n_used, n_experts)


def xq_gemm_q4k_id(y, slab, xq, ids, n_tokens: int, n_used: int, n_experts: int, rows: int,
                   K: int, x_per_slot: int = 0, workspace=None, stream=None) -> None:
    pairs = n_tokens * n_used
    xrows = pairs if x_per_slot else n_tokens
    wp, wb = _workspace(workspace, xq_gemm_q4k_id_workspace_bytes(n_tokens, n_used, n_experts))
    _check(lib().xq_gemm_q4k_id(_ptr(y, 4 * pairs * rows, "y"),
                                _ptr(slab, xq_q4k_bytes(n_experts * rows, K), "slab"),
                                _ptr(xq, xq_q8k_bytes(xrows, K), "xq"), _ptr(ids, 4 * pairs, "ids"),
                                n_tokens, n_used, n_experts, rows, K, x_per_slot, wp, wb,
                                _stream(stream)),
           "xq_gemm_q4k_id")


def xq_bench_sink_words(nbytes: int) -> int:
    return lib().xq_bench_sink_words(nbytes)


def xq_bench_stream_read(buf, nbytes: int, sink, stream=None) -> None:
    _check(lib().xq_bench_stream_read(_ptr(buf, nbytes, "buf"), nbytes,
                                      _ptr(sink, 4 * xq_bench_sink_words(nbytes), "sink"),
                                      _stream(stream)),
           "xq_bench_stream_read")
