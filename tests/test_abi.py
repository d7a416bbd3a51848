"""The C ABI on the host: the library loads, exports every function that
include/xq.h declares, sizes its layouts, and refuses bad arguments before any
HIP call (no GPU is touched by these tests)."""
import ctypes
import os
import re

import pytest

import quantized_decode_mat_amd as xq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "xq.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(xq_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    L = xq.lib()
    names = _declared()
    assert len(names) >= 11
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(xq.EXPORTS)


def test_layout_sizes():
    assert xq.xq_q8k_bytes(1, 4096) == 16 * 320
    assert xq.xq_q8k_bytes(512, 4096) == 2621440
    assert xq.xq_q4k_bytes(14336, 4096) == 33030144
    assert xq.xq_q4k_bytes(256, 1024) == 147456
    assert xq.xq_iq4nl_bytes(4096, 4096) == 9437184
    assert xq.xq_iq4nl_bytes(128256, 4096) == 295501824
    assert xq.xq_q8k_bytes(1, 1000) == 0 and xq.xq_q4k_bytes(0, 256) == 0


def test_workspace_sizes():
    """The bytes each workspace query gives, worked out from the plans they
    describe: a fixed region of 768 counter lines of 128 bytes (96 KiB, the
    same for every plan, so a reused workspace never reads another plan's
    partials as counters) then one partial slot per split workgroup (8 KiB on
    the 16-token tile, 32 KiB on the 64-token one); one counter line per q8_K
    block of the fused tail; the expert map's descriptors, pairs and two
    counts."""
    ws = xq.xq_gemm_q4k_small_m_workspace_bytes
    assert ws(1, 14336, 4096) == 0                 # the mat-vec
    assert ws(3, 14336, 4096) == 0                 # the batched mat-vec
    assert ws(512, 14336, 4096) == 0               # whole tiles only
    assert ws(16, 14336, 4096) == 0                # the wave-split tile (no hand-off)
    assert ws(4, 8192, 4096) == 0 and ws(7, 4096, 4096) == 0  # the batched mat-vec
    assert ws(9, 4096, 4096) > 0 and ws(7, 2048, 8192) > 0     # split MFMA tiles
    # 4 tokens x 14336 rows x 32 blocks: 112 tiles of 16 x 128, 4 splits each
    assert ws(4, 14336, 8192) == 768 * 128 + 112 * 4 * 8192
    # 16 tokens x 4096 rows x 56 blocks: 32 tiles of 16 x 128, 8 splits each
    assert ws(16, 4096, 14336) == 768 * 128 + 32 * 8 * 8192
    # 320 tokens x 14336 rows x 16 blocks: 560 tiles, 512 whole + 48 in 4 splits
    assert ws(320, 14336, 4096) == 768 * 128 + 48 * 4 * 32768
    assert ws(0, 8, 256) == 0 and ws(16, 4096, 1000) == 0
    # shapes the entry point refuses (sizes past 2^30 rows or 2 GiB) need nothing
    assert ws(2 ** 40, 4096, 4096) == 0 and ws(16, 2 ** 40, 4096) == 0
    assert ws(16, 2 ** 30, 2 ** 38) == 0 and ws(2 ** 30, 2 ** 30, 2 ** 62) == 0
    assert xq.xq_gemv_q4k_q8k_workspace_bytes(14336) == 56 * 128
    assert xq.xq_gemv_q4k_q8k_workspace_bytes(300) == 0
    # 16 pairs over 6 experts: 7 whole-tile and 14 small-tile descriptors of
    # 16 B, 16 pair indices, then two counts in a 16-byte slot
    assert xq.xq_gemm_q4k_id_workspace_bytes(8, 2, 6) == 7 * 16 + 14 * 16 + 64 + 16
    assert xq.xq_gemm_q4k_id_workspace_bytes(0, 2, 6) == 0
    # the largest split plan stays within 16 MiB + 96 KiB
    worst = max(ws(M, N, K) for M in (17, 33, 48, 64, 100, 200, 320, 400, 700)
                for N in (128, 1000, 4096, 14336, 30000) for K in (1024, 4096, 14336))
    assert 0 < worst <= (16 << 20) + (96 << 10)


def test_status_names():
    assert [xq.xq_status_name(s) for s in range(6)] == [
        "XQ_OK", "XQ_E_NULL", "XQ_E_SHAPE", "XQ_E_ALIGN", "XQ_E_DEVICE", "XQ_E_LAUNCH"]


# Fake device addresses: the gates tested here refuse before anything is
# dereferenced or launched.
A16 = 0x7F0000000000
A4 = A16 + 4
A1 = A16 + 1
W256 = 0x7F0000100000   # a 256-byte-aligned fake workspace
BIG = 1 << 30           # its claimed size


def _call(name, *args):
    L = xq.lib()
    s = getattr(L, name)(*args)
    return s, L.xq_last_error().decode()


@pytest.mark.parametrize("args,status,text", [
    ((0, A16, 1, 256, None), xq.XQ_E_NULL, "xq is NULL"),
    ((A16, 0, 1, 256, None), xq.XQ_E_NULL, "x is NULL"),
    ((A16, A16, 0, 256, None), xq.XQ_E_SHAPE, "rows=0"),
    ((A16, A16, 1, 1000, None), xq.XQ_E_SHAPE, "K=1000"),
    ((A16, A16, 1, 0, None), xq.XQ_E_SHAPE, "K=0"),
    ((A16, A16, 2 ** 40, 256, None), xq.XQ_E_SHAPE, "exceeds"),
    ((A4, A16, 1, 256, None), xq.XQ_E_ALIGN, "xq not 16-byte"),
    ((A16, A1, 1, 256, None), xq.XQ_E_ALIGN, "x not 4-byte"),
])
def test_quantize_refusals(args, status, text):
    s, err = _call("xq_quantize_q8k", *args)
    assert s == status and text in err


@pytest.mark.parametrize("fn", ["xq_gemv_q4k", "xq_gemv_iq4nl", "xq_gemv_q4_0"])
@pytest.mark.parametrize("args,status,text", [
    ((0, A16, A16, 8, 256, None), xq.XQ_E_NULL, "y is NULL"),
    ((A16, 0, A16, 8, 256, None), xq.XQ_E_NULL, "w is NULL"),
    ((A16, A16, 0, 8, 256, None), xq.XQ_E_NULL, "xq is NULL"),
    ((A16, A16, A16, 0, 256, None), xq.XQ_E_SHAPE, "N=0"),
    ((A16, A16, A16, 2 ** 30 + 1, 256, None), xq.XQ_E_SHAPE, "N=1073741825"),
    ((A16, A16, A16, 8, 300, None), xq.XQ_E_SHAPE, "K=300"),
    ((A16, A16, A16, 8, 1048576 + 256, None), xq.XQ_E_SHAPE, "above the largest"),
    ((A1, A16, A16, 8, 256, None), xq.XQ_E_ALIGN, "y not 4-byte"),
    ((A16, A4, A16, 8, 256, None), xq.XQ_E_ALIGN, "w not 16-byte"),
    ((A16, A16, A4, 8, 256, None), xq.XQ_E_ALIGN, "xq not 16-byte"),
])
def test_gemv_refusals(fn, args, status, text):
    s, err = _call(fn, *args)
    assert s == status and text in err


@pytest.mark.parametrize("args,status,text", [
    ((0, A16, A16, 4, 8, 256, None, 0, None), xq.XQ_E_NULL, "y is NULL"),
    ((A16, A16, A16, 0, 8, 256, None, 0, None), xq.XQ_E_SHAPE, "M=0"),
    ((A16, A16, A16, 4, 0, 256, None, 0, None), xq.XQ_E_SHAPE, "N=0"),
    ((A16, A16, A16, 4, 8, 257, None, 0, None), xq.XQ_E_SHAPE, "K=257"),
    ((A16, A4, A16, 4, 8, 256, None, 0, None), xq.XQ_E_ALIGN, "w not 16-byte"),
    ((A16, A16, A1, 4, 8, 256, None, 0, None), xq.XQ_E_ALIGN, "xq not 16-byte"),
    ((A16, A16, A16, 2 ** 20, 8, 2048, None, 0, None), xq.XQ_E_SHAPE, "reaches 2 GiB"),
    ((A16, A16, A16, 4, 2 ** 21, 2048, None, 0, None), xq.XQ_E_SHAPE, "reaches 2 GiB"),
    # rows x bytes per row past int64: refused by the size gate, not wrapped past it
    ((A16, A16, A16, 2 ** 30, 1, 2 ** 38, None, 0, None), xq.XQ_E_SHAPE,
     "xq of M=1073741824 rows reaches 2 GiB"),
    ((A16, A16, A16, 1, 2 ** 30, 2 ** 38, None, 0, None), xq.XQ_E_SHAPE, "reaches 2 GiB"),
])
def test_gemm_refusals(args, status, text):
    s, err = _call("xq_gemm_q4k_small_m", *args)
    assert s == status and text in err


# 16 tokens x 4096 x 14336 splits K: it needs a workspace.
_SPLIT = (A16, A16, A16, 16, 4096, 14336)
_SPLIT_NEED = 768 * 128 + 32 * 8 * 8192


@pytest.mark.parametrize("ws,nbytes,status,text", [
    (None, 0, xq.XQ_E_NULL, "workspace is NULL"),
    (None, BIG, xq.XQ_E_NULL, "workspace is NULL"),
    (W256, _SPLIT_NEED - 1, xq.XQ_E_SHAPE, "below the %d bytes" % _SPLIT_NEED),
    (W256 + 128, BIG, xq.XQ_E_ALIGN, "workspace not 256-byte"),
])
def test_gemm_workspace_refusals(ws, nbytes, status, text):
    s, err = _call("xq_gemm_q4k_small_m", *_SPLIT, ws, nbytes, None)
    assert s == status and text in err, (s, err)


def test_noalloc_scratch_limit():
    """The no-allocation product holds 8 MiB of split-K scratch: every plan of
    up to 32 tokens fits, and a shape that needs more is refused by name
    before the device gate (48 tokens x 14336 x 4096: 112 tiles of 64 x 128
    split four ways, 448 slots of 32 KiB after the 96 KiB of counters)."""
    ws = xq.xq_gemm_q4k_small_m_workspace_bytes
    assert xq.XQ_NOALLOC_SCRATCH_BYTES == 8 << 20
    assert max(ws(M, N, K) for M in range(2, 33) for N in (100, 1000, 4096, 14336, 100000)
               for K in (256, 1024, 4096, 14336, 49152)) <= xq.XQ_NOALLOC_SCRATCH_BYTES
    need = ws(48, 14336, 4096)
    assert need == 768 * 128 + 448 * 32768 > xq.XQ_NOALLOC_SCRATCH_BYTES
    s, err = _call("xq_gemm_q4k_small_m_noalloc", A16, A16, A16, 48, 14336, 4096, None)
    assert s == xq.XQ_E_SHAPE and "above the 8388608 bytes" in err, err
    s, err = _call("xq_gemm_q4k_small_m_noalloc", 0, A16, A16, 48, 14336, 4096, None)
    assert s == xq.XQ_E_NULL and "y is NULL" in err
    s, err = _call("xq_gemm_q4k_small_m_noalloc", A16, A4, A16, 32, 4096, 14336, None)
    assert s == xq.XQ_E_ALIGN and "w not 16-byte" in err


def test_gemm_workspace_not_needed_may_be_null():
    """A shape that splits nothing passes the workspace gates with NULL and
    stops only at the device gate (no GPU here) or runs (GPU)."""
    import torch
    if torch.cuda.device_count() != 0:
        pytest.skip("a GPU is visible; this gate is exercised only where none is")
    s, err = _call("xq_gemm_q4k_small_m", A16, A16, A16, 512, 14336, 4096, None, 0, None)
    assert s == xq.XQ_E_DEVICE, err
    s, err = _call("xq_gemm_q4k_small_m", *_SPLIT, W256, _SPLIT_NEED, None)
    assert s == xq.XQ_E_DEVICE, err


@pytest.mark.parametrize("fn", ["xq_gemv_q4k_id", "xq_gemv_iq4nl_id"])
@pytest.mark.parametrize("args,status,text", [
    ((0, A16, A16, A16, 6, 3, 64, 2048, 0, None), xq.XQ_E_NULL, "y is NULL"),
    ((A16, 0, A16, A16, 6, 3, 64, 2048, 0, None), xq.XQ_E_NULL, "slab is NULL"),
    ((A16, A16, 0, A16, 6, 3, 64, 2048, 0, None), xq.XQ_E_NULL, "xq is NULL"),
    ((A16, A16, A16, 0, 6, 3, 64, 2048, 0, None), xq.XQ_E_NULL, "sel is NULL"),
    ((A16, A16, A16, A16, 0, 3, 64, 2048, 0, None), xq.XQ_E_SHAPE, "n_experts=0"),
    ((A16, A16, A16, A16, 6, 0, 64, 2048, 0, None), xq.XQ_E_SHAPE, "used=0"),
    ((A16, A16, A16, A16, 6, 65536, 64, 2048, 0, None), xq.XQ_E_SHAPE, "used=65536"),
    ((A16, A16, A16, A16, 6, 3, 0, 2048, 0, None), xq.XQ_E_SHAPE, "rows=0"),
    ((A16, A16, A16, A16, 2 ** 20, 3, 2 ** 11, 2048, 0, None), xq.XQ_E_SHAPE, "above 2^30"),
    ((A16, A16, A16, A16, 6, 3, 64, 2000, 0, None), xq.XQ_E_SHAPE, "K=2000"),
    ((A16, A16, A16, A16, 6, 3, 64, 2048, 3, None), xq.XQ_E_SHAPE, "x_stride_blocks=3"),
    ((A4, A16, A16, A16, 6, 3, 64, 2048, 0, None), xq.XQ_E_ALIGN, None),
    ((A16, A4, A16, A16, 6, 3, 64, 2048, 0, None), xq.XQ_E_ALIGN, "slab not 16-byte"),
    ((A16, A16, A4, A16, 6, 3, 64, 2048, 8, None), xq.XQ_E_ALIGN, "xq not 16-byte"),
    ((A16, A16, A16, A1, 6, 3, 64, 2048, 0, None), xq.XQ_E_ALIGN, "sel not 4-byte"),
])
def test_id_refusals(fn, args, status, text):
    s, err = _call(fn, *args)
    if text is None:  # a 4-byte-aligned y passes its gate; the next gate decides
        assert s != xq.XQ_OK
        return
    assert s == status and text in err, (s, err)


@pytest.mark.parametrize("args,status,text", [
    ((0, A16, A16, A16, 8, 2, 6, 64, 2048, 0, W256, BIG, None), xq.XQ_E_NULL, "y is NULL"),
    ((A16, 0, A16, A16, 8, 2, 6, 64, 2048, 0, W256, BIG, None), xq.XQ_E_NULL, "slab is NULL"),
    ((A16, A16, 0, A16, 8, 2, 6, 64, 2048, 0, W256, BIG, None), xq.XQ_E_NULL, "xq is NULL"),
    ((A16, A16, A16, 0, 8, 2, 6, 64, 2048, 0, W256, BIG, None), xq.XQ_E_NULL, "ids is NULL"),
    ((A16, A16, A16, A16, 8, 0, 6, 64, 2048, 0, W256, BIG, None), xq.XQ_E_SHAPE, "n_used=0"),
    ((A16, A16, A16, A16, 0, 2, 6, 64, 2048, 0, W256, BIG, None), xq.XQ_E_SHAPE, "n_tokens*n_used"),
    ((A16, A16, A16, A16, 2 ** 19 + 1, 2, 6, 64, 2048, 0, W256, BIG, None), xq.XQ_E_SHAPE,
     "n_tokens*n_used"),
    ((A16, A16, A16, A16, 8, 2, 0, 64, 2048, 0, W256, BIG, None), xq.XQ_E_SHAPE, "n_experts=0"),
    ((A16, A16, A16, A16, 8, 2, 1025, 64, 2048, 0, W256, BIG, None), xq.XQ_E_SHAPE, "n_experts=1025"),
    ((A16, A16, A16, A16, 8, 2, 6, 0, 2048, 0, W256, BIG, None), xq.XQ_E_SHAPE, "rows=0"),
    ((A16, A16, A16, A16, 8, 2, 6, 64, 2000, 0, W256, BIG, None), xq.XQ_E_SHAPE, "K=2000"),
    ((A16, A16, A16, A16, 8, 2, 6, 64, 2048, 2, W256, BIG, None), xq.XQ_E_SHAPE, "x_per_slot=2"),
    ((A16, A16, A16, A16, 8, 2, 6, 2 ** 21, 2048, 0, W256, BIG, None), xq.XQ_E_SHAPE, "reaches 2 GiB"),
    ((A16, A16, A16, A16, 2 ** 19, 2, 6, 64, 4096, 1, W256, BIG, None), xq.XQ_E_SHAPE, "reaches 2 GiB"),
    ((A16 + 2, A16, A16, A16, 8, 2, 6, 64, 2048, 0, W256, BIG, None), xq.XQ_E_ALIGN, "y not 4-byte"),
    ((A16, A4, A16, A16, 8, 2, 6, 64, 2048, 0, W256, BIG, None), xq.XQ_E_ALIGN, "slab not 16-byte"),
    ((A16, A16, A4, A16, 8, 2, 6, 64, 2048, 0, W256, BIG, None), xq.XQ_E_ALIGN, "xq not 16-byte"),
    ((A16, A16, A16, A1, 8, 2, 6, 64, 2048, 0, W256, BIG, None), xq.XQ_E_ALIGN, "ids not 4-byte"),
    ((A16, A16, A16, A16, 8, 2, 6, 2 ** 30, 2 ** 38, 0, W256, BIG, None), xq.XQ_E_SHAPE,
     "one expert of rows=1073741824 reaches 2 GiB"),
])
def test_gemm_id_refusals(args, status, text):
    s, err = _call("xq_gemm_q4k_id", *args)
    assert s == status and text in err, (s, err)


@pytest.mark.parametrize("ws,nbytes,status,text", [
    (None, BIG, xq.XQ_E_NULL, "workspace is NULL"),
    (W256, 7 * 16 + 14 * 16 + 64 + 15, xq.XQ_E_SHAPE, "below the 416 bytes"),
    (W256 + 16, BIG, xq.XQ_E_ALIGN, "workspace not 256-byte"),
])
def test_gemm_id_workspace_refusals(ws, nbytes, status, text):
    s, err = _call("xq_gemm_q4k_id", A16, A16, A16, A16, 8, 2, 6, 64, 2048, 0, ws, nbytes, None)
    assert s == status and text in err, (s, err)


@pytest.mark.parametrize("args,status,text", [
    ((0, A16, A16, A16, 512, 4096, W256, BIG, None), xq.XQ_E_NULL, "y is NULL"),
    ((A16, 0, A16, A16, 512, 4096, W256, BIG, None), xq.XQ_E_NULL, "yq is NULL"),
    ((A16, A16, 0, A16, 512, 4096, W256, BIG, None), xq.XQ_E_NULL, "w is NULL"),
    ((A16, A16, A16, 0, 512, 4096, W256, BIG, None), xq.XQ_E_NULL, "xq is NULL"),
    ((A16, A16, A16, A16, 300, 4096, W256, BIG, None), xq.XQ_E_SHAPE, "N=300"),
    ((A16, A16, A16, A16, 0, 4096, W256, BIG, None), xq.XQ_E_SHAPE, "N=0"),
    ((A16, A16, A16, A16, 2 ** 22 + 256, 4096, W256, BIG, None), xq.XQ_E_SHAPE, "N=4194560"),
    ((A16, A16, A16, A16, 512, 4000, W256, BIG, None), xq.XQ_E_SHAPE, "K=4000"),
    ((A1, A16, A16, A16, 512, 4096, W256, BIG, None), xq.XQ_E_ALIGN, "y not 4-byte"),
    ((A16, A4, A16, A16, 512, 4096, W256, BIG, None), xq.XQ_E_ALIGN, "yq not 16-byte"),
    ((A16, A16, A4, A16, 512, 4096, W256, BIG, None), xq.XQ_E_ALIGN, "w not 16-byte"),
    ((A16, A16, A16, A4, 512, 4096, W256, BIG, None), xq.XQ_E_ALIGN, "xq not 16-byte"),
])
def test_gemv_q8k_refusals(args, status, text):
    s, err = _call("xq_gemv_q4k_q8k", *args)
    assert s == status and text in err, (s, err)


@pytest.mark.parametrize("ws,nbytes,status,text", [
    (None, BIG, xq.XQ_E_NULL, "workspace is NULL"),
    (W256, 255, xq.XQ_E_SHAPE, "below the 256 bytes"),
    (W256 + 64, BIG, xq.XQ_E_ALIGN, "workspace not 256-byte"),
])
def test_gemv_q8k_workspace_refusals(ws, nbytes, status, text):
    s, err = _call("xq_gemv_q4k_q8k", A16, A16, A16, A16, 512, 4096, ws, nbytes, None)
    assert s == status and text in err, (s, err)



@pytest.mark.parametrize("args,status,text", [
    ((0, A16, 10, 0, 9, None), xq.XQ_E_NULL, "resident is NULL"),
    ((A16, 0, 10, 0, 9, None), xq.XQ_E_NULL, "file_blocks is NULL"),
    ((A16, A16, 0, 0, 9, None), xq.XQ_E_SHAPE, "n_blocks=0"),
    ((A16, A16, 2 ** 29 + 1, 0, 9, None), xq.XQ_E_SHAPE, "n_blocks=536870913"),
    ((A16, A16, 10, -1, 9, None), xq.XQ_E_SHAPE, "block_base=-1"),
    ((A16, A16, 10, 0, 0, None), xq.XQ_E_SHAPE, "bpr=0"),
    ((A16, A16, 10, 0, 2 ** 24 + 1, None), xq.XQ_E_SHAPE, "bpr=16777217"),
    ((A16 + 2, A16, 10, 0, 9, None), xq.XQ_E_ALIGN, "resident not 4-byte"),
    ((A16, A1, 10, 0, 9, None), xq.XQ_E_ALIGN, "file_blocks not 2-byte"),
])
def test_repack_refusals(args, status, text):
    s, err = _call("xq_repack_iq4nl", *args)
    assert s == status and text in err, (s, err)


def test_refusal_raises_in_binding():
    with pytest.raises(xq.XQError) as e:
        xq.xq_gemv_q4k(A16, A16, A16, 8, 1000)
    assert e.value.status == xq.XQ_E_SHAPE and "K=1000" in str(e.value)


def test_binding_refuses_host_and_short_tensors():
    import torch
    with pytest.raises(ValueError):
        xq.xq_gemv_q4k(torch.zeros(8), A16, A16, 8, 256)   # host tensor


def test_device_gate_without_gpu():
    """With no HIP device visible, a call whose other arguments pass is refused
    at the device gate, before any launch."""
    import torch
    if torch.cuda.device_count() != 0:
        pytest.skip("a GPU is visible; this gate is exercised only where none is")
    s, err = _call("xq_gemv_q4k", A16, A16, A16, 8, 256, None)
    assert s == xq.XQ_E_DEVICE, err
    # 4-byte alignment is enough for the quantizer's x and the fused tail's y
    s, err = _call("xq_quantize_q8k", A16, A4, 1, 256, None)
    assert s == xq.XQ_E_DEVICE, err
    s, err = _call("xq_gemv_q4k_q8k", A4, A16, A16, A16, 512, 4096, W256, BIG, None)
    assert s == xq.XQ_E_DEVICE, err
