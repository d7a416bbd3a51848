"""Bind-time repack of IQ4_NL file blocks into resident rows (xq_repack_iq4nl)
through the C ABI, against the oracle's repack byte for byte.

The route pair is the pages' ("25 — Writing XPU Kernels", section 25.7.2): a
chunk that starts and ends on rows (13 rows of 317 blocks from block 0) must
take the dword-prefix route once, and a chunk that ends mid-row (from block
2000, 317 blocks per row) must not; both must write the same bytes as the
oracle, and nothing outside their blocks.
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_decode_mat_amd as xq
import workloads as wl
from test_gpu_parity import _note, assert_close, dev, poisoned_f32, take_f32

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def _poisoned(rows, bpr):
    return np.full((rows, xq.iq4nl_row_bytes(bpr)), 0xAB, dtype=np.uint8)


def _gpu_repack(resident_np, blocks, n, base, bpr):
    res = dev(resident_np)
    xq.xq_repack_iq4nl(res, dev(blocks), n, base, bpr)
    torch.cuda.synchronize()
    return res.cpu().numpy().reshape(resident_np.shape)


def test_repack_row_aligned_takes_the_dword_route():
    rows, bpr = 13, 317
    blocks = wl.iq4nl_file_blocks(rows * bpr, wl.rng(9500))
    _note("repack row-aligned rows=%d bpr=%d" % (rows, bpr))
    before = xq.xq_repack_dword_prefix_launches()
    got = _gpu_repack(_poisoned(rows, bpr), blocks, rows * bpr, 0, bpr)
    assert xq.xq_repack_dword_prefix_launches() - before == 1
    want = oracle.repack_iq4nl(blocks, rows * bpr, 0, bpr, resident=_poisoned(rows, bpr))
    assert np.array_equal(got, want)
    assert not (got == 0xAB).all(axis=1).any()


def test_repack_mid_row_chunk_keeps_the_half_route():
    bpr, first, n = 317, 2000, 1121          # blocks 2000..3120 end inside row 9
    rows = (first + n + bpr - 1) // bpr
    blocks = wl.iq4nl_file_blocks(n, wl.rng(9501))
    _note("repack mid-row chunk first=%d n=%d bpr=%d" % (first, n, bpr))
    before = xq.xq_repack_dword_prefix_launches()
    got = _gpu_repack(_poisoned(rows, bpr), blocks, n, first, bpr)
    assert xq.xq_repack_dword_prefix_launches() == before
    want = oracle.repack_iq4nl(blocks, n, first, bpr, resident=_poisoned(rows, bpr))
    assert np.array_equal(got, want)


@pytest.mark.parametrize("rows,bpr,cuts", [
    (7, 9, [0, 5, 9, 27, 40, 63]),            # odd bpr: pads, chunks on and off rows
    (5, 128, [0, 128, 300, 640]),             # K = 4096 rows
    (4, 1, [0, 1, 3, 4]),                     # one block per row
])
def test_repack_in_chunks_writes_every_byte(rows, bpr, cuts):
    blocks = wl.iq4nl_file_blocks(rows * bpr, wl.rng(9502 + bpr))
    res = dev(_poisoned(rows, bpr))
    _note("repack chunks rows=%d bpr=%d" % (rows, bpr))
    for a, b in zip(cuts[:-1], cuts[1:]):
        xq.xq_repack_iq4nl(res, dev(blocks[a:b]), b - a, a, bpr)
    torch.cuda.synchronize()
    got = res.cpu().numpy().reshape(rows, -1)
    assert np.array_equal(got, oracle.repack_iq4nl(blocks, rows * bpr, 0, bpr))


def test_repacked_rows_feed_the_mat_vec():
    N, K = 300, 4096
    bpr = K // 32
    g = wl.rng(9510)
    blocks = wl.iq4nl_file_blocks(N * bpr, g)
    res = dev(_poisoned(N, bpr))
    _note("repack then mat-vec N=%d K=%d" % (N, K))
    xq.xq_repack_iq4nl(res, dev(blocks), N * bpr, 0, bpr)
    x = wl.activations(1, K, g)
    xqb = oracle.quantize_q8k(x)
    y = poisoned_f32(N)
    xq.xq_gemv_iq4nl(y, res, dev(xqb), N, K)
    got = take_f32(y, N)
    w = oracle.repack_iq4nl(blocks, N * bpr, 0, bpr)
    assert np.array_equal(res.cpu().numpy().reshape(N, -1), w)
    ref, T = oracle.gemv_iq4nl(w, xqb, N, K)
    assert_close(got, ref, T, "repacked mat-vec")


def test_repack_head_round_trip():
    """The full 128256 x 4096 head: resident rows -> file blocks (the inverse
    of the layout map, by slicing) -> GPU repack gives the rows back."""
    N, K = 128256, 4096
    bpr, prefix, row_bytes = wl.iq4nl_row_geometry(K)
    w = wl.iq4nl_weights(N, K, wl.rng(wl.SEEDS["iq4nl_head"]))
    blocks = np.empty((N, bpr, 18), dtype=np.uint8)
    blocks[:, :, 0:2] = w[:, 0:2 * bpr].reshape(N, bpr, 2)
    blocks[:, :, 2:] = w[:, prefix:].reshape(N, bpr, 16)
    _note("repack head round trip")
    res = torch.full((N * row_bytes,), 0xAB, dtype=torch.uint8, device="cuda")
    before = xq.xq_repack_dword_prefix_launches()
    xq.xq_repack_iq4nl(res, dev(blocks), N * bpr, 0, bpr)
    torch.cuda.synchronize()
    assert xq.xq_repack_dword_prefix_launches() - before == 1
    assert np.array_equal(res.cpu().numpy().reshape(N, row_bytes), w)


@pytest.mark.parametrize("bpr,first,n,route", [
    (1 << 16, 1 << 32, 1 << 16, 1),           # one whole row at global block 2^32: dword route
    ((1 << 16) + 1, (1 << 32) + 7, 1000, 0),  # mid-row, odd bpr (row 65535, blocks 8..1007)
], ids=["whole_row", "mid_row"])
def test_repack_past_2_32_blocks(bpr, first, n, route):
    """A chunk whose global block indices pass 2^32 takes the 64-bit-index
    kernel. The resident base the library takes is row 0 of the matrix and it
    writes only the chunk's rows, so only those rows are allocated here and
    the base passed is that allocation shifted back by its first row. The
    bytes equal the oracle's repack of the same blocks in a frame that starts
    at that row, and nothing outside the chunk's blocks is written."""
    row0 = first // bpr
    rows = (first + n + bpr - 1) // bpr - row0
    rb = xq.iq4nl_row_bytes(bpr)
    blocks = wl.iq4nl_file_blocks(n, wl.rng(9520 + route))
    res = dev(_poisoned(rows, bpr))
    src = dev(blocks)
    _note("repack past 2^32 blocks first=%d n=%d bpr=%d" % (first, n, bpr))
    before = xq.xq_repack_dword_prefix_launches()
    st = xq.lib().xq_repack_iq4nl(res.data_ptr() - row0 * rb, src.data_ptr(), n, first, bpr,
                                  torch.cuda.current_stream().cuda_stream)
    assert st == xq.XQ_OK, xq.xq_last_error()
    torch.cuda.synchronize()
    assert xq.xq_repack_dword_prefix_launches() - before == route
    got = res.cpu().numpy().reshape(rows, rb)
    want = oracle.repack_iq4nl(blocks, n, first - row0 * bpr, bpr, resident=_poisoned(rows, bpr))
    assert np.array_equal(got, want)


@pytest.mark.parametrize("rows,bpr,cuts", [
    (7, 9, [0, 5, 9, 27, 40, 63]),            # odd bpr: pads, chunks on and off rows
    (3, 1100, [0, 1100, 1700, 3300]),         # tiles of 512 blocks inside and across rows
])
def test_repack_unaligned_source_takes_the_direct_route(rows, bpr, cuts):
    # A 16-byte aligned source is staged through LDS in tiles of 512 blocks;
    # any other source (2-byte aligned at least) is read directly as halves.
    # Both must write the oracle's bytes.
    blocks = wl.iq4nl_file_blocks(rows * bpr, wl.rng(9540 + bpr))
    _note("repack unaligned source rows=%d bpr=%d" % (rows, bpr))
    for offset in (2, 0):
        res = dev(_poisoned(rows, bpr))
        for a, b in zip(cuts[:-1], cuts[1:]):
            buf = torch.zeros(18 * (b - a) + 16, dtype=torch.uint8, device="cuda")
            buf[offset:offset + 18 * (b - a)] = dev(blocks[a:b].reshape(-1))
            xq.xq_repack_iq4nl(res, buf.data_ptr() + offset, b - a, a, bpr)
            torch.cuda.synchronize()
        got = res.cpu().numpy().reshape(rows, -1)
        assert np.array_equal(got, oracle.repack_iq4nl(blocks, rows * bpr, 0, bpr)), offset
