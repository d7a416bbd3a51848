"""Q4_0 x q8_K mat-vec (xq_gemv_q4_0) against the oracle through the C ABI.

Bars as for IQ4_NL: f32 outputs within 1e-5 * T of the oracle; per-block
integer partials D = sum (nibble-8)*code bit-exact, isolated through the entry
point with unit scales against an activation whose only nonzero 32-block has
q8_K scale 1; outputs poisoned and canaried.
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


Q40_SHAPES = [
    ("square_4096x4096", 4096, 4096, 8201),
    ("head_128256x4096", 128256, 4096, 8202),
    ("n5_k256", 5, 256, 8203),
    ("n33_k768", 33, 768, 8204),
    ("n1000_k2304", 1000, 2304, 8205),
    ("n8193_k2048", 8193, 2048, 8206),
    ("n16_k14336_staged", 16, 14336, 8207),
    ("n300_k8192_four_units", 300, 8192, 8208),
    ("n70_k10240_five_units", 70, 10240, 8209),
    ("n20000_k512_two_rows_per_wave", 20000, 512, 8210),
    ("n64_k49152_staged_max", 64, 49152, 8211),
    ("n40_k53248_unstaged", 40, 53248, 8212),
    ("n500_k6144_three_units", 500, 6144, 8213),
    ("n90_k12288_six_units", 90, 12288, 8214),
    ("n50_k16384_eight_units", 50, 16384, 8215),
]


@pytest.mark.parametrize("name,N,K,seed", Q40_SHAPES, ids=[s[0] for s in Q40_SHAPES])
def test_gemv_q4_0(name, N, K, seed):
    g = wl.rng(seed)
    w = wl.iq4nl_weights(N, K, g)     # the shared row shape: any payload is a valid Q4_0 row
    x = wl.activations(1, K, g)
    xqb = oracle.quantize_q8k(x)
    _note("gemv_q4_0 %s N=%d K=%d" % (name, N, K))
    y = poisoned_f32(N)
    xq.xq_gemv_q4_0(y, dev(w), dev(xqb), N, K)
    got = take_f32(y, N)
    ref, T = oracle.gemv_q4_0(w, xqb, N, K)
    assert_close(got, ref, T, name)


@pytest.mark.parametrize("N,K,blocks", [(4096, 4096, [0, 7, 8, 63, 64, 127]), (33, 768, [0, 5, 23]),
                                        (16, 14336, [0, 200, 447])])
def test_q4_0_partials_bit_exact(N, K, blocks):
    g = wl.rng(8300 + N)
    w = wl.iq4nl_unit_scale_weights(N, K, g)
    wd = dev(w)
    for c in blocks:
        x = wl.isolating_activation(1, K, g, c // 8, width=32, offset=32 * (c % 8))
        xqb = oracle.quantize_q8k(x)
        D = oracle.q4_0_partials(w, xqb, N, K)
        _note("gemv_q4_0 partial block %d (N=%d K=%d)" % (c, N, K))
        y = poisoned_f32(N)
        xq.xq_gemv_q4_0(y, wd, dev(xqb), N, K)
        got = take_f32(y, N)
        assert np.array_equal(got, D[:, c].astype(np.float64)), c


def test_q4_0_file_blocks_through_the_repack():
    """Q4_0 file blocks share IQ4_NL's 18-byte shape: the repack serves both."""
    N, K = 257, 2048
    bpr = K // 32
    g = wl.rng(8400)
    blocks = wl.iq4nl_file_blocks(N * bpr, g)
    res = torch.empty(N * xq.iq4nl_row_bytes(bpr), dtype=torch.uint8, device="cuda")
    _note("q4_0 repack then mat-vec")
    xq.xq_repack_iq4nl(res, dev(blocks), N * bpr, 0, bpr)
    xqb = oracle.quantize_q8k(wl.activations(1, K, g))
    y = poisoned_f32(N)
    xq.xq_gemv_q4_0(y, res, dev(xqb), N, K)
    got = take_f32(y, N)
    ref, T = oracle.gemv_q4_0(oracle.repack_iq4nl(blocks, N * bpr, 0, bpr), xqb, N, K)
    assert_close(got, ref, T, "q4_0 from file blocks")
