"""xq_gemm_q4k_small_m_noalloc (the product for callers that cannot allocate)
against xq_gemm_q4k_small_m with a caller workspace, through the C ABI: two
calls in a row, the second with a smaller input, both on split-K plans (so the
library's static scratch carries the partials and counters), then a shape
that splits nothing. Each output equals the workspace entry point's bit for
bit and is within the f32 bar of the oracle."""
import numpy as np
import pytest
import torch

import oracle
import quantized_decode_mat_amd as xq
import workloads as wl
from test_gpu_parity import _note, assert_close, dev, gemm_workspace, poisoned_f32, take_f32

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def _case(M, N, K, seed):
    g = wl.rng(seed)
    w = wl.q4k_weights(N, K, g)
    xqb = oracle.quantize_q8k(wl.activations(M, K, g))
    return w, xqb


def _both(w, xqb, M, N, K):
    wd, xd = dev(w), dev(xqb)
    y_ws = poisoned_f32(M * N)
    xq.xq_gemm_q4k_small_m(y_ws, wd, xd, M, N, K, workspace=gemm_workspace(M, N, K))
    want = take_f32(y_ws, M * N).reshape(M, N)
    y_na = poisoned_f32(M * N)
    xq.xq_gemm_q4k_small_m_noalloc(y_na, wd, xd, M, N, K)
    got = take_f32(y_na, M * N).reshape(M, N)
    return got, want


def test_noalloc_equals_workspace_entry_point():
    # 32 tokens x 4096 x 14336: 64 tiles of 16 x 128, each split 8 ways
    # (4.1 MB of scratch); then 9 tokens x 1000 x 4352: 8 tiles split 4 ways.
    for M, N, K, seed, full in ((32, 4096, 14336, 8801, False), (9, 1000, 4352, 8802, True)):
        need = xq.xq_gemm_q4k_small_m_workspace_bytes(M, N, K)
        assert 0 < need <= xq.XQ_NOALLOC_SCRATCH_BYTES, need
        w, xqb = _case(M, N, K, seed)
        _note("noalloc %dx%dx%d" % (M, N, K))
        got, want = _both(w, xqb, M, N, K)
        assert np.array_equal(got, want), "%dx%dx%d: %d outputs differ" % (
            M, N, K, int((got != want).sum()))
        if full:
            ref, T = oracle.gemm_q4k(w, xqb, M, N, K)
            assert_close(got.reshape(-1), ref.reshape(-1), T.reshape(-1), "noalloc full")
        else:
            s = wl.rng(seed + 1)
            ms = np.concatenate([s.integers(0, M, 600), [0, M - 1, 15, 16]])
            ns = np.concatenate([s.integers(0, N, 600), [0, N - 1, 127, 128]])
            ref, T = oracle.gemm_q4k(w, xqb, M, N, K, ms, ns)
            assert_close(got[ms, ns], ref, T, "noalloc sampled")
            ref, T = oracle.gemv_q4k(w, xqb[M - 1], N, K)
            assert_close(got[M - 1], ref, T, "noalloc last row")
    # A shape that splits nothing takes no scratch and still matches.
    M, N, K = 20, 256, 1024
    assert xq.xq_gemm_q4k_small_m_workspace_bytes(M, N, K) == 0
    w, xqb = _case(M, N, K, 8803)
    got, want = _both(w, xqb, M, N, K)
    assert np.array_equal(got, want)
    ref, T = oracle.gemm_q4k(w, xqb, M, N, K)
    assert_close(got.reshape(-1), ref.reshape(-1), T.reshape(-1), "noalloc unsplit")
