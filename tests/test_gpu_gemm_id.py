"""Grouped small-M product (xq_gemm_q4k_id) through the C ABI.

Every (token, slot) pair is held to the oracle's mat-vec of its expert's rows
against its own q8_K row (|y - ref| <= 1e-5 * T); outputs of out-of-range
selections must be NaN and nothing else may be; block partials are bit-exact
through the entry point (unit-scale isolation weights); and because each output
is computed from its own pair alone, permuting the tokens permutes the outputs
bit for bit (the pairs land in different tiles).
"""
import numpy as np
import pytest
import torch

import oracle
import quantized_decode_mat_amd as xq
import workloads as wl
from test_gpu_parity import _note, assert_close, dev, poisoned_f32, take_f32, zeroed_workspace

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def _slab(E, rows, K, seed):
    parts = [wl.q4k_weights(rows, K, wl.rng(seed + 31 * e)) for e in range(E)]
    return np.concatenate([p.reshape(rows, -1) for p in parts], axis=0)


def _run(slab, xqb, ids, E, rows, K, per_slot):
    T, U = ids.shape
    y = poisoned_f32(T * U * rows)
    ws = zeroed_workspace(xq.xq_gemm_q4k_id_workspace_bytes(T, U, E))
    xq.xq_gemm_q4k_id(y, dev(slab), dev(xqb), dev(ids.astype(np.int32)), T, U, E, rows, K,
                      per_slot, workspace=ws)
    return take_f32(y, T * U * rows).reshape(T, U, rows)


def _check(Y, slab, xqb, ids, E, rows, K, per_slot, pairs=None):
    T, U = ids.shape
    todo = [(t, k) for t in range(T) for k in range(U)] if pairs is None else pairs
    for t, k in todo:
        e = int(ids[t, k])
        got = Y[t, k]
        if not 0 <= e < E:
            assert np.isnan(got).all(), (t, k, e)
            continue
        assert not np.isnan(got).any(), (t, k)
        xrow = xqb[t * U + k] if per_slot else xqb[t]
        ref, Tm = oracle.gemv_q4k(slab[e * rows:(e + 1) * rows], xrow, rows, K)
        assert_close(got, ref, Tm, "pair (%d, %d) expert %d" % (t, k, e))


def _top_k(T, U, E, g):
    return np.stack([g.choice(E, size=U, replace=False) for _ in range(T)]).astype(np.int32)


def test_gemm_id_six_experts_three_slots():
    E, rows, K, T, U = 6, 64, 2048, 5, 3
    slab = _slab(E, rows, K, 9500)
    g = wl.rng(9501)
    xqb = oracle.quantize_q8k(wl.activations(T, K, g))
    ids = np.array([[4, 0, 3], [1, 4, 2], [0, 5, 3], [2, 1, 4], [3, 0, 5]], dtype=np.int32)
    _note("gemm id six experts")
    Y = _run(slab, xqb, ids, E, rows, K, 0)
    assert (Y != 0).any()
    _check(Y, slab, xqb, ids, E, rows, K, 0)


@pytest.mark.parametrize("T,U,E,rows,K,per_slot,seed", [
    (200, 2, 8, 200, 4096, 0, 9600),     # top-2 of 8, rows not a multiple of 128
    (150, 4, 16, 128, 1024, 1, 9610),    # a q8_K row per slot (down projection)
    (40, 8, 64, 96, 2048, 0, 9620),      # many experts, most with a few pairs
])
def test_gemm_id_routed(T, U, E, rows, K, per_slot, seed):
    slab = _slab(E, rows, K, seed)
    g = wl.rng(seed + 1)
    xrows = T * U if per_slot else T
    xqb = oracle.quantize_q8k(wl.activations(xrows, K, g))
    ids = _top_k(T, U, E, g)
    _note("gemm id routed T=%d U=%d E=%d rows=%d K=%d per_slot=%d" % (T, U, E, rows, K, per_slot))
    Y = _run(slab, xqb, ids, E, rows, K, per_slot)
    s = wl.rng(seed + 2)
    pairs = sorted({(int(s.integers(T)), int(s.integers(U))) for _ in range(60)} |
                   {(0, 0), (T - 1, U - 1)})
    _check(Y, slab, xqb, ids, E, rows, K, per_slot, pairs)
    # Each expert's outputs as a whole: the oracle's product over the
    # expert's gathered rows.
    for e in range(E):
        tk = np.argwhere(ids == e)
        if len(tk) == 0:
            continue
        xr = np.stack([xqb[t * U + k] if per_slot else xqb[t] for t, k in tk])
        ref, Tm = oracle.gemm_q4k(slab[e * rows:(e + 1) * rows], xr, len(tk), rows, K)
        got = np.stack([Y[t, k] for t, k in tk])
        assert_close(got.reshape(-1), ref.reshape(-1), Tm.reshape(-1), "expert %d" % e)


def test_gemm_id_skewed_and_out_of_range():
    """One expert takes 300 pairs (five tiles, the last ragged), others none;
    out-of-range selections give NaN rows and leave the rest intact."""
    E, rows, K, T, U = 5, 130, 1536, 150, 2
    slab = _slab(E, rows, K, 9700)
    g = wl.rng(9701)
    xqb = oracle.quantize_q8k(wl.activations(T, K, g))
    ids = np.full((T, U), 2, dtype=np.int32)
    ids[:, 1] = 2
    ids[7, 0], ids[8, 1], ids[100, 0] = -1, 5, 1 << 30
    ids[9, 1] = 4
    _note("gemm id skewed")
    Y = _run(slab, xqb, ids, E, rows, K, 0)
    bad = [(7, 0), (8, 1), (100, 0)]
    for t, k in bad:
        assert np.isnan(Y[t, k]).all()
    good = np.ones((T, U), bool)
    for t, k in bad:
        good[t, k] = False
    assert not np.isnan(Y[good]).any()
    _check(Y, slab, xqb, ids, E, rows, K, 0, [(0, 0), (7, 1), (9, 1), (63, 1), (64, 0), (149, 1)])


def test_gemm_id_ragged_tiles():
    """Experts whose pairs leave ragged last tiles: 70 pairs (64 + 6), 20 (one
    short tile), 100 (64 + 36), 96 (64 + 32), 33, and 5 out-of-range
    selections in a NaN tile. Every pair against the oracle; permuting the
    tokens moves pairs between tiles and must permute the outputs bit for
    bit."""
    E, rows, K = 6, 200, 2048
    counts = {0: 70, 1: 20, 2: 100, 3: 96, 4: 33, -1: 5}
    flat = np.concatenate([np.full(c, e, np.int32) for e, c in counts.items()])
    flat = flat[wl.rng(9851).permutation(flat.size)]
    U = 2
    T = flat.size // U
    ids = flat[: T * U].reshape(T, U)
    slab = _slab(E, rows, K, 9850)
    xqb = oracle.quantize_q8k(wl.activations(T, K, wl.rng(9852)))
    _note("gemm id ragged tiles T=%d" % T)
    Y = _run(slab, xqb, ids, E, rows, K, 0)
    _check(Y, slab, xqb, ids, E, rows, K, 0)
    perm = wl.rng(9853).permutation(T)
    Yp = _run(slab, xqb[perm], ids[perm], E, rows, K, 0)
    nan = np.isnan(Y[perm])
    assert np.array_equal(np.isnan(Yp), nan)
    assert np.array_equal(Yp[~nan], Y[perm][~nan])


def test_gemm_id_permutation_is_bit_exact():
    E, rows, K, T, U = 8, 256, 2048, 97, 2
    slab = _slab(E, rows, K, 9800)
    g = wl.rng(9801)
    xqb = oracle.quantize_q8k(wl.activations(T, K, g))
    ids = _top_k(T, U, E, g)
    perm = wl.rng(9802).permutation(T)
    _note("gemm id permutation")
    Y = _run(slab, xqb, ids, E, rows, K, 0)
    Yp = _run(slab, xqb[perm], ids[perm], E, rows, K, 0)
    assert np.array_equal(Yp, Y[perm])
    # and again on a second stream (its own routing workspace)
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        Y2 = _run(slab, xqb, ids, E, rows, K, 0)
    side.synchronize()
    assert np.array_equal(Y2, Y)


@pytest.mark.parametrize("which", ["S", "M"])
def test_gemm_id_partials_bit_exact(which):
    E, rows, K, T, U = 3, 40, 1024, 6, 2
    g = wl.rng(9900)
    slab = np.concatenate([wl.q4k_isolation_weights(rows, K, g, which).reshape(rows, -1)
                           for _ in range(E)], axis=0)
    ids = np.array([[0, 2], [1, 0], [2, 1], [0, 1], [2, 0], [1, 2]], dtype=np.int32)
    for b in range(K // 256):
        x = wl.isolating_activation(T, K, g, b)
        xqb = oracle.quantize_q8k(x)
        _note("gemm id partial %s block %d" % (which, b))
        Y = _run(slab, xqb, ids, E, rows, K, 0)
        for t in range(T):
            for k in range(U):
                e = ids[t, k]
                S, Mp = oracle.q4k_partials(slab[e * rows:(e + 1) * rows], xqb[t], rows, K)
                want = S[:, b] if which == "S" else -Mp[:, b]
                assert np.array_equal(Y[t, k], want.astype(np.float64)), (t, k, b)


@pytest.mark.parametrize("T,U,E,rows,K,seed", [
    (1100, 8, 64, 64, 256, 9950),    # 8800 pairs: past the routing kernel's 8192-pair window
    (300, 8, 1024, 32, 256, 9960),   # the largest expert count: most experts hold a few pairs
])
def test_gemm_id_many_pairs_many_experts(T, U, E, rows, K, seed):
    """Each expert's outputs against the oracle's product over that expert's
    gathered token rows; no output is left unwritten."""
    slab = _slab(E, rows, K, seed)
    g = wl.rng(seed + 1)
    xqb = oracle.quantize_q8k(wl.activations(T, K, g))
    ids = _top_k(T, U, E, g)
    _note("gemm id many pairs T=%d U=%d E=%d" % (T, U, E))
    Y = _run(slab, xqb, ids, E, rows, K, 0)
    assert not np.isnan(Y).any()
    for e in range(E):
        tk = np.argwhere(ids == e)
        if len(tk) == 0:
            continue
        xr = xqb[tk[:, 0]]
        ref, Tm = oracle.gemm_q4k(slab[e * rows:(e + 1) * rows], xr, len(tk), rows, K)
        got = Y[tk[:, 0], tk[:, 1]]
        assert_close(got.reshape(-1), ref.reshape(-1), Tm.reshape(-1), "expert %d" % e)


@pytest.mark.parametrize("T,U,E,seed", [
    (1024, 8, 16, 9970),   # exactly the routing kernel's 8192-pair window
    (1, 1, 1, 9971),       # one pair, one expert
])
def test_gemm_id_window_edges(T, U, E, seed):
    """The routing window's edge (every pair ranked by the counting atomic)
    and the smallest map; also one pair past the window with a single
    expert, where every pair lands in one bucket."""
    rows, K = 32, 256
    slab = _slab(E, rows, K, seed)
    g = wl.rng(seed + 1)
    xqb = oracle.quantize_q8k(wl.activations(T, K, g))
    ids = _top_k(T, U, E, g) if U <= E else g.integers(0, E, size=(T, U)).astype(np.int32)
    _note("gemm id window edge T=%d U=%d E=%d" % (T, U, E))
    Y = _run(slab, xqb, ids, E, rows, K, 0)
    assert not np.isnan(Y).any()
    for e in range(E):
        tk = np.argwhere(ids == e)
        if len(tk) == 0:
            continue
        ref, Tm = oracle.gemm_q4k(slab[e * rows:(e + 1) * rows], xqb[tk[:, 0]], len(tk), rows, K)
        assert_close(Y[tk[:, 0], tk[:, 1]].reshape(-1), ref.reshape(-1), Tm.reshape(-1), "expert %d" % e)


def test_gemm_id_one_expert_past_the_window():
    """8193 pairs all routed to one expert: the first 8192 ranked in the
    window, the last by the scatter's own atomic, every one in one bucket of
    129 tiles (the last a small one)."""
    E, rows, K, T, U = 1, 32, 256, 8193, 1
    slab = _slab(E, rows, K, 9972)
    xqb = oracle.quantize_q8k(wl.activations(T, K, wl.rng(9973)))
    ids = np.zeros((T, U), dtype=np.int32)
    _note("gemm id one expert past the window")
    Y = _run(slab, xqb, ids, E, rows, K, 0)
    ref, Tm = oracle.gemm_q4k(slab, xqb, T, rows, K)
    assert_close(Y.reshape(T, rows).reshape(-1), ref.reshape(-1), Tm.reshape(-1), "one expert")


def test_gemm_id_every_selection_out_of_range():
    E, rows, K, T, U = 4, 40, 512, 30, 2
    slab = _slab(E, rows, K, 9974)
    xqb = oracle.quantize_q8k(wl.activations(T, K, wl.rng(9975)))
    ids = np.full((T, U), -3, dtype=np.int32)
    ids[::2, 1] = 1 << 20
    _note("gemm id every selection out of range")
    Y = _run(slab, xqb, ids, E, rows, K, 0)
    assert np.isnan(Y).all()
