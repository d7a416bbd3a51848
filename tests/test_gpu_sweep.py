"""Seeded random shapes through every dispatch regime, against the oracle.

The fixed cases elsewhere pin each launch shape at chosen sizes; this sweep
draws further shapes from a fixed seed so that ragged edges land in new
places: mat-vecs of the three formats over ragged N and K, and the small-M
product on the batched mat-vec, the 16-token tile, split K, and launches
whose tiles run in whole rounds with a split remainder (the remainder and
the whole rounds in one grid, for both token tiles), and the grouped product
over skewed routings with stray selections, some past the expert map's
first batch of pairs. Outputs are compared to the oracle at the f32 bar
(whole outputs where the oracle is quick, sampled outputs with tile corners
and whole rows where not).
"""
import numpy as np
import pytest

import oracle
import quantized_decode_mat_amd as xq
import workloads as wl
from test_gpu_gemm_id import _check, _run, _slab
from test_gpu_parity import _note, assert_close, dev, gpu_gemm, poisoned_f32, take_f32

pytestmark = pytest.mark.gpu


def _matvec_shapes():
    g = wl.rng(8000)
    out = []
    for fmt in ("q4k", "iq4nl", "q4_0"):
        for _ in range(5):
            N = int(g.integers(1, 20001))
            K = 256 * int(g.integers(1, 65))
            out.append((fmt, N, K, int(g.integers(0, 2 ** 31))))
    return out


MATVEC = _matvec_shapes()


@pytest.mark.parametrize("fmt,N,K,seed", MATVEC,
                         ids=["%s_n%d_k%d" % (s[0], s[1], s[2]) for s in MATVEC])
def test_sweep_matvec(fmt, N, K, seed):
    g = wl.rng(seed)
    xqb = oracle.quantize_q8k(wl.activations(1, K, g))
    y = poisoned_f32(N)
    _note("sweep mat-vec %s N=%d K=%d" % (fmt, N, K))
    if fmt == "q4k":
        w = wl.q4k_weights(N, K, g)
        xq.xq_gemv_q4k(y, dev(w), dev(xqb), N, K)
        ref, T = oracle.gemv_q4k(w, xqb, N, K)
    elif fmt == "iq4nl":
        w = wl.iq4nl_weights(N, K, g)
        xq.xq_gemv_iq4nl(y, dev(w), dev(xqb), N, K)
        ref, T = oracle.gemv_iq4nl(w, xqb, N, K)
    else:
        w = wl.iq4nl_weights(N, K, g)
        xq.xq_gemv_q4_0(y, dev(w), dev(xqb), N, K)
        ref, T = oracle.gemv_q4_0(w, xqb, N, K)
    assert_close(take_f32(y, N), ref, T, "sweep %s" % fmt)


def _product_shapes():
    g = wl.rng(8100)
    out = []
    # (token range, rows range, K choices): short batches, the 16-token tile,
    # the 64-token tile with split K, grids past one round of workgroups, and
    # the wave-split tile's range (5-16 tokens, 256-512 row tiles of 32, 8-16
    # super-blocks; four tokens there take the batched mat-vec).
    regimes = [
        ((2, 4), (1000, 16000), (2048, 4096, 14336)),
        ((4, 33), (100, 16000), (1024, 4096, 7936)),
        ((33, 129), (100, 4200), (4096, 8192, 14336)),
        ((129, 320), (4000, 9000), (2048, 4096)),
        ((320, 700), (7000, 15000), (2048, 4096, 8192)),
        ((129, 200), (100, 2000), (4096, 14336)),      # the 64-token tile on few tiles, split K
        ((5, 17), (8161, 16385), tuple(256 * u for u in range(8, 17))),  # the wave-split tile
    ]
    for (m_lo, m_hi), (n_lo, n_hi), ks in regimes:
        for _ in range(3):
            M = int(g.integers(m_lo, m_hi))
            N = int(g.integers(n_lo, n_hi))
            K = int(ks[int(g.integers(0, len(ks)))])
            out.append((M, N, K, int(g.integers(0, 2 ** 31))))
    # Past whole rounds of the 16-token tile (768 resident): 20 tokens x
    # 100000 rows is 1564 tiles, two whole rounds and a remainder of 28.
    out.append((20, 100000, 4096, 8199))
    return out


PRODUCT = _product_shapes()


def _short_shapes():
    # Two to four tokens on rows of one unit (K <= 4096): the batched
    # mat-vec on its persistent grid; every token's row must be the mat-vec's.
    g = wl.rng(8200)
    out = []
    for _ in range(8):
        M = int(g.integers(2, 5))
        N = int(g.integers(1, 30000))
        K = 256 * int(g.integers(1, 17))
        out.append((M, N, K, int(g.integers(0, 2 ** 31))))
    return out


SHORT = _short_shapes()


@pytest.mark.parametrize("M,N,K,seed", SHORT, ids=["m%d_n%d_k%d" % s[:3] for s in SHORT])
def test_sweep_short_batch_rows_equal_matvec(M, N, K, seed):
    g = wl.rng(seed)
    w = wl.q4k_weights(N, K, g)
    xqb = oracle.quantize_q8k(wl.activations(M, K, g))
    _note("sweep short batch M=%d N=%d K=%d" % (M, N, K))
    Y = gpu_gemm(w, xqb, M, N, K)
    wd = dev(w)
    for m in range(M):
        y = poisoned_f32(N)
        xq.xq_gemv_q4k(y, wd, dev(xqb[m]), N, K)
        assert np.array_equal(Y[m], take_f32(y, N)), m
    ref, T = oracle.gemv_q4k(w, xqb[M - 1], N, K)
    assert_close(Y[M - 1], ref, T, "sweep short batch last row")


@pytest.mark.parametrize("M,N,K,seed", PRODUCT,
                         ids=["m%d_n%d_k%d" % s[:3] for s in PRODUCT])
def test_sweep_product(M, N, K, seed):
    g = wl.rng(seed)
    w = wl.q4k_weights(N, K, g)
    xqb = oracle.quantize_q8k(wl.activations(M, K, g))
    _note("sweep product M=%d N=%d K=%d" % (M, N, K))
    Y = gpu_gemm(w, xqb, M, N, K)
    assert not np.isnan(Y).any()
    if M * N * K <= 2 ** 27:
        ref, T = oracle.gemm_q4k(w, xqb, M, N, K)
        assert_close(Y.reshape(-1), ref.reshape(-1), T.reshape(-1), "sweep product")
        return
    s = wl.rng(seed + 1)
    corners_m = [0, M - 1] + [t for t in (15, 16, 63, 64) if t < M]
    corners_n = [0, N - 1] + [t for t in (127, 128) if t < N]
    ms = np.concatenate([s.integers(0, M, 800), np.repeat(corners_m, len(corners_n))])
    ns = np.concatenate([s.integers(0, N, 800), np.tile(corners_n, len(corners_m))])
    ref, T = oracle.gemm_q4k(w, xqb, M, N, K, ms, ns)
    assert_close(Y[ms, ns], ref, T, "sweep product sampled")
    for m in sorted({0, M - 1}):
        ref, T = oracle.gemv_q4k(w, xqb[m], N, K)
        assert_close(Y[m], ref, T, "sweep product row %d" % m)


def _grouped_shapes():
    # (tokens, slots, experts, rows per expert, K, q8_K row per slot); the
    # slab stays under 2^27 weights. The last regime passes 8192 pairs.
    g = wl.rng(8300)
    out = []
    regimes = [((1, 64), (1, 4), (1, 9)), ((64, 700), (1, 9), (8, 129)),
               ((1100, 1400), (8, 9), (16, 65))]
    for (t_lo, t_hi), (u_lo, u_hi), (e_lo, e_hi) in regimes:
        for _ in range(3):
            E = int(g.integers(e_lo, e_hi))
            U = min(E, int(g.integers(u_lo, u_hi)))
            T = int(g.integers(t_lo, t_hi))
            K = 256 * int(g.integers(1, 17))
            rows = int(g.integers(1, max(2, min(3000, 2 ** 27 // (E * K)))))
            out.append((T, U, E, rows, K, int(g.integers(0, 2)), int(g.integers(0, 2 ** 31))))
    return out


GROUPED = _grouped_shapes()


@pytest.mark.parametrize("T,U,E,rows,K,per_slot,seed", GROUPED,
                         ids=["t%d_u%d_e%d_r%d_k%d_s%d" % s[:6] for s in GROUPED])
def test_sweep_grouped_product(T, U, E, rows, K, per_slot, seed):
    g = wl.rng(seed)
    slab = _slab(E, rows, K, seed)
    xqb = oracle.quantize_q8k(wl.activations(T * U if per_slot else T, K, g))
    # Each token's U distinct experts drawn with weights falling as 1/(e+1),
    # so a few experts take most pairs; about 1 in 50 selections is replaced
    # by an expert number outside 0..E-1.
    w = 1.0 / np.arange(1, E + 1)
    ids = np.stack([g.choice(E, size=U, replace=False, p=w / w.sum()) for _ in range(T)])
    stray = g.random(ids.shape) < 0.02
    ids = np.where(stray, g.choice([-1, E, E + 7], size=ids.shape), ids).astype(np.int32)
    _note("sweep grouped T=%d U=%d E=%d rows=%d K=%d per_slot=%d" % (T, U, E, rows, K, per_slot))
    Y = _run(slab, xqb, ids, E, rows, K, per_slot)
    s = wl.rng(seed + 1)
    pairs = sorted({(int(s.integers(T)), int(s.integers(U))) for _ in range(80)} |
                   {(0, 0), (T - 1, U - 1)} | {tuple(int(v) for v in p) for p in np.argwhere(stray)[:8]})
    _check(Y, slab, xqb, ids, E, rows, K, per_slot, pairs)
    # Outputs outside the sample: NaN exactly where a selection is stray.
    assert np.array_equal(np.isnan(Y).all(axis=2), (ids < 0) | (ids >= E))
    assert not np.isnan(Y[(ids >= 0) & (ids < E)]).any()


def _repack_cases():
    g = wl.rng(8400)
    out = []
    for i in range(8):
        bpr = int(g.integers(1, 1200))
        rows = int(g.integers(1, 9))
        n = rows * bpr
        cuts = sorted(set([0, n] + [int(c) for c in g.integers(1, max(2, n), size=int(g.integers(0, 5)))]))
        out.append((rows, bpr, cuts, 0 if i % 2 == 0 else 2, int(g.integers(0, 2 ** 31))))
    return out


REPACK = _repack_cases()


@pytest.mark.parametrize("rows,bpr,cuts,offset,seed", REPACK,
                         ids=["r%d_bpr%d_c%d_off%d" % (s[0], s[1], len(s[2]) - 1, s[3]) for s in REPACK])
def test_sweep_repack(rows, bpr, cuts, offset, seed):
    # Random chunkings of a matrix's file blocks, each chunk from a 16-byte
    # aligned source (staged through LDS) or a 2-byte aligned one (read as
    # halves): the resident rows equal the oracle's byte for byte, and no
    # byte of the poisoned buffer is left unwritten.
    import torch
    blocks = wl.iq4nl_file_blocks(rows * bpr, wl.rng(seed))
    res = dev(np.full((rows, xq.iq4nl_row_bytes(bpr)), 0xAB, dtype=np.uint8))
    _note("sweep repack rows=%d bpr=%d cuts=%s offset=%d" % (rows, bpr, cuts, offset))
    for a, b in zip(cuts[:-1], cuts[1:]):
        buf = torch.zeros(18 * (b - a) + 16, dtype=torch.uint8, device="cuda")
        buf[offset:offset + 18 * (b - a)] = dev(blocks[a:b].reshape(-1))
        xq.xq_repack_iq4nl(res, buf.data_ptr() + offset, b - a, a, bpr)
        torch.cuda.synchronize()
    got = res.cpu().numpy().reshape(rows, -1)
    assert np.array_equal(got, oracle.repack_iq4nl(blocks, rows * bpr, 0, bpr))
