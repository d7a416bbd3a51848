"""Expert-grouped mat-vecs (xq_gemv_q4k_id, xq_gemv_iq4nl_id) through the C ABI.

The gate is the pages' ("25 — Writing XPU Kernels", section 25.7.1): a slab of
six experts that differ from one another (so a kernel that ignored the
selection could not agree by accident), one q8_K activation packed on the GPU
from x_j = ((j % 25) - 12) / 64, selection {4, 0, 3}, and the grouped launch
compared with the per-expert dense launches it replaces by equality, never a
tolerance, plus no NaN and at least one non-zero output. Each slot is also
held to the oracle's mat-vec on its expert's rows (|y - ref| <= 1e-5 * T).
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


FORMATS = {
    "q4k": dict(weights=wl.q4k_weights, nbytes=xq.xq_q4k_bytes, dense=xq.xq_gemv_q4k,
                grouped=xq.xq_gemv_q4k_id, oracle=oracle.gemv_q4k),
    "iq4nl": dict(weights=wl.iq4nl_weights, nbytes=xq.xq_iq4nl_bytes, dense=xq.xq_gemv_iq4nl,
                  grouped=xq.xq_gemv_iq4nl_id, oracle=oracle.gemv_iq4nl),
}


def _slab(fmt, E, rows, K, seed):
    """E experts of `rows` rows, each drawn from its own seed."""
    f = FORMATS[fmt]
    parts = [f["weights"](rows, K, wl.rng(seed + 17 * e)) for e in range(E)]
    return np.concatenate([p.reshape(rows, -1) for p in parts], axis=0)


def _gpu_q8k(x):
    rows, K = x.shape
    out = torch.empty(xq.xq_q8k_bytes(rows, K), dtype=torch.uint8, device="cuda")
    xq.xq_quantize_q8k(out, dev(x.astype(np.float32)), rows, K)
    return out


def _check_slots(fmt, slab, slab_d, xqd, xqb, ids, E, rows, K, stride, y_id):
    """Slot by slot: dense launch on the expert's rows (bit-equal) and the
    oracle (within 1e-5 * T); out-of-range selections must be NaN."""
    f = FORMATS[fmt]
    row_bytes = f["nbytes"](1, K)
    nb8 = xq.xq_q8k_bytes(1, K)
    for kk, e in enumerate(ids):
        got = y_id[kk * rows:(kk + 1) * rows]
        if not 0 <= e < E:
            assert np.isnan(got).all(), "slot %d (sel %d) not NaN" % (kk, e)
            continue
        assert not np.isnan(got).any()
        ex = slab_d[e * rows * row_bytes:(e + 1) * rows * row_bytes]
        xrow = xqd[kk * nb8:(kk + 1) * nb8] if stride else xqd
        yd = poisoned_f32(rows)
        f["dense"](yd, ex, xrow, rows, K)
        want = take_f32(yd, rows)
        assert np.array_equal(got, want), "slot %d: %d rows differ from the dense launch" % (
            kk, int((got != want).sum()))
        xo = xqb[kk:kk + 1] if stride else xqb[:1]
        ref, T = f["oracle"](slab[e * rows:(e + 1) * rows], xo, rows, K)
        assert_close(got, ref, T, "%s slot %d" % (fmt, kk))


@pytest.mark.parametrize("fmt", ["q4k", "iq4nl"])
def test_id_gate_of_the_pages(fmt):
    E, rows, K, used, ids = 6, 64, 2048, 3, [4, 0, 3]
    slab = _slab(fmt, E, rows, K, 9100)
    slab_d = dev(slab)
    x = wl.pages_activation(K).reshape(1, K)
    xqd = _gpu_q8k(x)
    torch.cuda.synchronize()
    xqb = xqd.cpu().numpy().reshape(1, K // 256, 320)
    assert np.array_equal(xqb[:, :, :292], oracle.quantize_q8k(x)[:, :, :292])
    sel = torch.tensor(ids, dtype=torch.int32, device="cuda")
    _note("id gate %s E=%d rows=%d K=%d ids=%s" % (fmt, E, rows, K, ids))
    y = poisoned_f32(used * rows)
    FORMATS[fmt]["grouped"](y, slab_d, xqd, sel, E, used, rows, K, 0)
    y_id = take_f32(y, used * rows)
    assert not np.isnan(y_id).any()
    assert (y_id != 0).any()
    _check_slots(fmt, slab, slab_d, xqd, xqb, ids, E, rows, K, 0, y_id)


@pytest.mark.parametrize("fmt", ["q4k", "iq4nl"])
def test_id_activation_per_slot(fmt):
    E, rows, K, used, ids = 5, 96, 1536, 4, [2, 2, 0, 4]
    g = wl.rng(9200)
    slab = _slab(fmt, E, rows, K, 9201)
    slab_d = dev(slab)
    x = wl.activations(used, K, g)
    xqd = _gpu_q8k(x)
    torch.cuda.synchronize()
    xqb = xqd.cpu().numpy().reshape(used, K // 256, 320)
    sel = torch.tensor(ids, dtype=torch.int32, device="cuda")
    _note("id per-slot activation %s" % fmt)
    y = poisoned_f32(used * rows)
    FORMATS[fmt]["grouped"](y, slab_d, xqd, sel, E, used, rows, K, K // 256)
    _check_slots(fmt, slab, slab_d, xqd, xqb, ids, E, rows, K, K // 256,
                 take_f32(y, used * rows))


@pytest.mark.parametrize("fmt", ["q4k", "iq4nl"])
def test_id_out_of_range_selection(fmt):
    E, rows, K, used, ids = 6, 40, 1024, 4, [1, 7, -1, 2]
    g = wl.rng(9300)
    slab = _slab(fmt, E, rows, K, 9301)
    slab_d = dev(slab)
    x = wl.activations(1, K, g)
    xqd = _gpu_q8k(x)
    torch.cuda.synchronize()
    xqb = xqd.cpu().numpy().reshape(1, K // 256, 320)
    sel = torch.tensor(ids, dtype=torch.int32, device="cuda")
    _note("id out-of-range selection %s" % fmt)
    y = poisoned_f32(used * rows)
    FORMATS[fmt]["grouped"](y, slab_d, xqd, sel, E, used, rows, K, 0)
    _check_slots(fmt, slab, slab_d, xqd, xqb, ids, E, rows, K, 0, take_f32(y, used * rows))


ID_SHAPES = [
    # fmt, E, rows, K, ids: the other launch shapes of the dense kernels
    ("q4k", 4, 8192, 4096, [3, 1]),         # two rows per wave
    ("q4k", 3, 300, 14336, [2, 0]),         # whole row in flight (four units)
    ("q4k", 3, 130, 20480, [1, 0]),         # loads past the row skipped (five units)
    ("q4k", 3, 257, 6144, [1, 2, 0]),       # two units, the last half full
    ("iq4nl", 3, 20000, 512, [2, 0]),       # persistent grid, waves take a second row
    ("iq4nl", 3, 4096, 2048, [2, 0]),       # single-unit rows, the most a grouped staged launch takes
    ("iq4nl", 3, 4097, 2048, [0, 1]),       # one row more: the persistent grid
    ("iq4nl", 3, 1000, 10240, [0, 2]),      # staged kernel (five units)
    ("iq4nl", 2, 130, 8192, [1, 0, 1]),     # four units
    ("q4k", 3, 70, 53248, [2, 0]),          # rows past the staged limit
    ("iq4nl", 3, 70, 53248, [1, 2]),        # rows past the staged limit
    ("q4k", 3, 1000, 4096, [2, 1]),         # one unit, one row per wave
    ("q4k", 2, 200, 8192, [1, 0]),          # two units
    ("q4k", 2, 100, 10240, [0, 1]),         # three units, the last half full
    ("q4k", 2, 100, 12288, [1, 0]),         # three units
    ("iq4nl", 3, 3000, 4096, [2, 0]),       # persistent grid, two units
    ("iq4nl", 2, 500, 6144, [1, 0]),        # persistent grid, three units
    ("iq4nl", 2, 100, 12288, [0, 1]),       # staged kernel, six units
    ("iq4nl", 3, 200, 14336, [0, 2]),       # staged kernel, seven units
    ("iq4nl", 2, 64, 20480, [1, 0]),        # staged kernel, batches of eight units
]


@pytest.mark.parametrize("fmt,E,rows,K,ids", ID_SHAPES,
                         ids=["%s_E%d_r%d_k%d" % (s[0], s[1], s[2], s[3]) for s in ID_SHAPES])
def test_id_shapes(fmt, E, rows, K, ids):
    g = wl.rng(9400 + rows)
    slab = _slab(fmt, E, rows, K, 9401 + K)
    slab_d = dev(slab)
    x = wl.activations(1, K, g)
    xqd = _gpu_q8k(x)
    torch.cuda.synchronize()
    xqb = xqd.cpu().numpy().reshape(1, K // 256, 320)
    used = len(ids)
    sel = torch.tensor(ids, dtype=torch.int32, device="cuda")
    _note("id shape %s E=%d rows=%d K=%d" % (fmt, E, rows, K))
    y = poisoned_f32(used * rows)
    FORMATS[fmt]["grouped"](y, slab_d, xqd, sel, E, used, rows, K, 0)
    _check_slots(fmt, slab, slab_d, xqd, xqb, ids, E, rows, K, 0, take_f32(y, used * rows))
