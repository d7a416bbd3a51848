"""HIP path against the oracle, element by element, through the C ABI.

Bars (the pages' comparison rules, "The kernel reference interpreter",
section Comparing against it, and "25 — Writing XPU Kernels", section 25.7):
  * q8_K bytes 0..291 of every block: bit-exact (bytes 292..319 carry no
    meaning and are skipped).
  * Per-block integer partials: bit-exact. They are isolated through the
    production entry points: weights with d = 1, dmin = 0 (or d = 0, dmin = 1)
    against an activation whose only nonzero block has scale 1 make each
    output equal one block's S (or -M) exactly.
  * f32 outputs: |y - y_oracle| <= 1e-5 * T per output, T the sum of the
    magnitudes of the terms the integer route adds for it: |d*xs*S| +
    |dmin*xs*M| per Q4_K block, |d_c*xs*D_c| per IQ4_NL or Q4_0 32-block.
    T = 0 demands y = 0. The largest |y - y_oracle| / T of each test is
    recorded (HEADROOM) and, when XQ_HEADROOM_OUT names a file, written
    there at the end of the session.
  * No NaN, and outputs written in full: every output buffer is poisoned with
    0xFF bytes first, and a canary tail past its end must stay untouched.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import quantized_decode_mat_amd as xq
import workloads as wl

pytestmark = pytest.mark.gpu

REL = 1e-5
CANARY = 64


def _note(msg):
    print("[gpu-case] " + msg, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).reshape(-1).copy()).cuda()


def poisoned_f32(n: int) -> torch.Tensor:
    return torch.full(((n + CANARY) * 4,), 255, dtype=torch.uint8, device="cuda").view(torch.float32)


def poisoned_u8(n: int) -> torch.Tensor:
    return torch.full((n + CANARY * 4,), 255, dtype=torch.uint8, device="cuda")


def take_f32(buf: torch.Tensor, n: int) -> np.ndarray:
    torch.cuda.synchronize()
    tail = buf[n:].view(torch.int32)
    assert bool((tail == -1).all()), "canary past the output was overwritten"
    return buf[:n].cpu().numpy().astype(np.float64)


def take_u8(buf: torch.Tensor, n: int) -> np.ndarray:
    torch.cuda.synchronize()
    assert bool((buf[n:] == 255).all()), "canary past the output was overwritten"
    return buf[:n].cpu().numpy()


# Largest |y - y_oracle| / T seen per test (the bar's headroom).
HEADROOM = {}


def _record_headroom(err: np.ndarray, T: np.ndarray):
    pos = T > 0
    if not pos.any():
        return
    test = os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0]
    r = float((err[pos] / T[pos]).max())
    HEADROOM[test] = max(HEADROOM.get(test, 0.0), r)


def assert_close(y: np.ndarray, ref: np.ndarray, T: np.ndarray, what: str):
    assert not np.isnan(y).any(), "%s: %d NaN outputs" % (what, int(np.isnan(y).sum()))
    err = np.abs(y - ref)
    _record_headroom(err, T)
    bad = err > REL * T
    assert not bad.any(), "%s: %d outputs outside 1e-5*T, first at %d: gpu %r oracle %r T %r" % (
        what, int(bad.sum()), int(np.argmax(bad)), y[bad][0], ref[bad][0], T[bad][0])
    assert np.all(y[T == 0] == 0)
    assert np.any(y != 0), "%s: all outputs zero" % what


def gpu_quantize(x: np.ndarray) -> np.ndarray:
    rows, K = x.shape
    n = xq.xq_q8k_bytes(rows, K)
    out = poisoned_u8(n)
    xq.xq_quantize_q8k(out, dev(x.astype(np.float32)), rows, K)
    return take_u8(out, n).reshape(rows, K // 256, 320)


def gpu_gemv_q4k(w: np.ndarray, xqb: np.ndarray, N: int, K: int) -> np.ndarray:
    y = poisoned_f32(N)
    xq.xq_gemv_q4k(y, dev(w), dev(xqb), N, K)
    return take_f32(y, N)


def gpu_gemv_iq4nl(w: np.ndarray, xqb: np.ndarray, N: int, K: int) -> np.ndarray:
    y = poisoned_f32(N)
    xq.xq_gemv_iq4nl(y, dev(w), dev(xqb), N, K)
    return take_f32(y, N)


def zeroed_workspace(nbytes: int):
    """A caller-owned device workspace of nbytes, zeroed before its first use
    (None when a call needs none)."""
    if nbytes == 0:
        return None
    return torch.zeros(nbytes, dtype=torch.uint8, device="cuda")


def gemm_workspace(M: int, N: int, K: int):
    return zeroed_workspace(xq.xq_gemm_q4k_small_m_workspace_bytes(M, N, K))


def gpu_gemm(w: np.ndarray, xqb: np.ndarray, M: int, N: int, K: int) -> np.ndarray:
    y = poisoned_f32(M * N)
    xq.xq_gemm_q4k_small_m(y, dev(w), dev(xqb), M, N, K, workspace=gemm_workspace(M, N, K))
    return take_f32(y, M * N).reshape(M, N)


# ---------------------------------------------------------------------------
# q8_K quantizer: bit-exact
# ---------------------------------------------------------------------------

def _quant_cases():
    cases = {}
    g = wl.rng(wl.SEEDS["q4k_tiny"])
    wl.q4k_weights(256, 1024, g)
    cases["tiny_1x1024"] = wl.activations(1, 1024, g)
    g = wl.rng(wl.SEEDS["q4k_4096"])
    wl.q4k_weights(1, 4096, g)
    cases["c1_1x4096"] = wl.activations(1, 4096, wl.rng(2001))
    cases["h_1x14336"] = 3.0 * wl.activations(1, 14336, wl.rng(2002))
    cases["prefill_512x4096"] = wl.activations(512, 4096, wl.rng(wl.SEEDS["prefill"]))
    cases["ragged_3x768"] = wl.activations(3, 768, wl.rng(2003))
    cases["pages_1x2048"] = wl.pages_activation(2048).reshape(1, -1)
    t = np.round(wl.rng(2004).uniform(-126, 126, 512) * 2) / 2
    t[0], t[1:8] = 127.0, [0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 62.5]
    t[256] = -127.0
    cases["ties_1x512"] = t.reshape(1, -1)
    z = np.zeros((2, 512), np.float32)
    z[1, :256] = 0.37
    z[1, 300] = -5.0
    cases["zero_const_2x512"] = z
    s = wl.activations(5, 256, wl.rng(2005))
    s *= np.array([[1e-37], [1e-30], [1e-3], [1e3], [1e30]], np.float32)
    cases["magnitudes_5x256"] = s
    return cases


QUANT_CASES = _quant_cases()


@pytest.mark.parametrize("name", sorted(QUANT_CASES))
def test_quantize_q8k_bit_exact(name):
    x = QUANT_CASES[name].astype(np.float32)
    _note("quantize %s" % name)
    got = gpu_quantize(x)
    want = oracle.quantize_q8k(x)
    diff = got[:, :, :292] != want[:, :, :292]
    assert not diff.any(), "%s: %d bytes differ, first block %s" % (
        name, int(diff.sum()), np.argwhere(diff.any(axis=2))[0])
    assert np.all(got[:, :, 292:] == 0)


@pytest.mark.parametrize("offset", [1, 2, 3])
def test_quantize_q8k_rows_4_byte_aligned(offset):
    """x needs only 4-byte alignment: rows that start 4, 8 or 12 bytes past a
    16-byte boundary take the 4-byte loads and give the same bytes."""
    rows, K = 3, 4096
    x = wl.activations(rows, K, wl.rng(2100 + offset)).astype(np.float32)
    x[1, 7] = 0.5 * np.abs(x[1]).max() / 127 * 3  # a tie one half past a code
    _note("quantize 4-byte aligned x, offset %d floats" % offset)
    buf = torch.full((rows * K + 4,), float("nan"), dtype=torch.float32, device="cuda")
    buf[offset:offset + rows * K] = torch.from_numpy(x.reshape(-1)).cuda()
    xv = buf[offset:offset + rows * K]
    assert xv.data_ptr() % 16 == 4 * offset
    n = xq.xq_q8k_bytes(rows, K)
    out = poisoned_u8(n)
    xq.xq_quantize_q8k(out, xv, rows, K)
    got = take_u8(out, n).reshape(rows, K // 256, 320)
    want = oracle.quantize_q8k(x)
    assert np.array_equal(got[:, :, :292], want[:, :, :292])
    assert np.array_equal(got, gpu_quantize(x))


# ---------------------------------------------------------------------------
# Q4_K mat-vec
# ---------------------------------------------------------------------------

Q4K_SHAPES = [
    ("tiny", 256, 1024, wl.SEEDS["q4k_tiny"]),
    ("c1_4096x4096", 4096, 4096, wl.SEEDS["q4k_4096"]),
    ("ffn_up_14336x4096", 14336, 4096, wl.SEEDS["ffn_up"]),
    ("ffn_down_4096x14336", 4096, 14336, wl.SEEDS["ffn_down"]),
    ("n1_k256", 1, 256, 3001),
    ("n37_k768", 37, 768, 3002),
    ("n130_k2304", 130, 2304, 3003),
    ("n9000_k4352", 9000, 4352, 3004),
    ("n8193_k2048_ragged_rows", 8193, 2048, 3005),
    ("n64_kmax", 64, 49152, 3006),                     # twelve units, batches of two
    ("n300_k8192_two_units", 300, 8192, 3016),
    ("n100_k7424_two_units_ragged", 100, 7424, 3017),  # 29 super-blocks: a last unit of 13
    ("n77_k10240_three_units_ragged", 77, 10240, 3007),
    ("n300_k9472_three_units_ragged", 300, 9472, 3008),
    ("n257_k12288_three_units", 257, 12288, 3009),
    ("n33_k11264_three_units_ragged", 33, 11264, 3010),
    ("n1000_k14080_four_units_ragged", 1000, 14080, 3011),
    ("n50_k16384_four_units", 50, 16384, 3012),
    ("n90_k17408_five_units_ragged", 90, 17408, 3018),  # batches of two, loads past the row skipped
    ("n45_k20736_six_units_ragged", 45, 20736, 3019),   # the last unit one block
    ("n64_k49408_unstaged", 64, 49408, 3013),          # one block past the staged limit
    ("n40_k53248_unstaged", 40, 53248, 3014),
    ("n3_k1048576_max", 3, 1048576, 3015),             # the largest K accepted
]


@pytest.mark.parametrize("name,N,K,seed", Q4K_SHAPES, ids=[s[0] for s in Q4K_SHAPES])
def test_gemv_q4k(name, N, K, seed):
    g = wl.rng(seed)
    w = wl.q4k_weights(N, K, g)
    x = wl.activations(1, K, g)
    xqb = oracle.quantize_q8k(x)
    _note("gemv_q4k %s N=%d K=%d" % (name, N, K))
    y = gpu_gemv_q4k(w, xqb, N, K)
    ref, T = oracle.gemv_q4k(w, xqb, N, K)
    assert_close(y, ref, T, name)


ISO_Q4K = [
    ("c1", 4096, 4096, list(range(16))),
    ("ffn_down", 4096, 14336, [0, 13, 27, 41, 55]),
    ("ragged", 37, 768, [0, 1, 2]),
]


@pytest.mark.parametrize("which", ["S", "M"])
@pytest.mark.parametrize("name,N,K,blocks", ISO_Q4K, ids=[s[0] for s in ISO_Q4K])
def test_gemv_q4k_partials_bit_exact(name, N, K, blocks, which):
    g = wl.rng(4000 + N + K)
    w = wl.q4k_isolation_weights(N, K, g, which)
    wd = dev(w)
    for b in blocks:
        x = wl.isolating_activation(1, K, g, b)
        xqb = oracle.quantize_q8k(x)
        assert xqb[0, b, 288:292].view("<f4")[0] == 1.0
        S, Mp = oracle.q4k_partials(w, xqb, N, K)
        want = S[:, b] if which == "S" else -Mp[:, b]
        _note("gemv_q4k partial %s %s block %d" % (name, which, b))
        y = poisoned_f32(N)
        xq.xq_gemv_q4k(y, wd, dev(xqb), N, K)
        got = take_f32(y, N)
        assert np.array_equal(got, want.astype(np.float64)), (
            "block %d: %d rows differ" % (b, int((got != want).sum())))


def test_ffn_pair_chain():
    """The FFN pair with the GPU quantizer in the loop: x -> q8_K -> up ->
    h -> q8_K -> down. Each quantization is bit-exact against the oracle
    quantizing the same f32 input (the GPU's own h for the second)."""
    K, H = 4096, 14336
    gu = wl.rng(wl.SEEDS["ffn_up"])
    wu = wl.q4k_weights(H, K, gu)
    x = wl.activations(1, K, gu)
    wdn = wl.q4k_weights(K, H, wl.rng(wl.SEEDS["ffn_down"]))
    _note("ffn chain")
    xq1 = torch.full((xq.xq_q8k_bytes(1, K),), 255, dtype=torch.uint8, device="cuda")
    h = torch.empty(H, dtype=torch.float32, device="cuda")
    xq2 = torch.full((xq.xq_q8k_bytes(1, H),), 255, dtype=torch.uint8, device="cuda")
    y = torch.empty(K, dtype=torch.float32, device="cuda")
    wu_d, wd_d, x_d = dev(wu), dev(wdn), dev(x)
    xq.xq_quantize_q8k(xq1, x_d, 1, K)
    xq.xq_gemv_q4k(h, wu_d, xq1, H, K)
    xq.xq_quantize_q8k(xq2, h, 1, H)
    xq.xq_gemv_q4k(y, wd_d, xq2, K, H)
    torch.cuda.synchronize()
    q1 = xq1.cpu().numpy().reshape(1, K // 256, 320)
    q1o = oracle.quantize_q8k(x)
    assert np.array_equal(q1[:, :, :292], q1o[:, :, :292])
    hh = h.cpu().numpy().astype(np.float64)
    ref, T = oracle.gemv_q4k(wu, q1o, H, K)
    assert_close(hh, ref, T, "up")
    q2 = xq2.cpu().numpy().reshape(1, H // 256, 320)
    q2o = oracle.quantize_q8k(h.cpu().numpy().reshape(1, H))
    assert np.array_equal(q2[:, :, :292], q2o[:, :, :292])
    ref2, T2 = oracle.gemv_q4k(wdn, q2o, K, H)
    assert_close(y.cpu().numpy().astype(np.float64), ref2, T2, "down")


# The mat-vec with its output quantized in the same launch (the FFN pair's
# fused tail): y is xq_gemv_q4k's, bit for bit, and yq is what
# xq_quantize_q8k writes for that y.
GEMV_Q8K = [
    ("up_14336x4096", 14336, 4096, wl.SEEDS["ffn_up"]),        # one unit, 8 rows per workgroup
    ("down_4096x14336", 4096, 14336, wl.SEEDS["ffn_down"]),    # four units, whole row in flight
    ("n256_k1024", 256, 1024, 7601),                           # one ragged unit
    ("n512_k20480", 512, 20480, 7602),                         # loads past the row skipped
    ("n1280_k2304", 1280, 2304, 7603),                         # ragged unit tail
    ("n512_k7424", 512, 7424, 7605),                           # two units, the last ragged
    ("n512_k53248", 512, 53248, 7604),                         # activation from global memory
    ("n8192_k2048", 8192, 2048, 7606),                         # one unit, two rows per wave
    ("n768_k6144", 768, 6144, 7607),                           # two units, the last half full
    ("n256_k10240", 256, 10240, 7608),                         # three units
    ("n512_k12288", 512, 12288, 7609),                         # three units
]


@pytest.mark.parametrize("name,N,K,seed", GEMV_Q8K, ids=[c[0] for c in GEMV_Q8K])
def test_gemv_q4k_q8k(name, N, K, seed):
    g = wl.rng(seed)
    w = wl.q4k_weights(N, K, g)
    xqb = oracle.quantize_q8k(wl.activations(1, K, g))
    wd, xd = dev(w), dev(xqb)
    _note("gemv q8k %s" % name)
    nq = xq.xq_q8k_bytes(1, N)
    outs = []
    side = torch.cuda.Stream()
    ws = zeroed_workspace(xq.xq_gemv_q4k_q8k_workspace_bytes(N))
    ws_side = zeroed_workspace(xq.xq_gemv_q4k_q8k_workspace_bytes(N))
    for call in range(3):  # repeated calls (counters reset), the last on a second stream
        y = poisoned_f32(N)
        yq = poisoned_u8(nq)
        if call < 2:
            xq.xq_gemv_q4k_q8k(y, yq, wd, xd, N, K, workspace=ws)
        else:
            with torch.cuda.stream(side):
                xq.xq_gemv_q4k_q8k(y, yq, wd, xd, N, K, workspace=ws_side)
            side.synchronize()
        outs.append((take_f32(y, N), take_u8(yq, nq).reshape(N // 256, 320)))
    y0 = poisoned_f32(N)
    xq.xq_gemv_q4k(y0, wd, xd, N, K)
    ref_y = take_f32(y0, N)
    yq0 = poisoned_u8(nq)
    xq.xq_quantize_q8k(yq0, y0[:N], 1, N)
    ref_q = take_u8(yq0, nq).reshape(N // 256, 320)
    oq = oracle.quantize_q8k(ref_y.astype(np.float32).reshape(1, N))[0]
    for yy, qq in outs:
        assert np.array_equal(yy, ref_y)
        assert np.array_equal(qq[:, :292], ref_q[:, :292])
        assert np.array_equal(qq[:, :292], oq[:, :292])
        assert not qq[:, 292:].any()


def test_gemv_q4k_q8k_y_4_byte_aligned():
    """The fused tail's y needs only 4-byte alignment: y 4 bytes past a
    16-byte boundary gets the bits of the aligned call, and yq the same bytes."""
    N, K = 14336, 4096
    g = wl.rng(7611)
    w = wl.q4k_weights(N, K, g)
    xqb = oracle.quantize_q8k(wl.activations(1, K, g))
    wd, xd = dev(w), dev(xqb)
    _note("gemv q8k with y at +4 bytes")
    nq = xq.xq_q8k_bytes(1, N)
    ws = zeroed_workspace(xq.xq_gemv_q4k_q8k_workspace_bytes(N))
    ya, yqa = poisoned_f32(N), poisoned_u8(nq)
    xq.xq_gemv_q4k_q8k(ya, yqa, wd, xd, N, K, workspace=ws)
    buf, yqb = poisoned_f32(N + 1), poisoned_u8(nq)
    yv = buf[1:1 + N]
    assert yv.data_ptr() % 16 == 4
    xq.xq_gemv_q4k_q8k(yv, yqb, wd, xd, N, K, workspace=ws)
    yb = take_f32(buf, N + 1)
    assert bool((buf[:1].view(torch.int32) == -1).all()), "the word before y was written"
    assert np.array_equal(yb[1:], take_f32(ya, N))
    assert np.array_equal(take_u8(yqb, nq), take_u8(yqa, nq))


def test_ffn_pair_fused_tail_equals_four_launches():
    """quantize x -> up with its q8_K tail -> down gives the four-launch
    chain's h, q8_K(h) and y bit for bit."""
    K, H = 4096, 14336
    gu = wl.rng(wl.SEEDS["ffn_up"])
    wu = dev(wl.q4k_weights(H, K, gu))
    x = dev(wl.activations(1, K, gu))
    wdn = dev(wl.q4k_weights(K, H, wl.rng(wl.SEEDS["ffn_down"])))
    _note("ffn fused tail")
    xq1 = torch.empty(xq.xq_q8k_bytes(1, K), dtype=torch.uint8, device="cuda")
    ws = zeroed_workspace(xq.xq_gemv_q4k_q8k_workspace_bytes(H))
    outs = []
    for fused in (False, True):
        h = torch.empty(H, dtype=torch.float32, device="cuda")
        xq2 = torch.zeros(xq.xq_q8k_bytes(1, H), dtype=torch.uint8, device="cuda")
        y = torch.empty(K, dtype=torch.float32, device="cuda")
        xq.xq_quantize_q8k(xq1, x, 1, K)
        if fused:
            xq.xq_gemv_q4k_q8k(h, xq2, wu, xq1, H, K, workspace=ws)
        else:
            xq.xq_gemv_q4k(h, wu, xq1, H, K)
            xq.xq_quantize_q8k(xq2, h, 1, H)
        xq.xq_gemv_q4k(y, wdn, xq2, K, H)
        torch.cuda.synchronize()
        outs.append((h.cpu(), xq2.cpu(), y.cpu()))
    for a, b in zip(*outs):
        assert torch.equal(a, b)


# ---------------------------------------------------------------------------
# IQ4_NL mat-vec
# ---------------------------------------------------------------------------

IQ4_SHAPES = [
    ("c3_4096x4096", 4096, 4096, wl.SEEDS["iq4nl_4096"]),
    ("c3_head_128256x4096", 128256, 4096, wl.SEEDS["iq4nl_head"]),
    ("n5_k256", 5, 256, 5001),
    ("n33_k768", 33, 768, 5002),
    ("n1000_k2304", 1000, 2304, 5003),
    ("n8193_k2048_tworow", 8193, 2048, 5004),
    ("n16_k14336", 16, 14336, 5005),
    ("n300_k8192_four_units", 300, 8192, 5006),
    ("n70_k10240_five_units", 70, 10240, 5007),
    ("n20000_k512_two_rows_per_wave", 20000, 512, 5008),
    ("n16384_k4096_grid_one_per_cu", 16384, 4096, 5012),
    ("n16385_k2048_grid_two_per_cu", 16385, 2048, 5013),
    ("n65537_k2048_grid_two_rounds", 65537, 2048, 5014),
    ("n64_k49152_staged_max", 64, 49152, 5009),
    ("n40_k53248_unstaged", 40, 53248, 5010),
    ("n3_k1048576_max", 3, 1048576, 5011),
]


@pytest.mark.parametrize("name,N,K,seed", IQ4_SHAPES, ids=[s[0] for s in IQ4_SHAPES])
def test_gemv_iq4nl(name, N, K, seed):
    g = wl.rng(seed)
    w = wl.iq4nl_weights(N, K, g)
    x = wl.activations(1, K, g)
    xqb = oracle.quantize_q8k(x)
    _note("gemv_iq4nl %s N=%d K=%d" % (name, N, K))
    y = gpu_gemv_iq4nl(w, xqb, N, K)
    ref, T = oracle.gemv_iq4nl(w, xqb, N, K)
    assert_close(y, ref, T, name)


@pytest.mark.parametrize("N,K,blocks", [(4096, 4096, [0, 7, 8, 63, 64, 127]), (33, 768, [0, 5, 23])])
def test_gemv_iq4nl_partials_bit_exact(N, K, blocks):
    g = wl.rng(6000 + N)
    w = wl.iq4nl_unit_scale_weights(N, K, g)
    wd = dev(w)
    for c in blocks:
        x = wl.isolating_activation(1, K, g, c // 8, width=32, offset=32 * (c % 8))
        xqb = oracle.quantize_q8k(x)
        D = oracle.iq4nl_partials(w, xqb, N, K)
        _note("gemv_iq4nl partial block %d" % c)
        y = poisoned_f32(N)
        xq.xq_gemv_iq4nl(y, wd, dev(xqb), N, K)
        got = take_f32(y, N)
        assert np.array_equal(got, D[:, c].astype(np.float64)), c


# ---------------------------------------------------------------------------
# Small-M product (int8 MFMA)
# ---------------------------------------------------------------------------

GEMM_SMALL = [
    (1, 37, 256, 7001),
    (3, 130, 768, 7002),
    (130, 200, 512, 7003),
    (129, 128, 1024, 7004),
    (256, 256, 2048, 7005),
]


@pytest.mark.parametrize("M,N,K,seed", GEMM_SMALL)
def test_gemm_full_compare(M, N, K, seed):
    g = wl.rng(seed)
    w = wl.q4k_weights(N, K, g)
    x = wl.activations(M, K, g)
    xqb = oracle.quantize_q8k(x)
    _note("gemm M=%d N=%d K=%d" % (M, N, K))
    Y = gpu_gemm(w, xqb, M, N, K)
    ref, T = oracle.gemm_q4k(w, xqb, M, N, K)
    assert_close(Y.reshape(-1), ref.reshape(-1), T.reshape(-1), "gemm")


# Split-K shapes (few tiles: the grid is tiles x splits; the last split of a
# tile to arrive sums the partials in split order).
GEMM_SPLIT = [
    (37, 1000, 4352, 7011),    # 16-token tile: 17 super-blocks in four splits
    (16, 300, 14336, 7012),    # eight splits of seven super-blocks
    (70, 129, 7936, 7013),     # 31 super-blocks, seven splits, ragged M and N
    (150, 129, 7936, 7014),    # 64-token tile: 31 super-blocks, seven splits, ragged M and N
    (137, 1000, 4352, 7015),   # 64-token tile: 17 super-blocks in four splits (4, 4, 4, 5)
]


@pytest.mark.parametrize("M,N,K,seed", GEMM_SPLIT)
def test_gemm_split_full_compare(M, N, K, seed):
    g = wl.rng(seed)
    w = wl.q4k_weights(N, K, g)
    x = wl.activations(M, K, g)
    xqb = oracle.quantize_q8k(x)
    _note("gemm split M=%d N=%d K=%d" % (M, N, K))
    Y = gpu_gemm(w, xqb, M, N, K)
    ref, T = oracle.gemm_q4k(w, xqb, M, N, K)
    assert_close(Y.reshape(-1), ref.reshape(-1), T.reshape(-1), "gemm split")


@pytest.mark.parametrize("M,N,K", [(1, 14336, 4096), (64, 4096, 14336), (65, 4096, 14336),
                                   (256, 4096, 14336)])
def test_gemm_split_full_size(M, N, K):
    """The FFN shapes at token counts that split K: sampled outputs with the
    tile corners, plus whole rows against the mat-vec oracle."""
    g = wl.rng(7300 + M)
    w = wl.q4k_weights(N, K, g)
    x = wl.activations(M, K, g)
    xqb = oracle.quantize_q8k(x)
    _note("gemm split full size M=%d N=%d K=%d" % (M, N, K))
    Y = gpu_gemm(w, xqb, M, N, K)
    assert not np.isnan(Y).any()
    s = wl.rng(7310 + M)
    ms = np.concatenate([s.integers(0, M, 600), [0, M - 1, min(63, M - 1), min(64, M - 1)]])
    ns = np.concatenate([s.integers(0, N, 600), [0, N - 1, 127, 128]])
    ref, T = oracle.gemm_q4k(w, xqb, M, N, K, ms, ns)
    assert_close(Y[ms, ns], ref, T, "split sampled")
    for m in sorted({0, M - 1}):
        ref, T = oracle.gemv_q4k(w, xqb[m], N, K)
        assert_close(Y[m], ref, T, "split row %d" % m)


@pytest.mark.parametrize("M,N,K,first_split_row", [(320, 14336, 4096, 13056), (576, 8192, 4096, 7168),
                                                    (1024, 14336, 4096, 12288)])
def test_gemm_whole_and_split_tiles(M, N, K, first_split_row):
    """More tiles than whole rounds of resident workgroups, with a short
    remainder: the whole rounds run whole tiles and the remainder splits K in
    the same launch (320 tokens: 512 of 560 tiles whole, the rest in four
    splits from weight tile 102 on; 576 tokens: 512 of 576 whole, four
    splits from weight tile 56 on; 1024 tokens: 1536 of 1792 whole, two
    splits from weight tile 96 on). Sampled outputs on both sides of that
    boundary, and whole rows against the mat-vec."""
    g = wl.rng(7600 + M)
    w = wl.q4k_weights(N, K, g)
    xqb = oracle.quantize_q8k(wl.activations(M, K, g))
    _note("gemm whole and split tiles M=%d N=%d K=%d" % (M, N, K))
    Y = gpu_gemm(w, xqb, M, N, K)
    assert not np.isnan(Y).any()
    s = wl.rng(7610 + M)
    ms = np.concatenate([s.integers(0, M, 1200), [0, M - 1, 63, 64, 127, 128, M - 1]])
    ns = np.concatenate([s.integers(0, N, 600), s.integers(first_split_row, N, 600),
                         [first_split_row - 1, first_split_row, N - 1, 0, 127, 128,
                          first_split_row + 127]])
    ref, T = oracle.gemm_q4k(w, xqb, M, N, K, ms, ns)
    assert_close(Y[ms, ns], ref, T, "whole/split sampled")
    for m in sorted({0, 130, M - 1}):
        ref, T = oracle.gemv_q4k(w, xqb[m], N, K)
        assert_close(Y[m], ref, T, "whole/split row %d" % m)


# Short batches run on the mat-vec kernels: one pass over the weights for all
# M tokens, each token's row bit-identical to xq_gemv_q4k on that token.
GEMM_SHORT = [
    (2, 14336, 4096, 7501),    # two rows per wave, clamped
    (3, 14336, 4096, 7502),    # the longest batch on this shape
    (3, 4096, 14336, 7503),    # four units split across a workgroup's waves, three tokens
    (6, 4096, 4096, 7504),     # six tokens on a 2^24-weight matrix (the eight-token instance)
    (5, 300, 2304, 7505),      # ragged unit tail
    (2, 130, 20480, 7506),     # five units (two tokens fit): batches of two, loads past the row skipped
    (6, 8191, 2048, 7507),     # two rows per wave with an odd tail
    (4, 4096, 4096, 7508),     # persistent grid, activation in registers, four tokens
    (3, 3000, 1280, 7509),     # persistent grid, one ragged unit
    (2, 20000, 3840, 7510),    # persistent grid, the unit ragged, rows past one pass
    (4, 100, 256, 7511),       # persistent grid smaller than a workgroup's waves allow
    (2, 4096, 14336, 7512),    # two tokens on four-unit rows: the LDS form
    (2, 1000, 7424, 7519),     # two units (the last ragged) on the LDS form
    (4, 3000, 8192, 7541),     # four tokens, two units (a 2^25-weight matrix)
    (6, 2000, 8192, 7542),     # six tokens fill the LDS at two units
    (6, 2000, 6144, 7543),     # two units, the last half full, the eight-token instance
    (3, 2500, 10240, 7544),    # three units, the four-token instance
    (2, 1500, 12288, 7545),    # three units, below the unit split's row lengths
    (2, 1001, 12544, 7513),    # four units, the last one block, rows past a workgroup's eight
    (3, 4099, 13312, 7514),    # three tokens split over four units, eight rows per workgroup, a ragged row tail
    (8, 4096, 4096, 7562),     # eight tokens on the persistent grid
    (7, 3000, 1280, 7563),     # seven tokens (the eight-token instance), one ragged unit
    (5, 2048, 4096, 7565),     # five tokens (the six-token instance)
]


@pytest.mark.parametrize("M,N,K,seed", GEMM_SHORT)
def test_gemm_short_batch_rows_equal_matvec(M, N, K, seed):
    g = wl.rng(seed)
    w = wl.q4k_weights(N, K, g)
    xqb = oracle.quantize_q8k(wl.activations(M, K, g))
    wd = dev(w)
    _note("gemm short batch M=%d N=%d K=%d" % (M, N, K))
    Y = gpu_gemm(w, xqb, M, N, K)
    for m in range(M):
        y = poisoned_f32(N)
        xq.xq_gemv_q4k(y, wd, dev(xqb[m]), N, K)
        assert np.array_equal(Y[m], take_f32(y, N)), m
    for m in sorted({0, M - 1}):
        ref, T = oracle.gemv_q4k(w, xqb[m], N, K)
        assert_close(Y[m], ref, T, "short batch row %d" % m)


# The 16-token MFMA tile (M <= 32, or M <= 64 on matrices of at most 2^25
# weights), split over K where the tile grid is short of the device.
GEMM_TILE16 = [
    (4, 14336, 8192, 7521),    # four tokens in one 16-token tile, four splits of 8 super-blocks
    (16, 14336, 6144, 7522),   # a full tile, four splits of 6 super-blocks
    (31, 4096, 14336, 7523),   # two tiles, the second ragged, eight splits
    (17, 300, 2304, 7524),     # ragged tokens and rows, nine super-blocks
    (64, 4096, 4096, 7525),    # four tiles on a 2^24-weight matrix
    (16, 4096, 14336, 7526),   # one workgroup per CU: the three-stage ring, 8 splits of 7 super-blocks
    (10, 2000, 2816, 7527),    # the three-stage ring over uneven splits (5 and 6 super-blocks)
    (9, 1000, 4096, 7528),     # the three-stage ring, 4 super-blocks per split
]


@pytest.mark.parametrize("M,N,K,seed", GEMM_TILE16)
def test_gemm_token_tile_16(M, N, K, seed):
    g = wl.rng(seed)
    w = wl.q4k_weights(N, K, g)
    xqb = oracle.quantize_q8k(wl.activations(M, K, g))
    _note("gemm tile16 M=%d N=%d K=%d" % (M, N, K))
    Y = gpu_gemm(w, xqb, M, N, K)
    assert not np.isnan(Y).any()
    if M * N * K <= 2 ** 28:
        ref, T = oracle.gemm_q4k(w, xqb, M, N, K)
        assert_close(Y.reshape(-1), ref.reshape(-1), T.reshape(-1), "tile16")
    else:
        s = wl.rng(seed + 1)
        ms = np.concatenate([s.integers(0, M, 500), [0, M - 1, min(15, M - 1), min(16, M - 1)]])
        ns = np.concatenate([s.integers(0, N, 500), [0, N - 1, 127, 128]])
        ref, T = oracle.gemm_q4k(w, xqb, M, N, K, ms, ns)
        assert_close(Y[ms, ns], ref, T, "tile16 sampled")
        for m in sorted({0, M - 1}):
            ref, T = oracle.gemv_q4k(w, xqb[m], N, K)
            assert_close(Y[m], ref, T, "tile16 row %d" % m)


# Short batches on tall matrices: the wave-split tile (four waves split K,
# their partial tiles summed in LDS; no workspace).
GEMM_WAVE_SPLIT = [
    (6, 14336, 4096, 7551),    # 448 workgroups, four super-blocks per wave
    (16, 14336, 4096, 7552),   # a full token tile
    (7, 8192, 4096, 7553),     # one workgroup per CU
    (16, 8200, 2304, 7554),    # a last row tile of 8 rows; 9 super-blocks (2, 2, 2, 3 per wave)
    (12, 16384, 3840, 7555),   # 512 workgroups; 15 super-blocks (3, 4, 4, 4)
    (5, 11008, 2048, 7556),    # two super-blocks per wave
]


@pytest.mark.parametrize("M,N,K,seed", GEMM_WAVE_SPLIT, ids=["m%d_n%d_k%d" % c[:3] for c in GEMM_WAVE_SPLIT])
def test_gemm_wave_split(M, N, K, seed):
    g = wl.rng(seed)
    w = wl.q4k_weights(N, K, g)
    xqb = oracle.quantize_q8k(wl.activations(M, K, g))
    assert xq.xq_gemm_q4k_small_m_workspace_bytes(M, N, K) == 0
    _note("gemm wave split M=%d N=%d K=%d" % (M, N, K))
    wd, xd = dev(w), dev(xqb)
    outs = []
    for _ in range(2):
        y = poisoned_f32(M * N)
        xq.xq_gemm_q4k_small_m(y, wd, xd, M, N, K)
        outs.append(take_f32(y, M * N).reshape(M, N))
    Y = outs[0]
    assert np.array_equal(outs[1], Y)
    assert not np.isnan(Y).any()
    s = wl.rng(seed + 1)
    corners_m = sorted({0, 3, 4, M - 1} & set(range(M)))
    corners_n = [0, 31, 32, N - 32, N - 1]
    ms = np.concatenate([s.integers(0, M, 800), np.repeat(corners_m, len(corners_n))])
    ns = np.concatenate([s.integers(0, N, 800), np.tile(corners_n, len(corners_m))])
    ref, T = oracle.gemm_q4k(w, xqb, M, N, K, ms, ns)
    assert_close(Y[ms, ns], ref, T, "wave split sampled")
    for m in sorted({0, M - 1}):
        ref, T = oracle.gemv_q4k(w, xqb[m], N, K)
        assert_close(Y[m], ref, T, "wave split row %d" % m)


# Both sides of every dispatch boundary of the small-M product: the batched
# mat-vec against the MFMA tiles (4|5 tokens on rows of one unit, 16 and 8
# super-blocks, where five take the wave-split tile, and 8|9 on such rows of
# 2^24 weights; 3|4 on a large matrix of longer rows, 4|5 on 2^25 weights,
# 6|7 on 2^24, 8|9 on 2^23), the wave-split tile against the 16-token
# tile (16|17 tokens), the 16-token tile against the 64-token tile (32|33 on a
# large matrix, 64|65 on 4096 rows of a long K, 96|97 on 2^25 weights, 128|129
# on 2^24).
GEMM_BOUNDARY = [
    (4, 14336, 4096, 7531),
    (5, 14336, 4096, 7559),
    (5, 11008, 2048, 7560),
    (4, 4096, 14336, 7561),
    (4, 4096, 8192, 7538),
    (5, 4096, 8192, 7539),
    (6, 4096, 4096, 7540),
    (7, 4096, 4096, 7532),
    (9, 4096, 4096, 7564),
    (6, 2048, 8192, 7566),
    (7, 2048, 8192, 7567),
    (4, 8192, 4096, 7546),
    (4, 11008, 2048, 7547),
    (17, 14336, 4096, 7548),
    (32, 14336, 4096, 7533),
    (33, 14336, 4096, 7534),
    (8, 4096, 2048, 7549),
    (64, 4096, 14336, 7550),
    (65, 4096, 14336, 7557),
    (96, 8192, 4096, 7536),
    (97, 8192, 4096, 7537),
    (128, 4096, 4096, 7535),
    (129, 4096, 4096, 7558),
]


@pytest.mark.parametrize("M,N,K,seed", GEMM_BOUNDARY, ids=["m%d_n%d_k%d" % c[:3] for c in GEMM_BOUNDARY])
def test_gemm_dispatch_boundaries(M, N, K, seed):
    g = wl.rng(seed)
    w = wl.q4k_weights(N, K, g)
    xqb = oracle.quantize_q8k(wl.activations(M, K, g))
    _note("gemm dispatch boundary M=%d N=%d K=%d" % (M, N, K))
    Y = gpu_gemm(w, xqb, M, N, K)
    s = wl.rng(seed + 1)
    corners_m = sorted({0, 15, 16, 31, 32, M - 1} & set(range(M)))
    corners_n = [0, 127, 128, N - 1]
    ms = np.concatenate([s.integers(0, M, 600), np.repeat(corners_m, len(corners_n))])
    ns = np.concatenate([s.integers(0, N, 600), np.tile(corners_n, len(corners_m))])
    ref, T = oracle.gemm_q4k(w, xqb, M, N, K, ms, ns)
    assert_close(Y[ms, ns], ref, T, "boundary sampled")
    ref, T = oracle.gemv_q4k(w, xqb[M - 1], N, K)
    assert_close(Y[M - 1], ref, T, "boundary last row")


def test_gemm_mfma_below_eight_tokens():
    """Five tokens whose q8_K rows exceed the mat-vec's LDS cap (K = 14336
    holds three): the MFMA product, split over K."""
    M, N, K = 5, 200, 14336
    g = wl.rng(7510)
    w = wl.q4k_weights(N, K, g)
    xqb = oracle.quantize_q8k(wl.activations(M, K, g))
    _note("gemm mfma five tokens")
    Y = gpu_gemm(w, xqb, M, N, K)
    ref, T = oracle.gemm_q4k(w, xqb, M, N, K)
    assert_close(Y.reshape(-1), ref.reshape(-1), T.reshape(-1), "mfma five tokens")


def test_gemm_split_repeatable_across_calls_and_streams():
    """Bit-identical results on repeated calls through one workspace (the
    arrival counters reset themselves), through a workspace at another
    address, on a second stream with its own workspace, and after the
    workspace served a call of another shape."""
    M, N, K = 40, 640, 8192
    g = wl.rng(7400)
    wd = dev(wl.q4k_weights(N, K, g))
    xd = dev(oracle.quantize_q8k(wl.activations(M, K, g)))
    need = xq.xq_gemm_q4k_small_m_workspace_bytes(M, N, K)
    assert need > 0
    _note("gemm split repeat")
    ws = zeroed_workspace(need + 4096)
    outs = []
    for _ in range(3):
        y = poisoned_f32(M * N)
        xq.xq_gemm_q4k_small_m(y, wd, xd, M, N, K, workspace=ws)
        outs.append(take_f32(y, M * N))
    other = zeroed_workspace(need + 4096)[1024:]          # another address, 256-aligned
    y = poisoned_f32(M * N)
    xq.xq_gemm_q4k_small_m(y, wd, xd, M, N, K, workspace=other)
    outs.append(take_f32(y, M * N))
    side = torch.cuda.Stream()
    ws_side = zeroed_workspace(need)
    with torch.cuda.stream(side):
        y = poisoned_f32(M * N)
        xq.xq_gemm_q4k_small_m(y, wd, xd, M, N, K, workspace=ws_side)
    side.synchronize()
    outs.append(take_f32(y, M * N))
    # the first workspace serves a smaller split shape, then this one again
    M2, K2 = 20, 4096
    assert 0 < xq.xq_gemm_q4k_small_m_workspace_bytes(M2, N, K2) <= need + 4096
    y2 = poisoned_f32(M2 * N)
    xq.xq_gemm_q4k_small_m(y2, wd, dev(oracle.quantize_q8k(wl.activations(M2, K2, g))), M2, N,
                           K2, workspace=ws)
    take_f32(y2, M2 * N)
    y = poisoned_f32(M * N)
    xq.xq_gemm_q4k_small_m(y, wd, xd, M, N, K, workspace=ws)
    outs.append(take_f32(y, M * N))
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])
    assert not np.isnan(outs[0]).any()


def test_gemm_split_graph_capture_first_use():
    """A split call captured into a HIP graph on its workspace's first use
    (the caller zeroed it before the capture) replays to the eager result bit
    for bit, three times, with eager work between the replays."""
    M, N, K = 16, 4096, 14336
    g = wl.rng(7410)
    wd = dev(wl.q4k_weights(N, K, g))
    xd = dev(oracle.quantize_q8k(wl.activations(M, K, g)))
    need = xq.xq_gemm_q4k_small_m_workspace_bytes(M, N, K)
    assert need > 0
    _note("gemm split graph capture")
    y_eager = poisoned_f32(M * N)
    xq.xq_gemm_q4k_small_m(y_eager, wd, xd, M, N, K, workspace=zeroed_workspace(need))
    want = take_f32(y_eager, M * N)
    ws = zeroed_workspace(need)
    y = poisoned_f32(M * N)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        xq.xq_gemm_q4k_small_m(y, wd, xd, M, N, K, workspace=ws)
    for r in range(3):
        y[:M * N].fill_(float("nan"))
        graph.replay()
        assert np.array_equal(take_f32(y, M * N), want), "replay %d" % r
        y_e = poisoned_f32(M * N)                            # eager work between replays
        xq.xq_gemm_q4k_small_m(y_e, wd, xd, M, N, K, workspace=zeroed_workspace(need))
        assert np.array_equal(take_f32(y_e, M * N), want)


def test_gemm_prefill_512x14336x4096():
    M, N, K = 512, 14336, 4096
    g = wl.rng(wl.SEEDS["prefill"])
    w = wl.q4k_weights(N, K, g)
    x = wl.activations(M, K, g)
    xqb = oracle.quantize_q8k(x)
    _note("gemm prefill full size")
    Y = gpu_gemm(w, xqb, M, N, K)
    assert not np.isnan(Y).any()
    # Sampled outputs, including every tile corner.
    s = wl.rng(7100)
    ms = np.concatenate([s.integers(0, M, 3000), [0, 0, M - 1, M - 1, 127, 128, 255, 256]])
    ns = np.concatenate([s.integers(0, N, 3000), [0, N - 1, 0, N - 1, 127, 128, 14207, 14208]])
    ref, T = oracle.gemm_q4k(w, xqb, M, N, K, ms, ns)
    assert_close(Y[ms, ns], ref, T, "prefill sampled")
    # Whole rows of Y for a few tokens.
    for m in (0, 200, 511):
        ref, T = oracle.gemv_q4k(w, xqb[m], N, K)
        assert_close(Y[m], ref, T, "prefill row %d" % m)


@pytest.mark.parametrize("which", ["S", "M"])
@pytest.mark.parametrize("M,N,K", [(3, 200, 1024), (9, 200, 1024), (9, 200, 3584), (130, 200, 1024),
                                   (9, 8192, 2048)])
def test_gemm_partials_bit_exact(which, M, N, K):
    """M = 3 runs on the batched mat-vec, M = 9 on the 16-token MFMA tile
    (K = 3584: three splits) or, on 8192 rows, the wave-split tile (two
    super-blocks per wave), M = 130 on the 64-token tile."""
    g = wl.rng(7200)
    w = wl.q4k_isolation_weights(N, K, g, which)
    wd = dev(w)
    for b in range(K // 256):
        x = wl.isolating_activation(M, K, g, b)
        xqb = oracle.quantize_q8k(x)
        _note("gemm partial %s block %d" % (which, b))
        y = poisoned_f32(M * N)
        xq.xq_gemm_q4k_small_m(y, wd, dev(xqb), M, N, K, workspace=gemm_workspace(M, N, K))
        got = take_f32(y, M * N).reshape(M, N)
        for m in range(M):
            S, Mp = oracle.q4k_partials(w, xqb[m], N, K)
            want = S[:, b] if which == "S" else -Mp[:, b]
            assert np.array_equal(got[m], want.astype(np.float64)), (m, b)


def _stream_fold_model(words: np.ndarray) -> np.ndarray:
    """Host model of the streaming probe's fold: 512 lanes per workgroup, lane t
    reads 16-byte chunks g*1024+t and g*1024+512+t (chunks past the end count
    zero), xors each chunk's four words, adds the two (mod 2^32), and the
    workgroup stores the xor of its eight wave sums of (acc & 0xFFFF) as f32 bits."""
    n16 = words.size // 4
    chunk = np.bitwise_xor.reduce(words.reshape(n16, 4).astype(np.uint32), axis=1)
    groups = (n16 + 1023) // 1024
    padded = np.zeros(groups * 1024, dtype=np.uint32)
    padded[:n16] = chunk
    per = padded.reshape(groups, 2, 512)
    acc = (per[:, 0, :].astype(np.uint64) + per[:, 1, :]) & 0xFFFFFFFF
    lo = (acc & 0xFFFF).astype(np.float64).reshape(groups, 8, 64).sum(axis=2)
    bits = lo.astype(np.float32).view(np.uint32)
    return np.bitwise_xor.reduce(bits, axis=1).view(np.int32)


@pytest.mark.parametrize("nbytes", [1 << 24, (1 << 20) + 16 * 777])
def test_stream_read_probe_reads_every_chunk(nbytes):
    g = wl.rng(9100 + nbytes % 1000)
    words = g.integers(0, 2**32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(words.view(np.int32)).to("cuda")
    sink = torch.zeros(xq.xq_bench_sink_words(nbytes), dtype=torch.int32, device="cuda")
    _note("stream_read probe nbytes=%d" % nbytes)
    xq.xq_bench_stream_read(buf, nbytes, sink)
    torch.cuda.synchronize()
    assert np.array_equal(sink.cpu().numpy(), _stream_fold_model(words))


# ---------------------------------------------------------------------------
# Degenerate inputs
# ---------------------------------------------------------------------------

def _subnormal_scales(g, shape):
    """f16 bit patterns: a random half subnormal (0x0001..0x03FF), the rest
    small normals (0x0400..0x2400, up to about 0.0156); a random quarter of
    either kind negative (the formats store signed f16 scales)."""
    sub = g.integers(1, 0x400, size=shape, dtype=np.uint16)
    nor = g.integers(0x400, 0x2401, size=shape, dtype=np.uint16)
    bits = np.where(g.random(shape) < 0.5, sub, nor)
    bits = np.where(g.random(shape) < 0.25, bits | 0x8000, bits)
    return bits.astype("<u2")


def test_subnormal_block_scales():
    """f16 block scales that are subnormal or negative (valid f16 numbers the
    weights' scales can take) decode as the oracle's f16 decoder does, on the Q4_K
    mat-vec, the batched mat-vec, the 16- and 64-token MFMA tiles, and the
    IQ4_NL and Q4_0 mat-vecs."""
    g = wl.rng(7700)
    N, K = 1000, 2048
    nb = K // 256
    w = wl.q4k_weights(N, K, g)
    w[:, :, 0:2] = _subnormal_scales(g, (N, nb)).view(np.uint8).reshape(N, nb, 2)
    w[:, :, 2:4] = _subnormal_scales(g, (N, nb)).view(np.uint8).reshape(N, nb, 2)
    _note("subnormal scales: Q4_K mat-vec")
    xqb = oracle.quantize_q8k(wl.activations(1, K, g))
    ref, T = oracle.gemv_q4k(w, xqb, N, K)
    assert_close(gpu_gemv_q4k(w, xqb, N, K), ref, T, "q4k subnormal")
    for M in (3, 70, 130):
        _note("subnormal scales: Q4_K product M=%d" % M)
        xqm = oracle.quantize_q8k(wl.activations(M, K, g))
        ref, T = oracle.gemm_q4k(w, xqm, M, N, K)
        Y = gpu_gemm(w, xqm, M, N, K)
        assert_close(Y.reshape(-1), ref.reshape(-1), T.reshape(-1), "gemm subnormal M=%d" % M)
    wi = wl.iq4nl_weights(N, K, g)
    bpr = K // 32
    wi[:, 0:2 * bpr] = _subnormal_scales(g, (N, bpr)).view(np.uint8).reshape(N, 2 * bpr)
    _note("subnormal scales: IQ4_NL and Q4_0 mat-vecs")
    ref, T = oracle.gemv_iq4nl(wi, xqb, N, K)
    assert_close(gpu_gemv_iq4nl(wi, xqb, N, K), ref, T, "iq4nl subnormal")
    y = poisoned_f32(N)
    xq.xq_gemv_q4_0(y, dev(wi), dev(xqb), N, K)
    ref, T = oracle.gemv_q4_0(wi, xqb, N, K)
    assert_close(take_f32(y, N), ref, T, "q4_0 subnormal")


def test_zero_activations_give_exact_zeros():
    """An all-zero activation quantizes to d = 0 and codes 0 (the quantizer's
    zero-block case); every path then outputs exactly 0.0, with no NaN from
    the zero scale. Zero token rows inside a batch stay exactly zero while
    the other rows match the oracle."""
    N, K = 300, 4096
    g = wl.rng(7700)
    wq = wl.q4k_weights(N, K, g)
    wi = wl.iq4nl_weights(N, K, g)
    zero = np.zeros((1, K), np.float32)
    zq = oracle.quantize_q8k(zero)
    assert not zq[:, :, :292].any()
    _note("zero activations")
    for name, fn, w in (("q4k", xq.xq_gemv_q4k, wq), ("iq4nl", xq.xq_gemv_iq4nl, wi),
                        ("q4_0", xq.xq_gemv_q4_0, wi)):
        y = poisoned_f32(N)
        fn(y, dev(w), dev(zq), N, K)
        got = take_f32(y, N)
        assert np.array_equal(got, np.zeros(N)), name
    for M in (3, 16, 130):  # batched mat-vec, 16-token tile, 64-token tile
        x = wl.activations(M, K, g)
        x[1::2] = 0.0
        xqb = oracle.quantize_q8k(x)
        Y = gpu_gemm(wq, xqb, M, N, K)
        assert np.array_equal(Y[1::2], np.zeros_like(Y[1::2])), M
        ref, T = oracle.gemm_q4k(wq, xqb, M, N, K)
        assert_close(Y.reshape(-1), ref.reshape(-1), T.reshape(-1), "zero rows M=%d" % M)


@pytest.mark.parametrize("K", [49152, 53248])
def test_gemm_max_k(K):
    """The product at K = 49152 (192 super-blocks, the longest row the
    mat-vecs stage in LDS) and past it, with ragged tokens and rows."""
    M, N = 20, 130
    g = wl.rng(7710)
    w = wl.q4k_weights(N, K, g)
    xqb = oracle.quantize_q8k(wl.activations(M, K, g))
    _note("gemm max K %d" % K)
    Y = gpu_gemm(w, xqb, M, N, K)
    ref, T = oracle.gemm_q4k(w, xqb, M, N, K)
    assert_close(Y.reshape(-1), ref.reshape(-1), T.reshape(-1), "gemm max K")
