"""Pins of the CPU oracle: checks against closed forms, invariants, special
cases, brute force and the pages' own deterministic activation.

Each ``pin_*`` takes a loaded oracle build and raises AssertionError when the
build disagrees with what the pages or the mathematics fix. The default build
must pass all of them; builds with one planted mistake must fail at least one
(``test_oracle_instrument.py``).

None of these checks retypes the oracle's formula: each compares it with a
value fixed some other way (an exact rational, a constructed block whose
dequantized values are known by construction, numpy's own float16 decoder,
a brute-force dot of separately dequantized operands, or an error bound
against the unquantized input).
"""

from __future__ import annotations

import os
from fractions import Fraction

import numpy as np

import workloads as wl

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _f32(v) -> np.float32:
    return np.float32(v)


def _q8k_fields(blk: np.ndarray):
    """(codes int8[256], sums int32[8], scale f32) of one stored q8_K block,
    read straight from the byte offsets of section 25.2.1 of "25 — Writing
    XPU Kernels" (+0 codes, +256 sums, +288 scale)."""
    blk = np.ascontiguousarray(blk, dtype=np.uint8)
    codes = blk[0:256].view(np.int8).astype(np.int64)
    sums = blk[256:288].view("<i4").astype(np.int64)
    scale = blk[288:292].view("<f4")[0]
    return codes, sums, scale


# ---------------------------------------------------------------------------
# f16
# ---------------------------------------------------------------------------

def pin_f16_exhaustive(o):
    """All 65536 binary16 patterns against numpy's float16 -> float64."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([o.f16_to_f64(int(b)) for b in bits], dtype=np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # signed zero is kept
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


# ---------------------------------------------------------------------------
# q8_K quantizer
# ---------------------------------------------------------------------------

def pin_q8k_constant(o):
    """x == c in a block: every code is sign(c)*127, every sum is 32x that and
    the scale is the f32 quotient |c|/127."""
    for c in (0.37, 1e-3, 5.0, -2.25, 3.0e-20):
        x = np.full((1, 256), c, dtype=np.float32)
        codes, sums, scale = _q8k_fields(o.quantize_q8k(x)[0, 0])
        s = 1 if c > 0 else -1
        assert np.all(codes == 127 * s), c
        assert np.all(sums == 4064 * s), c
        assert scale == _f32(abs(_f32(c))) / _f32(127.0), c


def pin_q8k_zero(o):
    """An all-zero block has scale 0, codes 0 and sums 0."""
    blk = o.quantize_q8k(np.zeros((1, 256), dtype=np.float32))[0, 0]
    assert np.all(blk[:292] == 0)


def pin_q8k_unit_scale_ties(o):
    """With one element equal to 127 and the rest in [-127, 127] the scale is
    exactly 1, so each code is its input rounded to nearest. Halves separate
    ties-to-even (0.5 -> 0, 1.5 -> 2, 2.5 -> 2) from ties-away (1, 2, 3)."""
    g = wl.rng(7)
    x = np.round(g.uniform(-126.0, 126.0, size=256) * 4.0) / 4.0
    specials = [127.0, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 62.5, -126.5, 3.25, -3.75,
                125.5, -125.5, 0.0, -0.0, 63.5]
    x[: len(specials)] = specials
    x = x.astype(np.float32).reshape(1, 256)
    codes, sums, scale = _q8k_fields(o.quantize_q8k(x)[0, 0])
    assert scale == np.float32(1.0)
    # Python's round() on an exactly representable float rounds half to even.
    want = np.array([round(float(v)) for v in x[0]], dtype=np.int64)
    assert np.array_equal(codes, want), np.nonzero(codes != want)
    assert codes[1] == 0 and codes[2] == 2 and codes[3] == 2
    assert np.array_equal(sums, want.reshape(8, 32).sum(axis=1))


def pin_q8k_pages_pattern(o):
    """The activation x_j = ((j mod 25) - 12)/64 of section 25.7.1 of "25 —
    Writing XPU Kernels" at 2048 columns. amax = 12/64, so the exact code of an
    element with k = (j mod 25) - 12 is k*127/12 rounded; k = +-6 lands on the
    tie +-63.5 exactly in f32, which both tie rules send to +-64. Every other
    k is at least 1/12 away from a half, so f32 rounding cannot move it."""
    K = 2048
    x = wl.pages_activation(K).reshape(1, K)
    xq = o.quantize_q8k(x)[0]
    with open(os.path.join(GOLDEN, "pages_pattern_q8k.txt")) as f:
        gold = {}
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, val = line.split("=")
            gold[key.strip()] = val.strip()
    scale_bits = int(gold["scale_bits"], 16)
    table = [int(v) for v in gold["codes_k_minus12_to_12"].split(",")]
    for b in range(K // 256):
        codes, sums, scale = _q8k_fields(xq[b])
        assert int(np.array(scale).view(np.uint32)) == scale_bits
        j = np.arange(b * 256, (b + 1) * 256)
        k = (j % 25) - 12
        want = np.array([table[kk + 12] for kk in k], dtype=np.int64)
        # the stored table is the exact rational rounding
        assert all(table[kk + 12] == round(Fraction(kk * 127, 12)) for kk in range(-12, 13))
        assert np.array_equal(codes, want)
        assert np.array_equal(sums, want.reshape(8, 32).sum(axis=1))


def pin_q8k_invariants(o):
    """Random rows: |code| <= 127, max |code| = 127, |x - d*code| <= d*(1/2 +
    2^-17) (round to nearest, the slack covering the f32 quotient's rounding),
    the scale is the f32 quotient amax/127, sums are the sums of the codes and
    the undefined tail is zero."""
    g = wl.rng(11)
    x = g.standard_normal((4, 1024)).astype(np.float32)
    x[1] *= np.float32(1e-3)
    x[2, 5] = np.float32(40.0)             # an outlier
    x[3] = np.abs(x[3])                    # all positive
    xq = o.quantize_q8k(x)
    for r in range(4):
        for b in range(4):
            codes, sums, scale = _q8k_fields(xq[r, b])
            xb = x[r, b * 256:(b + 1) * 256]
            amax = np.max(np.abs(xb))
            assert scale == _f32(amax) / _f32(127.0)
            assert np.all(np.abs(codes) <= 127)
            assert np.max(np.abs(codes)) == 127
            err = np.abs(xb.astype(np.float64) - float(scale) * codes.astype(np.float64))
            assert np.all(err <= float(scale) * (0.5 + 2.0 ** -17))
            assert np.array_equal(sums, codes.reshape(8, 32).sum(axis=1))
            assert np.all(xq[r, b, 292:] == 0)


# ---------------------------------------------------------------------------
# Q4_K
# ---------------------------------------------------------------------------

def pin_q4k_pack_roundtrip(o):
    """The 6-bit header packing: unpack(pack(sc, m)) == (sc, m) for random
    fields, and pack(unpack(bytes)) == bytes for random header bytes (the
    packing is a bijection of 96 bits)."""
    g = wl.rng(13)
    for _ in range(50):
        sc = g.integers(0, 64, 8)
        m = g.integers(0, 64, 8)
        blk = wl.q4k_block(0.5, 0.25, sc, m, np.zeros(128, np.uint8))
        for j in range(8):
            assert o.q4k_scale_min(blk, j) == (sc[j], m[j]), (j, sc, m)
    for _ in range(50):
        blk = np.zeros(144, np.uint8)
        blk[4:16] = g.integers(0, 256, 12, dtype=np.uint8)
        pairs = [o.q4k_scale_min(blk, j) for j in range(8)]
        sc = [p[0] for p in pairs]
        m = [p[1] for p in pairs]
        assert np.array_equal(wl.pack_q4k_scales(sc, m), blk[4:16])


def pin_q4k_closed_forms(o):
    """Constructed blocks whose dequantized weights are known by construction:
    nibbles 0 give -dmin*m_j; nibbles 15 with m = 0 give 15*d*sc_j; distinct
    nibble patterns with unit scale give back the nibbles in the stated order
    (group g at byte 16+32g, low nibble = sub-block 2g, high = 2g+1)."""
    sc = np.arange(1, 9)
    m = np.arange(10, 18)
    # all nibbles zero
    blk = wl.q4k_block(2.0, 0.5, sc, m, np.zeros(128, np.uint8))
    w = o.dequant_q4k(blk, 1, 256)[0]
    want = np.repeat(-0.5 * m.astype(np.float64), 32)
    assert np.array_equal(w, want)
    # all nibbles 15, no mins
    blk = wl.q4k_block(0.125, 0.5, sc, np.zeros(8, int), np.full(128, 0xFF, np.uint8))
    w = o.dequant_q4k(blk, 1, 256)[0]
    assert np.array_equal(w, np.repeat(15 * 0.125 * sc.astype(np.float64), 32))
    # distinct nibbles, unit scale
    nib = np.zeros(128, np.uint8)
    want = np.zeros(256, np.float64)
    for gidx in range(4):
        for t in range(32):
            lo = (t + gidx) % 16
            hi = (t + 3 * gidx + 5) % 16
            nib[32 * gidx + t] = lo | (hi << 4)
            want[64 * gidx + t] = lo
            want[64 * gidx + 32 + t] = hi
    blk = wl.q4k_block(1.0, 0.0, np.ones(8, int), np.zeros(8, int), nib)
    assert np.array_equal(o.dequant_q4k(blk, 1, 256)[0], want)
    for i in (0, 31, 32, 63, 64, 200, 255):
        assert o.q4k_code(blk, i) == want[i]


def _rand_q4k_case(seed, N, K, R=1):
    g = wl.rng(seed)
    w = wl.q4k_weights(N, K, g)
    x = wl.activations(R, K, g)
    return w, x


def pin_q4k_one_hot(o):
    """A one-hot activation x = 127*e_p quantizes to scale 1 and code 127 at p
    (other blocks zero), so y_r = 127*w_rp exactly and the partials of p's
    block are S = 127*sc_j*q_p, M = 127*m_j."""
    N, K = 3, 512
    w, _ = _rand_q4k_case(17, N, K)
    wd = o.dequant_q4k(w, N, K)
    for p in (0, 31, 32, 100, 255, 256, 300, 511):
        x = np.zeros((1, K), np.float32)
        x[0, p] = 127.0
        xq = o.quantize_q8k(x)
        y, _ = o.gemv_q4k(w, xq, N, K)
        assert np.array_equal(y, 127.0 * wd[:, p]), p
        S, M = o.q4k_partials(w, xq, N, K)
        b = p // 256
        for r in range(N):
            blk = w[r, b]
            i = p % 256
            j = (i // 64) * 2 + ((i % 64) >= 32)
            sc, mm = o.q4k_scale_min(blk, j)
            q = o.q4k_code(blk, i)
            assert S[r, b] == 127 * sc * q and M[r, b] == 127 * mm
            assert np.all(S[r, np.arange(K // 256) != b] == 0)


def pin_q4k_brute_force(o):
    """The mat-vec against a numpy f64 dot of the separately dequantized
    weights and activation, within 1e-12 of the magnitude sum."""
    for seed, N, K in ((19, 5, 768), (23, 2, 256), (29, 4, 2048)):
        w, x = _rand_q4k_case(seed, N, K)
        xq = o.quantize_q8k(x)
        y, T = o.gemv_q4k(w, xq, N, K)
        ref = o.dequant_q4k(w, N, K) @ o.dequant_q8k(xq, 1, K)[0]
        assert np.all(np.abs(y - ref) <= 1e-12 * T)


def pin_q4k_error_bound(o):
    """Against the unquantized activation: |y_r - sum_i w_ri x_i| <=
    sum_i |w_ri| * d_b(i) * (1/2 + 2^-17), the quantizer's round-to-nearest
    bound carried through the dot."""
    N, K = 6, 1024
    w, x = _rand_q4k_case(31, N, K)
    xq = o.quantize_q8k(x)
    y, T = o.gemv_q4k(w, xq, N, K)
    wd = o.dequant_q4k(w, N, K)
    d = np.repeat(xq[0, :, 288:292].copy().view("<f4").astype(np.float64).reshape(-1), 256)
    exact = wd @ x[0].astype(np.float64)
    bound = np.abs(wd) @ (d * (0.5 + 2.0 ** -17))
    assert np.all(np.abs(y - exact) <= bound + 1e-12 * T)


def pin_q4k_partials(o):
    """Partials against values fixed elsewhere: the plain-definition output is
    sum_b xs_b*(d*S - dmin*M); M equals sum_j m_j*s_j over the sums stored in
    the q8_K block; nibbles 15 with m = 0 give S = 15*sum_j sc_j*s_j."""
    N, K = 4, 1024
    w, x = _rand_q4k_case(37, N, K)
    xq = o.quantize_q8k(x)
    S, M = o.q4k_partials(w, xq, N, K)
    y, T = o.gemv_q4k(w, xq, N, K)
    nb = K // 256
    xs = np.array([_q8k_fields(xq[0, b])[2] for b in range(nb)], np.float64)
    sums = np.array([_q8k_fields(xq[0, b])[1] for b in range(nb)])
    d = w[:, :, 0:2].copy().view("<f2").astype(np.float64).reshape(N, nb)
    dmin = w[:, :, 2:4].copy().view("<f2").astype(np.float64).reshape(N, nb)
    yp = (xs[None, :] * (d * S - dmin * M)).sum(axis=1)
    assert np.all(np.abs(yp - y) <= 1e-12 * T)
    for r in range(N):
        for b in range(nb):
            mins = np.array([o.q4k_scale_min(w[r, b], j)[1] for j in range(8)])
            assert M[r, b] == int((mins * sums[b]).sum())
    # nibbles all 15, no mins
    g = wl.rng(41)
    sc = g.integers(0, 64, 8)
    blk = wl.q4k_block(1.0, 1.0, sc, np.zeros(8, int), np.full(128, 0xFF, np.uint8))
    x1 = g.standard_normal((1, 256)).astype(np.float32)
    xq1 = o.quantize_q8k(x1)
    S1, M1 = o.q4k_partials(blk, xq1, 1, 256)
    s1 = _q8k_fields(xq1[0, 0])[1]
    assert S1[0, 0] == 15 * int((sc * s1).sum()) and M1[0, 0] == 0


# ---------------------------------------------------------------------------
# The magnitude sums that scale the f32 bar
# ---------------------------------------------------------------------------
# T: over the row's blocks, |d*xs*S| + |dmin*xs*M| (Q4_K) or |d_c*xs*D_c|
# (IQ4_NL, Q4_0): the magnitudes of the terms the integer route adds.
# Te: over the row's elements, |d*sc*q*xhat| + |dmin*m*xhat| (or |d_c*kv*xhat|).
# Both are fixed here by construction, never by retyping them.

def _q4k_parts(o, w, N, K):
    """The scale part d*sc*q and the min part -dmin*m of every weight, each
    through the oracle's dequantizer (pinned above) on a copy of the blocks
    with the other f16 zeroed: dmin = 0 leaves d*sc*q, d = 0 leaves -dmin*m."""
    w = np.array(w, dtype=np.uint8, copy=True).reshape(N, K // 256, 144)
    ws = w.copy()
    ws[:, :, 2:4] = 0
    wm = w.copy()
    wm[:, :, 0:2] = 0
    return o.dequant_q4k(ws, N, K), o.dequant_q4k(wm, N, K)


def pin_q4k_magnitudes_one_hot(o):
    """x = 127*e_p: one element and one block contribute, xhat = 127, so
    T = Te = 127*(|d*sc_j*q_p| + |dmin*m_j|) for every row, exactly."""
    N, K = 3, 512
    w, _ = _rand_q4k_case(17, N, K)
    ws, wm = _q4k_parts(o, w, N, K)
    for p in (0, 31, 32, 100, 255, 256, 300, 511):
        x = np.zeros((1, K), np.float32)
        x[0, p] = 127.0
        y, T, Te = o.gemv_q4k(w, o.quantize_q8k(x), N, K, elem=True)
        want = 127.0 * (np.abs(ws[:, p]) + np.abs(wm[:, p]))
        assert np.array_equal(T, want), (p, T, want)
        assert np.array_equal(Te, want), (p, Te, want)


def pin_q4k_magnitudes_cancel(o):
    """Codes +127 and -127 (scale 1) on two weights of one block whose scale
    parts are equal and whose mins are equal: S = M = 0, so y = 0 and T = 0,
    while Te = 2*127*(|d*sc*q| + |dmin*m|). Once within one sub-block (equal
    nibbles), once across two sub-blocks of one block (sc_1*q_1 = sc_2*q_2,
    m_1 = m_2): T is per block, not per sub-block. The same pair in two
    different blocks does not cancel: T = Te. Unequal nibbles in one sub-block
    leave S = 127*sc*(q1 - q2) and M = 0."""
    sc = np.array([6, 3, 9, 2, 5, 7, 1, 4])
    m = np.array([11, 11, 20, 8, 3, 63, 0, 17])
    nib = np.zeros(128, np.uint8)
    nib[0:32] = 4 | (8 << 4)       # sub-block 0: q = 4 (sc*q = 24); sub-block 1: q = 8 (24)
    nib[32:64] = 9 | (2 << 4)      # sub-block 2: q = 9; sub-block 3: q = 2
    nib[5] = 13 | (8 << 4)         # weight 5 of sub-block 0 gets q = 13
    d, dmin = 0.5, 0.25
    blk = wl.q4k_block(d, dmin, sc, m, nib)

    def run(w, K, plus, minus):
        x = np.zeros((1, K), np.float32)
        x[0, plus] = 127.0
        x[0, minus] = -127.0
        return o.gemv_q4k(w, o.quantize_q8k(x), 1, K, elem=True)

    one_pair = 2 * 127.0 * (d * 24 + dmin * 11)
    y, T, Te = run(blk, 256, 0, 7)          # same sub-block, equal nibbles
    assert y[0] == 0.0 and T[0] == 0.0 and Te[0] == one_pair, (y, T, Te)
    y, T, Te = run(blk, 256, 1, 40)         # sub-blocks 0 and 1, 6*4 == 3*8, m equal
    assert y[0] == 0.0 and T[0] == 0.0 and Te[0] == one_pair, (y, T, Te)
    two = np.stack([blk, blk]).reshape(1, 2, 144)
    y, T, Te = run(two, 512, 0, 256 + 7)    # the same weights in two blocks
    assert y[0] == 0.0 and T[0] == one_pair and Te[0] == one_pair, (y, T, Te)
    y, T, Te = run(blk, 256, 5, 0)          # q 13 against q 4 in sub-block 0
    assert T[0] == 127.0 * d * 6 * (13 - 4), T
    assert Te[0] == 127.0 * (d * 6 * (13 + 4) + 2 * dmin * 11), Te


def pin_q4k_magnitudes_brute_force(o):
    """Random rows: Te = |scale parts| . |xhat| + |min parts| . |xhat| and
    T = sum over blocks of |scale parts . xhat| + |min parts . xhat|, from
    the separately dequantized operands; |y| <= T <= Te; with every xhat >= 0
    and no mins every term is non-negative, so y = T = Te."""
    for seed, N, K in ((71, 4, 1024), (73, 3, 256)):
        w, x = _rand_q4k_case(seed, N, K)
        xq = o.quantize_q8k(x)
        y, T, Te = o.gemv_q4k(w, xq, N, K, elem=True)
        ws, wm = _q4k_parts(o, w, N, K)
        xh = o.dequant_q8k(xq, 1, K)[0]
        te = np.abs(ws) @ np.abs(xh) + np.abs(wm) @ np.abs(xh)
        assert np.all(np.abs(Te - te) <= 1e-12 * te)
        nb = K // 256
        tb = (np.abs((ws * xh).reshape(N, nb, 256).sum(axis=2)).sum(axis=1) +
              np.abs((wm * xh).reshape(N, nb, 256).sum(axis=2)).sum(axis=1))
        assert np.all(np.abs(T - tb) <= 1e-12 * te)
        assert np.all(np.abs(y) <= T * (1 + 1e-12)) and np.all(T <= Te * (1 + 1e-12))
        # one sign everywhere: mins 0, activation >= 0
        wz = np.array(w, copy=True).reshape(N, nb, 144)
        wz[:, :, 2:4] = 0
        xq_pos = o.quantize_q8k(np.abs(x))
        y, T, Te = o.gemv_q4k(wz, xq_pos, N, K, elem=True)
        assert np.all(np.abs(y - T) <= 1e-12 * T) and np.all(np.abs(T - Te) <= 1e-12 * T)


def pin_iq4nl_magnitudes(o):
    """A row of nibbles t with unit scales: each 32-block's D_c = kv[t]*s_c
    (s_c the q8_K's stored sum of the block's 32 codes), so
    T = sum_c |kv[t]|*xs*|s_c| and Te = |kv[t]| * sum |xhat|. A pair of codes
    +127/-127 on equal nibbles of one 32-block cancels: T = 0, y = 0,
    Te = 2*127*|d*kv|. The same for Q4_0, with kv[t] replaced by t - 8."""
    kv = _codebook_golden()
    K = 512
    x = wl.activations(1, K, wl.rng(79))
    xq = o.quantize_q8k(x)
    xh = o.dequant_q8k(xq, 1, K)[0]
    sums = np.concatenate([_q8k_fields(xq[0, b])[1] for b in range(K // 256)])
    xs = np.repeat(np.array([_q8k_fields(xq[0, b])[2] for b in range(K // 256)], np.float64), 8)
    for fmt, val, gemv in (("iq4nl", lambda t: kv[t], o.gemv_iq4nl),
                           ("q4_0", lambda t: t - 8, o.gemv_q4_0)):
        for t in range(16):
            row = _iq4nl_row(K, np.ones(K // 32), np.full(16 * (K // 32), t | (t << 4), np.uint8))
            y, T, Te = gemv(row, xq, 1, K, elem=True)
            v = abs(val(t))
            tb = float((v * xs * np.abs(sums)).sum())
            te = float(v * np.abs(xh).sum())
            assert abs(T[0] - tb) <= 1e-12 * te and abs(Te[0] - te) <= 1e-12 * te, (fmt, t)
        scales = np.full(K // 32, 0.5)
        pay = np.full(16 * (K // 32), 3 | (12 << 4), np.uint8)
        row = _iq4nl_row(K, scales, pay)
        xc = np.zeros((1, K), np.float32)
        xc[0, 33] = 127.0                   # block 1, low nibble 3
        xc[0, 40] = -127.0                  # block 1, low nibble 3
        y, T, Te = gemv(row, o.quantize_q8k(xc), 1, K, elem=True)
        assert y[0] == 0.0 and T[0] == 0.0, (fmt, y, T)
        assert Te[0] == 2 * 127.0 * 0.5 * abs(val(3)), (fmt, Te)


def pin_q4k_gemm_rows(o):
    """Each output of the small-M product equals the mat-vec of that token's
    activation row, and sampled pairs equal the full product."""
    M_, N, K = 3, 5, 512
    w, x = _rand_q4k_case(43, N, K, R=M_)
    xq = o.quantize_q8k(x)
    Y, T, Te = o.gemm_q4k(w, xq, M_, N, K, elem=True)
    for m in range(M_):
        y, t, te = o.gemv_q4k(w, xq[m], N, K, elem=True)
        assert np.array_equal(Y[m], y) and np.array_equal(T[m], t) and np.array_equal(Te[m], te)
    ms = np.array([2, 0, 1, 2])
    ns = np.array([4, 0, 3, 1])
    Ys, _ = o.gemm_q4k(w, xq, M_, N, K, ms, ns)
    assert np.array_equal(Ys, Y[ms, ns])


# ---------------------------------------------------------------------------
# IQ4_NL
# ---------------------------------------------------------------------------

def _codebook_golden():
    with open(os.path.join(GOLDEN, "iq4nl_codebook.txt")) as f:
        vals = [ln.strip() for ln in f if ln.strip() and not ln.startswith("#")]
    return [int(v) for v in vals[0].split(",")]


def _iq4nl_row(K, scales, payload):
    bpr, prefix, row_bytes = wl.iq4nl_row_geometry(K)
    row = np.zeros(row_bytes, np.uint8)
    row[0:2 * bpr] = np.asarray(scales, np.float32).astype(np.float16).view(np.uint8)
    row[prefix:] = np.asarray(payload, np.uint8).reshape(-1)
    return row


def pin_iq4nl_table(o):
    """Every nibble value t: a row of nibbles t with unit scales dequantizes to
    kv[t] everywhere, and its dot with an activation is kv[t]*sum(xhat). The
    table itself matches the stored codebook."""
    kv = _codebook_golden()
    assert [o.iq4nl_codebook(t) for t in range(16)] == kv
    assert kv == list(wl.IQ4NL_CODEBOOK)
    K = 256
    x = wl.activations(1, K, wl.rng(47))
    xq = o.quantize_q8k(x)
    xh = o.dequant_q8k(xq, 1, K)[0]
    for t in range(16):
        row = _iq4nl_row(K, np.ones(K // 32), np.full(16 * (K // 32), t | (t << 4), np.uint8))
        wd = o.dequant_iq4nl(row, 1, K)[0]
        assert np.all(wd == kv[t])
        y, T = o.gemv_iq4nl(row, xq, 1, K)
        assert abs(y[0] - kv[t] * xh.sum()) <= 1e-12 * T[0]


def pin_iq4nl_layout(o):
    """A constructed resident row: block c has scale (c+1)/8 (exact in f16),
    payload byte t holds nibble lo_t for weight t and hi_t for weight t+16.
    The dequantized row and a one-hot dot read them back."""
    kv = _codebook_golden()
    K = 512
    bpr = K // 32
    scales = (np.arange(bpr) + 1) / 8.0
    payload = np.zeros((bpr, 16), np.uint8)
    want = np.zeros(K, np.float64)
    for c in range(bpr):
        for t in range(16):
            lo = (t + c) % 16
            hi = (3 * t + 7 * c + 1) % 16
            payload[c, t] = lo | (hi << 4)
            want[32 * c + t] = scales[c] * kv[lo]
            want[32 * c + 16 + t] = scales[c] * kv[hi]
    row = _iq4nl_row(K, scales, payload)
    assert np.array_equal(o.dequant_iq4nl(row, 1, K)[0], want)
    for p in (0, 15, 16, 31, 32, 300, 511):
        x = np.zeros((1, K), np.float32)
        x[0, p] = 127.0
        y, _ = o.gemv_iq4nl(row, o.quantize_q8k(x), 1, K)
        assert y[0] == 127.0 * want[p], p


def pin_iq4nl_brute_force_and_partials(o):
    """Random resident rows: the mat-vec against a numpy f64 dot of the
    separately dequantized operands; the partials recombine to it as
    sum_c d_c*xs*D_c; the error bound against the unquantized activation."""
    g = wl.rng(53)
    N, K = 5, 1024
    w = wl.iq4nl_weights(N, K, g)
    x = wl.activations(1, K, g)
    xq = o.quantize_q8k(x)
    y, T = o.gemv_iq4nl(w, xq, N, K)
    wd = o.dequant_iq4nl(w, N, K)
    ref = wd @ o.dequant_q8k(xq, 1, K)[0]
    assert np.all(np.abs(y - ref) <= 1e-12 * T)
    D = o.iq4nl_partials(w, xq, N, K)
    bpr, prefix, _ = wl.iq4nl_row_geometry(K)
    dc = w[:, 0:2 * bpr].copy().view("<f2").astype(np.float64)
    xs = np.repeat(xq[0, :, 288:292].copy().view("<f4").astype(np.float64).reshape(-1), 8)
    yp = (dc * xs[None, :] * D).sum(axis=1)
    assert np.all(np.abs(yp - y) <= 1e-12 * T)
    dx = np.repeat(xq[0, :, 288:292].copy().view("<f4").astype(np.float64).reshape(-1), 256)
    bound = np.abs(wd) @ (dx * (0.5 + 2.0 ** -17))
    assert np.all(np.abs(y - wd @ x[0].astype(np.float64)) <= bound + 1e-12 * T)


def pin_q4_0_layout(o):
    """A constructed Q4_0 row (the IQ4_NL row shape): block c has scale
    (c+1)/8, payload byte t holds nibble lo_t for weight t and hi_t for weight
    t+16, so the weights are scale*(nibble-8) by construction; one-hot dots read
    them back, and a row of nibbles 8 is zero against any activation."""
    K = 512
    bpr = K // 32
    scales = (np.arange(bpr) + 1) / 8.0
    payload = np.zeros((bpr, 16), np.uint8)
    want = np.zeros(K, np.float64)
    for c in range(bpr):
        for t in range(16):
            lo = (5 * t + c) % 16
            hi = (t + 3 * c + 2) % 16
            payload[c, t] = lo | (hi << 4)
            want[32 * c + t] = scales[c] * (lo - 8)
            want[32 * c + 16 + t] = scales[c] * (hi - 8)
    row = _iq4nl_row(K, scales, payload)
    assert np.array_equal(o.dequant_q4_0(row, 1, K)[0], want)
    for p in (0, 15, 16, 31, 32, 300, 511):
        x = np.zeros((1, K), np.float32)
        x[0, p] = 127.0
        y, _ = o.gemv_q4_0(row, o.quantize_q8k(x), 1, K)
        assert y[0] == 127.0 * want[p], p
    eight = _iq4nl_row(K, scales, np.full((bpr, 16), 0x88, np.uint8))
    xq = o.quantize_q8k(wl.activations(1, K, wl.rng(61)))
    y, T = o.gemv_q4_0(eight, xq, 1, K)
    assert y[0] == 0.0 and T[0] == 0.0
    assert not o.q4_0_partials(eight, xq, 1, K).any()


def pin_q4_0_brute_force_and_partials(o):
    """Random rows: the mat-vec against a numpy f64 dot of the separately
    dequantized operands; the partials equal sum(nibble*code) - 8*s_c with s_c
    the activation's stored 32-code sums (the -8 riding on the activation sum)
    and recombine to the mat-vec."""
    g = wl.rng(67)
    N, K = 5, 1024
    w = wl.iq4nl_weights(N, K, g)
    x = wl.activations(1, K, g)
    xq = o.quantize_q8k(x)
    y, T = o.gemv_q4_0(w, xq, N, K)
    wd = o.dequant_q4_0(w, N, K)
    assert np.all(np.abs(y - wd @ o.dequant_q8k(xq, 1, K)[0]) <= 1e-12 * T)
    bpr, prefix, _ = wl.iq4nl_row_geometry(K)
    pay = w[:, prefix:].reshape(N, bpr, 16).astype(np.int64)
    nib = np.concatenate([pay & 15, pay >> 4], axis=2)                      # [N, bpr, 32]
    codes = np.stack([_q8k_fields(xq[0, b])[0] for b in range(K // 256)]).reshape(bpr, 32)
    sums = np.stack([_q8k_fields(xq[0, b])[1] for b in range(K // 256)]).reshape(bpr)
    D = o.q4_0_partials(w, xq, N, K)
    assert np.array_equal(D, (nib * codes[None]).sum(axis=2) - 8 * sums[None])
    dc = w[:, 0:2 * bpr].copy().view("<f2").astype(np.float64)
    xs = np.repeat(xq[0, :, 288:292].copy().view("<f4").astype(np.float64).reshape(-1), 8)
    assert np.all(np.abs((dc * xs[None, :] * D).sum(axis=1) - y) <= 1e-12 * T)


def _iq4nl_file_dequant(blocks: np.ndarray, rows: int, bpr: int) -> np.ndarray:
    """Weights of IQ4_NL file blocks straight from the format: block c of a row
    holds w[32c + t] = d * kv[low nibble of payload byte t] and
    w[32c + 16 + t] = d * kv[high nibble of byte t] for t < 16, d the f16 at
    the block's first two bytes (numpy's float16 decoder), kv the table in
    tests/golden/iq4nl_codebook.txt."""
    kv = np.array(_codebook_golden(), dtype=np.float64)
    b = np.ascontiguousarray(blocks, dtype=np.uint8).reshape(rows, bpr, 18)
    d = b[:, :, 0:2].copy().view("<f2").astype(np.float64)
    q = b[:, :, 2:18]
    w = np.concatenate([kv[q & 15], kv[q >> 4]], axis=2) * d
    return w.reshape(rows, 32 * bpr)


def pin_iq4nl_repack_layout(o):
    """Repacked rows dequantize (through the oracle's resident-row decoder) to
    the weights the file blocks define; a row's pad bytes are zero."""
    import oracle
    for rows, bpr in ((3, 9), (2, 8), (1, 1), (2, 317)):
        blocks = wl.iq4nl_file_blocks(rows * bpr, wl.rng(7000 + 10 * rows + bpr))
        res = oracle.repack_iq4nl(blocks, rows * bpr, 0, bpr)
        K = 32 * bpr
        got = o.dequant_iq4nl(res, rows, K).reshape(rows, K)
        assert np.array_equal(got, _iq4nl_file_dequant(blocks, rows, bpr)), (rows, bpr)
        prefix = ((2 * bpr + 3) // 4) * 4
        assert not res[:, 2 * bpr:prefix].any()


def pin_iq4nl_repack_chunks(o):
    """Repacking in chunks that start and end mid-row writes every byte of the
    resident rows (a poisoned buffer comes out whole) and equals one chunk."""
    import oracle
    rows, bpr = 3, 9
    blocks = wl.iq4nl_file_blocks(rows * bpr, wl.rng(7100))
    whole = oracle.repack_iq4nl(blocks, rows * bpr, 0, bpr)
    part = np.full_like(whole, 0xAB)
    for a, b in ((0, 5), (5, 17), (17, 27)):
        oracle.repack_iq4nl(blocks[a:b], b - a, a, bpr, resident=part)
    assert np.array_equal(whole, part)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
