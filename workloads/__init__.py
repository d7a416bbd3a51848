"""Seeded synthetic inputs for the quantized decode mat-vec.

This module produces input *bytes* only. It holds none of the method's
arithmetic: no quantizer, no decoder and no dot. Both the CPU oracle (under
``oracle/``) and the HIP library consume what it returns; neither imports the
other.

Formats written here (byte layouts only):

* Q4_K super-block, 144 bytes per 256 weights. Bytes 0-1 hold the f16 scale
  ``d``, bytes 2-3 the f16 ``dmin``, bytes 4-15 the twelve bytes of packed
  6-bit sub-block scales and mins, bytes 16-143 the 128 bytes of nibbles; the
  nibble group ``g`` sits at ``16 + 32*g`` ("cajeta.xpu — one kernel, any
  device", section 2.3, the load-alignment example).  Drawing the twelve
  packed bytes uniformly is the same as drawing each of the sixteen 6-bit
  fields uniformly from 0..63, because the 96 bits hold exactly those sixteen
  fields.
* IQ4_NL resident row ("25 — Writing XPU Kernels", section 25.2.1): the row's
  f16 block scales first, padded to a dword, then one 16-byte payload per
  32-weight block.
* f32 activations, row-major.

Random draws use numpy ``Generator(PCG64(seed))`` in a fixed order: for a
Q4_K matrix ``d``, ``dmin``, the twelve scale bytes, the nibble bytes; for an
IQ4_NL matrix the scales, then the payload bytes; activations last.
"""

from __future__ import annotations

import numpy as np

Q4K_BLOCK_BYTES = 144
Q4K_BLOCK_WEIGHTS = 256
Q8K_BLOCK_BYTES = 320
IQ4NL_BLOCK_WEIGHTS = 32

# The sixteen signed int8 values of the IQ4_NL codebook. The pages name the
# table (the codebook accessor in section 25.2.1 of "25 — Writing XPU
# Kernels") but do not print it; these are the published IQ4_NL values that
# the codebook workload specifies.
IQ4NL_CODEBOOK = (-127, -104, -83, -65, -49, -35, -22, -10,
                  1, 13, 25, 38, 53, 69, 89, 113)

# Seeds of the five workloads (tiny Q4_K, Q4_K 4096x4096, FFN up/down,
# IQ4_NL square/head, small-M prefill).
SEEDS = {
    "q4k_tiny": 1000,
    "q4k_4096": 1001,
    "ffn_up": 1002,
    "ffn_down": 1003,
    "iq4nl_4096": 1004,
    "iq4nl_head": 1005,
    "prefill": 1006,
    "grouped": 1007,
}


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def _f16_bytes(values: np.ndarray) -> np.ndarray:
    """f32 values -> their f16 (round-to-nearest-even, numpy astype) bytes."""
    h = np.ascontiguousarray(values.astype(np.float32).astype(np.float16))
    return h.view(np.uint8).reshape(values.shape + (2,))


def q4k_weights(N: int, K: int, g: np.random.Generator,
                d_range=(0.001, 0.02)) -> np.ndarray:
    """Q4_K matrix of N rows and K columns as uint8[N, K/256, 144]."""
    assert K % Q4K_BLOCK_WEIGHTS == 0
    nb = K // Q4K_BLOCK_WEIGHTS
    d = g.uniform(d_range[0], d_range[1], size=(N, nb))
    dmin = g.uniform(d_range[0], d_range[1], size=(N, nb))
    scale_bytes = g.integers(0, 256, size=(N, nb, 12), dtype=np.uint8)
    nibbles = g.integers(0, 256, size=(N, nb, 128), dtype=np.uint8)
    out = np.empty((N, nb, Q4K_BLOCK_BYTES), dtype=np.uint8)
    out[:, :, 0:2] = _f16_bytes(d)
    out[:, :, 2:4] = _f16_bytes(dmin)
    out[:, :, 4:16] = scale_bytes
    out[:, :, 16:144] = nibbles
    return out


def iq4nl_row_geometry(K: int):
    """(blocks per row, scale-prefix bytes, row bytes) of the resident row."""
    assert K % IQ4NL_BLOCK_WEIGHTS == 0
    bpr = K // IQ4NL_BLOCK_WEIGHTS
    prefix = ((bpr * 2 + 3) // 4) * 4
    return bpr, prefix, prefix + 16 * bpr


def iq4nl_weights(N: int, K: int, g: np.random.Generator,
                  d_range=(0.001, 0.02)) -> np.ndarray:
    """IQ4_NL matrix in resident rows as uint8[N, rowBytes]."""
    bpr, prefix, row_bytes = iq4nl_row_geometry(K)
    d = g.uniform(d_range[0], d_range[1], size=(N, bpr))
    payload = g.integers(0, 256, size=(N, bpr * 16), dtype=np.uint8)
    out = np.zeros((N, row_bytes), dtype=np.uint8)
    out[:, 0:2 * bpr] = _f16_bytes(d).reshape(N, 2 * bpr)
    out[:, prefix:] = payload
    return out


def iq4nl_file_blocks(n_blocks: int, g: np.random.Generator,
                      d_range=(0.001, 0.02)) -> np.ndarray:
    """IQ4_NL blocks in the file layout as uint8[n_blocks, 18]: the f16 scale,
    then 16 payload bytes (uniform)."""
    d = g.uniform(d_range[0], d_range[1], size=n_blocks)
    out = np.empty((n_blocks, 18), dtype=np.uint8)
    out[:, 0:2] = _f16_bytes(d)
    out[:, 2:] = g.integers(0, 256, size=(n_blocks, 16), dtype=np.uint8)
    return out


def activations(R: int, K: int, g: np.random.Generator) -> np.ndarray:
    """f32 [R, K] drawn from N(0, 1)."""
    return g.standard_normal(size=(R, K), dtype=np.float32)


def pages_activation(K: int) -> np.ndarray:
    """The deterministic activation of the grouped-kernel bit gate in
    section 25.7.1 of "25 — Writing XPU Kernels": element j is
    ((j mod 25) - 12) / 64, formed in f32."""
    j = np.arange(K, dtype=np.int64)
    return (((j % 25) - 12).astype(np.float32) / np.float32(64.0)).astype(np.float32)


# ---------------------------------------------------------------------------
# Constructed (non-random) inputs for special cases.
# ---------------------------------------------------------------------------

def pack_q4k_scales(sc, m) -> np.ndarray:
    """Pack eight 6-bit scales and eight 6-bit mins into the twelve header
    bytes of a Q4_K block (bytes 4-15 of the block).

    The pages give the block size and the header offset but not this packing;
    it follows the public GGUF Q4_K convention. For k = 0..3:
      byte 4+k  = sc[k]   | (sc[k+4] >> 4) << 6
      byte 8+k  = m[k]    | (m[k+4]  >> 4) << 6
      byte 12+k = (sc[k+4] & 15) | (m[k+4] & 15) << 4
    """
    sc = np.asarray(sc, dtype=np.int64)
    m = np.asarray(m, dtype=np.int64)
    assert sc.shape[-1] == 8 and m.shape == sc.shape
    assert sc.min() >= 0 and sc.max() < 64 and m.min() >= 0 and m.max() < 64
    out = np.zeros(sc.shape[:-1] + (12,), dtype=np.int64)
    for k in range(4):
        out[..., k] = sc[..., k] | ((sc[..., k + 4] >> 4) << 6)
        out[..., 4 + k] = m[..., k] | ((m[..., k + 4] >> 4) << 6)
        out[..., 8 + k] = (sc[..., k + 4] & 15) | ((m[..., k + 4] & 15) << 4)
    return out.astype(np.uint8)


def q4k_block(d: float, dmin: float, sc, m, nibble_bytes) -> np.ndarray:
    """One constructed 144-byte Q4_K block."""
    blk = np.zeros(Q4K_BLOCK_BYTES, dtype=np.uint8)
    blk[0:2] = _f16_bytes(np.array(d))
    blk[2:4] = _f16_bytes(np.array(dmin))
    blk[4:16] = pack_q4k_scales(sc, m)
    nb = np.asarray(nibble_bytes, dtype=np.uint8)
    assert nb.shape == (128,)
    blk[16:] = nb
    return blk


def f16_bits(value: float) -> int:
    """The binary16 bit pattern of ``value`` (numpy round-to-nearest-even)."""
    return int(np.array(value, dtype=np.float16).view(np.uint16))


def q4k_from_fields(d, dmin, sc, m, nibble_bytes) -> np.ndarray:
    """A Q4_K matrix [N, nb, 144] assembled from its fields: f32 d and dmin
    [N, nb] (stored as f16), 6-bit sc and m [N, nb, 8], nibble bytes
    [N, nb, 128]."""
    d = np.asarray(d, dtype=np.float32)
    N, nb = d.shape
    out = np.empty((N, nb, Q4K_BLOCK_BYTES), dtype=np.uint8)
    out[:, :, 0:2] = _f16_bytes(d)
    out[:, :, 2:4] = _f16_bytes(np.asarray(dmin, dtype=np.float32))
    out[:, :, 4:16] = pack_q4k_scales(sc, m)
    out[:, :, 16:] = np.asarray(nibble_bytes, dtype=np.uint8)
    return out


def q4k_isolation_weights(N: int, K: int, g: np.random.Generator, which: str) -> np.ndarray:
    """Weights that make a mat-vec output equal one exact integer partial.

    which == "S": d = 1, dmin = 0, sub-block scales in 0..31, so against an
    activation whose only nonzero block has scale 1 the output is that block's
    S partial exactly (|S| < 2^24). which == "M": d = 0, dmin = 1, so the
    output is minus the block's M partial."""
    nb = K // Q4K_BLOCK_WEIGHTS
    sc = g.integers(0, 32 if which == "S" else 64, size=(N, nb, 8))
    m = g.integers(0, 64, size=(N, nb, 8))
    nib = g.integers(0, 256, size=(N, nb, 128), dtype=np.uint8)
    one = np.ones((N, nb), np.float32)
    zero = np.zeros((N, nb), np.float32)
    if which == "S":
        return q4k_from_fields(one, zero, sc, m, nib)
    if which == "M":
        return q4k_from_fields(zero, one, sc, m, nib)
    raise ValueError(which)


def isolating_activation(R: int, K: int, g: np.random.Generator, block: int,
                         width: int = 256, offset: int = 0) -> np.ndarray:
    """f32 [R, K], zero except elements [block*256 + offset, + width) of every
    row, which hold values in [-127, 127] with one element exactly 127, so
    that the block's q8_K scale is exactly 1 and its codes are the values
    rounded to integers."""
    x = np.zeros((R, K), np.float32)
    lo = block * 256 + offset
    vals = g.uniform(-127.0, 127.0, size=(R, width)).astype(np.float32)
    vals[:, g.integers(0, width)] = 127.0
    x[:, lo:lo + width] = vals
    return x


def iq4nl_unit_scale_weights(N: int, K: int, g: np.random.Generator) -> np.ndarray:
    """Resident IQ4_NL rows with every block scale 1.0 and random payloads."""
    bpr, prefix, row_bytes = iq4nl_row_geometry(K)
    out = np.zeros((N, row_bytes), dtype=np.uint8)
    out[:, 0:2 * bpr] = _f16_bytes(np.ones((N, bpr), np.float32)).reshape(N, 2 * bpr)
    out[:, prefix:] = g.integers(0, 256, size=(N, bpr * 16), dtype=np.uint8)
    return out
