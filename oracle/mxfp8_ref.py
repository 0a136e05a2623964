"""MXFP8 latent KV rows: the format, its exact decode and the quantiser.

TEST INFRASTRUCTURE ONLY (see the package docstring for who may import it).

The VRAM page ("cell_size" section: the low-precision corrections of the
per-token cost) gives mxfp8 KV as one byte per element plus one scale per
32 elements.  Readings, after the OCP MX format the name refers to:

* Element: OCP e4m3fn (the FP8 codes of the FP8 pools; largest 448).
* Block scale: one byte per 32 consecutive elements, an unsigned biased
  exponent (E8M0): code c scales the block by 2^(c - 127).  As for the FP4
  rows, the valid codes are 63 .. 191 (2^-64 .. 2^64).
* Row of one token, 608 bytes: bytes 0..575 the codes (element i in byte
  i), bytes 576..593 the 18 block scales (block k = elements 32 k .. 32 k +
  31: 16 blocks of c_kv, 2 of k_rope), bytes 594..607 zero padding (rows
  stay 16-byte aligned).
* Value = e4m3fn(code) * 2^(c - 127), exact in float64 (and in BF16).
* Quantiser of a block with largest magnitude a: e is the smallest integer
  with a <= 448 * 2^e (no element clips), clamped to [-64, 64] (a = 0 takes
  -64); each code is the e4m3fn value nearest to x * 2^-e, ties to the even
  code, clamped to +-448.
"""

from __future__ import annotations

import numpy as np

from .mla_ref import E4M3FN_TABLE

D_K = 576
BLOCK = 32
N_BLOCKS = D_K // BLOCK            # 18
ROW_BYTES = 608                    # 576 codes + 18 scales + 14 padding
SCALE_BIAS = 127
SCALE_MIN_CODE = SCALE_BIAS - 64
SCALE_MAX_CODE = SCALE_BIAS + 64
E4M3_MAX = 448.0


def block_exponents(raw: np.ndarray) -> np.ndarray:
    """Block exponents e = code - 127, int64 [n, 18]; invalid codes raise."""
    c = np.asarray(raw, dtype=np.uint8)[:, D_K:D_K + N_BLOCKS].astype(np.int64)
    if np.any((c < SCALE_MIN_CODE) | (c > SCALE_MAX_CODE)):
        raise ValueError("MXFP8 block-scale code outside 63..191")
    return c - SCALE_BIAS


def decode_mxfp8_rows(raw: np.ndarray) -> np.ndarray:
    """Exact float64 latent rows [n, 576] of MXFP8 rows [n, 608]."""
    raw = np.asarray(raw, dtype=np.uint8)
    if raw.ndim != 2 or raw.shape[1] != ROW_BYTES:
        raise ValueError(f"MXFP8 rows must be [n, {ROW_BYTES}] bytes")
    vals = E4M3FN_TABLE[raw[:, :D_K].astype(np.intp)]
    scale = np.ldexp(1.0, block_exponents(raw))              # [n, 18]
    return vals * np.repeat(scale, BLOCK, axis=1)


def block_exponent_of(amax) -> np.ndarray:
    """Smallest integer e with amax <= 448 * 2^e, clamped to [-64, 64] (0 -> -64)."""
    a = np.asarray(amax, dtype=np.float64)
    e = np.full(a.shape, -64, dtype=np.int64)
    nz = a > 0
    est = np.ceil(np.log2(a[nz] / E4M3_MAX)).astype(np.int64)
    # settle the estimate with exact comparisons (448 * 2^k is exact)
    est = np.where(a[nz] > E4M3_MAX * np.ldexp(1.0, est), est + 1, est)
    est = np.where(a[nz] <= E4M3_MAX * np.ldexp(1.0, est - 1), est - 1, est)
    e[nz] = est
    return np.clip(e, -64, 64)


def mxfp8_quantise_rows(x) -> np.ndarray:
    """MXFP8 rows [n, 608] of float rows x [n, 576] (values exact in float32)."""
    from .prepare_ref import e4m3fn_encode    # the pinned e4m3fn rounding
    x = np.asarray(x, dtype=np.float64)
    if x.ndim != 2 or x.shape[1] != D_K:
        raise ValueError("rows must be [n, 576]")
    n = x.shape[0]
    blocks = x.reshape(n, N_BLOCKS, BLOCK)
    e = block_exponent_of(np.max(np.abs(blocks), axis=2))      # [n, 18]
    y = np.clip(blocks * np.ldexp(1.0, -e)[:, :, None], -E4M3_MAX, E4M3_MAX)
    out = np.zeros((n, ROW_BYTES), dtype=np.uint8)
    out[:, :D_K] = e4m3fn_encode(y.astype(np.float32)).reshape(n, D_K)
    out[:, D_K:D_K + N_BLOCKS] = (e + SCALE_BIAS).astype(np.uint8)
    return out
