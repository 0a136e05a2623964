"""FP4 latent KV rows: the format, its exact decode and the quantiser.

TEST INFRASTRUCTURE ONLY (see the package docstring for who may import it).

The pages give FP4 KV as 0.5 byte per element (two codes packed per byte)
plus one block scale per 16 elements, which puts a token's cost a little
above a quarter of BF16 (VRAM page, "KV ledger" section on the KV dtype;
"cell_size" section: the FP4 correction halves the bytes and then adds one
scale per 16 elements).  They name neither the element encoding nor the
scale encoding.  Readings:

* Element: OCP e2m1 (sign, 2 exponent bits with bias 1, 1 mantissa bit):
  0, 0.5, 1, 1.5, 2, 3, 4, 6 and their negatives; no infinity or NaN.
* Block scale: one byte per 16 consecutive elements (which is what "a little
  above a quarter" allows), read as an unsigned biased exponent (UE8M0, the
  OCP MX scale type): code c scales the block by 2^(c - 127).  Valid codes
  are 63 .. 191 (2^-64 .. 2^64); others are rejected.
* Row of one token, 336 bytes: bytes 0..287 hold the 576 codes (element
  2 i in the low nibble of byte i, element 2 i + 1 in the high nibble),
  bytes 288..323 the 36 block-scale codes (block k = elements 16 k .. 16 k +
  15: the 32 blocks of c_kv, then the 4 of k_rope), bytes 324..335 are zero
  padding so that rows stay 16-byte aligned.
* Value = e2m1(code) * 2^(c - 127), exact in float64 (and in BF16).
* Quantiser of a block with largest magnitude a: the exponent e is the
  smallest integer with a <= 6 * 2^e (so no element clips), clamped to
  [-64, 64] (a = 0 takes -64); each code is the e2m1 value nearest to
  x * 2^-e, ties to the code with an even mantissa bit, clamped to +-6.
"""

from __future__ import annotations

import numpy as np

D_K = 576
BLOCK = 16
N_BLOCKS = D_K // BLOCK            # 36
CODE_BYTES = D_K // 2              # 288
ROW_BYTES = 336                    # 288 codes + 36 scales + 12 padding
SCALE_BIAS = 127
SCALE_MIN_CODE = SCALE_BIAS - 64   # 63
SCALE_MAX_CODE = SCALE_BIAS + 64   # 191
E2M1_MAX = 6.0


def e2m1_decode_table() -> np.ndarray:
    """Value of each of the 16 e2m1 codes as float64, from the bit fields."""
    table = np.empty(16, dtype=np.float64)
    for code in range(16):
        sign = -1.0 if code & 0x8 else 1.0
        exp_field = (code >> 1) & 0x3
        mant = code & 0x1
        if exp_field == 0:
            mag = 0.5 * mant                      # subnormal: m * 2^(1 - bias) / 2
        else:
            mag = (1.0 + 0.5 * mant) * 2.0 ** (exp_field - 1)
        table[code] = sign * mag
    return table


E2M1_TABLE = e2m1_decode_table()

# The 8 non-negative codes in increasing value (0x0..0x7).
_POS_CODES = np.arange(8, dtype=np.uint8)
_POS_VALUES = E2M1_TABLE[:8]


def unpack_codes(raw: np.ndarray) -> np.ndarray:
    """e2m1 codes [n, 576] (uint8 0..15) of rows [n, 336]."""
    b = np.asarray(raw, dtype=np.uint8)[:, :CODE_BYTES]
    codes = np.empty((b.shape[0], D_K), dtype=np.uint8)
    codes[:, 0::2] = b & 0x0F
    codes[:, 1::2] = b >> 4
    return codes


def block_exponents(raw: np.ndarray) -> np.ndarray:
    """Block exponents e = code - 127, int64 [n, 36]; invalid codes raise."""
    c = np.asarray(raw, dtype=np.uint8)[:, CODE_BYTES:CODE_BYTES + N_BLOCKS].astype(np.int64)
    if np.any((c < SCALE_MIN_CODE) | (c > SCALE_MAX_CODE)):
        raise ValueError("FP4 block-scale code outside 63..191")
    return c - SCALE_BIAS


def decode_fp4_rows(raw: np.ndarray) -> np.ndarray:
    """Exact float64 latent rows [n, 576] of FP4 rows [n, 336]."""
    raw = np.asarray(raw, dtype=np.uint8)
    if raw.ndim != 2 or raw.shape[1] != ROW_BYTES:
        raise ValueError(f"FP4 rows must be [n, {ROW_BYTES}] bytes")
    vals = E2M1_TABLE[unpack_codes(raw).astype(np.intp)]
    scale = np.ldexp(1.0, block_exponents(raw))              # [n, 36]
    return vals * np.repeat(scale, BLOCK, axis=1)


def e2m1_encode(y) -> np.ndarray:
    """e2m1 code of each value in [-6, 6]: the nearest code value, ties to the
    code with an even mantissa bit; the sign bit is the value's own."""
    v = np.asarray(y, dtype=np.float64)
    if np.any(np.abs(v) > E2M1_MAX) or np.any(np.isnan(v)):
        raise ValueError("e2m1_encode expects finite values in [-6, 6]")
    mag = np.abs(v)
    hi = np.minimum(np.searchsorted(_POS_VALUES, mag, side="left"), 7)
    lo = np.maximum(hi - 1, 0)
    d_lo = mag - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (_POS_CODES[hi] % 2 == 0))
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo]).astype(np.uint8)
    return np.where(np.signbit(v), code | np.uint8(0x8), code).astype(np.uint8)


def block_exponent_of(amax) -> np.ndarray:
    """Smallest integer e with amax <= 6 * 2^e, clamped to [-64, 64] (0 -> -64)."""
    a = np.asarray(amax, dtype=np.float64)
    e = np.full(a.shape, -64, dtype=np.int64)
    nz = a > 0
    est = np.ceil(np.log2(a[nz] / E2M1_MAX)).astype(np.int64)
    # The estimate is exact or off by one near powers of two; settle it with
    # exact comparisons (6 * 2^k is exact in float64).
    est = np.where(a[nz] > E2M1_MAX * np.ldexp(1.0, est), est + 1, est)
    est = np.where(a[nz] <= E2M1_MAX * np.ldexp(1.0, est - 1), est - 1, est)
    e[nz] = est
    return np.clip(e, -64, 64)


def fp4_quantise_rows(x) -> np.ndarray:
    """FP4 rows [n, 336] of float rows x [n, 576] (values exact in float32)."""
    x = np.asarray(x, dtype=np.float64)
    if x.ndim != 2 or x.shape[1] != D_K:
        raise ValueError("rows must be [n, 576]")
    n = x.shape[0]
    blocks = x.reshape(n, N_BLOCKS, BLOCK)
    e = block_exponent_of(np.max(np.abs(blocks), axis=2))      # [n, 36]
    y = np.clip(blocks * np.ldexp(1.0, -e)[:, :, None], -E2M1_MAX, E2M1_MAX)
    codes = e2m1_encode(y).reshape(n, D_K)
    out = np.zeros((n, ROW_BYTES), dtype=np.uint8)
    out[:, :CODE_BYTES] = codes[:, 0::2] | (codes[:, 1::2] << 4)
    out[:, CODE_BYTES:CODE_BYTES + N_BLOCKS] = (e + SCALE_BIAS).astype(np.uint8)
    return out
