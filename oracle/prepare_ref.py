"""Plain CPU oracle of the MLA prepare step that feeds absorbed decode.

TEST INFRASTRUCTURE ONLY (see the package docstring for who may import it).

The step runs once per decode step and layer, on the T = B * q_len new query
tokens, before the attention kernel:

1. Q absorption.  The 128-wide no-RoPE query of every head is multiplied by
   that head's w_kc (128 x 512), into which kv_b_proj was absorbed, giving
   the 512-wide q_nope_absorbed the attention scores against c_kv.  (Page
   "Kimi K3 decode: DP16 vs DP2 x DCP8": kv_b_proj is absorbed into w_kc /
   w_vc (section on the weight AllGather); w_kc is 96 x 128 x 512 in bf16
   (VRAM-ledger section, replicated Q projection bullet); the step is
   mla_prepare (section "MLA", per-layer overheads of DP2).)
2. RoPE on the 64-wide decoupled parts: every head's q_rope and the new
   tokens' k_rope, at the tokens' positions.
3. KV append: the new tokens' latent rows [c_kv (512) | roped k_rope (64)]
   are written into the paged pool at the slots the caller gives, as BF16,
   or as OCP e4m3fn codes with one fp32 scale per token (VRAM page, "KV
   ledger" MLA bullet and "cell_size": one 576-wide row per token; FP8 KV at
   576 B per token, so the scale is kept beside the row).

Readings where the pages are silent:
* RoPE rotates interleaved pairs (x[2i], x[2i+1]) by the angle of frequency
  i; the caller passes the cos / sin of every (position, i), so the base
  and any context-extension scaling stay the caller's choice.
* The RoPE output is rounded to BF16 (the query the attention reads is
  BF16, and the BF16 pool stores BF16); the FP8 append quantises those BF16
  values.
* FP8 per-token scale = amax / 448 over the token's 576 values (1 if all are
  zero), code = e4m3fn round-to-nearest-even of x / scale, clamped to +-448.
* FP4 and MXFP8 rows (formats and quantisers in fp4_ref and mxfp8_ref):
  the BF16 row values are quantised block by block; every step is exact
  (power-of-two scaling, comparisons, one nearest-even rounding of an exact
  value), so the stored bytes are compared bit for bit.

Where floating point decides a stored code (the FP8 bytes, the BF16 bits of
the roped values), the stored code is defined by float32 arithmetic, so that
codes can be compared bit for bit: RoPE is y0 = x0 c - x1 s, y1 = x0 s + x1 c
with every product and every sum a correctly rounded float32 operation (no
fused multiply-add), then round-to-nearest-even to BF16; the FP8 scale and
the quotient x / scale are correctly rounded float32 divisions.  This is the
definition the library header states for mla_prepare; rope_f32 is pinned to
it bit for bit by a test that evaluates every product and sum from exact
rationals.  The absorbed query, a sum of 128 products, is computed in
float64 and compared within one BF16 unit in the last place.
"""

from __future__ import annotations

import numpy as np

from .fp4_ref import fp4_quantise_rows
from .mxfp8_ref import mxfp8_quantise_rows
from .mla_ref import E4M3FN_TABLE, bf16_bits_to_f64

D_NOPE = 128    # qk_nope_head_dim: the no-RoPE query width before absorption
D_C = 512       # kv_lora_rank
D_R = 64        # qk_rope_head_dim
E4M3_MAX = 448.0

# The 127 non-negative finite e4m3fn codes in increasing value (0x00..0x7E).
_POS_CODES = np.arange(0x7F, dtype=np.uint8)
_POS_VALUES = E4M3FN_TABLE[:0x7F]


def bf16_bits_to_f32(bits) -> np.ndarray:
    """Float32 value of BF16 bit patterns (exact)."""
    a = np.asarray(bits).view(np.uint16).astype(np.uint32) << np.uint32(16)
    return a.view(np.float32)


def f32_to_bf16_bits(x) -> np.ndarray:
    """Round float32 values to BF16 bit patterns, nearest-even (finite inputs)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def e4m3fn_encode(x) -> np.ndarray:
    """e4m3fn code of each float32 value in [-448, 448], round-to-nearest-even.

    The nearest of the finite values of the format (the decode table built
    from its definition); a value halfway between two neighbours takes the
    code with the even mantissa.  The sign bit is the value's own, so a
    negative value that rounds to zero gives 0x80.
    """
    v = np.asarray(x, dtype=np.float32).astype(np.float64)
    if np.any(np.abs(v) > E4M3_MAX) or np.any(np.isnan(v)):
        raise ValueError("e4m3fn_encode expects finite values in [-448, 448]")
    mag = np.abs(v)
    hi = np.searchsorted(_POS_VALUES, mag, side="left")  # first value >= mag
    hi = np.minimum(hi, len(_POS_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = mag - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (_POS_CODES[hi] % 2 == 0))
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo]).astype(np.uint8)
    neg = np.signbit(np.asarray(x, dtype=np.float32))
    return np.where(neg, code | np.uint8(0x80), code).astype(np.uint8)


def rope_f32(x, cos, sin) -> np.ndarray:
    """Rotate interleaved pairs of float32 x[..., 64] by the given cos / sin.

    cos, sin: float32 [..., 32], broadcast against x's leading dimensions.
    Pair i = (x[2i], x[2i+1]) -> (x0 c - x1 s, x0 s + x1 c), each product and
    each sum rounded to float32.
    """
    x = np.asarray(x, dtype=np.float32)
    c = np.asarray(cos, dtype=np.float32)
    s = np.asarray(sin, dtype=np.float32)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    y = np.empty_like(x)
    y[..., 0::2] = (x0 * c) - (x1 * s)
    y[..., 1::2] = (x0 * s) + (x1 * c)
    return y


def q_absorb_ref(q_nope_bits, w_kc_t_bits) -> np.ndarray:
    """q_nope_absorbed[t, h, n] = sum_k q_nope[t, h, k] * w_kc[h, k, n], float64.

    q_nope_bits: BF16 bits [T, H, 128]; w_kc_t_bits: BF16 bits [H, 512, 128],
    each head's w_kc transposed (element (h, n, k) = w_kc[h, k, n]).
    """
    q = bf16_bits_to_f64(q_nope_bits)                    # [T, H, 128]
    wt = bf16_bits_to_f64(w_kc_t_bits)                   # [H, 512, 128]
    out = np.empty(q.shape[:2] + (wt.shape[1],), dtype=np.float64)
    for h in range(q.shape[1]):
        out[:, h, :] = q[:, h, :] @ wt[h].T
    return out


def rope_table_rows(cos_sin, positions):
    """cos and sin [T, 32] of the given positions from a [max_pos, 64] table."""
    tab = np.asarray(cos_sin, dtype=np.float32)
    p = np.asarray(positions, dtype=np.int64)
    return tab[p, :32], tab[p, 32:]


def q_rope_ref(q_rope_bits, cos_sin, positions) -> np.ndarray:
    """BF16 bits [T, H, 64] of the roped query parts."""
    c, s = rope_table_rows(cos_sin, positions)
    x = bf16_bits_to_f32(q_rope_bits)                    # [T, H, 64]
    return f32_to_bf16_bits(rope_f32(x, c[:, None, :], s[:, None, :]))


def latent_rows_ref(c_kv_bits, k_rope_bits, cos_sin, positions) -> np.ndarray:
    """BF16 bits [T, 576] of the rows to append: [c_kv | bf16(rope(k_rope))]."""
    c, s = rope_table_rows(cos_sin, positions)
    k = f32_to_bf16_bits(rope_f32(bf16_bits_to_f32(k_rope_bits), c, s))
    return np.concatenate([np.asarray(c_kv_bits).view(np.uint16), k], axis=1)


def fp8_quantise_rows(row_bits):
    """(codes uint8 [T, 576], scale float32 [T]) of BF16 rows, per-token scale."""
    x = bf16_bits_to_f32(row_bits)                       # exact
    amax = np.max(np.abs(x), axis=1)
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    q = (x / scale[:, None]).astype(np.float32)
    q = np.clip(q, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
    return e4m3fn_encode(q), scale


def kv_append_ref(pool, kv_scale, c_kv_bits, k_rope_bits, cos_sin, positions, slots,
                  kv_dtype: str):
    """Pool (and scales) after appending the T new rows at `slots`.

    pool: uint16 BF16 bits [num_slots, 576], uint8 e4m3fn codes, uint8 FP4
    rows [num_slots, 336] or MXFP8 rows [num_slots, 608]; kv_scale: float32
    [num_slots] (FP8) or None.
    Slots outside [0, num_slots) are skipped (a token another DCP shard
    holds); the others must be distinct.
    Returns new arrays; the inputs are not modified.
    """
    rows = latent_rows_ref(c_kv_bits, k_rope_bits, cos_sin, positions)
    sl = np.asarray(slots, dtype=np.int64)
    pool = np.array(pool, copy=True)
    keep = (sl >= 0) & (sl < pool.shape[0])
    if kv_dtype == "bf16":
        pool[sl[keep]] = rows[keep]
        return pool, None
    if kv_dtype == "fp4":
        pool[sl[keep]] = fp4_quantise_rows(bf16_bits_to_f32(rows[keep]))
        return pool, None
    if kv_dtype == "mxfp8":
        pool[sl[keep]] = mxfp8_quantise_rows(bf16_bits_to_f32(rows[keep]))
        return pool, None
    if kv_dtype != "fp8":
        raise ValueError(f"unknown kv_dtype {kv_dtype!r}")
    codes, scale = fp8_quantise_rows(rows)
    kv_scale = np.array(kv_scale, dtype=np.float32, copy=True)
    pool[sl[keep]] = codes[keep]
    kv_scale[sl[keep]] = scale[keep]
    return pool, kv_scale


def mla_prepare_ref(q_nope_bits, q_rope_bits, w_kc_t_bits, c_kv_bits, k_rope_bits,
                    cos_sin, positions, slots, pool, kv_scale, kv_dtype: str):
    """The whole step: (q_nope_absorbed float64 [T, H, 512], q_rope_out BF16
    bits [T, H, 64], pool, kv_scale) after the append."""
    qa = q_absorb_ref(q_nope_bits, w_kc_t_bits)
    qr = q_rope_ref(q_rope_bits, cos_sin, positions)
    pool2, sc2 = kv_append_ref(pool, kv_scale, c_kv_bits, k_rope_bits, cos_sin, positions,
                               slots, kv_dtype)
    return qa, qr, pool2, sc2
