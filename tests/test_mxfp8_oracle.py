"""Pins of the MXFP8 KV format in the oracle (oracle/mxfp8_ref.py).

The format (VRAM page, "cell_size" section: one byte per element plus one
scale per 32 elements; the encodings are readings, stated in mxfp8_ref):
the decode is pinned to a row worked out by hand and to the BF16 decode of
the same values (the e4m3fn table itself is pinned in test_oracle); the
quantiser to exact round trips, the exponent rule at its edges, clamps and
a brute-force nearest-value search.
"""

import numpy as np
import pytest

from oracle import (E4M3FN_TABLE, bf16_bits_to_f64, decode_mxfp8_rows, mla_decode_ref,
                    mxfp8_quantise_rows)
from oracle.mxfp8_ref import block_exponent_of
from workload import make_inputs


def _blank_row():
    row = np.zeros(608, dtype=np.uint8)
    row[576:594] = 127                          # every block scale 2^0
    return row


def test_hand_worked_row():
    row = _blank_row()
    row[0] = 0x38          # 1.0
    row[1] = 0xBC          # -1.5
    row[31] = 0x7E         # 448, last element of block 0
    row[32] = 0x01         # 2^-9 (smallest subnormal), first of block 1
    row[575] = 0x40        # 2.0, last element (block 17)
    row[576] = 128         # block 0 x 2
    row[577] = 126         # block 1 x 1/2
    row[593] = 124         # block 17 x 1/8
    v = decode_mxfp8_rows(row[None])[0]
    want = np.zeros(576)
    want[0], want[1], want[31] = 2.0, -3.0, 896.0
    want[32] = 2.0 ** -10
    want[575] = 0.25
    assert np.array_equal(v, want)


def test_decode_rejects_out_of_range_scales_and_bad_shapes():
    row = _blank_row()
    row[580] = 255
    with pytest.raises(ValueError):
        decode_mxfp8_rows(row[None])
    row[580] = 62
    with pytest.raises(ValueError):
        decode_mxfp8_rows(row[None])
    with pytest.raises(ValueError):
        decode_mxfp8_rows(np.zeros((1, 594), dtype=np.uint8))


def test_mxfp8_decode_is_the_bf16_decode_of_the_decoded_values():
    """Every e4m3fn value times 2^(-64..64) is a BF16 value, so an MXFP8 pool
    attends exactly like a BF16 pool holding its values."""
    x = make_inputs(13, [200, 77, 5], 5, 4, "mxfp8", page_size=16)
    nb = x.numpy_bits()
    pool = nb["pool"]
    used = np.concatenate([nb["req_to_token"][b, :n] for b, n in enumerate(x.local_lens)])
    vals = decode_mxfp8_rows(pool[used])
    f = vals.astype(np.float32)
    assert np.array_equal(f.astype(np.float64), vals)
    bits = (f.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(bf16_bits_to_f64(bits), vals)
    bf = np.full((pool.shape[0], 576), 0x7FC0, dtype=np.uint16)
    bf[used] = bits
    args = (nb["q_nope"], nb["q_rope"])
    o8, l8 = mla_decode_ref(*args, pool, None, nb["req_to_token"], nb["seq_lens"], 5,
                            x.softmax_scale, "mxfp8")
    ob, lb = mla_decode_ref(*args, bf, None, nb["req_to_token"], nb["seq_lens"], 5,
                            x.softmax_scale, "bf16")
    assert np.array_equal(o8, ob) and np.array_equal(l8, lb)
    assert np.all(np.isfinite(o8))


def test_unreferenced_mxfp8_rows_are_poisoned():
    x = make_inputs(14, [100, 40], 1, 2, "mxfp8", page_size=64)
    nb = x.numpy_bits()
    used = np.zeros(x.num_slots, dtype=bool)
    for b, n in enumerate(x.local_lens):
        used[nb["req_to_token"][b, :n]] = True
    assert np.all(nb["pool"][~used, :576] == 0x7F)
    assert np.all(nb["pool"][~used, 576:594] == 0xFF)
    assert np.all(nb["pool"][:, 594:] == 0)
    sc = nb["pool"][used, 576:594]
    assert sc.min() >= 122 and sc.max() <= 124
    assert not np.any(np.isin(nb["pool"][used, :576], [0x7F, 0xFF]))


# ----------------------------------------------------------------- quantiser

def test_quantiser_round_trips_representable_rows():
    rng = np.random.default_rng(6)
    n = 5
    e = rng.integers(-12, 12, size=(n, 18))
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)])
    codes = finite[rng.integers(0, len(finite), size=(n, 576))]
    codes[:, ::32] = 0x7E                                # each block reaches 448 * 2^e
    codes[codes == 0x80] = 0                             # no -0 in the input
    x = E4M3FN_TABLE[codes] * np.repeat(np.ldexp(1.0, e), 32, axis=1)
    rows = mxfp8_quantise_rows(x)
    assert np.array_equal(rows[:, 576:594], (e + 127).astype(np.uint8))
    assert np.array_equal(decode_mxfp8_rows(rows), x)
    assert np.array_equal(rows[:, :576], codes.astype(np.uint8))
    assert np.all(rows[:, 594:] == 0)


def test_exponent_rule_at_its_edges():
    f32 = np.float32
    up448 = float(np.nextafter(f32(448.0), f32(np.inf)))
    assert list(block_exponent_of([448.0, up448, 224.0, 1.0, 0.0, 1e-30])) == \
        [0, 1, -1, -8, -64, -64]
    assert list(block_exponent_of([448.0 * 2.0 ** 64, 1e30])) == [64, 64]


def test_quantiser_ties_clamps_and_zero_blocks():
    x = np.zeros((2, 576))
    x[0, 0] = 448.0                                      # block 0 at 2^0
    x[0, 1] = 1.0 + 1.0 / 16                             # halfway 1 and 1.125: even code (1)
    x[0, 2] = 1.0 + 3.0 / 16                             # halfway 1.125 and 1.25: even (1.25)
    x[0, 32:64] = 1e30                                   # saturates at 448 * 2^64
    x[1, 64:96] = 1e-30                                  # below the smallest step at 2^-64
    rows = mxfp8_quantise_rows(x)
    v = decode_mxfp8_rows(rows)
    assert v[0, 1] == 1.0 and v[0, 2] == 1.25
    assert np.all(v[0, 32:64] == 448.0 * 2.0 ** 64) and rows[0, 577] == 191
    assert np.all(v[1] == 0.0) and rows[1, 578] == 63


def test_quantiser_is_nearest_by_brute_force():
    rng = np.random.default_rng(10)
    x = (rng.standard_normal((4, 576)) * np.exp(rng.uniform(-8, 8, size=(4, 1)))).astype(
        np.float32).astype(np.float64)
    rows = mxfp8_quantise_rows(x)
    v = decode_mxfp8_rows(rows)
    e = rows[:, 576:594].astype(np.int64) - 127
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)])
    for t in range(4):
        for k in range(18):
            a = np.abs(x[t, 32 * k:32 * k + 32]).max()
            assert a <= 448.0 * 2.0 ** e[t, k] and not a <= 448.0 * 2.0 ** (e[t, k] - 1)
            cand = E4M3FN_TABLE[finite] * 2.0 ** e[t, k]
            for d in range(32 * k, 32 * k + 32):
                dist = np.abs(cand - x[t, d])
                best = dist.min()
                assert abs(v[t, d] - x[t, d]) == best
                ties = finite[dist == best]
                if np.unique(cand[dist == best]).size > 1:
                    assert rows[t, d] % 2 == 0 and rows[t, d] in ties   # even code of the tie
