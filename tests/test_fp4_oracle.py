"""Pins of the FP4 KV format in the oracle (oracle/fp4_ref.py).

The format (VRAM page, "KV ledger" and "cell_size" sections: two e2m1
codes per byte plus one scale per 16 elements; the element and scale
encodings are readings, stated in fp4_ref): the decode is pinned to the
e2m1 value list of the OCP MX specification and to a row worked out by
hand; the quantiser to exact round trips, the tie rule, the exponent rule
at its edges and a brute-force nearest-value search.
"""

import numpy as np
import pytest

from oracle import (bf16_bits_to_f64, decode_fp4_rows, e2m1_encode, fp4_quantise_rows,
                    block_exponent_of, mla_decode_ref, E2M1_TABLE)
from workload import make_inputs

# OCP MX specification, FP4 (E2M1) element values by code 0b0000 .. 0b0111;
# codes 0b1000 .. 0b1111 are their negatives.
SPEC_E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_table_is_the_format_value_list():
    assert list(E2M1_TABLE[:8]) == SPEC_E2M1
    assert list(E2M1_TABLE[8:]) == [-v for v in SPEC_E2M1]
    assert np.signbit(E2M1_TABLE[8])            # code 0b1000 is -0


def _blank_row():
    row = np.zeros(336, dtype=np.uint8)
    row[288:324] = 127                          # every block scale 2^0
    return row


def test_hand_worked_row():
    row = _blank_row()
    row[0] = 0x72          # element 0 = code 2 (1.0), element 1 = code 7 (6.0)
    row[1] = 0x9F          # element 2 = code 15 (-6), element 3 = code 9 (-0.5)
    row[9] = 0x05          # element 18 = code 5 (3.0), in block 1
    row[287] = 0x1E        # element 574 = code 14 (-4), element 575 = code 1 (0.5)
    row[288] = 128         # block 0 (elements 0..15) x 2
    row[289] = 125         # block 1 (elements 16..31) x 1/4
    row[323] = 124         # block 35 (elements 560..575) x 1/8
    v = decode_fp4_rows(row[None])[0]
    want = np.zeros(576)
    want[0], want[1], want[2], want[3] = 2.0, 12.0, -12.0, -1.0
    want[18] = 0.75
    want[574], want[575] = -0.5, 0.0625
    assert np.array_equal(v, want)


def test_decode_rejects_out_of_range_scales_and_bad_shapes():
    row = _blank_row()
    row[300] = 255
    with pytest.raises(ValueError):
        decode_fp4_rows(row[None])
    row[300] = 62
    with pytest.raises(ValueError):
        decode_fp4_rows(row[None])
    with pytest.raises(ValueError):
        decode_fp4_rows(np.zeros((1, 324), dtype=np.uint8))


def _bf16_bits_of(values: np.ndarray) -> np.ndarray:
    """BF16 bits of values that BF16 holds exactly (checked)."""
    f = values.astype(np.float32)
    assert np.array_equal(f.astype(np.float64), values)
    bits = (f.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(bf16_bits_to_f64(bits), values)
    return bits


def test_fp4_decode_is_the_bf16_decode_of_the_decoded_values():
    """An FP4 pool attends exactly like a BF16 pool holding its values (every
    FP4 value with these scales is a BF16 value), so the FP4 branch reduces
    to the BF16 one, pinned in test_oracle."""
    x = make_inputs(11, [200, 77, 5], 5, 4, "fp4", page_size=16)
    nb = x.numpy_bits()
    pool = nb["pool"]
    used = np.concatenate([nb["req_to_token"][b, :n] for b, n in enumerate(x.local_lens)])
    bf = np.full((pool.shape[0], 576), 0x7FC0, dtype=np.uint16)
    bf[used] = _bf16_bits_of(decode_fp4_rows(pool[used]))
    args = (nb["q_nope"], nb["q_rope"])
    o4, l4 = mla_decode_ref(*args, pool, None, nb["req_to_token"], nb["seq_lens"], 5,
                            x.softmax_scale, "fp4")
    ob, lb = mla_decode_ref(*args, bf, None, nb["req_to_token"], nb["seq_lens"], 5,
                            x.softmax_scale, "bf16")
    assert np.array_equal(o4, ob) and np.array_equal(l4, lb)
    assert np.all(np.isfinite(o4))


def test_unreferenced_fp4_rows_are_poisoned():
    x = make_inputs(12, [100, 40], 1, 2, "fp4", page_size=64)
    nb = x.numpy_bits()
    used = np.zeros(x.num_slots, dtype=bool)
    for b, n in enumerate(x.local_lens):
        used[nb["req_to_token"][b, :n]] = True
    assert np.all(nb["pool"][~used, :288] == 0x77)
    assert np.all(nb["pool"][~used, 288:324] == 0xFF)
    assert np.all(nb["pool"][:, 324:] == 0)
    sc = nb["pool"][used, 288:324]
    assert sc.min() >= 121 and sc.max() <= 123


# ----------------------------------------------------------------- quantiser

def test_quantiser_round_trips_representable_rows():
    rng = np.random.default_rng(5)
    n = 6
    e = rng.integers(-10, 10, size=(n, 36))
    codes = rng.integers(0, 8, size=(n, 576))
    sign = rng.integers(0, 2, size=(n, 576))
    codes[:, ::16] = 7                                   # each block reaches 6 * 2^e
    vals = np.array(SPEC_E2M1)[codes] * np.where(sign == 1, -1.0, 1.0)
    vals = np.where(codes == 0, 0.0, vals)               # no -0 in the input
    x = vals * np.repeat(np.ldexp(1.0, e), 16, axis=1)
    rows = fp4_quantise_rows(x)
    assert np.array_equal(rows[:, 288:324], (e + 127).astype(np.uint8))
    assert np.array_equal(decode_fp4_rows(rows), x)
    assert np.all(rows[:, 324:] == 0)


def test_quantiser_ties_go_to_the_even_code():
    x = np.zeros((1, 576))
    x[0, 0] = 6.0                                        # block exponent 0
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    x[0, 1:8] = mids
    x[0, 8:15] = [-m for m in mids]
    got = decode_fp4_rows(fp4_quantise_rows(x))[0]
    want = [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0]          # the neighbour with mantissa bit 0
    assert list(got[1:8]) == want
    assert list(got[8:15]) == [-w for w in want]
    assert np.signbit(got[8])                            # -0.25 -> -0
    # Just off the midpoints the nearest value wins.
    x[0, 1:8] = np.nextafter(np.array(mids), np.inf)
    got = decode_fp4_rows(fp4_quantise_rows(x))[0]
    assert list(got[1:8]) == [0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_exponent_rule_at_its_edges():
    f32 = np.float32
    six_up = float(np.nextafter(f32(6.0), f32(np.inf)))
    three_up = float(np.nextafter(f32(3.0), f32(np.inf)))
    assert list(block_exponent_of([6.0, six_up, 3.0, three_up, 0.75, 1e-30, 0.0])) == \
        [0, 1, -1, 0, -3, -64, -64]
    assert list(block_exponent_of([6.0 * 2.0 ** 64, 6.0 * 2.0 ** 64 * 1.5, 1e30])) == \
        [64, 64, 64]


def test_quantiser_clamps_and_zero_blocks():
    x = np.zeros((2, 576))
    x[0, :16] = 1e30                                     # beyond 6 * 2^64: saturates
    x[0, 16:32] = -1e30
    x[1, 32:48] = 1e-30                                  # below the smallest grid step
    rows = fp4_quantise_rows(x)
    v = decode_fp4_rows(rows)
    assert np.all(v[0, :16] == 6.0 * 2.0 ** 64) and np.all(v[0, 16:32] == -6.0 * 2.0 ** 64)
    assert rows[0, 288] == 191 and rows[1, 288] == 63 and rows[1, 290] == 63
    assert np.all(v[1] == 0.0)


def test_quantiser_is_nearest_by_brute_force():
    """Each element's decoded value is a nearest one among the 16 values of
    its block's grid (ties to an even code), and the block exponent is the
    smallest that keeps the block's largest magnitude within 6 * 2^e."""
    rng = np.random.default_rng(9)
    x = (rng.standard_normal((8, 576)) * np.exp(rng.uniform(-6, 6, size=(8, 1)))).astype(
        np.float32).astype(np.float64)
    rows = fp4_quantise_rows(x)
    v = decode_fp4_rows(rows)
    e = rows[:, 288:324].astype(np.int64) - 127
    grid = np.array(SPEC_E2M1 + [-s for s in SPEC_E2M1])
    for t in range(8):
        for k in range(36):
            a = np.abs(x[t, 16 * k:16 * k + 16]).max()
            assert a <= 6.0 * 2.0 ** e[t, k] and not a <= 6.0 * 2.0 ** (e[t, k] - 1)
            for d in range(16 * k, 16 * k + 16):
                cand = grid * 2.0 ** e[t, k]
                dist = np.abs(cand - x[t, d])
                best = dist.min()
                assert abs(v[t, d] - x[t, d]) == best
                ties = np.flatnonzero(dist == best)
                if len(ties) > 1 and np.any(cand[ties] != cand[ties][0]):
                    idx = [i for i in ties if cand[i] == v[t, d]]
                    assert any(i % 2 == 0 for i in idx)          # even code of the tie


def test_e2m1_encode_sign_and_range():
    assert list(e2m1_encode(np.array([0.0, -0.0, -6.0, 6.0, -0.2]))) == [0, 8, 15, 7, 8]
    with pytest.raises(ValueError):
        e2m1_encode(np.array([6.5]))
