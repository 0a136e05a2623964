"""Pins of the MLA-prepare oracle against things other than itself (CPU only).

Library cross-checks of the two encoders (torch's float32 -> bfloat16 and
float32 -> float8_e4m3fn conversions, both round-to-nearest-even), a scalar
brute-force e4m3fn encoder, the rotation written as a complex product in
float64, closed forms (identity rotations and weights, unit vectors), a
50-digit brute force of the absorption GEMM on tiny inputs, and the FP8
append's own invariants.  A last test plants plausible mistakes in single
oracle steps and checks that these pins catch every one of them.
"""

import math
import struct

import mpmath
import numpy as np
import pytest
import torch

import oracle
from oracle import prepare_ref as P

mpmath.mp.dps = 50
_FP8 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()


def _rng(k):
    return np.random.default_rng(np.random.SeedSequence([77, k]))


def _bf16_bits(rng, shape, std=1.0):
    x = torch.from_numpy((rng.standard_normal(shape) * std).astype(np.float32))
    return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _near_ties(rng, n):
    # Random values in [-448, 448] plus exact midpoints of neighbouring
    # e4m3fn values and their float32 neighbours.
    vals = np.sort(_FP8[:0x7F])
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    around = np.concatenate([mids, np.nextafter(mids, np.float32(0)),
                             np.nextafter(mids, np.float32(1e9))])
    r = (rng.uniform(-448, 448, n) * rng.choice([1, 1e-2, 1e-4], n)).astype(np.float32)
    allv = np.concatenate([r, around, -around])
    return allv[np.abs(allv) <= 448].astype(np.float32)


def _brute_e4m3(x: float) -> int:
    best, best_d = None, None
    for code in range(256):
        v = _FP8[code]
        if math.isnan(v):
            continue
        d = abs(v - x)
        if best is None or d < best_d or (d == best_d and (code & 1) == 0 and (best & 1)):
            best, best_d = code, d
    # the sign of zero follows the input
    if best in (0x00, 0x80):
        best = 0x80 if math.copysign(1.0, x) < 0 else 0x00
    return best


# ---------------------------------------------------------------- encoders

def test_e4m3fn_encode_inverts_the_decode_table():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = oracle.E4M3FN_TABLE[codes].astype(np.float32)
    vals[codes == 0x80] = np.float32(-0.0)
    np.testing.assert_array_equal(P.e4m3fn_encode(vals), codes)


def test_e4m3fn_encode_matches_torch_and_brute_force():
    x = _near_ties(_rng(1), 20000)
    got = P.e4m3fn_encode(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(got, ref)
    sub = x[::37]
    np.testing.assert_array_equal(P.e4m3fn_encode(sub),
                                  np.array([_brute_e4m3(float(v)) for v in sub], np.uint8))


def test_e4m3fn_encode_ties_and_edges():
    # 1.0625 lies halfway between 1.0 (0x38) and 1.125 (0x39): even mantissa.
    assert P.e4m3fn_encode(np.float32(1.0625)) == 0x38
    assert P.e4m3fn_encode(np.float32(1.1875)) == 0x3A
    assert P.e4m3fn_encode(np.float32(448.0)) == 0x7E
    assert P.e4m3fn_encode(np.float32(-448.0)) == 0xFE
    # Half the smallest subnormal (2^-9) ties to zero; a hair above goes up.
    assert P.e4m3fn_encode(np.float32(2.0 ** -10)) == 0x00
    assert P.e4m3fn_encode(np.nextafter(np.float32(2.0 ** -10), np.float32(1))) == 0x01
    assert P.e4m3fn_encode(np.float32(-1e-30)) == 0x80
    with pytest.raises(ValueError):
        P.e4m3fn_encode(np.float32(449.0))


def test_bf16_rounding_matches_torch():
    rng = _rng(2)
    x = (rng.standard_normal(50000) * rng.choice([1, 1e3, 1e-3], 50000)).astype(np.float32)
    # exact ties: low 16 bits 0x8000
    u = x.view(np.uint32)
    ties = ((u & np.uint32(0xFFFF0000)) | np.uint32(0x8000)).view(np.float32)
    x = np.concatenate([x, ties])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(P.f32_to_bf16_bits(x), ref)


# ---------------------------------------------------------------- RoPE

def test_rope_identity_and_unit_vectors():
    rng = _rng(3)
    x = rng.standard_normal((5, 64)).astype(np.float32)
    one, zero = np.ones((5, 32), np.float32), np.zeros((5, 32), np.float32)
    np.testing.assert_array_equal(P.rope_f32(x, one, zero), x)
    th = rng.uniform(-3, 3, (5, 32))
    c, s = np.cos(th).astype(np.float32), np.sin(th).astype(np.float32)
    for i in (0, 7, 31):
        e = np.zeros((5, 64), np.float32)
        e[:, 2 * i] = 1.0
        y = P.rope_f32(e, c, s)
        np.testing.assert_array_equal(y[:, 2 * i], c[:, i])
        np.testing.assert_array_equal(y[:, 2 * i + 1], s[:, i])
        e[:, 2 * i], e[:, 2 * i + 1] = 0.0, 1.0
        y = P.rope_f32(e, c, s)
        np.testing.assert_array_equal(y[:, 2 * i], -s[:, i])
        np.testing.assert_array_equal(y[:, 2 * i + 1], c[:, i])


def test_rope_is_a_complex_rotation():
    rng = _rng(4)
    x = rng.standard_normal((200, 64)).astype(np.float32)
    th = rng.uniform(-100, 100, (200, 32))
    c, s = np.cos(th).astype(np.float32), np.sin(th).astype(np.float32)
    y = P.rope_f32(x, c, s).astype(np.float64)
    z = (x[:, 0::2].astype(np.float64) + 1j * x[:, 1::2]) * (c + 1j * s.astype(np.float64))
    np.testing.assert_allclose(y[:, 0::2], z.real, rtol=0, atol=2e-6)
    np.testing.assert_allclose(y[:, 1::2], z.imag, rtol=0, atol=2e-6)


def _round_f32(q):
    """Nearest float32 (ties to even) of an exact rational q, by integer
    arithmetic: an independent statement of a correctly rounded float32
    operation."""
    from fractions import Fraction
    if q == 0:
        return 0.0
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, -126)                       # subnormals share the smallest exponent
    scaled = a / Fraction(2) ** (e - 23)   # mantissa with 23 fraction bits
    m = scaled.numerator // scaled.denominator
    rem = scaled - m
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and m % 2 == 1):
        m += 1
    return sign * float(Fraction(m) * Fraction(2) ** (e - 23))


def test_rope_bits_match_exact_rational_rounding():
    """Every output bit of rope_f32 against the definition: each product
    x0 c, x1 s, x0 s, x1 c correctly rounded to float32, then the difference
    / sum of the rounded products correctly rounded to float32 (no fused
    multiply-add), with each rounding computed from exact rationals."""
    from fractions import Fraction
    rng = _rng(41)
    n = 300
    x = rng.standard_normal((n, 2)).astype(np.float32) * np.float32(3.0)
    th = rng.uniform(-50, 50, n)
    c, s = np.cos(th).astype(np.float32), np.sin(th).astype(np.float32)
    # Cases where the two products nearly cancel (the difference is exact in
    # float32 but not in a wider rounding of the operands), and tiny values.
    x[:40, 1] = (x[:40, 0] * c[:40] / np.where(s[:40] == 0, 1, s[:40])).astype(np.float32)
    x[40:60] *= np.float32(1e-30)
    xx = np.zeros((n, 64), np.float32)
    xx[:, 0:2] = x
    cc = np.zeros((n, 32), np.float32)
    ss = np.zeros((n, 32), np.float32)
    cc[:, 0], ss[:, 0] = c, s
    y = P.rope_f32(xx, cc, ss)
    for k in range(n):
        F = [Fraction(float(v)) for v in (x[k, 0], x[k, 1], c[k], s[k])]
        p0c, p1s = _round_f32(F[0] * F[2]), _round_f32(F[1] * F[3])
        p0s, p1c = _round_f32(F[0] * F[3]), _round_f32(F[1] * F[2])
        y0 = np.float32(_round_f32(Fraction(p0c) - Fraction(p1s)))
        y1 = np.float32(_round_f32(Fraction(p0s) + Fraction(p1c)))
        assert y[k, 0].view(np.uint32) == y0.view(np.uint32), k
        assert y[k, 1].view(np.uint32) == y1.view(np.uint32), k


def test_q_rope_uses_each_tokens_position():
    rng = _rng(5)
    T, H = 4, 3
    q = _bf16_bits(rng, (T, H, 64))
    th = rng.uniform(-3, 3, (10, 32))
    tab = np.concatenate([np.cos(th), np.sin(th)], axis=1).astype(np.float32)
    pos = np.array([9, 0, 3, 3])
    got = P.q_rope_ref(q, tab, pos)
    for t in range(T):
        for h in range(H):
            y = P.rope_f32(P.bf16_bits_to_f32(q[t, h]), tab[pos[t], :32], tab[pos[t], 32:])
            np.testing.assert_array_equal(got[t, h], P.f32_to_bf16_bits(y))


# ---------------------------------------------------------------- absorption

def test_q_absorb_matches_50_digit_brute_force():
    rng = _rng(6)
    T, H = 3, 2
    q = _bf16_bits(rng, (T, H, 128))
    w = _bf16_bits(rng, (H, 128, 512), std=0.05)          # w_kc[h, k, n]
    wt = np.ascontiguousarray(np.transpose(w, (0, 2, 1)))   # [h, n, k]
    got = P.q_absorb_ref(q, wt)

    def f(b):
        return struct.unpack("<f", struct.pack("<I", int(b) << 16))[0]
    for t in range(T):
        for h in range(H):
            for n in (0, 1, 127, 128, 300, 511):
                ref = mpmath.fsum(mpmath.mpf(f(q[t, h, k])) * mpmath.mpf(f(w[h, k, n]))
                                  for k in range(128))
                assert abs(got[t, h, n] - float(ref)) <= 1e-12 * (1 + abs(float(ref)))


def test_q_absorb_identity_weights():
    rng = _rng(7)
    q = _bf16_bits(rng, (4, 3, 128))
    wt = np.zeros((3, 512, 128), np.uint16)
    wt[:, np.arange(128), np.arange(128)] = 0x3F80  # BF16 1.0
    got = P.q_absorb_ref(q, wt)
    np.testing.assert_array_equal(got[..., :128], oracle.bf16_bits_to_f64(q))
    assert not got[..., 128:].any()


# ---------------------------------------------------------------- KV append

def _append_case(kv, seed=8, T=6, n=20):
    rng = _rng(seed)
    c_kv = _bf16_bits(rng, (T, 512))
    k_rope = _bf16_bits(rng, (T, 64))
    th = rng.uniform(-3, 3, (50, 32))
    tab = np.concatenate([np.cos(th), np.sin(th)], axis=1).astype(np.float32)
    pos = rng.integers(0, 50, T)
    slots = rng.permutation(n)[:T].astype(np.int32)
    slots[2] = -1
    if kv == "bf16":
        pool = _bf16_bits(rng, (n, 576))
        sc = None
    elif kv == "fp4":
        pool = rng.integers(0, 255, (n, 336)).astype(np.uint8)
        sc = None
    elif kv == "mxfp8":
        pool = rng.integers(0, 255, (n, 608)).astype(np.uint8)
        sc = None
    else:
        pool = rng.integers(0, 255, (n, 576)).astype(np.uint8)
        sc = rng.uniform(0.01, 0.05, n).astype(np.float32)
    return c_kv, k_rope, tab, pos, slots, pool, sc


def test_bf16_append_copies_c_kv_and_ropes_k():
    c_kv, k_rope, tab, pos, slots, pool, _ = _append_case("bf16")
    new, _ = P.kv_append_ref(pool, None, c_kv, k_rope, tab, pos, slots, "bf16")
    qr = P.q_rope_ref(k_rope[:, None, :], tab, pos)[:, 0]   # same rotation as a 1-head query
    for t, sl in enumerate(slots):
        if sl < 0:
            continue
        np.testing.assert_array_equal(new[sl, :512], c_kv[t])
        np.testing.assert_array_equal(new[sl, 512:], qr[t])
    untouched = np.setdiff1d(np.arange(len(pool)), slots[slots >= 0])
    np.testing.assert_array_equal(new[untouched], pool[untouched])


def test_fp8_append_scale_codes_and_error():
    c_kv, k_rope, tab, pos, slots, pool, sc = _append_case("fp8")
    new, nsc = P.kv_append_ref(pool, sc, c_kv, k_rope, tab, pos, slots, "fp8")
    rows = P.bf16_bits_to_f32(P.latent_rows_ref(c_kv, k_rope, tab, pos)).astype(np.float64)
    for t, sl in enumerate(slots):
        if sl < 0:
            continue
        amax = np.abs(rows[t]).max()
        assert nsc[sl] == np.float32(np.float32(amax) / np.float32(448.0))
        j = int(np.argmax(np.abs(rows[t])))
        assert new[sl, j] in (0x7E, 0xFE)
        dec = oracle.E4M3FN_TABLE[new[sl]] * np.float64(nsc[sl])
        # e4m3: 3 mantissa bits (half-ulp 2^-4 relative), subnormal step 2^-9.
        bound = np.maximum(np.abs(rows[t]) * 2.0 ** -4, 2.0 ** -10 * nsc[sl]) * 1.0001
        assert np.all(np.abs(dec - rows[t]) <= bound)
    untouched = np.setdiff1d(np.arange(len(pool)), slots[slots >= 0])
    np.testing.assert_array_equal(new[untouched], pool[untouched])
    np.testing.assert_array_equal(nsc[untouched], sc[untouched])


def test_fp4_append_writes_rows_within_half_a_grid_step():
    # FP4 rows of the roped latent rows: within half of the e2m1 grid gap
    # (at most 2^e, between the codes 4 and 6) of every value, each block's
    # exponent the smallest that holds its largest value, the padding zero;
    # other slots untouched.
    c_kv, k_rope, tab, pos, slots, pool, _ = _append_case("fp4")
    new, nsc = P.kv_append_ref(pool, None, c_kv, k_rope, tab, pos, slots, "fp4")
    assert nsc is None
    rows = P.bf16_bits_to_f32(P.latent_rows_ref(c_kv, k_rope, tab, pos)).astype(np.float64)
    for t, sl in enumerate(slots):
        if sl < 0:
            continue
        dec = oracle.decode_fp4_rows(new[sl][None])[0]
        e = new[sl, 288:324].astype(np.int64) - 127
        step = np.repeat(np.ldexp(1.0, e), 16)
        assert np.all(np.abs(dec - rows[t]) <= step)
        amax = np.abs(rows[t]).reshape(36, 16).max(axis=1)
        assert np.all(amax <= 6.0 * np.ldexp(1.0, e)) and np.all(amax > 3.0 * np.ldexp(1.0, e))
        assert not new[sl, 324:].any()
    untouched = np.setdiff1d(np.arange(len(pool)), slots[slots >= 0])
    np.testing.assert_array_equal(new[untouched], pool[untouched])


def test_mxfp8_append_writes_rows_within_half_a_step():
    # MXFP8 rows: within half an e4m3 step of every value (2^-4 relative,
    # 2^-10 * 2^e below the normal range), each block's exponent the
    # smallest that holds its largest value, the padding zero.
    c_kv, k_rope, tab, pos, slots, pool, _ = _append_case("mxfp8")
    new, nsc = P.kv_append_ref(pool, None, c_kv, k_rope, tab, pos, slots, "mxfp8")
    assert nsc is None
    rows = P.bf16_bits_to_f32(P.latent_rows_ref(c_kv, k_rope, tab, pos)).astype(np.float64)
    for t, sl in enumerate(slots):
        if sl < 0:
            continue
        dec = oracle.decode_mxfp8_rows(new[sl][None])[0]
        e = new[sl, 576:594].astype(np.int64) - 127
        sc = np.repeat(np.ldexp(1.0, e), 32)
        bound = np.maximum(np.abs(rows[t]) * 2.0 ** -4, 2.0 ** -10 * sc) * 1.0001
        assert np.all(np.abs(dec - rows[t]) <= bound)
        amax = np.abs(rows[t]).reshape(18, 32).max(axis=1)
        assert np.all(amax <= 448.0 * np.ldexp(1.0, e)) and np.all(amax > 224.0 * np.ldexp(1.0, e))
        assert not new[sl, 594:].any()
    untouched = np.setdiff1d(np.arange(len(pool)), slots[slots >= 0])
    np.testing.assert_array_equal(new[untouched], pool[untouched])


def test_fp8_append_zero_row():
    c_kv = np.zeros((1, 512), np.uint16)
    k_rope = np.zeros((1, 64), np.uint16)
    tab = np.ones((1, 64), np.float32)
    new, nsc = P.kv_append_ref(np.full((2, 576), 7, np.uint8), np.ones(2, np.float32),
                               c_kv, k_rope, tab, [0], [1], "fp8")
    assert nsc[1] == 1.0 and not new[1].any() and np.all(new[0] == 7)


# ---------------------------------------------------------------- planted mistakes

def _run_pins():
    for f in (test_e4m3fn_encode_inverts_the_decode_table,
              test_e4m3fn_encode_matches_torch_and_brute_force,
              test_e4m3fn_encode_ties_and_edges, test_bf16_rounding_matches_torch,
              test_rope_identity_and_unit_vectors, test_rope_is_a_complex_rotation,
              test_q_rope_uses_each_tokens_position, test_q_absorb_matches_50_digit_brute_force,
              test_q_absorb_identity_weights, test_bf16_append_copies_c_kv_and_ropes_k,
              test_fp8_append_scale_codes_and_error, test_fp8_append_zero_row):
        f()


def _rope_halves(x, cos, sin):  # rotates (x[i], x[i + 32]) instead of interleaved pairs
    x = np.asarray(x, np.float32)
    c, s = np.asarray(cos, np.float32), np.asarray(sin, np.float32)
    y = np.empty_like(x)
    y[..., :32] = x[..., :32] * c - x[..., 32:] * s
    y[..., 32:] = x[..., :32] * s + x[..., 32:] * c
    return y


def _encode_ties_away(x):  # ties away from zero instead of to even
    v = np.asarray(x, np.float32).astype(np.float64)
    mag = np.abs(v)
    vals = P._POS_VALUES
    hi = np.minimum(np.searchsorted(vals, mag, side="left"), len(vals) - 1)
    lo = np.maximum(hi - 1, 0)
    pick_hi = (vals[hi] - mag) <= (mag - vals[lo])
    code = np.where(pick_hi, P._POS_CODES[hi], P._POS_CODES[lo]).astype(np.uint8)
    return np.where(np.signbit(np.asarray(x, np.float32)), code | np.uint8(0x80), code)


def _bf16_truncate(x):  # truncation instead of nearest-even
    return (np.asarray(x, np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _quantise_447(row_bits):  # scale off by one code
    x = P.bf16_bits_to_f32(row_bits)
    amax = np.max(np.abs(x), axis=1)
    scale = np.where(amax > 0, amax / np.float32(447.0), np.float32(1)).astype(np.float32)
    q = np.clip((x / scale[:, None]).astype(np.float32), -448, 448).astype(np.float32)
    return P.e4m3fn_encode(q), scale


def _absorb_no_transpose(q_bits, wt_bits):  # reads w_kc_t as if it were [h, k, n]
    q = oracle.bf16_bits_to_f64(q_bits)
    wt = oracle.bf16_bits_to_f64(wt_bits).reshape(wt_bits.shape[0], 128, 512)
    return np.einsum("thk,hkn->thn", q, wt)


@pytest.mark.parametrize("name,patch", [
    ("rope_f32", _rope_halves), ("rope_f32", "sign"), ("e4m3fn_encode", _encode_ties_away),
    ("f32_to_bf16_bits", _bf16_truncate), ("fp8_quantise_rows", _quantise_447),
    ("q_absorb_ref", _absorb_no_transpose)])
def test_planted_mistakes_are_caught(monkeypatch, name, patch):
    orig = getattr(P, name)
    if patch == "sign":
        def patch(x, cos, sin):
            return orig(x, cos, -np.asarray(sin, np.float32))
    monkeypatch.setattr(P, name, patch)
    with pytest.raises(AssertionError):
        _run_pins()
