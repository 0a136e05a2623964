"""Pins of the up-projection oracle (CPU only).

A 50-digit brute force of merge-then-project on tiny inputs, the closed forms
(one part is no merge, identity weights copy the first 128 latent features,
all-empty rows give zeros), the identity that merging and projecting commute
(the projection is linear and the merge weights sum to one), and planted
mistakes that these pins catch.
"""

import struct

import mpmath
import numpy as np
import pytest
import torch

import oracle
from oracle import project_ref as PR

mpmath.mp.dps = 50


def _rng(k):
    return np.random.default_rng(np.random.SeedSequence([88, k]))


def _bf16_bits(rng, shape, std=1.0):
    x = torch.from_numpy((rng.standard_normal(shape) * std).astype(np.float32))
    return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _f(b):
    return struct.unpack("<f", struct.pack("<I", int(b) << 16))[0]


def test_merge_then_project_matches_50_digit_brute_force():
    rng = _rng(1)
    P, T, H = 3, 2, 2
    po = rng.standard_normal((P, T, H, 512))
    pl = rng.standard_normal((P, T, H)) * 3
    pl[1, 0, 1] = -np.inf
    wt = _bf16_bits(rng, (H, 128, 512), 0.05)
    out, lse = PR.lse_combine_project_ref(po, pl, wt)
    for t in range(T):
        for h in range(H):
            ls = [mpmath.mpf(float(v)) if np.isfinite(v) else None for v in pl[:, t, h]]
            m = max(v for v in ls if v is not None)
            wts = [mpmath.e ** (v - m) if v is not None else mpmath.mpf(0) for v in ls]
            sw = mpmath.fsum(wts)
            assert abs(float(m + mpmath.log(sw)) - lse[t, h]) < 1e-12
            for n in (0, 5, 127):
                ref = mpmath.fsum(
                    mpmath.fsum(wts[j] * mpmath.mpf(float(po[j, t, h, k])) for j in range(P)) / sw
                    * mpmath.mpf(_f(wt[h, n, k])) for k in range(512))
                assert abs(float(ref) - out[t, h, n]) <= 1e-10 * (1 + abs(float(ref)))


def test_one_part_and_identity_weights():
    rng = _rng(2)
    po = rng.standard_normal((1, 3, 4, 512))
    pl = rng.standard_normal((1, 3, 4))
    wt = np.zeros((4, 128, 512), np.uint16)
    wt[:, np.arange(128), np.arange(128)] = 0x3F80
    out, lse = PR.lse_combine_project_ref(po, pl, wt)
    np.testing.assert_array_equal(lse, pl[0])
    np.testing.assert_allclose(out, po[0, :, :, :128], rtol=1e-15, atol=0)


def test_empty_rows_give_zero():
    rng = _rng(3)
    po = rng.standard_normal((4, 2, 3, 512))
    pl = np.full((4, 2, 3), -np.inf)
    wt = _bf16_bits(rng, (3, 128, 512))
    out, lse = PR.lse_combine_project_ref(po, pl, wt)
    assert np.all(np.isneginf(lse)) and not out.any()


def test_merging_and_projecting_commute():
    rng = _rng(4)
    P, T, H = 5, 3, 2
    po = rng.standard_normal((P, T, H, 512))
    pl = rng.standard_normal((P, T, H)) * 2
    wt = _bf16_bits(rng, (H, 128, 512), 0.05)
    out, lse = PR.lse_combine_project_ref(po, pl, wt)
    proj_parts = np.stack([PR.vc_project_ref(po[j], wt) for j in range(P)])
    out2, lse2 = oracle.lse_combine_ref(proj_parts, pl)
    np.testing.assert_allclose(out, out2, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(lse, lse2)


def _run_pins():
    test_merge_then_project_matches_50_digit_brute_force()
    test_one_part_and_identity_weights()
    test_empty_rows_give_zero()
    test_merging_and_projecting_commute()


def _project_untransposed(o, wt_bits):  # reads w_vc_t as [h, k, n]
    o = np.asarray(o, np.float64)
    w = oracle.bf16_bits_to_f64(wt_bits).reshape(wt_bits.shape[0], 512, 128)
    return np.einsum("thk,hkn->thn", o, w)


def _project_wrong_head(o, wt_bits):  # every head uses head 0's weights
    o = np.asarray(o, np.float64)
    wt = oracle.bf16_bits_to_f64(wt_bits)
    return np.einsum("thk,nk->thn", o, wt[0])


@pytest.mark.parametrize("patch", [_project_untransposed, _project_wrong_head])
def test_planted_mistakes_are_caught(monkeypatch, patch):
    monkeypatch.setattr(PR, "vc_project_ref", patch)
    with pytest.raises(AssertionError):
        _run_pins()
