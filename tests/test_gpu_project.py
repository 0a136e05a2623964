"""GPU parity of mla_lse_combine_project (LSE merge + w_vc up-projection).

The kernel rounds the merged latent O to bf16 before its MFMAs and rounds the
fp32 sums to bf16, so each output element may differ from the float64
reference by at most 2^-9 of |out| plus 2^-9 of sum_k |O_k w_k| (the two
roundings); the check allows twice that, 2^-8 (|ref| + sum_k |O_k w_k|),
plus 1e-6 of the largest |ref|.  The merged LSE must match within 1e-5.
Rows whose parts are all empty must give out = 0 and LSE = -inf.
"""

import numpy as np
import pytest
import torch

import mla_latent_kv_absorbed_amd as mla
from oracle import lse_combine_project_ref, lse_combine_ref, vc_project_ref

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _case(seed, P, T, H):
    rng = np.random.default_rng(np.random.SeedSequence([92, seed]))
    po = rng.standard_normal((P, T, H, 512)).astype(np.float32)
    pl = (rng.standard_normal((P, T, H)) * 3).astype(np.float32)
    if P > 1:
        pl[rng.random((P, T, H)) < 0.2] = -np.inf      # empty parts
        po[np.isneginf(pl)] = np.nan                   # their O must never be read
    if T > 2:
        pl[:, 1, :] = -np.inf                          # a token with no visible key anywhere
        po[:, 1, :] = 0.0
    w = (rng.standard_normal((H, 128, 512)) * 0.05).astype(np.float32)
    wt = torch.from_numpy(w).to(torch.bfloat16)
    return po, pl, wt


def _check(P, T, H, seed):
    po, pl, wt = _case(seed, P, T, H)
    wt_bits = wt.view(torch.int16).numpy().view(np.uint16)
    ref, lse_ref = lse_combine_project_ref(np.nan_to_num(po, nan=0.0), pl, wt_bits)
    o, _ = lse_combine_ref(np.nan_to_num(po, nan=0.0), pl)
    absdot = vc_project_ref(np.abs(o), np.abs(wt.float()).to(torch.bfloat16)
                            .view(torch.int16).numpy().view(np.uint16))
    out, lse = mla.lse_combine_project(torch.from_numpy(po).to(DEV), torch.from_numpy(pl).to(DEV),
                                       wt.to(DEV))
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    l = lse.cpu().numpy()
    tag = f"P{P} T{T} H{H}"
    bound = 2.0 ** -8 * (np.abs(ref) + absdot) + 1e-6 * np.abs(ref).max()
    err = np.abs(got - ref)
    print(f"[project] {tag}: max err / bound {float((err / bound).max()):.3f}", flush=True)
    assert np.all(err <= bound), tag
    empty = np.isneginf(lse_ref)
    assert np.array_equal(np.isneginf(l), empty), tag
    assert not got[empty].any(), tag
    np.testing.assert_allclose(l[~empty], lse_ref[~empty], rtol=0, atol=1e-5)


@pytest.mark.parametrize("P,T,H", [(1, 37, 16), (2, 80, 96), (8, 640, 96), (8, 33, 128),
                                   (3, 1, 8), (16, 64, 4)])
def test_combine_project_matches_oracle(P, T, H):
    _check(P, T, H, seed=P * 1000 + T + H)
