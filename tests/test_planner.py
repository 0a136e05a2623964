"""Host planner (mla_decode_plan) and wave arithmetic: CPU only."""

import json
import os

import numpy as np
import pytest

import mla_latent_kv_absorbed_amd as mla
from mla_latent_kv_absorbed_amd import waves
from workload import local_lengths, ragged_lengths

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_numbers.json")))


def check_plan(plan, seq_lens, q_len, H, W=1, r=0):
    h = plan.header
    n = local_lengths(seq_lens, W, r)
    G = -(-q_len * H // 128)
    assert h["row_groups"] == G and h["rows"] == q_len * H
    u = plan.units()
    wgb = plan.wg_begin()
    assert wgb[0] == 0 and wgb[-1] == h["num_units"] and np.all(np.diff(wgb) >= 0)
    assert len(u) == h["num_units"]
    rp = plan.req_parts()
    sr = plan.split_reqs()
    split = set(sr[:, 0].tolist())
    assert len(split) == len(sr) and np.all(sr[:, 3] == 0)
    for b, first, nparts in sr[:, :3].tolist():   # each record repeats its request's slots
        assert first == rp[b, 0] and nparts == rp[b, 1]
    seen_parts = set()
    for b in range(len(seq_lens)):
        ub = u[u[:, 0] == b]
        cuts_by_g = []
        for g in range(G):
            s = ub[ub[:, 1] == g]
            s = s[np.argsort(s[:, 2])]
            assert len(s) >= 1
            if n[b] == 0:
                assert len(s) == 1 and s[0, 2] == 0 and s[0, 3] == 0
            else:
                assert s[0, 2] == 0 and s[-1, 3] == n[b]
                assert np.all(s[1:, 2] == s[:-1, 3]) and np.all(s[:, 3] > s[:, 2])
                assert np.all(s[:, 2] % 32 == 0)
            cuts_by_g.append(s[:, 2:5].tolist())
        assert all(c == cuts_by_g[0] for c in cuts_by_g)  # row groups share cuts and parts
        parts = [c[2] for c in cuts_by_g[0]]
        if len(parts) == 1:
            assert parts[0] == -1 and rp[b, 1] == 1 and b not in split
        else:
            assert b in split and rp[b, 1] == len(parts)
            assert parts == list(range(rp[b, 0], rp[b, 0] + len(parts)))
            seen_parts |= set(parts)
    assert seen_parts == set(range(h["num_parts"]))
    assert h["num_split_reqs"] == len(split)


CASES = [
    ([100000] * 16, 5, 96, 1, 0),
    ([4096] * 32, 1, 128, 1, 0),
    ([1024, 1536], 1, 16, 1, 0),
    ([100000] * 128, 5, 96, 8, 3),
    ([200000], 5, 96, 1, 0),
    ([5, 6, 8, 9, 100], 5, 32, 8, 7),   # shard 7 holds nothing of the short requests
    (list(ragged_lengths(5, 64, 1024, 400000)), 5, 96, 1, 0),
]


@pytest.mark.parametrize("case", CASES, ids=range(len(CASES)))
@pytest.mark.parametrize("force", [0, 1, 3])
def test_plan_covers_every_token_once(case, force):
    lens, q, H, W, r = case
    d = mla.make_desc(len(lens), q, H, "fp8", dcp_size=W, dcp_rank=r, num_cus=256,
                      force_splits=force)
    check_plan(mla.make_plan(d, lens), lens, q, H, W, r)


def test_random_plans_cover_every_token_once():
    rng = np.random.default_rng(9)
    for _ in range(40):
        B = int(rng.integers(1, 40))
        q = int(rng.integers(1, 9))
        H = int(rng.choice([1, 16, 40, 96, 128, 200]))
        W = int(rng.choice([1, 2, 8]))
        r = int(rng.integers(0, W))
        lens = rng.integers(q, 300000, size=B)
        cus = int(rng.choice([8, 100, 256, 304]))
        d = mla.make_desc(B, q, H, "bf16", dcp_size=W, dcp_rank=r, num_cus=cus)
        check_plan(mla.make_plan(d, lens), lens, q, H, W, r)


def test_siblings_share_an_xcd_and_grid_fits_the_chip():
    d = mla.make_desc(16, 5, 96, "fp8", num_cus=256)
    p = mla.make_plan(d, [100000] * 16)
    assert p.header["num_wgs"] == 256
    wgb, u = p.wg_begin(), p.units()
    owner = {}
    for x in range(len(wgb) - 1):
        for k in range(wgb[x], wgb[x + 1]):
            owner.setdefault((u[k, 0], u[k, 2], u[k, 3]), []).append(x)
    for key, xs in owner.items():
        assert len(xs) == 4 and len({x % 8 for x in xs}) == 1, key


def _owners(p):
    wgb, u = p.wg_begin(), p.units()
    return [(x, u[k]) for x in range(len(wgb) - 1) for k in range(wgb[x], wgb[x + 1])]


def test_pieces_of_a_request_share_an_xcd():
    # 32 requests cut into 8 pieces each on 256 CUs: the 8 pieces of a request
    # run on one XCD (ids congruent modulo 8), which then loads its Q once.
    p = mla.make_plan(mla.make_desc(32, 1, 128, "bf16", num_cus=256), [4096] * 32)
    assert p.header["num_wgs"] == 256
    xcds = {}
    for x, unit in _owners(p):
        xcds.setdefault(int(unit[0]), set()).add(x % 8)
    assert all(len(v) == 1 for v in xcds.values())
    assert sorted(len([b for b in xcds if xcds[b] == {k}]) for k in range(8)) == [4] * 8


def test_grid_never_exceeds_the_compute_units():
    rng = np.random.default_rng(11)
    for _ in range(60):
        B = int(rng.integers(1, 40))
        q = int(rng.integers(1, 9))
        H = int(rng.choice([16, 32, 96, 128]))
        lens = rng.integers(q, 300000, size=B)
        cus = int(rng.choice([8, 100, 120, 256, 304]))
        p = mla.make_plan(mla.make_desc(B, q, H, "fp8", num_cus=cus), lens)
        assert p.header["num_wgs"] <= cus


@pytest.mark.parametrize("lens", [[100000] * 16, [4096] * 32, [200000] * 24,
                                  list(ragged_lengths(5, 64, 1024, 400000))])
def test_plan_is_balanced(lens):
    q, H = (1, 128) if lens[0] == 4096 else (5, 96)
    p = mla.make_plan(mla.make_desc(len(lens), q, H, "fp8", num_cus=256), lens)
    assert waves.plan_efficiency(p, 256) > 0.95


def test_no_wave_cliff_across_batch_1_to_24():
    eff, work = [], []
    for B in range(1, 25):
        p = mla.make_plan(mla.make_desc(B, 5, 96, "fp8", num_cus=256), [200000] * B)
        eff.append(waves.plan_efficiency(p, 256))
        work.append(waves.plan_wg_costs(p).max())
    assert max(eff) - min(eff) <= 0.05
    assert all(b >= a for a, b in zip(work, work[1:]))  # busiest workgroup never shrinks


def test_prior_art_wave_arithmetic_matches_the_page():
    g = GOLDEN["prior_art_split"]
    sms, t = g["sms"], g["t_wave_us"]
    for c in g["cases"]:
        B, q = c["batch"], c["q_len"]
        if B <= 24 and q == 5:
            assert waves.prior_art_ctas(B, q, sms) == c["ctas"]
            assert waves.waves(c["ctas"], sms) == c["waves"]
            assert round(waves.wave_rounded_time(B, q, sms, t)) == c["wave_rounded_us"]
        if "waves_fractional" in c:
            assert abs(c["ctas"] / sms - c["waves_fractional"]) < 0.06
        if "time_us" in c:
            assert waves.prior_art_time(B, q, sms, t) == c["time_us"]
    # The DP2 grid (2, 640, 1) and the old (bs 24 x q_len 6) grid.
    assert 2 * 128 * 5 == 1280 and 2 * 24 * 6 == 288


def test_prior_art_rule_has_a_cliff_on_256_cus():
    # The same rule on 256 CUs: 240 CTAs at B = 24 fit one wave, 26 requests spill.
    t = [waves.prior_art_time(B, 5, 256, 1.0) for B in range(1, 40)]
    assert max(b / a for a, b in zip(t, t[1:])) >= 1.9
