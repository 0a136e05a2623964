"""Pins of the CPU oracle against things other than itself (CPU only).

Brute force at 50 digits on tiny inputs, the exact-merge invariants the pages
rely on (split partials and the p % 8 shards merge back to full attention by
LSE), closed forms, the causal rule, page-permutation invariance, and library
cross-checks of the two bit decoders.  A last test plants plausible mistakes
in single oracle steps and checks that these pins catch every one of them.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle import mla_ref
from workload import make_inputs, shard_from_full

from bruteforce import brute_decode

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _run_oracle(x, **kw):
    nb = x.numpy_bits()
    return mla_ref.mla_decode_ref(nb["q_nope"], nb["q_rope"], nb["pool"], nb["kv_scale"],
                                  nb["req_to_token"], nb["seq_lens"], x.q_len,
                                  x.softmax_scale, x.kv_dtype, x.dcp_size, x.dcp_rank, **kw)


# ---------------------------------------------------------------- decoders

def test_e4m3fn_table_matches_torch_float8():
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    nan = np.isnan(t)
    assert set(np.nonzero(nan)[0]) == {0x7F, 0xFF}
    assert set(np.nonzero(np.isnan(oracle.E4M3FN_TABLE))[0]) == {0x7F, 0xFF}
    np.testing.assert_array_equal(oracle.E4M3FN_TABLE[~nan], t[~nan])
    assert oracle.E4M3FN_TABLE[0x7E] == 448.0 and oracle.E4M3FN_TABLE[0x01] == 2.0 ** -9


def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 1 << 16, size=100000, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    got = oracle.bf16_bits_to_f64(bits)
    ok = ~np.isnan(ref)
    assert np.array_equal(np.isnan(got), ~ok)
    np.testing.assert_array_equal(got[ok], ref[ok])


# ---------------------------------------------------------------- brute force

TINY = [
    # (kv_dtype, seq_lens, q_len, dcp_size, dcp_rank, p_range, page_size)
    ("bf16", [5, 8], 1, 1, 0, None, 4),
    ("bf16", [6, 7], 3, 1, 0, None, 2),
    ("fp8", [4, 8], 2, 1, 0, None, 4),
    ("fp8", [8, 5], 3, 1, 0, None, 1),
    ("bf16", [8, 7], 2, 2, 1, None, 2),
    ("fp8", [8, 6], 3, 3, 2, None, 2),
    ("fp8", [8, 8], 3, 3, 0, None, 4),
    ("bf16", [8, 8], 2, 1, 0, (2, 5), 4),
    ("fp8", [8, 8], 1, 2, 0, (3, 8), 2),
]


@pytest.mark.parametrize("case", TINY, ids=[f"{c[0]}-q{c[2]}-w{c[3]}r{c[4]}-{c[5]}" for c in TINY])
def test_oracle_matches_bruteforce(case):
    kv, lens, q, W, r, pr, ps = case
    x = make_inputs(11, lens, q, 2, kv, page_size=ps, dcp_size=W, dcp_rank=r, variant=None,
                    q_std=1.0, kv_std=1.0)
    o, lse = _run_oracle(x, p_range=pr)
    bo, blse = brute_decode(x.numpy_bits(), q, x.softmax_scale, kv, W, r, pr)
    assert np.array_equal(np.isinf(lse), np.isinf(blse))
    fin = np.isfinite(blse)
    np.testing.assert_allclose(lse[fin], blse[fin], rtol=0, atol=1e-12)
    np.testing.assert_allclose(o, bo, rtol=0, atol=1e-12)


# ---------------------------------------------------------------- invariants

def test_probabilities_sum_to_one():
    x = make_inputs(12, [300, 77, 5], 5, 4, "fp8", page_size=16, variant="qx30")
    _, _, probs = _run_oracle(x, return_probs=True)
    for (b, i), (pos, p) in probs.items():
        assert p.shape == (4, len(pos))
        np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-12)


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_split_then_merge_equals_unsplit(kv):
    x = make_inputs(13, [400, 257, 64], 5, 3, kv, page_size=16, variant="qx30")
    o, lse = _run_oracle(x)
    rng = np.random.default_rng(5)
    for _ in range(3):
        cuts = np.sort(rng.integers(0, 401, size=6))
        edges = [0] + list(cuts) + [400]  # repeated cuts give empty pieces
        parts = [_run_oracle(x, p_range=(a, b)) for a, b in zip(edges[:-1], edges[1:])]
        mo, ml = oracle.lse_combine_ref(np.stack([p[0] for p in parts]),
                                        np.stack([p[1] for p in parts]))
        np.testing.assert_allclose(ml, lse, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(mo, o, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_eight_interleaved_shards_merge_to_full(kv):
    full = make_inputs(14, [700, 389, 8, 64], 5, 4, kv, page_size=16, variant="qx30")
    o, lse = _run_oracle(full)
    shards = [shard_from_full(full, 8, r) for r in range(8)]
    for r, s in enumerate(shards):
        assert list(s.local_lens) == [len(range(r, L, 8)) for L in full.seq_lens]
    parts = [_run_oracle(s) for s in shards]
    mo, ml = oracle.lse_combine_ref(np.stack([p[0] for p in parts]),
                                    np.stack([p[1] for p in parts]))
    np.testing.assert_allclose(ml, lse, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(mo, o, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- closed forms

def _keys_values(x, b, positions):
    nb = x.numpy_bits()
    slots = nb["req_to_token"][b, positions]
    k = mla_ref.dequant_rows(nb["pool"], nb["kv_scale"], slots, x.kv_dtype)
    return k


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_zero_query_gives_uniform_mean(kv):
    x = make_inputs(15, [50, 33], 3, 2, kv, page_size=8)
    x.q_nope.zero_()
    x.q_rope.zero_()
    o, lse = _run_oracle(x)
    for b, L in enumerate(x.seq_lens):
        for i in range(3):
            n = L - 3 + i + 1
            k = _keys_values(x, b, np.arange(n))
            np.testing.assert_allclose(lse[b, i], math.log(n), rtol=0, atol=1e-14)
            np.testing.assert_allclose(o[b, i], np.broadcast_to(k[:, :512].mean(0), (2, 512)),
                                       rtol=0, atol=1e-14)


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_single_visible_token(kv):
    # seq_len == q_len: draft row 0 sees exactly position 0.
    x = make_inputs(16, [4, 4], 4, 3, kv, page_size=2, q_std=1.0)
    o, lse = _run_oracle(x)
    nb = x.numpy_bits()
    for b in range(2):
        k = _keys_values(x, b, np.array([0]))[0]
        qv = mla_ref.query_rows(nb["q_nope"], nb["q_rope"], b, 0)
        s0 = np.float64(np.float32(x.softmax_scale)) * (qv @ k)
        np.testing.assert_allclose(lse[b, 0], s0, rtol=0, atol=1e-15)
        np.testing.assert_array_equal(o[b, 0], np.broadcast_to(k[:512], (3, 512)))


def test_all_keys_equal_gives_that_value():
    x = make_inputs(17, [40], 2, 3, "bf16", page_size=8, q_std=1.0)
    nb = x.numpy_bits()
    used = nb["req_to_token"][0, :40]
    x.pool[torch.from_numpy(used.astype(np.int64))] = x.pool[int(used[0])].clone()
    o, lse = _run_oracle(x)
    k = _keys_values(x, 0, np.array([0]))[0]
    for i in range(2):
        n = 40 - 2 + i + 1
        qv = mla_ref.query_rows(nb["q_nope"], nb["q_rope"], 0, i)
        s = np.float64(np.float32(x.softmax_scale)) * (qv @ k)
        np.testing.assert_allclose(lse[0, i], s + math.log(n), rtol=0, atol=1e-12)
        np.testing.assert_allclose(o[0, i], np.broadcast_to(k[:512], (3, 512)), rtol=0,
                                   atol=1e-15)


def test_planted_key_dominates():
    x = make_inputs(18, [200], 1, 1, "bf16", page_size=16, q_std=1.0, kv_std=0.01)
    nb = x.numpy_bits()
    qv = mla_ref.query_rows(nb["q_nope"], nb["q_rope"], 0, 0)[0]
    slot = nb["req_to_token"][0, 123]
    x.pool[slot] = torch.from_numpy(qv * 3.0).to(torch.bfloat16)
    o, lse = _run_oracle(x)
    k = _keys_values(x, 0, np.array([123]))[0]
    s_star = np.float64(np.float32(x.softmax_scale)) * (qv @ k)
    assert s_star > 100
    np.testing.assert_allclose(lse[0, 0, 0], s_star, rtol=0, atol=1e-9)
    np.testing.assert_allclose(o[0, 0, 0], k[:512], rtol=0, atol=1e-9)


# ---------------------------------------------------------------- structure

@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_causal_rows_equal_shorter_q1_calls(kv):
    x = make_inputs(19, [130, 71], 5, 3, kv, page_size=16, variant="qx30")
    o, lse = _run_oracle(x)
    nb = x.numpy_bits()
    for i in range(5):
        lens = x.seq_lens - 5 + i + 1
        o1, l1 = mla_ref.mla_decode_ref(nb["q_nope"][:, i:i + 1], nb["q_rope"][:, i:i + 1],
                                        nb["pool"], nb["kv_scale"], nb["req_to_token"], lens,
                                        1, x.softmax_scale, kv)
        np.testing.assert_allclose(l1[:, 0], lse[:, i], rtol=0, atol=1e-13)
        np.testing.assert_allclose(o1[:, 0], o[:, i], rtol=0, atol=1e-15)


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_page_permutation_does_not_change_output(kv):
    x = make_inputs(20, [150, 90], 2, 2, kv, page_size=16)
    o, lse = _run_oracle(x)
    y = make_inputs(21, [150, 90], 2, 2, kv, page_size=16)  # other page permutation
    ty, tx = y.req_to_token.numpy(), x.req_to_token.numpy()
    for b, n in enumerate(x.local_lens):
        y.pool[torch.from_numpy(ty[b, :n].astype(np.int64))] = \
            x.pool[torch.from_numpy(tx[b, :n].astype(np.int64))]
        if kv == "fp8":
            y.kv_scale[torch.from_numpy(ty[b, :n].astype(np.int64))] = \
                x.kv_scale[torch.from_numpy(tx[b, :n].astype(np.int64))]
    y.q_nope, y.q_rope = x.q_nope, x.q_rope
    assert not np.array_equal(tx, ty)
    o2, l2 = _run_oracle(y)
    np.testing.assert_array_equal(o2, o)
    np.testing.assert_array_equal(l2, lse)


def test_combine_edge_cases():
    rng = np.random.default_rng(3)
    o = rng.standard_normal((3, 4, 8))
    l = np.array([[0.5, -np.inf, 2.0, -np.inf],
                  [-np.inf, -np.inf, 1.0, -np.inf],
                  [0.1, -np.inf, -np.inf, -np.inf]])
    mo, ml = oracle.lse_combine_ref(o, l)
    assert ml[1] == -np.inf and ml[3] == -np.inf
    np.testing.assert_array_equal(mo[3], 0.0)
    np.testing.assert_allclose(mo[2], (math.exp(2.0) * o[0, 2] + math.exp(1.0) * o[1, 2]) /
                               (math.exp(2.0) + math.exp(1.0)), rtol=1e-14)
    np.testing.assert_allclose(ml[0], math.log(math.exp(0.5) + math.exp(0.1)), rtol=1e-15)
    single_o, single_l = oracle.lse_combine_ref(o[:1], l[:1])
    fin = np.isfinite(l[0])
    np.testing.assert_array_equal(single_o[fin], o[0][fin])
    np.testing.assert_array_equal(single_l, l[0])


# ---------------------------------------------------------------- planted mistakes

def _wrong_visible_offbyone(seq_len, q_len, i, dcp_size=1, dcp_rank=0):
    last = seq_len - q_len + i + 1
    return np.arange(dcp_rank, max(dcp_rank, last + 1), dcp_size, dtype=np.int64) \
        if last >= dcp_rank else np.empty(0, np.int64)


def _wrong_visible_noncausal(seq_len, q_len, i, dcp_size=1, dcp_rank=0):
    return np.arange(dcp_rank, seq_len, dcp_size, dtype=np.int64)


def _wrong_local_index(p, dcp_size, dcp_rank):
    return (p + dcp_rank) // dcp_size


def _wrong_query_no_rope(q_nope, q_rope, b, i):
    return np.concatenate([oracle.bf16_bits_to_f64(q_nope[b, i]),
                           0.0 * oracle.bf16_bits_to_f64(q_rope[b, i])], axis=-1)


def _wrong_dequant_no_scale(pool, kv_scale, slots, kv_dtype):
    if kv_dtype == "fp8":
        return mla_ref.E4M3FN_TABLE[pool[slots].astype(np.intp)]
    return oracle.bf16_bits_to_f64(pool[slots])


def _wrong_scores_sign(q, keys, softmax_scale):
    return -np.float64(np.float32(softmax_scale)) * (q @ keys.T)


def _wrong_softmax_log2(s, values):
    o, lse, p = _orig_softmax(s, values)
    return o, lse / math.log(2.0), p


def _wrong_softmax_values_transposed(s, values):
    return _orig_softmax(s, values[::-1])


_orig_softmax = mla_ref.softmax_reduce

MUTATIONS = {
    "visible_offbyone": ("visible_positions", _wrong_visible_offbyone),
    "visible_noncausal": ("visible_positions", _wrong_visible_noncausal),
    "local_index_sign": ("local_index", _wrong_local_index),
    "dropped_rope_term": ("query_rows", _wrong_query_no_rope),
    "dropped_fp8_scale": ("dequant_rows", _wrong_dequant_no_scale),
    "score_sign": ("scores", _wrong_scores_sign),
    "lse_base2": ("softmax_reduce", _wrong_softmax_log2),
    "values_reversed": ("softmax_reduce", _wrong_softmax_values_transposed),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    fn_name, wrong = MUTATIONS[name]
    caught = False
    for kv, lens, q, W, r, pr, ps in [("fp8", [8, 6], 3, 3, 2, None, 2),
                                       ("fp8", [8, 7], 2, 1, 0, None, 2)]:
        x = make_inputs(11, lens, q, 2, kv, page_size=ps, dcp_size=W, dcp_rank=r,
                        q_std=1.0, kv_std=1.0)
        bo, blse = brute_decode(x.numpy_bits(), q, x.softmax_scale, kv, W, r, pr)
        with monkeypatch.context() as m:
            m.setattr(mla_ref, fn_name, wrong)
            try:
                o, lse = _run_oracle(x, p_range=pr)
            except (IndexError, ValueError):
                caught = True
                continue
        if not (np.allclose(o, bo, atol=1e-12, rtol=0) and
                np.allclose(lse, blse, atol=1e-12, rtol=0, equal_nan=True)):
            caught = True
    assert caught, f"planted mistake {name} was not caught by the brute-force pin"
