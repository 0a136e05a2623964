"""Seeded input generator: structure, poisoning, determinism, byte model (CPU only)."""

import json
import math
import os

import numpy as np
import pytest
import torch

from workload import (CONFIGS, config_inputs, kv_bytes_per_token, local_lengths, make_inputs,
                      ragged_lengths, shard_from_full, softmax_scale_default)

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_numbers.json")))


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_table_slots_unique_in_range_and_page_aligned(kv):
    x = make_inputs(30, [1000, 64, 1, 129], 1, 2, kv, page_size=64)
    t = x.req_to_token.numpy()
    slots = np.concatenate([t[b, :n] for b, n in enumerate(x.local_lens)])
    assert len(np.unique(slots)) == len(slots)
    assert slots.min() >= 64 and slots.max() < x.num_slots  # page 0 never referenced
    for b, n in enumerate(x.local_lens):
        for j0 in range(0, n, 64):
            run = t[b, j0:min(n, j0 + 64)]
            assert run[0] % 64 == 0 and np.array_equal(run, run[0] + np.arange(len(run)))


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_unused_slots_are_poisoned_and_used_slots_finite(kv):
    x = make_inputs(31, [100, 37], 1, 2, kv, page_size=16)
    t = x.req_to_token.numpy()
    used = np.zeros(x.num_slots, bool)
    for b, n in enumerate(x.local_lens):
        used[t[b, :n]] = True
    if kv == "bf16":
        vals = x.pool.float().numpy()
    else:
        vals = x.pool.view(torch.float8_e4m3fn).float().numpy() * x.kv_scale.numpy()[:, None]
    assert np.isnan(vals[~used]).all()
    assert np.isfinite(vals[used]).all()


def test_deterministic_and_seed_dependent():
    a = make_inputs(32, [300], 5, 4, "fp8")
    b = make_inputs(32, [300], 5, 4, "fp8")
    c = make_inputs(33, [300], 5, 4, "fp8")
    assert torch.equal(a.pool, b.pool) and torch.equal(a.q_nope, b.q_nope)
    assert torch.equal(a.req_to_token, b.req_to_token)
    assert not torch.equal(a.req_to_token, c.req_to_token)


def test_value_distributions():
    x = make_inputs(34, [20000], 1, 128, "bf16")
    v = x.pool[x.req_to_token[0, :20000].long()].float()
    assert abs(v.std().item() - 0.1) < 0.002 and abs(v.mean().item()) < 0.002
    y = make_inputs(35, [20000], 1, 8, "fp8")
    s = y.kv_scale[y.req_to_token[0, :20000].long()]
    assert 0.01 <= s.min().item() and s.max().item() <= 0.05
    f = y.pool[y.req_to_token[0, :20000].long()].view(torch.float8_e4m3fn).float()
    assert abs(f.std().item() - 1.0) < 0.02
    assert abs(x.q_nope.float().std().item() - 0.1) < 0.005


def test_dcp_local_lengths_follow_p_mod_8():
    g = GOLDEN["dcp"]
    n = local_lengths([g["context"]] * 3, g["shards"], 5)
    assert list(n) == [g["tokens_per_shard"]] * 3
    for L in [1, 7, 8, 9, 100003]:
        assert sum(local_lengths([L], 8, r)[0] for r in range(8)) == L
        for r in range(8):
            assert local_lengths([L], 8, r)[0] == len(range(r, L, 8))


def test_shard_from_full_copies_rows_bit_exact():
    full = make_inputs(36, [300, 17], 2, 2, "fp8", page_size=16)
    ft = full.req_to_token.numpy()
    for r in range(8):
        s = shard_from_full(full, 8, r)
        st = s.req_to_token.numpy()
        for b, n in enumerate(s.local_lens):
            p = np.arange(n) * 8 + r
            assert torch.equal(s.pool[torch.from_numpy(st[b, :n].astype(np.int64))],
                               full.pool[torch.from_numpy(ft[b, p].astype(np.int64))])


def test_ragged_lengths_log_uniform_range():
    L = ragged_lengths(5, 64, 1024, 400000)
    assert L.min() >= 1024 and L.max() < 400000 and len(L) == 64
    assert np.array_equal(L, ragged_lengths(5, 64, 1024, 400000))


def test_softmax_scale_is_fp32_of_inverse_sqrt_192():
    qk = GOLDEN["latent_row"]["qk_head_dim"]
    assert softmax_scale_default() == float(np.float32(1 / math.sqrt(qk)))


def test_byte_model_matches_pages():
    g = GOLDEN["capacity"]
    lat = GOLDEN["latent_row"]
    assert lat["kv_lora_rank"] + lat["qk_rope_head_dim"] == g["bytes_per_token_per_layer"]
    assert kv_bytes_per_token("fp8") == g["bytes_per_token_per_layer"] + 4  # + fp32 scale
    assert kv_bytes_per_token("bf16") == 2 * g["bytes_per_token_per_layer"]
    per_gpu_tokens = g["pool_gib_per_gpu_dp16"] * 2 ** 30 / (g["mla_layers"] * 576)
    assert abs(per_gpu_tokens / 1e6 - 3.19) < 0.01
    assert abs(per_gpu_tokens * g["gpus"] / 1e6 - g["instance_tokens_millions_dp16"]) < 0.1
    r = GOLDEN["req_to_token_row"]
    assert r["context_len"] * 4 == r["row_bytes"]
    assert abs(r["rows_dp2"] * r["row_bytes"] / 2 ** 30 - r["gib_dp2"]) < 0.005
    assert abs(r["rows_dp16"] * r["row_bytes"] / 2 ** 30 - r["gib_dp16"]) < 0.005
    # The 100k MTP workload reads 16 x 100000 x 576 B = 921.6 MB of latent rows.
    assert 16 * 100000 * g["bytes_per_token_per_layer"] == 921_600_000


def test_config_shapes_small():
    x = config_inputs(1)
    assert x.q_nope.shape == (2, 1, 16, 512) and x.q_rope.shape == (2, 1, 16, 64)
    assert list(x.seq_lens) == [1024, 1536] and x.kv_dtype == "bf16"
    assert x.num_slots == (16 + 24 + 1) * 64
    assert CONFIGS[3]["num_heads"] == GOLDEN["latent_row"]["heads"]
