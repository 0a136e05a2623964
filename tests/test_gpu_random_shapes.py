"""GPU parity over seeded random small shapes: every KV format, q_len 1-5,
head counts whose row groups end in partial waves, page sizes 1-128 (paged
and general tables), DCP shards, forced splits, small CU counts (several
units per workgroup) and the peaked variants, each against the float64
oracle at the stated tolerances.  The cases are drawn once, at collection,
from a fixed seed, so every run checks the same ones."""

import numpy as np
import pytest
import torch

import mla_latent_kv_absorbed_amd as mla
from oracle import mla_decode_ref
from workload import make_inputs

pytestmark = pytest.mark.gpu

TOL_O_MAX, TOL_O_REL, TOL_LSE = 2e-2, 1e-2, 1e-3
DEV = "cuda"


def _cases(seed=7, n=40):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        kv = ["bf16", "fp8", "fp4", "mxfp8"][rng.integers(4)]
        q = int(rng.integers(1, 6))
        heads = int(rng.choice([8, 16, 32, 40, 64, 96, 112, 128]))
        lens = [int(max(q, rng.integers(1, 1800))) for _ in range(int(rng.integers(1, 7)))]
        page = int(rng.choice([16, 32, 64, 128, 1]))
        dcp = int(rng.choice([1, 1, 1, 2, 4, 8]))
        rank = int(rng.integers(dcp))
        variant = [None, None, "qx30", "planted", "offset"][rng.integers(5)]
        if kv in ("fp4", "mxfp8") and variant == "offset":
            variant = None   # the offset variant is defined for BF16 / FP8 pools
        splits = int(rng.choice([0, 0, 2, 3, 7]))
        cus = int(rng.choice([0, 0, 8, 24]))
        out.append(pytest.param(1000 + i, kv, q, heads, lens, page, dcp, rank, variant, splits, cus,
                                id=f"{i}-{kv}-q{q}-h{heads}-p{page}-dcp{dcp}-{variant}"))
    return out


@pytest.mark.parametrize("seed,kv,q,heads,lens,page,dcp,rank,variant,splits,cus", _cases())
def test_random_shape(seed, kv, q, heads, lens, page, dcp, rank, variant, splits, cus):
    tag = (f"{kv} q{q} h{heads} lens {lens} page {page} dcp {dcp}/{rank} {variant} "
           f"splits {splits} cus {cus}")
    print(f"\n[random] {tag}", flush=True)
    x = make_inputs(seed, lens, q, heads, kv, page_size=page, dcp_size=dcp, dcp_rank=rank,
                    kv_std=0.1 if kv == "bf16" else 1.0, variant=variant)
    desc = mla.make_desc(x.batch, x.q_len, x.num_heads, kv, page_size=page, dcp_size=dcp,
                         dcp_rank=rank, force_splits=splits, num_cus=cus)
    plan = mla.make_plan(desc, x.seq_lens, device=DEV)
    g = x.to(DEV)
    out, lse = mla.decode(plan, g.q_nope, g.q_rope, g.pool, g.kv_scale, g.req_to_token,
                          torch.from_numpy(np.asarray(x.seq_lens, np.int32)).to(DEV),
                          x.softmax_scale)
    torch.cuda.synchronize()
    nb = x.numpy_bits()
    o_ref, l_ref = mla_decode_ref(nb["q_nope"], nb["q_rope"], nb["pool"], nb["kv_scale"],
                                  nb["req_to_token"], nb["seq_lens"], x.q_len, x.softmax_scale,
                                  x.kv_dtype, x.dcp_size, x.dcp_rank)
    o = out.double().cpu().numpy()
    l = lse.double().cpu().numpy()
    empty = np.isneginf(l_ref)
    assert np.array_equal(np.isneginf(l), empty), f"{tag}: empty-row pattern differs"
    assert np.all(o[empty] == 0.0) and np.isfinite(o).all(), f"{tag}: empty or non-finite rows"
    d = o - o_ref
    nrm = np.linalg.norm(o_ref)
    assert np.abs(d).max() <= TOL_O_MAX, tag
    assert (np.linalg.norm(d) / nrm if nrm > 0 else 0.0) <= TOL_O_REL, tag
    if (~empty).any():
        assert np.abs(l[~empty] - l_ref[~empty]).max() <= TOL_LSE, tag
