"""GPU parity of mla_prepare (Q absorption, RoPE, KV append) against the oracle.

The absorbed query is a float32-accumulated sum rounded to BF16: each element
must lie within one BF16 unit in the last place of the float64 reference.
The roped query, the appended pool rows (BF16 bits, e4m3fn codes or FP4
rows) and the FP8 scales are bytes decided by correctly rounded float32
steps that the oracle repeats in the same order (FP4: power-of-two scaling
and comparisons, exact on both sides), so they must match bit for bit, and
every slot the call does not store must be left as it was.
"""

import numpy as np
import pytest
import torch

import mla_latent_kv_absorbed_amd as mla
from oracle import prepare_ref as P

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _case(seed, T, H, kv, num_slots=None, max_pos=4096, skip=True):
    rng = np.random.default_rng(np.random.SeedSequence([91, seed]))

    def bf16(shape, std):
        return torch.from_numpy((rng.standard_normal(shape) * std).astype(np.float32)).to(torch.bfloat16)
    num_slots = num_slots or 4 * T + 7
    x = dict(
        q_nope=bf16((T, H, 128), 1.0), q_rope_in=bf16((T, H, 64), 1.0),
        w_kc_t=bf16((H, 512, 128), 0.05), c_kv_new=bf16((T, 512), 0.5),
        k_rope_new=bf16((T, 64), 1.0),
        positions=torch.from_numpy(rng.integers(0, max_pos, T).astype(np.int32)))
    inv = 10000.0 ** (-np.arange(32) / 32.0)
    ang = np.arange(max_pos)[:, None] * inv[None, :]
    x["cos_sin"] = torch.from_numpy(np.concatenate([np.cos(ang), np.sin(ang)], 1).astype(np.float32))
    slots = rng.permutation(num_slots)[:T].astype(np.int32)
    if skip and T >= 4:
        slots[1] = -1                 # not stored (another shard's token)
        slots[T - 2] = num_slots + 5  # outside the pool: not stored
    x["slots"] = torch.from_numpy(slots)
    if kv == "bf16":
        x["kv_pool"] = bf16((num_slots, 576), 1.0)
        x["kv_scale"] = None
    elif kv in ("fp4", "mxfp8"):
        rb = 336 if kv == "fp4" else 608
        x["kv_pool"] = torch.from_numpy(rng.integers(0, 256, (num_slots, rb)).astype(np.uint8))
        x["kv_scale"] = None
    else:
        x["kv_pool"] = torch.from_numpy(rng.integers(0, 0x7E, (num_slots, 576)).astype(np.uint8))
        x["kv_scale"] = torch.from_numpy(rng.uniform(0.01, 0.05, num_slots).astype(np.float32))
    return x


def _oracle(x, kv):
    pool = _bits(x["kv_pool"]) if kv == "bf16" else x["kv_pool"].numpy()
    sc = None if x["kv_scale"] is None else x["kv_scale"].numpy()
    return P.mla_prepare_ref(_bits(x["q_nope"]), _bits(x["q_rope_in"]), _bits(x["w_kc_t"]),
                             _bits(x["c_kv_new"]), _bits(x["k_rope_new"]), x["cos_sin"].numpy(),
                             np.clip(x["positions"].numpy(), 0, x["cos_sin"].shape[0] - 1),
                             x["slots"].numpy(), pool, sc, kv)


def _gpu(x):
    g = {k: (v.to(DEV) if v is not None else None) for k, v in x.items()}
    qa, qr = mla.prepare(g["q_nope"], g["q_rope_in"], g["w_kc_t"], g["c_kv_new"], g["k_rope_new"],
                         g["positions"], g["cos_sin"], g["slots"], g["kv_pool"], g["kv_scale"])
    torch.cuda.synchronize()
    return qa, qr, g["kv_pool"], g["kv_scale"]


def _check(x, kv, tag):
    print(f"[prepare] {tag}", flush=True)
    qa_ref, qr_ref, pool_ref, sc_ref = _oracle(x, kv)
    qa, qr, pool, sc = _gpu(x)
    got = qa.float().cpu().numpy().astype(np.float64)
    # one BF16 ulp of the reference (2^(e - 7) for |ref| in [2^e, 2^(e+1)))
    e = np.floor(np.log2(np.maximum(np.abs(qa_ref), 1e-30)))
    ulp = np.exp2(e - 7)
    err = np.abs(got - qa_ref)
    assert np.all(err <= ulp * 1.0001 + 1e-6 * np.abs(qa_ref).max()), \
        f"{tag}: absorbed query off by {float((err / ulp).max()):.2f} ulp"
    np.testing.assert_array_equal(_bits(qr), qr_ref, err_msg=f"{tag}: roped query")
    if kv == "bf16":
        np.testing.assert_array_equal(_bits(pool), pool_ref, err_msg=f"{tag}: pool")
    else:
        np.testing.assert_array_equal(pool.cpu().numpy(), pool_ref, err_msg=f"{tag}: pool codes")
    if sc_ref is not None:
        np.testing.assert_array_equal(sc.cpu().numpy().view(np.uint32), sc_ref.view(np.uint32),
                                      err_msg=f"{tag}: scales")


@pytest.mark.parametrize("kv", ["bf16", "fp8", "fp4", "mxfp8"])
@pytest.mark.parametrize("T,H", [(80, 96), (37, 128), (1, 16), (640, 96), (33, 1)])
def test_prepare_matches_oracle(kv, T, H):
    _check(_case(10 * T + H, T, H, kv), kv, f"{kv} T{T} H{H}")


@pytest.mark.parametrize("kv", ["bf16", "fp8", "fp4", "mxfp8"])
def test_prepare_edge_inputs(kv):
    x = _case(5, 12, 8, kv, max_pos=64)
    pos = x["positions"].numpy()
    pos[0], pos[1], pos[2] = -3, 64, 1 << 30        # clamped into [0, max_pos)
    x["positions"] = torch.from_numpy(pos)
    c = x["c_kv_new"].float().numpy()
    c[3] = 0.0                                         # a zero c_kv row ...
    x["c_kv_new"] = torch.from_numpy(c).to(torch.bfloat16)
    k = x["k_rope_new"].float().numpy()
    k[3] = 0.0                                         # ... and a zero k_rope: scale 1, codes 0
    k[4] = 1e-30                                       # values that round to (signed) zero
    k[5, :] = 300.0                                    # one token dominated by its RoPE part
    x["k_rope_new"] = torch.from_numpy(k).to(torch.bfloat16)
    _check(x, kv, f"{kv} edge inputs")


def test_prepare_fp4_block_edges():
    # FP4 blocks whose largest value sits exactly on 6 * 2^e and just above
    # it, elements on the midpoints of the e2m1 grid (ties to the even code)
    # and just off them, a block of zeros and tiny values, and a huge block.
    x = _case(6, 8, 4, "fp4")
    c = np.zeros((8, 512), np.float32)
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], np.float32)
    for t in range(8):
        e = t - 4
        c[t, 0] = 6.0 * 2.0 ** e
        c[t, 1:8] = mids * 2.0 ** e
        c[t, 8:15] = -mids * 2.0 ** e
        # one BF16 unit in the last place above (the inputs are BF16)
        c[t, 16] = (6.0 + 2.0 ** -5) * 2.0 ** e
        c[t, 17:24] = (mids + np.exp2(np.floor(np.log2(mids)) - 7)) * 2.0 ** e
        c[t, 48:64] = 1e-30
        c[t, 64:80] = 3e38 if t == 0 else 1.0
        c[t, 80:] = np.random.default_rng(t).standard_normal(432) * 2.0 ** e
    x["c_kv_new"] = torch.from_numpy(c).to(torch.bfloat16)
    _check(x, "fp4", "fp4 block edges")


def test_prepare_mxfp8_block_edges():
    # MXFP8 blocks whose largest value sits exactly on 448 * 2^e and one BF16
    # ulp above it, values halfway between e4m3 neighbours (ties to even) and
    # one ulp off, subnormal-range values, a block of tiny values and a
    # saturating block.
    x = _case(7, 8, 4, "mxfp8")
    c = np.zeros((8, 512), np.float32)
    for t in range(8):
        e = 2 * t - 8
        c[t, 0] = 448.0 * 2.0 ** e
        c[t, 32] = (448.0 + 2.0) * 2.0 ** e                 # 448 + 1 BF16 ulp
        c[t, 1:5] = np.array([1.0 + 1 / 16, 1.0 + 3 / 16, 3.0 + 1 / 8, 2.0 ** -7], np.float32) * 2.0 ** e
        c[t, 5:9] = np.array([1.0 + 1 / 16 + 2 ** -7, 1.25 + 1 / 16, 2.0 ** -9 * 1.5, -2.0 ** -10],
                             np.float32) * 2.0 ** e
        c[t, 64:96] = 1e-30
        c[t, 96:128] = 3e38 if t == 0 else 1.0
        c[t, 128:] = np.random.default_rng(t).standard_normal(384) * 2.0 ** e
    x["c_kv_new"] = torch.from_numpy(c).to(torch.bfloat16)
    _check(x, "mxfp8", "mxfp8 block edges")
