"""mla_decode_noalloc (the decode entry point that allocates nothing) against
mla_decode, through the C ABI, on two calls in a row, the second with a
smaller input.  Both entry points run the same kernels on the same plan, so
the outputs must be identical; they are also held to the oracle's
tolerances against the oracle."""

import numpy as np
import pytest
import torch

import mla_latent_kv_absorbed_amd as mla
from mla_latent_kv_absorbed_amd._binding import MlaError
from oracle import mla_decode_ref
from workload import make_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _both(x, force_splits=0):
    desc = mla.make_desc(x.batch, x.q_len, x.num_heads, x.kv_dtype, page_size=x.page_size,
                         force_splits=force_splits)
    plan = mla.make_plan(desc, x.seq_lens, device=DEV)
    g = x.to(DEV)
    seq = torch.from_numpy(np.asarray(x.seq_lens, np.int32)).to(DEV)
    args = (plan, g.q_nope, g.q_rope, g.pool, g.kv_scale, g.req_to_token, seq, x.softmax_scale)
    o1, l1 = mla.decode(*args)
    o2 = torch.full_like(o1, float("nan"))
    l2 = torch.full_like(l1, float("nan"))
    mla.decode_noalloc(*args, out=o2, lse=l2)
    torch.cuda.synchronize()
    return plan, (o1, l1), (o2, l2)


def _check_oracle(x, out, lse):
    nb = x.numpy_bits()
    o_ref, l_ref = mla_decode_ref(nb["q_nope"], nb["q_rope"], nb["pool"], nb["kv_scale"],
                                  nb["req_to_token"], nb["seq_lens"], x.q_len, x.softmax_scale,
                                  x.kv_dtype)
    o = out.double().cpu().numpy()
    l = lse.double().cpu().numpy()
    assert np.abs(o - o_ref).max() <= 2e-2
    assert np.linalg.norm(o - o_ref) / np.linalg.norm(o_ref) <= 1e-2
    assert np.abs(l - l_ref).max() <= 1e-3


@pytest.mark.parametrize("kv", ["fp8", "bf16"])
def test_noalloc_matches_decode_on_two_calls(kv):
    std = 0.1 if kv == "bf16" else 1.0
    # First call: 3 requests, split by the planner (the partials use the scratch).
    x1 = make_inputs(80, [5000, 3100, 900], 5, 96, kv, kv_std=std)
    plan1, (o1, l1), (o2, l2) = _both(x1, force_splits=4)
    assert plan1.workspace_bytes > 0
    assert torch.equal(o1, o2) and torch.equal(l1, l2), "first call differs from mla_decode"
    _check_oracle(x1, o2, l2)
    # Second call, smaller: the scratch still holds the first call's partials.
    x2 = make_inputs(81, [700, 64], 1, 16, kv, kv_std=std)
    plan2, (o3, l3), (o4, l4) = _both(x2, force_splits=3)
    assert 0 < plan2.workspace_bytes < plan1.workspace_bytes
    assert torch.equal(o3, o4) and torch.equal(l3, l4), "second call differs from mla_decode"
    _check_oracle(x2, o4, l4)


def test_noalloc_rejects_plans_beyond_the_scratch():
    # 64 requests x 8 splits x 1024 rows of fp16 partials (512 MiB): beyond 128 MiB.
    lens = [4096] * 64
    desc = mla.make_desc(64, 8, 128, "bf16", page_size=64, force_splits=8)
    plan = mla.make_plan(desc, lens, device=DEV)
    assert plan.workspace_bytes > (128 << 20)
    q = torch.zeros((64, 8, 128, 512), dtype=torch.bfloat16, device=DEV)
    qr = torch.zeros((64, 8, 128, 64), dtype=torch.bfloat16, device=DEV)
    pool = torch.zeros((64, 576), dtype=torch.bfloat16, device=DEV)
    table = torch.zeros((64, 4096), dtype=torch.int32, device=DEV)
    seq = torch.full((64,), 4096, dtype=torch.int32, device=DEV)
    out = torch.empty((64, 8, 128, 512), dtype=torch.float32, device=DEV)
    lse = torch.empty((64, 8, 128), dtype=torch.float32, device=DEV)
    with pytest.raises(MlaError, match="too small"):
        mla.decode_noalloc(plan, q, qr, pool, None, table, seq, 0.07, out=out, lse=lse)
