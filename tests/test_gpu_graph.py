"""mla_decode under HIP graph capture (through torch.cuda.CUDAGraph, which
drives hipGraph on ROCm).

A decode step (the decode kernel and the merge of the split requests) is
captured once and replayed.  The library allocates nothing, records no memset
and never synchronizes inside a call, so the captured graph holds only its
kernels.  Each replay, with other eager decodes and synchronizations between
the replays, must give exactly the eager result of the same call, and the
eager result is held to the oracle's tolerances.  The same holds for
mla_decode_noalloc, whose split partials live in the library's scratch array.
"""

import numpy as np
import pytest
import torch

import mla_latent_kv_absorbed_amd as mla
from oracle import mla_decode_ref
from workload import make_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _setup(seed, lens, q, H, kv, force_splits):
    x = make_inputs(seed, lens, q, H, kv, kv_std=0.1 if kv == "bf16" else 1.0)
    desc = mla.make_desc(x.batch, x.q_len, x.num_heads, kv, page_size=x.page_size,
                         force_splits=force_splits)
    plan = mla.make_plan(desc, x.seq_lens, device=DEV)
    g = x.to(DEV)
    seq = torch.from_numpy(np.asarray(x.seq_lens, np.int32)).to(DEV)
    args = (plan, g.q_nope, g.q_rope, g.pool, g.kv_scale, g.req_to_token, seq, x.softmax_scale)
    o_shape = (x.batch, x.q_len, x.num_heads, 512)
    return x, plan, args, o_shape


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


@pytest.mark.parametrize("entry", ["decode", "decode_noalloc"])
@pytest.mark.parametrize("kv", ["fp8", "bf16"])
def test_captured_decode_replays_equal_the_eager_call(kv, entry):
    print(f"\n[graph] {entry} {kv}", flush=True)
    x, plan, args, o_shape = _setup(90, [3000, 1200, 64], 5, 32, kv, force_splits=3)
    assert plan.workspace_bytes > 0  # split requests: the merge is in the graph too
    ws = torch.zeros(plan.workspace_bytes, dtype=torch.uint8, device=DEV)

    def call(out, lse):
        if entry == "decode":
            mla.decode(*args, workspace=ws, out=out, lse=lse)
        else:
            mla.decode_noalloc(*args, out=out, lse=lse)

    # The eager call first (it also sets up the scratch address of the
    # no-alloc entry point on this device).
    o_e = torch.empty(o_shape, dtype=torch.float32, device=DEV)
    l_e = torch.empty(o_shape[:3], dtype=torch.float32, device=DEV)
    call(o_e, l_e)
    torch.cuda.synchronize()

    o_g = torch.empty_like(o_e)
    l_g = torch.empty_like(l_e)
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(graph, stream=side):
        call(o_g, l_g)
    torch.cuda.current_stream().wait_stream(side)

    # Other eager work between the replays: a different decode with its own
    # plan and buffers.
    x2, plan2, args2, o_shape2 = _setup(91, [900, 2500], 1, 16, kv, force_splits=2)
    o2 = torch.empty(o_shape2, dtype=torch.float32, device=DEV)
    l2 = torch.empty(o_shape2[:3], dtype=torch.float32, device=DEV)
    for r in range(3):
        o_g.fill_(float("nan"))
        l_g.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o_g, o_e) and torch.equal(l_g, l_e), f"replay {r} differs"
        mla.decode(*args2, out=o2, lse=l2)
        torch.cuda.synchronize()
    _check_oracle(x, o_e, l_e)
    _check_oracle(x2, o2, l2)
