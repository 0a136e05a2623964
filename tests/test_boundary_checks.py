"""Host-side guards of the boundary (CPU only; nothing here launches a kernel).

- tile_asm.inc is exactly what gen_tile_asm.py emits (the committed statements
  are the generated ones).
- mla_check_table reports tables that break the contract the decode kernel
  relies on: slots inside the pool, and, for page sizes that are multiples of
  32, 32 consecutive slots behind every entry the kernel reads.
- The Python binding rejects caller-supplied out / lse / workspace / seq_lens
  of the wrong shape, dtype or device before anything reaches the library.
"""

import importlib.util
import os

import numpy as np
import pytest
import torch

import mla_latent_kv_absorbed_amd as mla
from mla_latent_kv_absorbed_amd._binding import MlaError
from workload import make_inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mla_latent_kv_absorbed_amd", "csrc")


def test_tile_asm_is_what_the_generator_emits():
    spec = importlib.util.spec_from_file_location("gen_tile_asm",
                                                  os.path.join(CSRC, "gen_tile_asm.py"))
    gen = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(gen)
    with open(os.path.join(CSRC, "tile_asm.inc")) as f:
        committed = f.read()
    assert gen.generate() == committed, "tile_asm.inc is stale: run gen_tile_asm.py"


# ------------------------------------------------------------ table contract

def _paged_table(lens, page_size, pages_per_req, seed=0):
    rng = np.random.default_rng(seed)
    B = len(lens)
    perm = rng.permutation(B * pages_per_req) + 1
    stride = pages_per_req * page_size
    table = np.zeros((B, stride), dtype=np.int32)
    for b, n in enumerate(lens):
        j = np.arange(n)
        phys = perm[b * pages_per_req:(b + 1) * pages_per_req]
        table[b, :n] = phys[j // page_size] * page_size + j % page_size
    return table, (B * pages_per_req + 1) * page_size


@pytest.mark.parametrize("page_size", [32, 64, 128])
def test_check_table_accepts_paged_layouts(page_size):
    lens = [1000, 33, 5]
    table, slots = _paged_table(lens, page_size, -(-1000 // page_size))
    desc = mla.make_desc(3, 5, 16, "fp8", page_size=page_size, num_cus=256)
    mla.check_table(desc, lens, table, slots)


def test_check_table_reports_a_broken_32_slot_run():
    lens = [1000, 700]
    table, slots = _paged_table(lens, 64, 16)
    table[1, 37], table[1, 38] = table[1, 38], table[1, 37]  # inside one 32-run
    desc = mla.make_desc(2, 1, 16, "bf16", page_size=64, num_cus=256)
    with pytest.raises(MlaError, match="request 1, index 37"):
        mla.check_table(desc, lens, table, slots)
    # The same table is fine for a general-gather page size (not a multiple of 32).
    mla.check_table(mla.make_desc(2, 1, 16, "bf16", page_size=16, num_cus=256), lens, table,
                    slots)


def test_check_table_reports_slots_outside_the_pool():
    lens = [100, 200]
    table, slots = _paged_table(lens, 16, 13)
    desc = mla.make_desc(2, 1, 16, "bf16", page_size=16, num_cus=256)
    t = table.copy()
    t[0, 99] = slots
    with pytest.raises(MlaError, match="request 0, index 99"):
        mla.check_table(desc, lens, t, slots)
    t = table.copy()
    t[1, 0] = -1
    with pytest.raises(MlaError, match="request 1, index 0"):
        mla.check_table(desc, lens, t, slots)
    # Entries past a request's length are not read by the kernel, so not checked.
    t = table.copy()
    t[0, 150] = -5
    mla.check_table(desc, lens, t, slots)


def test_check_table_uses_the_shard_local_lengths():
    # DCP 8, rank 3: L = 1000 holds positions 3, 11, ..., 995: 125 local indices.
    lens = [1000]
    table, slots = _paged_table([125], 64, 2)
    desc = mla.make_desc(1, 5, 16, "fp8", page_size=64, dcp_size=8, dcp_rank=3, num_cus=256)
    mla.check_table(desc, lens, table, slots)
    t = table.copy()
    t[0, 124] = t[0, 96] + 29   # breaks the run of index 124 = 96 + 28
    with pytest.raises(MlaError, match="index 124"):
        mla.check_table(desc, lens, t, slots)


def test_check_table_rejects_bad_arguments():
    table, slots = _paged_table([100], 64, 2)
    desc = mla.make_desc(1, 1, 16, "bf16", page_size=64, num_cus=256)
    with pytest.raises(MlaError):
        mla.check_table(desc, [100], table[:, :64], slots)  # stride shorter than the length
    with pytest.raises(MlaError):
        mla.check_table(desc, [0], table, slots)            # length below q_len
    with pytest.raises(MlaError):
        mla.check_table(desc, [100, 5], table, slots)       # wrong number of lengths


def test_generated_tables_satisfy_the_contract():
    for kv, ps in (("fp8", 64), ("bf16", 16), ("fp4", 128)):
        x = make_inputs(5, [300, 77, 5], 5, 16, kv, page_size=ps)
        desc = mla.make_desc(x.batch, x.q_len, x.num_heads, kv, page_size=ps, num_cus=256)
        mla.check_table(desc, x.seq_lens, x.req_to_token.numpy(), x.num_slots)


# ------------------------------------------------------------ binding guards

def _cpu_call():
    x = make_inputs(9, [100, 40], 1, 16, "bf16")
    desc = mla.make_desc(x.batch, x.q_len, x.num_heads, "bf16", page_size=64, num_cus=256,
                         force_splits=2)
    plan = mla.make_plan(desc, x.seq_lens, device="cpu")
    seq = torch.from_numpy(np.asarray(x.seq_lens, np.int32))
    return x, plan, seq


@pytest.mark.parametrize("what", ["out_shape", "out_dtype", "lse_shape", "lse_dtype",
                                  "ws_dtype", "seq_lens_short", "seq_lens_long"])
def test_decode_rejects_bad_caller_buffers(what):
    x, plan, seq = _cpu_call()
    B, q, H = x.batch, x.q_len, x.num_heads
    kw = {}
    if what == "out_shape":
        kw["out"] = torch.empty((B, q, H, 256), dtype=torch.float32)
    elif what == "out_dtype":
        kw["out"] = torch.empty((B, q, H, 512), dtype=torch.bfloat16)
    elif what == "lse_shape":
        kw["lse"] = torch.empty((B, q, H - 1), dtype=torch.float32)
    elif what == "lse_dtype":
        kw["lse"] = torch.empty((B, q, H), dtype=torch.float64)
    elif what == "ws_dtype":
        kw["workspace"] = torch.empty(plan.workspace_bytes // 4, dtype=torch.float32)
    elif what == "seq_lens_short":
        seq = seq[:1].clone()
    else:
        seq = torch.cat([seq, seq])
    with pytest.raises(MlaError):
        mla.decode(plan, x.q_nope, x.q_rope, x.pool, x.kv_scale, x.req_to_token, seq,
                   x.softmax_scale, **kw)


def test_decode_verify_table_reports_before_any_launch():
    x, plan, seq = _cpu_call()
    t = x.req_to_token.clone()
    t[0, 3] = t[0, 4]
    with pytest.raises(MlaError, match="request 0, index 3"):
        mla.decode(plan, x.q_nope, x.q_rope, x.pool, x.kv_scale, t, seq, x.softmax_scale,
                   verify_table=True)
