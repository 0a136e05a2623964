"""GPU parity: the HIP path through the C ABI against the float64 oracle.

Tolerances (stated for this method): max |dO| <= 2e-2, ||dO||_F / ||O||_F <=
1e-2, max |dLSE| <= 1e-3.  Rows with no visible token must come back as
exactly (0, -inf).
"""

import numpy as np
import pytest
import torch

import mla_latent_kv_absorbed_amd as mla
from oracle import lse_combine_ref, mla_decode_ref
from workload import config_inputs, make_inputs, shard_from_full

pytestmark = pytest.mark.gpu

TOL_O_MAX, TOL_O_REL, TOL_LSE = 2e-2, 1e-2, 1e-3
DEV = "cuda"
KV_DTYPES = ["bf16", "fp8", "fp4", "mxfp8"]


def oracle(x, reqs=None, **kw):
    nb = x.numpy_bits()
    if reqs is not None:
        for k in ("q_nope", "q_rope", "req_to_token", "seq_lens"):
            nb[k] = nb[k][reqs]
    return mla_decode_ref(nb["q_nope"], nb["q_rope"], nb["pool"], nb["kv_scale"],
                          nb["req_to_token"], nb["seq_lens"], x.q_len, x.softmax_scale,
                          x.kv_dtype, x.dcp_size, x.dcp_rank, **kw)


def gpu_decode(x, force_splits=0, page_size=None, plan_out=None, num_cus=0):
    ps = x.page_size if page_size is None else page_size
    desc = mla.make_desc(x.batch, x.q_len, x.num_heads, x.kv_dtype, page_size=ps,
                         dcp_size=x.dcp_size, dcp_rank=x.dcp_rank, force_splits=force_splits,
                         num_cus=num_cus)
    plan = mla.make_plan(desc, x.seq_lens, device=DEV)
    if plan_out is not None:
        plan_out.append(plan)
    g = x.to(DEV) if x.pool.device.type != "cuda" else x
    out, lse = mla.decode(plan, g.q_nope, g.q_rope, g.pool, g.kv_scale, g.req_to_token,
                          torch.from_numpy(np.asarray(x.seq_lens, np.int32)).to(DEV),
                          x.softmax_scale)
    torch.cuda.synchronize()
    return out, lse


def check(out, lse, o_ref, l_ref, tag=""):
    o = out.double().cpu().numpy() if torch.is_tensor(out) else out
    l = lse.double().cpu().numpy() if torch.is_tensor(lse) else lse
    empty = np.isneginf(l_ref)
    assert np.array_equal(np.isneginf(l), empty), f"{tag}: empty-row pattern differs"
    assert np.all(o[empty] == 0.0), f"{tag}: empty rows must have O = 0"
    assert np.isfinite(o).all() and np.isfinite(l[~empty]).all(), f"{tag}: non-finite output"
    d = o - o_ref
    err_o = float(np.abs(d).max()) if d.size else 0.0
    nrm = float(np.linalg.norm(o_ref))
    rel = float(np.linalg.norm(d) / nrm) if nrm > 0 else 0.0
    err_l = float(np.abs(l[~empty] - l_ref[~empty]).max()) if (~empty).any() else 0.0
    print(f"[parity] {tag}: max|dO|={err_o:.3e} rel={rel:.3e} max|dLSE|={err_l:.3e}", flush=True)
    assert err_o <= TOL_O_MAX, f"{tag}: max|dO| {err_o}"
    assert rel <= TOL_O_REL, f"{tag}: rel {rel}"
    assert err_l <= TOL_LSE, f"{tag}: max|dLSE| {err_l}"


# ------------------------------------------------------------------ small

def test_tiny_workload_exact_config():
    x = config_inputs(1)
    out, lse = gpu_decode(x)
    check(out, lse, *oracle(x), tag="tiny 2x{1024,1536} q1 h16 bf16")


@pytest.mark.parametrize("kv", KV_DTYPES)
@pytest.mark.parametrize("q,H", [(1, 128), (5, 96), (2, 16), (3, 40)])
def test_small_shapes(kv, q, H):
    lens = [700, 33, q, 1000] if q > 1 else [700, 33, 1, 1000]
    x = make_inputs(40 + q, lens, q, H, kv, kv_std=0.1 if kv == "bf16" else 1.0)
    out, lse = gpu_decode(x)
    check(out, lse, *oracle(x), tag=f"{kv} q{q} h{H} lens {lens}")


@pytest.mark.parametrize("kv", KV_DTYPES)
@pytest.mark.parametrize("q,H,splits", [(1, 8, 5), (5, 96, 9), (2, 112, 3), (5, 96, 0)])
@pytest.mark.parametrize("page_size", [64, 16])
def test_rows_past_the_request_end(kv, q, H, splits, page_size):
    # Row groups whose last waves hold no valid row (8 rows: waves 1-3 of
    # the group are empty; 480 rows: wave 3 of group 3; 224 rows: wave 3 of
    # group 1), with units of a single tile (32-token cuts of short
    # requests) and a 1-token request.  splits 0 plans for 8 compute units,
    # so that each workgroup runs several units in a row.  Page size 16
    # takes the general-table kernels (a table load per lane and tile).
    lens = [q, 40, 95, 64 * 3 + 1, 900]
    x = make_inputs(60 + q, lens, q, H, kv, kv_std=0.1 if kv == "bf16" else 1.0,
                    page_size=page_size)
    out, lse = gpu_decode(x, force_splits=splits, num_cus=8 if splits == 0 else 0)
    check(out, lse, *oracle(x), tag=f"{kv} q{q} h{H} splits {splits} lens {lens}")


@pytest.mark.parametrize("kv", KV_DTYPES)
@pytest.mark.parametrize("variant", ["qx30", "planted", "offset"])
@pytest.mark.parametrize("q", [1, 5])
@pytest.mark.parametrize("splits", [1, 2, 7, 40])
def test_peaked_variants_and_forced_splits(kv, variant, q, splits):
    x = make_inputs(50, [1300, 257], q, 32, kv, variant=variant,
                    kv_std=0.1 if kv == "bf16" else 1.0)
    out, lse = gpu_decode(x, force_splits=splits)
    check(out, lse, *oracle(x), tag=f"{kv} {variant} q{q} splits {splits}")


@pytest.mark.parametrize("kv", KV_DTYPES)
@pytest.mark.parametrize("page_size", [1, 16, 64, 128])
def test_page_sizes_and_general_tables(kv, page_size):
    # page_size 1 and 16 exercise the per-token table path.
    x = make_inputs(60, [500, 129, 64], 5, 24, kv, page_size=page_size,
                    kv_std=0.1 if kv == "bf16" else 1.0)
    out, lse = gpu_decode(x)
    check(out, lse, *oracle(x), tag=f"{kv} page {page_size}")


@pytest.mark.parametrize("kv", KV_DTYPES)
def test_edge_lengths(kv):
    # seq_len == q_len (one visible token for draft 0), exact tile multiples, +1 tails.
    lens = [5, 6, 32, 33, 64, 65, 95, 96, 97]
    x = make_inputs(61, lens, 5, 20, kv, kv_std=0.1 if kv == "bf16" else 1.0)
    for fs in (0, 3):
        out, lse = gpu_decode(x, force_splits=fs)
        check(out, lse, *oracle(x), tag=f"{kv} edge lengths splits {fs}")


@pytest.mark.parametrize("kv", KV_DTYPES)
def test_planner_cuts_match_unsplit(kv):
    x = make_inputs(62, [3000, 100, 4097], 5, 96, kv, kv_std=0.1 if kv == "bf16" else 1.0)
    o1, l1 = gpu_decode(x, force_splits=1)
    o2, l2 = gpu_decode(x)  # planner: one workgroup per CU, cut into pieces
    o_ref, l_ref = oracle(x)
    check(o1, l1, o_ref, l_ref, tag=f"{kv} unsplit")
    check(o2, l2, o_ref, l_ref, tag=f"{kv} planner")


@pytest.mark.parametrize("kv", KV_DTYPES)
def test_attend_then_merge_equals_decode(kv):
    # The two halves of mla_decode, enqueued apart, give the same bits.
    x = make_inputs(63, [2000, 77, 900], 5, 48, kv, kv_std=0.1 if kv == "bf16" else 1.0)
    plans = []
    o1, l1 = gpu_decode(x, force_splits=3, plan_out=plans)
    plan = plans[0]
    g = x.to(DEV)
    seq = torch.from_numpy(np.asarray(x.seq_lens, np.int32)).to(DEV)
    ws = torch.zeros(plan.workspace_bytes, dtype=torch.uint8, device=DEV)
    o2 = torch.full_like(o1, float("nan"))
    l2 = torch.full_like(l1, float("nan"))
    args = (plan, g.q_nope, g.q_rope, g.pool, g.kv_scale, g.req_to_token, seq, x.softmax_scale)
    mla.decode(*args, workspace=ws, out=o2, lse=l2, phase="attend")
    mla.decode(*args, workspace=ws, out=o2, lse=l2, phase="merge")
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("kv", KV_DTYPES)
def test_dcp_shards_merge_to_full_context(kv):
    full = make_inputs(63, [1500, 700, 9, 8, 5], 5, 32, kv, kv_std=0.1 if kv == "bf16" else 1.0)
    o_full, l_full = oracle(full)
    parts_o, parts_l = [], []
    for r in range(8):
        s = shard_from_full(full, 8, r)
        out, lse = gpu_decode(s)
        check(out, lse, *oracle(s), tag=f"{kv} shard {r}")
        parts_o.append(out)
        parts_l.append(lse)
    po = torch.stack(parts_o).contiguous()
    pl = torch.stack(parts_l).contiguous()
    mo, ml = mla.lse_combine(po, pl)
    torch.cuda.synchronize()
    check(mo, ml, o_full, l_full, tag=f"{kv} 8-shard merge vs full context")


@pytest.mark.parametrize("kv", KV_DTYPES)
@pytest.mark.parametrize("W", [2, 3, 4])
def test_other_dcp_widths_merge_to_full_context(kv, W):
    # Shard counts other than 8 (3 does not divide the page size): every
    # shard against the oracle, and their LSE merge against full context.
    full = make_inputs(64 + W, [900, 301, 7, 5], 5, 24, kv, kv_std=0.1 if kv == "bf16" else 1.0)
    o_full, l_full = oracle(full)
    parts_o, parts_l = [], []
    for r in range(W):
        s = shard_from_full(full, W, r)
        out, lse = gpu_decode(s)
        check(out, lse, *oracle(s), tag=f"{kv} W{W} shard {r}")
        parts_o.append(out)
        parts_l.append(lse)
    mo, ml = mla.lse_combine(torch.stack(parts_o).contiguous(), torch.stack(parts_l).contiguous())
    torch.cuda.synchronize()
    check(mo, ml, o_full, l_full, tag=f"{kv} {W}-shard merge vs full context")


@pytest.mark.parametrize("kv", KV_DTYPES)
def test_largest_q_len_and_many_row_groups(kv):
    # q_len 8 (the largest) x 128 heads = 1024 rows: 8 row groups per request.
    x = make_inputs(66, [700, 64, 8], 8, 128, kv, kv_std=0.1 if kv == "bf16" else 1.0)
    for splits in (0, 3):
        out, lse = gpu_decode(x, force_splits=splits)
        check(out, lse, *oracle(x), tag=f"{kv} q8 h128 splits {splits}")


def test_lse_combine_edge_cases():
    rng = np.random.default_rng(4)
    P, rows = 5, 300
    o = rng.standard_normal((P, rows, 512)).astype(np.float32)
    l = (rng.standard_normal((P, rows)) * 3).astype(np.float32)
    l[:, :7] = -np.inf            # rows with no part at all
    l[1:, 7:20] = -np.inf         # rows with a single part
    l[rng.random((P, rows)) < 0.2] = -np.inf
    o[np.isneginf(l)] = np.nan    # weights of 0 must never touch these
    mo, ml = mla.lse_combine(torch.from_numpy(o).to(DEV), torch.from_numpy(l).to(DEV))
    torch.cuda.synchronize()
    ref_o, ref_l = lse_combine_ref(np.where(np.isneginf(l)[..., None], 0.0, o), l)
    check(mo, ml, ref_o, ref_l, tag="lse_combine edge cases")


# ------------------------------------------------------------------ full sizes

def test_standard_workload_full():
    x = config_inputs(2, device=DEV)
    out, lse = gpu_decode(x)
    check(out, lse, *oracle(x), tag="standard 32x4096 q1 h128 bf16 (all requests)")


def test_mtp_100k_workload_sampled():
    """The mtp workload in the plan bench.py times: requests 0 and 11 against the
    oracle, and all 16 requests against a run of the same inputs with every
    request in one piece (no split, no merge)."""
    x = config_inputs(3, device=DEV)
    out, lse = gpu_decode(x)
    reqs = [0, 11]
    o_ref, l_ref = oracle(x, reqs=reqs)
    check(out[reqs], lse[reqs], o_ref, l_ref, tag="mtp 16x100k q5 h96 fp8 (requests 0, 11)")
    o1, l1 = gpu_decode(x, force_splits=1)
    check(out, lse, o1.double().cpu().numpy(), l1.double().cpu().numpy(),
          tag="mtp 16x100k: planner cuts vs unsplit, all 16 requests")


@pytest.mark.parametrize("variant", ["planted", "qx30"])
def test_mtp_100k_peaked_sampled(variant):
    """The mtp shape (16 x 100k, q5, h96, FP8) at full size with a peaked score
    distribution, in the plan bench.py times: two requests against the oracle."""
    x = make_inputs(3, [100000] * 16, 5, 96, "fp8", device=DEV, kv_std=1.0, variant=variant)
    out, lse = gpu_decode(x)
    reqs = [2, 13]
    o_ref, l_ref = oracle(x, reqs=reqs)
    check(out[reqs], lse[reqs], o_ref, l_ref, tag=f"mtp 16x100k {variant} (requests 2, 13)")


def test_mtp_q1_companion_sampled():
    """The q_len 1 companion of the mtp shape (16 x 100k, 96 heads, FP8), in the
    plan bench.py times: requests 0 and 15 against the oracle."""
    x = config_inputs(9, device=DEV)
    out, lse = gpu_decode(x)
    reqs = [0, 15]
    o_ref, l_ref = oracle(x, reqs=reqs)
    check(out[reqs], lse[reqs], o_ref, l_ref, tag="mtp-q1 16x100k q1 h96 fp8 (requests 0, 15)")


def test_dcp_shard_workload_sampled():
    """A dcp8 shard (128 x 12500 local tokens, q5, h96, FP8) in the plan
    bench.py times (every request in one piece: 512 units fill the chip):
    three requests against the oracle, and all 128 against a run of the same
    inputs with every request cut in three pieces and merged."""
    x = config_inputs(4, device=DEV, dcp_rank=3)
    out, lse = gpu_decode(x)
    reqs = [0, 77, 127]
    o_ref, l_ref = oracle(x, reqs=reqs)
    check(out[reqs], lse[reqs], o_ref, l_ref, tag="dcp8 shard 3, 128x12500 (requests 0, 77, 127)")
    o3, l3 = gpu_decode(x, force_splits=3)
    check(o3, l3, out.double().cpu().numpy(), lse.double().cpu().numpy(),
          tag="dcp8 shard 3: three pieces merged vs one piece, all 128 requests")


def test_dcp8_all_shards_and_combine_sampled():
    """All 8 shards of the dcp8 workload (128 x 12500-token shards, q5, h96, FP8)
    at full size, each in the plan bench.py times, then mla_lse_combine over
    all 61440 rows of the 8 parts.  Three requests are checked: each shard's
    oracle result, merged by the oracle's combine (its equality with
    full-context attention is pinned on the CPU)."""
    reqs = [0, 64, 127]
    parts_o, parts_l, ref_o, ref_l = [], [], [], []
    for r in range(8):
        x = config_inputs(4, device=DEV, dcp_rank=r)
        out, lse = gpu_decode(x)
        o_r, l_r = oracle(x, reqs=reqs)
        check(out[reqs], lse[reqs], o_r, l_r, tag=f"dcp8 shard {r} (requests 0, 64, 127)")
        parts_o.append(out)
        parts_l.append(lse)
        ref_o.append(o_r)
        ref_l.append(l_r)
        del x
    mo, ml = mla.lse_combine(torch.stack(parts_o).contiguous(), torch.stack(parts_l).contiguous())
    torch.cuda.synchronize()
    assert mo.shape == parts_o[0].shape and ml.shape == parts_l[0].shape
    o_ref, l_ref = lse_combine_ref(np.stack(ref_o), np.stack(ref_l))
    check(mo[reqs], ml[reqs], o_ref, l_ref, tag="dcp8 8-shard combine (requests 0, 64, 127)")


def test_sweep_batch1_200k():
    x = config_inputs(5, device=DEV, batch=1)
    out, lse = gpu_decode(x)
    check(out, lse, *oracle(x), tag="sweep 1x200k q5 h96 fp8")


@pytest.mark.parametrize("B", [2, 4, 8, 12, 16, 20])
def test_sweep_batches_200k_sampled(B):
    """Sweep batches 2..20 at 200k (q5, h96, FP8) in the plans the sweep times:
    the last request of each against the oracle."""
    x = config_inputs(5, device=DEV, batch=B)
    out, lse = gpu_decode(x)
    reqs = [B - 1]
    o_ref, l_ref = oracle(x, reqs=reqs)
    check(out[reqs], lse[reqs], o_ref, l_ref, tag=f"sweep {B}x200k (request {B - 1})")
    del x


def test_sweep_batch24_200k_sampled():
    """The largest fixed sweep batch (24 x 200k, q5, h96, FP8) at full size, in
    the plan the sweep times: the last request against the oracle, and all 24
    against a run of the same inputs with every request in one piece."""
    x = config_inputs(5, device=DEV, batch=24)
    out, lse = gpu_decode(x)
    reqs = [23]
    o_ref, l_ref = oracle(x, reqs=reqs)
    check(out[reqs], lse[reqs], o_ref, l_ref, tag="sweep 24x200k q5 h96 fp8 (request 23)")
    o1, l1 = gpu_decode(x, force_splits=1)
    check(out, lse, o1.double().cpu().numpy(), l1.double().cpu().numpy(),
          tag="sweep 24x200k: planner cuts vs unsplit, all 24 requests")


def test_sweep_ragged64_sampled():
    """The ragged 64-request sweep batch (contexts log-uniform in [1024, 400000],
    4.4M tokens) at full size, in the plan the sweep times.  Five requests are
    checked against the oracle, from the shortest (1031 tokens) to the longest
    (398038 tokens, the largest context of any workload here)."""
    x = config_inputs(5, device=DEV, ragged=True)
    out, lse = gpu_decode(x)
    reqs = [31, 38, 63, 58, 9]
    assert list(np.asarray(x.seq_lens)[reqs]) == [1031, 2492, 46931, 85484, 398038]
    o_ref, l_ref = oracle(x, reqs=reqs)
    check(out[reqs], lse[reqs], o_ref, l_ref, tag="sweep ragged64 q5 h96 fp8 (5 requests)")


@pytest.mark.parametrize("kv", KV_DTYPES)
def test_paged_tile_at_the_end_of_a_short_pool(kv):
    """A paged table (page size 32) whose last valid tile starts 4 slots before
    the end of a pool that is not a multiple of 32 slots: the tile must read
    its own slots, not slots re-based into the pool."""
    x = make_inputs(70, [36, 40], 1, 16, kv, page_size=32, kv_std=0.1 if kv == "bf16" else 1.0)
    # Move request 0's second page (its 4 valid tokens) to the last 4 slots of
    # a pool cut to 100 slots more than it needs.
    n_slots = x.num_slots
    extra = 100 - n_slots % 32 if n_slots % 32 else 68
    pool = torch.cat([x.pool, x.pool[:extra].clone()], 0)
    sc = None if x.kv_scale is None else torch.cat([x.kv_scale, x.kv_scale[:extra].clone()], 0)
    end = pool.shape[0]
    assert end % 32 != 0
    table = x.req_to_token.clone()
    src = table[0, 32:36].long()
    dst = torch.arange(end - 4, end)
    pool[dst] = pool[src]
    if sc is not None:
        sc[dst] = sc[src]
    table[0, 32:36] = dst.to(torch.int32)
    table[0, 36:64] = 0
    x = type(x)(**dict(x.__dict__, pool=pool, kv_scale=sc, req_to_token=table))
    out, lse = gpu_decode(x)
    check(out, lse, *oracle(x), tag=f"{kv} paged tile at the end of a {end}-slot pool")


def test_fp8_every_code_decodes_exactly():
    # One visible token and q_len 1: the softmax weight is 1 (up to one fp32
    # rounding in the exponent), so O is that token's value row, which holds
    # every non-NaN e4m3fn code.  Adjacent codes differ by >= 1/8 relative
    # (subnormals: >= 1/7), so rtol 1e-5 (a few fp32 ulps) still pins every code.
    from oracle import E4M3FN_TABLE
    x = make_inputs(64, [1], 1, 32, "fp8")
    slot = int(x.req_to_token[0, 0])
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    row = np.concatenate([codes, codes[::-1], codes[:68]])
    x.pool[slot] = torch.from_numpy(row)
    x.kv_scale[slot] = 1.0
    out, lse = gpu_decode(x, force_splits=1)
    o = out[0, 0].double().cpu().numpy()
    want = E4M3FN_TABLE[row[:512]]
    np.testing.assert_allclose(o, np.broadcast_to(want, o.shape), rtol=1e-5, atol=0)


def test_fp4_every_code_and_scale_decodes_exactly():
    # One visible token and q_len 1: O is that token's c_kv, whose 16-element
    # blocks hold every e2m1 code under block scales that span the valid
    # range 2^-64 .. 2^64 (the dequantized BF16 value is exact, so only the
    # fp32 division by the softmax weight rounds).  The query is zero so that
    # the score stays 0 whatever the key: fp32 softmax arithmetic is not
    # meant for scores near 2^64.
    from oracle import decode_fp4_rows
    x = make_inputs(67, [1], 1, 32, "fp4")
    x.q_nope.zero_()
    x.q_rope.zero_()
    slot = int(x.req_to_token[0, 0])
    row = np.zeros(336, dtype=np.uint8)
    codes = np.arange(576) % 16
    codes[16:32] = codes[16:32][::-1]
    row[:288] = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)
    row[288:324] = np.linspace(63, 191, 36).round().astype(np.uint8)
    row[288 + 32:] = 127           # k_rope blocks at 2^0
    row[288 + 33:288 + 36] = 127
    x.pool[slot] = torch.from_numpy(row)
    out, lse = gpu_decode(x, force_splits=1)
    o = out[0, 0].double().cpu().numpy()
    want = decode_fp4_rows(row[None])[0, :512]
    np.testing.assert_allclose(o, np.broadcast_to(want, o.shape), rtol=1e-5, atol=0)


def test_fp4_mtp_100k_workload_sampled():
    x = config_inputs(6, device=DEV)
    out, lse = gpu_decode(x)
    reqs = [0, 11]
    o_ref, l_ref = oracle(x, reqs=reqs)
    check(out[reqs], lse[reqs], o_ref, l_ref, tag="mtp 16x100k q5 h96 fp4 (requests 0, 11)")


def test_fp4_standard_workload_full():
    x = config_inputs(7, device=DEV)
    out, lse = gpu_decode(x)
    check(out, lse, *oracle(x), tag="standard 32x4096 q1 h128 fp4 (all requests)")


def test_mxfp8_every_code_and_scale_decodes_exactly():
    # One visible token, q_len 1, zero query: O is that token's c_kv, whose
    # 32-element blocks hold every finite e4m3fn code under block scales
    # spanning the valid range 2^-64 .. 2^64.
    from oracle import decode_mxfp8_rows
    x = make_inputs(68, [1], 1, 32, "mxfp8")
    x.q_nope.zero_()
    x.q_rope.zero_()
    slot = int(x.req_to_token[0, 0])
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    row = np.zeros(608, dtype=np.uint8)
    row[:512] = np.resize(np.concatenate([finite, finite[::-1]]), 512)
    row[512:576] = finite[:64]
    row[576:592] = np.linspace(63, 191, 16).round().astype(np.uint8)
    row[592:594] = 127
    x.pool[slot] = torch.from_numpy(row)
    out, lse = gpu_decode(x, force_splits=1)
    o = out[0, 0].double().cpu().numpy()
    want = decode_mxfp8_rows(row[None])[0, :512]
    np.testing.assert_allclose(o, np.broadcast_to(want, o.shape), rtol=1e-5, atol=0)


def test_mxfp8_mtp_100k_workload_sampled():
    x = config_inputs(8, device=DEV)
    out, lse = gpu_decode(x)
    reqs = [0, 11]
    o_ref, l_ref = oracle(x, reqs=reqs)
    check(out[reqs], lse[reqs], o_ref, l_ref, tag="mtp 16x100k q5 h96 mxfp8 (requests 0, 11)")
