"""Seeded generators of paged latent-KV decode inputs.

Shapes and structure follow the workloads on the page "Kimi K3 decode: DP16 vs
DP2 x DCP8": 96 query heads, 5 verified tokens per request, a 576-wide latent
row per token (512 c_kv + 64 k_rope) stored once per token (VRAM page,
"cell_size": pool shape (size + page_size, 1, 576)), an int32 request-to-slot
table (VRAM page, "where the req_to_token size comes from"), FP8 storage at
one byte per element (DP16-vs-DP2 page, "capacity": 24 layers x 576 B), and
DCP shards holding positions p % 8 == r (same page, "problem" section).

Every random draw is seeded from (config id, tensor id).  Index structure
(lengths, page permutations, per-token scales) comes from numpy's
SeedSequence-seeded generator and is identical on every machine; bulk values
(queries and latent rows) come from a seeded torch generator on the target
device, so large pools can be generated directly in GPU memory.

Poisoning: page 0 is a padding page that no table entry references (the extra
page_size slots of the pool), and slots past a request's length in its last
page are filled with NaN (BF16 0x7FC0, e4m3fn 0x7F, scale NaN), so any read of
a slot that should not be visible shows up as a NaN in the output.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

D_C = 512
D_R = 64
D_K = 576

BF16_NAN_BITS = 0x7FC0
E4M3FN_NAN_CODE = 0x7F
# FP4 rows: 576 e2m1 codes packed two per byte (element 2 i in the low
# nibble of byte i), 36 block-scale bytes (power-of-two exponents with bias
# 127, one per 16 elements), 12 bytes of zero padding.
FP4_ROW_BYTES = 336
FP4_CODE_BYTES = 288
FP4_POISON_CODES = 0x77     # e2m1 6.0 in both nibbles
FP4_POISON_SCALE = 0xFF     # not a valid scale code
# MXFP8 rows: 576 e4m3fn codes, 18 block-scale bytes (one per 32 elements,
# bias 127), 14 bytes of zero padding.
MXFP8_ROW_BYTES = 608

# Tensor ids for the seed sequences.
_T_LENGTHS, _T_PAGES, _T_SCALE, _T_KV, _T_QNOPE, _T_QROPE, _T_PLANT = range(7)


def softmax_scale_default() -> float:
    """fp32(1 / sqrt(192)); 192 = qk_nope_head_dim 128 + qk_rope_head_dim 64."""
    return float(np.float32(1.0 / math.sqrt(192.0)))


def kv_bytes_per_token(kv_dtype: str) -> int:
    """Algorithmic KV bytes read per visible token: 576 elements (+ fp32 scale
    for FP8); FP4 rows are 336 bytes (288 of codes, 36 block scales,
    padding), MXFP8 rows 608 (576 codes, 18 block scales, padding)."""
    if kv_dtype == "fp4":
        return FP4_ROW_BYTES
    if kv_dtype == "mxfp8":
        return MXFP8_ROW_BYTES
    return D_K * 2 if kv_dtype == "bf16" else D_K * 1 + 4


def _np_rng(cfg_id: int, tensor_id: int, extra: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([cfg_id, tensor_id, extra]))


def _torch_gen(cfg_id: int, tensor_id: int, extra: int, device) -> torch.Generator:
    seed = int(np.random.SeedSequence([cfg_id, tensor_id, extra]).generate_state(1, np.uint64)[0]
               & ((1 << 63) - 1))
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def local_lengths(seq_lens, dcp_size: int, dcp_rank: int) -> np.ndarray:
    """Number of positions p < L with p % W == r, for each global length L."""
    L = np.asarray(seq_lens, dtype=np.int64)
    n = (L - dcp_rank + dcp_size - 1) // dcp_size
    return np.maximum(n, 0).astype(np.int64)


def ragged_lengths(cfg_id: int, batch: int, lo: int, hi: int) -> np.ndarray:
    """floor(exp(U(ln lo, ln hi))), seeded."""
    u = _np_rng(cfg_id, _T_LENGTHS).uniform(math.log(lo), math.log(hi), size=batch)
    return np.floor(np.exp(u)).astype(np.int64)


@dataclass
class DecodeInputs:
    batch: int
    q_len: int
    num_heads: int
    kv_dtype: str  # "bf16" | "fp8" | "fp4" | "mxfp8"
    page_size: int
    seq_lens: np.ndarray  # int64 [B], global lengths including the q drafts
    local_lens: np.ndarray  # int64 [B], table columns used on this shard
    q_nope: torch.Tensor  # bf16 [B, q, H, 512]
    q_rope: torch.Tensor  # bf16 [B, q, H, 64]
    pool: torch.Tensor  # bf16 [S, 576], uint8 [S, 576] (e4m3fn), [S, 336] (FP4) or [S, 608] (MXFP8)
    kv_scale: torch.Tensor | None  # float32 [S] (FP8 only)
    req_to_token: torch.Tensor  # int32 [B, stride]
    softmax_scale: float
    dcp_size: int = 1
    dcp_rank: int = 0
    name: str = ""
    meta: dict = field(default_factory=dict)

    @property
    def num_slots(self) -> int:
        return int(self.pool.shape[0])

    @property
    def rows_per_request(self) -> int:
        return self.q_len * self.num_heads

    def kv_bytes(self) -> int:
        """Algorithmic KV bytes: every stored token of every request read once."""
        return int(self.local_lens.sum()) * kv_bytes_per_token(self.kv_dtype)

    def to(self, device) -> "DecodeInputs":
        d = dict(self.__dict__)
        for k in ("q_nope", "q_rope", "pool", "kv_scale", "req_to_token"):
            if d[k] is not None:
                d[k] = d[k].to(device)
        return DecodeInputs(**d)

    def numpy_bits(self) -> dict:
        """Stored bit patterns as numpy arrays, the form the oracle takes."""
        return dict(
            q_nope=self.q_nope.cpu().view(torch.int16).numpy().view(np.uint16),
            q_rope=self.q_rope.cpu().view(torch.int16).numpy().view(np.uint16),
            pool=(self.pool.cpu().view(torch.int16).numpy().view(np.uint16)
                  if self.kv_dtype == "bf16" else self.pool.cpu().numpy()),
            kv_scale=None if self.kv_scale is None else self.kv_scale.cpu().numpy(),
            req_to_token=self.req_to_token.cpu().numpy(),
            seq_lens=np.asarray(self.seq_lens, dtype=np.int64),
        )


def _page_table(cfg_id: int, local_lens: np.ndarray, page_size: int, extra: int):
    """Request-to-slot table over a randomly permuted set of physical pages.

    Page 0 is never referenced.  Returns (table int32 [B, stride], num_slots,
    used bool [num_slots]).
    """
    B = len(local_lens)
    pages = [int(math.ceil(n / page_size)) for n in local_lens]
    total = sum(pages)
    perm = _np_rng(cfg_id, _T_PAGES, extra).permutation(total) + 1
    stride = max(page_size, int(math.ceil(max(local_lens, default=1) / page_size)) * page_size)
    table = np.zeros((B, stride), dtype=np.int32)
    used = np.zeros((total + 1) * page_size, dtype=bool)
    k = 0
    for b in range(B):
        n = int(local_lens[b])
        if n == 0:
            continue
        phys = perm[k:k + pages[b]]
        k += pages[b]
        j = np.arange(n)
        slots = phys[j // page_size] * page_size + j % page_size
        table[b, :n] = slots
        used[slots] = True
    return table, (total + 1) * page_size, used


def _fill_values(shape, gen, device, dtype_out: str, std: float) -> torch.Tensor:
    """N(0, 1) * std rounded to BF16 (RNE), or N(0, 1) rounded to e4m3fn bits."""
    rows = shape[0]
    out = torch.empty(shape, dtype=torch.bfloat16 if dtype_out == "bf16" else torch.uint8,
                      device=device)
    chunk = max(1, (1 << 26) // max(1, int(np.prod(shape[1:]))))
    for r0 in range(0, rows, chunk):
        r1 = min(rows, r0 + chunk)
        x = torch.randn((r1 - r0,) + tuple(shape[1:]), generator=gen, device=device,
                        dtype=torch.float32)
        if dtype_out == "bf16":
            out[r0:r1] = (x * std).to(torch.bfloat16)
        else:
            out[r0:r1] = x.to(torch.float8_e4m3fn).view(torch.uint8)
    return out


def _fill_fp4(rows: int, gen, device, exp_lo: int, exp_hi: int) -> torch.Tensor:
    """FP4 rows: uniformly random codes, block-scale exponents uniform in
    [exp_lo, exp_hi] (as codes 127 + e), zero padding."""
    out = torch.zeros((rows, FP4_ROW_BYTES), dtype=torch.uint8, device=device)
    chunk = 1 << 18
    for r0 in range(0, rows, chunk):
        r1 = min(rows, r0 + chunk)
        out[r0:r1, :FP4_CODE_BYTES] = torch.randint(
            0, 256, (r1 - r0, FP4_CODE_BYTES), generator=gen, device=device,
            dtype=torch.int32).to(torch.uint8)
        out[r0:r1, FP4_CODE_BYTES:FP4_CODE_BYTES + 36] = torch.randint(
            127 + exp_lo, 127 + exp_hi + 1, (r1 - r0, 36), generator=gen, device=device,
            dtype=torch.int32).to(torch.uint8)
    return out


def _fill_mxfp8(rows: int, gen, device, exp_lo: int, exp_hi: int) -> torch.Tensor:
    """MXFP8 rows: N(0, 1) rounded to e4m3fn codes, block-scale exponents
    uniform in [exp_lo, exp_hi] (as codes 127 + e), zero padding."""
    out = torch.zeros((rows, MXFP8_ROW_BYTES), dtype=torch.uint8, device=device)
    out[:, :D_K] = _fill_values((rows, D_K), gen, device, "fp8", 1.0)
    chunk = 1 << 18
    for r0 in range(0, rows, chunk):
        r1 = min(rows, r0 + chunk)
        out[r0:r1, D_K:D_K + 18] = torch.randint(
            127 + exp_lo, 127 + exp_hi + 1, (r1 - r0, 18), generator=gen, device=device,
            dtype=torch.int32).to(torch.uint8)
    return out


def make_inputs(cfg_id: int, seq_lens, q_len: int, num_heads: int, kv_dtype: str,
                page_size: int = 64, device="cpu", dcp_size: int = 1, dcp_rank: int = 0,
                q_std: float = 0.1, kv_std: float = 0.1, scale_lo: float = 0.01,
                scale_hi: float = 0.05, variant: str | None = None,
                name: str = "") -> DecodeInputs:
    """Build one decode call's inputs.

    seq_lens are global lengths L_b (>= q_len).  With dcp_size > 1 the pool
    and table hold only shard dcp_rank's positions p % W == r, at local index
    (p - r) / W.  `variant` selects a peaked distribution for parity runs:
    "qx30" (queries x 30), "planted" (1% of keys aligned with head 0's query),
    "offset" (a large common score offset through the RoPE part).
    """
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    B = len(seq_lens)
    local = local_lengths(seq_lens, dcp_size, dcp_rank)
    extra = dcp_rank if dcp_size > 1 else 0
    table, num_slots, used = _page_table(cfg_id, local, page_size, extra)

    kv_gen = _torch_gen(cfg_id, _T_KV, extra, device)
    if kv_dtype == "fp4":
        # Elements up to 6 * 2^-4; typical magnitudes near those of the BF16
        # pools (N(0, 1) * 0.1).
        pool = _fill_fp4(num_slots, kv_gen, device, -6, -4)
    elif kv_dtype == "mxfp8":
        # N(0, 1) * 2^(-5 .. -3): magnitudes near those of the BF16 pools.
        pool = _fill_mxfp8(num_slots, kv_gen, device, -5, -3)
    else:
        pool = _fill_values((num_slots, D_K), kv_gen, device, kv_dtype, kv_std)
    kv_scale = None
    if kv_dtype == "fp8":
        sc = _np_rng(cfg_id, _T_SCALE, extra).uniform(scale_lo, scale_hi, size=num_slots)
        kv_scale = torch.from_numpy(sc.astype(np.float32)).to(device)

    q_mult = 30.0 if variant == "qx30" else 1.0
    qn = _fill_values((B, q_len, num_heads, D_C), _torch_gen(cfg_id, _T_QNOPE, 0, device),
                      device, "bf16", q_std * q_mult)
    qr = _fill_values((B, q_len, num_heads, D_R), _torch_gen(cfg_id, _T_QROPE, 0, device),
                      device, "bf16", q_std * q_mult)

    if variant == "offset":
        # A shared component along RoPE element 0 adds roughly the same large
        # amount to every score, so exp() overflows unless the max is removed.
        qr[..., 0] = 100.0
        if kv_dtype == "bf16":
            pool[:, D_C] = 40.0
        elif kv_dtype == "fp4":
            # Element 512 (low nibble of byte 256) = 6 * 2^3 = 48; the rest of
            # its block scales up by 2^3 with it.
            pool[:, D_C // 2] = (pool[:, D_C // 2] & 0xF0) | 0x7
            pool[:, FP4_CODE_BYTES + D_C // 16] = 127 + 3
        elif kv_dtype == "mxfp8":
            # Element 512 = 448 * 2^-5 = 14 (its block at scale 2^-5).
            pool[:, D_C] = 0x7E
            pool[:, D_K + D_C // 32] = 127 - 5
        else:
            pool[:, D_C] = 0x7E  # e4m3fn 448
    elif variant == "planted":
        rng = _np_rng(cfg_id, _T_PLANT, extra)
        q0 = torch.cat([qn[:, 0, 0].float(), qr[:, 0, 0].float()], dim=-1).cpu()  # [B, 576]
        for b in range(B):
            n = int(local[b])
            k = max(1, n // 100)
            js = rng.choice(n, size=k, replace=False)
            slots = torch.from_numpy(table[b, js].astype(np.int64))
            direction = q0[b] / q0[b].norm()
            if kv_dtype == "bf16":
                vals = (direction * 40.0).to(torch.bfloat16)
                pool[slots.to(device)] = vals.to(device).expand(len(js), D_K)
            elif kv_dtype in ("fp4", "mxfp8"):
                enc = _encode_fp4_row if kv_dtype == "fp4" else _encode_mxfp8_row
                row = torch.from_numpy(enc(direction.numpy().astype(np.float64) * 40.0))
                pool[slots.to(device)] = row.to(device).expand(len(js), row.numel())
            else:
                sc = kv_scale[slots.to(device)].cpu()
                vals = (direction[None, :] * 40.0 / sc[:, None]).clamp(-448, 448)
                pool[slots.to(device)] = vals.to(torch.float8_e4m3fn).view(torch.uint8).to(device)

    _poison(pool, kv_scale, torch.from_numpy(~used).to(device), kv_dtype)

    return DecodeInputs(
        batch=B, q_len=q_len, num_heads=num_heads, kv_dtype=kv_dtype, page_size=page_size,
        seq_lens=seq_lens, local_lens=local, q_nope=qn, q_rope=qr, pool=pool,
        kv_scale=kv_scale, req_to_token=torch.from_numpy(table).to(device),
        softmax_scale=softmax_scale_default(), dcp_size=dcp_size, dcp_rank=dcp_rank,
        name=name, meta=dict(cfg_id=cfg_id, variant=variant))


# e2m1 magnitudes by code (0..7); code | 8 is the negative value.
_E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _block_exponent(amax: float, top: float) -> int:
    """Smallest e in [-64, 64] with amax <= top * 2^e (-64 for amax = 0)."""
    if amax == 0.0:
        return -64
    e = int(math.ceil(math.log2(amax / top)))
    while amax > top * 2.0 ** e:
        e += 1
    while e > -64 and amax <= top * 2.0 ** (e - 1):
        e -= 1
    return max(-64, min(64, e))


def _encode_fp4_row(v: np.ndarray) -> np.ndarray:
    """One FP4 row (336 bytes) holding the 576 values v: per 16-element block
    a power-of-two scale 2^e (byte 127 + e) and e2m1 codes of v / 2^e, each
    the nearest magnitude (ties to the even code), so that the stored row is
    a close copy of v.  Input construction only: the decode path and the
    oracle read whatever bytes are stored."""
    out = np.zeros(FP4_ROW_BYTES, dtype=np.uint8)
    codes = np.zeros(D_K, dtype=np.uint8)
    for k in range(D_K // 16):
        blk = v[16 * k:16 * k + 16]
        e = _block_exponent(float(np.abs(blk).max()), 6.0)
        out[FP4_CODE_BYTES + k] = 127 + e
        mag = np.minimum(np.abs(blk) / 2.0 ** e, 6.0)
        d = np.abs(mag[:, None] - _E2M1[None, :])
        best = d.min(axis=1, keepdims=True)
        ties = np.isclose(d, best, rtol=0.0, atol=0.0)
        # among the nearest codes prefer the even one
        c = np.where(ties & (np.arange(8)[None, :] % 2 == 0), np.arange(8)[None, :], 99).min(1)
        c = np.where(c == 99, d.argmin(axis=1), c)
        codes[16 * k:16 * k + 16] = c | np.where(blk < 0, 8, 0)
    out[:FP4_CODE_BYTES] = codes[0::2] | (codes[1::2] << 4)
    return out


def _encode_mxfp8_row(v: np.ndarray) -> np.ndarray:
    """One MXFP8 row (608 bytes) holding the 576 values v: per 32-element
    block a power-of-two scale 2^e (byte 127 + e) and e4m3fn codes of v / 2^e
    rounded to nearest even (torch's conversion).  Input construction only."""
    out = np.zeros(MXFP8_ROW_BYTES, dtype=np.uint8)
    for k in range(D_K // 32):
        blk = v[32 * k:32 * k + 32]
        e = _block_exponent(float(np.abs(blk).max()), 448.0)
        out[D_K + k] = 127 + e
        q = torch.from_numpy((blk / 2.0 ** e).astype(np.float32)).to(torch.float8_e4m3fn)
        out[32 * k:32 * k + 32] = q.view(torch.uint8).numpy()
    return out


def _poison(pool, kv_scale, unused, kv_dtype: str) -> None:
    """Fill the slots no table entry references with values that would show."""
    if kv_dtype == "bf16":
        pool.view(torch.int16)[unused] = BF16_NAN_BITS
    elif kv_dtype == "fp4":
        pool[unused, :FP4_CODE_BYTES] = FP4_POISON_CODES
        pool[unused, FP4_CODE_BYTES:FP4_CODE_BYTES + 36] = FP4_POISON_SCALE
    elif kv_dtype == "mxfp8":
        pool[unused, :D_K] = E4M3FN_NAN_CODE
        pool[unused, D_K:D_K + 18] = FP4_POISON_SCALE
    else:
        pool[unused] = E4M3FN_NAN_CODE
        if kv_scale is not None:
            kv_scale[unused] = float("nan")


def shard_from_full(full: DecodeInputs, dcp_size: int, dcp_rank: int,
                    cfg_id: int = 99) -> DecodeInputs:
    """Shard dcp_rank of a full-context input: its own pool, pages and table.

    Position p of request b (p % W == r) moves to local index (p - r) / W of a
    freshly permuted shard pool; the latent rows and scales are copied
    bit-for-bit, and the queries are shared (replicated on every shard).
    """
    W, r = dcp_size, dcp_rank
    local = local_lengths(full.seq_lens, W, r)
    table, num_slots, used = _page_table(cfg_id, local, full.page_size, 1000 + r)
    dev = full.pool.device
    pool = torch.empty((num_slots,) + tuple(full.pool.shape[1:]), dtype=full.pool.dtype,
                       device=dev)
    kv_scale = None if full.kv_scale is None else torch.full(
        (num_slots,), float("nan"), dtype=torch.float32, device=dev)
    full_table = full.req_to_token.cpu().numpy()
    for b in range(full.batch):
        n = int(local[b])
        if n == 0:
            continue
        p = np.arange(n) * W + r
        src = torch.from_numpy(full_table[b, p].astype(np.int64)).to(dev)
        dst = torch.from_numpy(table[b, :n].astype(np.int64)).to(dev)
        pool[dst] = full.pool[src]
        if kv_scale is not None:
            kv_scale[dst] = full.kv_scale[src]
    _poison(pool, kv_scale, torch.from_numpy(~used).to(dev), full.kv_dtype)
    return DecodeInputs(
        batch=full.batch, q_len=full.q_len, num_heads=full.num_heads, kv_dtype=full.kv_dtype,
        page_size=full.page_size, seq_lens=full.seq_lens.copy(), local_lens=local,
        q_nope=full.q_nope, q_rope=full.q_rope, pool=pool, kv_scale=kv_scale,
        req_to_token=torch.from_numpy(table).to(dev), softmax_scale=full.softmax_scale,
        dcp_size=W, dcp_rank=r, name=f"{full.name}/shard{r}", meta=dict(full.meta, shard=r))


# The five workloads, companions of the same shapes over FP4 pools (6, 7) and
# an MXFP8 pool (8), and the mtp shape at q_len 1 (9: 96 query rows per
# request, below the e4m3 ridge, so bound by HBM rather than by the MFMAs).
# Each is a decode call (or, for DCP, eight shard calls and one merge) on one
# GPU.
CONFIGS = {
    1: dict(name="tiny-2x1.3k-q1-h16-bf16", seq_lens=[1024, 1536], q_len=1, num_heads=16,
            kv_dtype="bf16"),
    2: dict(name="standard-32x4096-q1-h128-bf16", seq_lens=[4096] * 32, q_len=1,
            num_heads=128, kv_dtype="bf16"),
    3: dict(name="mtp-16x100k-q5-h96-fp8", seq_lens=[100000] * 16, q_len=5, num_heads=96,
            kv_dtype="fp8"),
    4: dict(name="dcp8-128x100k-q5-h96-fp8", seq_lens=[100000] * 128, q_len=5, num_heads=96,
            kv_dtype="fp8", dcp_size=8),
    5: dict(name="sweep-200k-q5-h96-fp8", seq_len=200000, q_len=5, num_heads=96,
            kv_dtype="fp8"),
    6: dict(name="mtp-16x100k-q5-h96-fp4", seq_lens=[100000] * 16, q_len=5, num_heads=96,
            kv_dtype="fp4"),
    7: dict(name="standard-32x4096-q1-h128-fp4", seq_lens=[4096] * 32, q_len=1,
            num_heads=128, kv_dtype="fp4"),
    8: dict(name="mtp-16x100k-q5-h96-mxfp8", seq_lens=[100000] * 16, q_len=5, num_heads=96,
            kv_dtype="mxfp8"),
    9: dict(name="mtp-q1-16x100k-q1-h96-fp8", seq_lens=[100000] * 16, q_len=1, num_heads=96,
            kv_dtype="fp8"),
}
SWEEP_BATCHES = (1, 2, 4, 8, 12, 16, 20, 24)


def config_inputs(cfg_id: int, device="cpu", dcp_rank: int = 0, batch: int | None = None,
                  ragged: bool = False) -> DecodeInputs:
    """Inputs of workload `cfg_id` (for 4: shard `dcp_rank`; for 5: `batch` or ragged)."""
    c = CONFIGS[cfg_id]
    if cfg_id == 5:
        if ragged:
            lens = ragged_lengths(5, 64, 1024, 400000)
            name = "sweep-ragged64-q5-h96-fp8"
        else:
            lens = [c["seq_len"]] * int(batch)
            name = f"sweep-{batch}x200k-q5-h96-fp8"
        return make_inputs(5, lens, c["q_len"], c["num_heads"], c["kv_dtype"], device=device,
                           name=name)
    kv_std = 0.1 if c["kv_dtype"] == "bf16" else 1.0
    return make_inputs(cfg_id, c["seq_lens"], c["q_len"], c["num_heads"], c["kv_dtype"],
                       device=device, dcp_size=c.get("dcp_size", 1), dcp_rank=dcp_rank,
                       kv_std=kv_std, name=c["name"])


# Inputs of the MLA prepare step (the T = B * q_len new tokens of a decode
# step): seeded like the decode workloads, with a RoPE cos / sin table of
# the usual geometric frequencies (base 10000) over max_pos positions.
PREPARE_CONFIGS = {
    "mtp": dict(name="prepare-mtp-80x96-fp8", T=16 * 5, H=96, kv_dtype="fp8"),
    "dcp8": dict(name="prepare-dcp8-640x96-fp8", T=128 * 5, H=96, kv_dtype="fp8"),
    "standard": dict(name="prepare-standard-32x128-bf16", T=32, H=128, kv_dtype="bf16"),
    "mtp-fp4": dict(name="prepare-mtp-80x96-fp4", T=16 * 5, H=96, kv_dtype="fp4"),
    "mtp-mxfp8": dict(name="prepare-mtp-80x96-mxfp8", T=16 * 5, H=96, kv_dtype="mxfp8"),
}


def prepare_inputs(key: str, device="cpu", num_slots: int = 1 << 18, max_pos: int = 1 << 17):
    """Tensors of one mla_prepare call for PREPARE_CONFIGS[key]."""
    c = PREPARE_CONFIGS[key]
    T, H, kv = c["T"], c["H"], c["kv_dtype"]
    rng = _np_rng(200, 0, sum(map(ord, key)))

    def bf16(shape, std):
        return torch.from_numpy((rng.standard_normal(shape) * std).astype(np.float32)).to(torch.bfloat16)
    x = dict(q_nope=bf16((T, H, 128), 1.0), q_rope_in=bf16((T, H, 64), 1.0),
             w_kc_t=bf16((H, 512, 128), 0.05), c_kv_new=bf16((T, 512), 0.5),
             k_rope_new=bf16((T, 64), 1.0))
    x["positions"] = torch.from_numpy(rng.integers(0, max_pos, T).astype(np.int32))
    inv = 10000.0 ** (-np.arange(32) / 32.0)
    ang = np.arange(max_pos)[:, None] * inv[None, :]
    x["cos_sin"] = torch.from_numpy(np.concatenate([np.cos(ang), np.sin(ang)], 1).astype(np.float32))
    x["slots"] = torch.from_numpy(rng.permutation(num_slots)[:T].astype(np.int32))
    if kv == "bf16":
        x["kv_pool"] = torch.zeros((num_slots, 576), dtype=torch.bfloat16)
        x["kv_scale"] = None
    elif kv in ("fp4", "mxfp8"):
        rb = FP4_ROW_BYTES if kv == "fp4" else MXFP8_ROW_BYTES
        x["kv_pool"] = torch.zeros((num_slots, rb), dtype=torch.uint8)
        x["kv_scale"] = None
    else:
        x["kv_pool"] = torch.zeros((num_slots, 576), dtype=torch.uint8)
        x["kv_scale"] = torch.ones(num_slots, dtype=torch.float32)
    out = {k: (v.to(device) if v is not None else None) for k, v in x.items()}
    out.update(name=c["name"], T=T, H=H, kv_dtype=kv)
    return out

