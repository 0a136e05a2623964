"""Plain float64 oracle of absorbed MLA decode attention and of the LSE merge.

TEST INFRASTRUCTURE ONLY (see the package docstring for who may import it).

What is computed, for request b, draft position i in [0, q) and head h:

1. Visible positions.  L = seq_lens[b] counts the q draft tokens, whose
   latent rows are already in the pool.  Row i sees global positions
   0 <= p <= L - q + i (causal among the drafts).  Under DCP with W shards,
   shard r only holds positions with p % W == r, addressed by the local index
   j = (p - r) / W.  (DP16-vs-DP2 page: introduction for the 5 verified
   tokens; section "problem: how to split" for slot p -> rank p % 8.)
2. Keys.  slot = req_to_token[b, j]; the key is the whole 576-wide latent row
   [c_kv (512) | k_rope (64)] of that slot, decoded exactly to float64: BF16
   bits, OCP e4m3fn codes times the slot's fp32 scale, or FP4 / MXFP8
   codes times their block scale (formats and readings in fp4_ref and
   mxfp8_ref).  (VRAM page,
   "KV ledger" MLA bullet and the "cell_size" MLA pool shape
   (size + page_size, 1, kv_lora_rank + qk_rope_head_dim).)
3. Values.  The first 512 elements of the same row (the latent c_kv).
   (DP16-vs-DP2 page: kv_b_proj is absorbed into w_kc / w_vc, so the value
   projection is applied after attention and the attended value is c_kv.)
4. Query.  [q_nope_absorbed (512) | q_rope (64)] decoded exactly from BF16.
   (Same page, VRAM-ledger section: w_kc is 96 x 128 x 512, i.e. the
   absorbed query is 512 wide.)
5. Scores.  s_p = scale * (q . k_p), dot product in float64, with scale the
   float32 value the caller passes.
6. Reduce.  Empty visible set -> (O, LSE) = (0, -inf).  Otherwise
   m = max s, LSE = m + ln sum exp(s - m), O = sum exp(s - LSE) v_p.
7. Merge of parts (O_j, LSE_j): M* = max LSE_j; if M* = -inf the result is
   (0, -inf); else w_j = exp(LSE_j - M*), LSE = M* + ln sum w_j and
   O = sum w_j O_j / sum w_j.  (DP16-vs-DP2 page, section "MLA": the
   per-shard (O, LSE) are exchanged and merged by LSE.)

Readings where the pages are silent: the natural log is used for LSE, the
scale is applied before the exponent and is included in LSE, the pool row
order is c_kv then k_rope, the FP8 per-token scale multiplies all 576
elements, FP8 means the OCP e4m3fn variant, and seq_lens hold global lengths
also under DCP.
"""

from __future__ import annotations

import numpy as np

from .fp4_ref import decode_fp4_rows

D_C = 512  # kv_lora_rank: width of the latent c_kv
D_R = 64  # qk_rope_head_dim: width of the decoupled RoPE key
D_K = D_C + D_R  # 576 elements cached per token per layer
D_V = D_C  # the attended value is the latent itself


def e4m3fn_decode_table() -> np.ndarray:
    """Value of every OCP FP8 E4M3 ("fn": finite, NaN only) code as float64.

    From the format definition: 1 sign bit, 4 exponent bits with bias 7,
    3 mantissa bits; exponent field 0 encodes subnormals (m/8) * 2^-6; the
    codes with all exponent and mantissa bits set (0x7F, 0xFF) are NaN; there
    is no infinity, so the largest finite magnitude is 1.75 * 2^8 = 448.
    """
    table = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        exp_field = (code >> 3) & 0xF
        mant = code & 0x7
        if exp_field == 0xF and mant == 0x7:
            table[code] = np.nan
        elif exp_field == 0:
            table[code] = sign * (mant / 8.0) * 2.0 ** -6
        else:
            table[code] = sign * (1.0 + mant / 8.0) * 2.0 ** (exp_field - 7)
    return table


E4M3FN_TABLE = e4m3fn_decode_table()


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact float64 value of BF16 bit patterns (the upper half of a float32)."""
    a = np.asarray(bits)
    if a.dtype.itemsize != 2:
        raise TypeError("BF16 bit patterns must be a 16-bit integer array")
    u32 = a.view(np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def visible_positions(seq_len: int, q_len: int, i: int,
                      dcp_size: int = 1, dcp_rank: int = 0) -> np.ndarray:
    """Global positions p that draft row i may attend to on shard dcp_rank.

    0 <= p <= seq_len - q_len + i, and p % dcp_size == dcp_rank.
    """
    last = seq_len - q_len + i
    if last < dcp_rank:
        return np.empty(0, dtype=np.int64)
    return np.arange(dcp_rank, last + 1, dcp_size, dtype=np.int64)


def local_index(p: np.ndarray, dcp_size: int, dcp_rank: int) -> np.ndarray:
    """Index of global position p inside shard dcp_rank's table: (p - r) / W."""
    return (p - dcp_rank) // dcp_size


def gather_slots(req_to_token: np.ndarray, b: int, j: np.ndarray) -> np.ndarray:
    """Pool slots of request b at table columns j."""
    return req_to_token[b, j].astype(np.int64)


def dequant_rows(pool: np.ndarray, kv_scale, slots: np.ndarray,
                 kv_dtype: str) -> np.ndarray:
    """Exact float64 latent rows [n, 576] of the given slots."""
    raw = pool[slots]
    if kv_dtype == "bf16":
        return bf16_bits_to_f64(raw)
    if kv_dtype == "fp8":
        scale = np.asarray(kv_scale, dtype=np.float32)[slots].astype(np.float64)
        return E4M3FN_TABLE[raw.astype(np.intp)] * scale[:, None]
    if kv_dtype == "fp4":
        return decode_fp4_rows(raw)
    if kv_dtype == "mxfp8":
        from .mxfp8_ref import decode_mxfp8_rows   # (it imports this module)
        return decode_mxfp8_rows(raw)
    raise ValueError(f"unknown kv_dtype {kv_dtype!r}")


def query_rows(q_nope: np.ndarray, q_rope: np.ndarray, b: int, i: int) -> np.ndarray:
    """Exact float64 query rows [H, 576] = [q_nope_absorbed | q_rope] of (b, i)."""
    return np.concatenate([bf16_bits_to_f64(q_nope[b, i]),
                           bf16_bits_to_f64(q_rope[b, i])], axis=-1)


def scores(q: np.ndarray, keys: np.ndarray, softmax_scale: float) -> np.ndarray:
    """s[h, p] = scale * (q[h] . k[p]) in float64; scale is the float32 value."""
    scale = np.float64(np.float32(softmax_scale))
    return scale * (q @ keys.T)


def softmax_reduce(s: np.ndarray, values: np.ndarray):
    """(O, LSE, P) of score rows s [H, n] over values [n, 512].

    n == 0 gives O = 0, LSE = -inf and an empty P.
    """
    rows = s.shape[0]
    if s.shape[1] == 0:
        return (np.zeros((rows, values.shape[1])),
                np.full(rows, -np.inf), np.zeros((rows, 0)))
    m = s.max(axis=1)
    z = np.exp(s - m[:, None]).sum(axis=1)
    lse = m + np.log(z)
    p = np.exp(s - lse[:, None])
    return p @ values, lse, p


def mla_decode_ref(q_nope, q_rope, pool, kv_scale, req_to_token, seq_lens,
                   q_len: int, softmax_scale: float, kv_dtype: str,
                   dcp_size: int = 1, dcp_rank: int = 0,
                   p_range=None, return_probs: bool = False):
    """Absorbed MLA decode over one (possibly DCP-sharded) paged latent pool.

    Arguments are the stored bit patterns, as numpy arrays:
      q_nope        uint16 [B, q, H, 512]  BF16 bits of the absorbed no-RoPE query
      q_rope        uint16 [B, q, H, 64]   BF16 bits of the RoPE query
      pool          uint16 [S, 576] (BF16 bits), uint8 [S, 576] (e4m3fn codes),
                    uint8 [S, 336] (FP4 rows, format in fp4_ref) or uint8
                    [S, 608] (MXFP8 rows, format in mxfp8_ref)
      kv_scale      float32 [S] for FP8, ignored otherwise
      req_to_token  int32 [B, >= local length]; column j is local index j
      seq_lens      int [B]; global lengths L_b including the q drafts
    p_range=(lo, hi) keeps only global positions lo <= p < hi (a partial).
    Returns O float64 [B, q, H, 512] and LSE float64 [B, q, H]
    (plus, if return_probs, a dict {(b, i): (positions, P[H, n])}).
    """
    B, q, H, _ = q_nope.shape
    assert q == q_len
    out = np.zeros((B, q, H, D_V), dtype=np.float64)
    lse = np.full((B, q, H), -np.inf, dtype=np.float64)
    probs = {}
    for b in range(B):
        L = int(seq_lens[b])
        for i in range(q):
            p = visible_positions(L, q, i, dcp_size, dcp_rank)
            if p_range is not None:
                p = p[(p >= p_range[0]) & (p < p_range[1])]
            slots = gather_slots(req_to_token, b, local_index(p, dcp_size, dcp_rank))
            keys = dequant_rows(pool, kv_scale, slots, kv_dtype)
            s = scores(query_rows(q_nope, q_rope, b, i), keys, softmax_scale)
            o_bi, lse_bi, p_bi = softmax_reduce(s, keys[:, :D_V])
            out[b, i] = o_bi
            lse[b, i] = lse_bi
            if return_probs:
                probs[(b, i)] = (p, p_bi)
    if return_probs:
        return out, lse, probs
    return out, lse


def lse_combine_ref(parts_o, parts_lse):
    """Merge parts (O_j, LSE_j) along axis 0 by log-sum-exp, in float64.

    parts_o: [P, ..., D], parts_lse: [P, ...].  Rows whose parts all have
    LSE = -inf come out as (0, -inf).
    """
    o = np.asarray(parts_o, dtype=np.float64)
    l = np.asarray(parts_lse, dtype=np.float64)
    m_star = l.max(axis=0)
    finite = np.isfinite(m_star)
    shift = np.where(finite, m_star, 0.0)
    w = np.where(np.isfinite(l), np.exp(l - shift[None]), 0.0)
    wsum = w.sum(axis=0)
    safe = np.where(finite, wsum, 1.0)
    lse = np.where(finite, shift + np.log(safe), -np.inf)
    out = (w[..., None] * o).sum(axis=0) / safe[..., None]
    out = np.where(finite[..., None], out, 0.0)
    return out, lse
