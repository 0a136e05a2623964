"""50-digit brute force of absorbed MLA decode, for tiny inputs only.

Independent of the oracle: BF16 values are decoded with ``struct`` and e4m3fn
codes with torch's float8 type, the visible set is an explicit loop over all
positions, and every sum, exp and log is taken in mpmath at 50 digits.
"""

import struct

import mpmath
import numpy as np
import torch

mpmath.mp.dps = 50

_FP8 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()


def _bf16(bits) -> float:
    return struct.unpack("<f", struct.pack("<I", (int(bits) & 0xFFFF) << 16))[0]


def brute_decode(nb: dict, q_len: int, softmax_scale: float, kv_dtype: str,
                 dcp_size: int = 1, dcp_rank: int = 0, p_range=None):
    """Returns (O [B, q, H, 512], LSE [B, q, H]) as float64 arrays."""
    qn, qr = nb["q_nope"], nb["q_rope"]
    pool, table, lens = nb["pool"], nb["req_to_token"], nb["seq_lens"]
    scale_f32 = float(np.float32(softmax_scale))
    B, q, H, _ = qn.shape
    out = np.zeros((B, q, H, 512))
    lse = np.full((B, q, H), -np.inf)
    for b in range(B):
        L = int(lens[b])
        for i in range(q):
            vis = []
            for p in range(L):
                if p > L - q_len + i or p % dcp_size != dcp_rank:
                    continue
                if p_range is not None and not (p_range[0] <= p < p_range[1]):
                    continue
                vis.append(p)
            keys = []
            for p in vis:
                slot = int(table[b, (p - dcp_rank) // dcp_size])
                if kv_dtype == "bf16":
                    k = [mpmath.mpf(_bf16(x)) for x in pool[slot]]
                else:
                    sc = mpmath.mpf(float(nb["kv_scale"][slot]))
                    k = [mpmath.mpf(float(_FP8[int(x)])) * sc for x in pool[slot]]
                keys.append(k)
            for h in range(H):
                if not vis:
                    continue
                qv = [mpmath.mpf(_bf16(x)) for x in qn[b, i, h]] + \
                     [mpmath.mpf(_bf16(x)) for x in qr[b, i, h]]
                s = [mpmath.mpf(scale_f32) * mpmath.fsum(a * c for a, c in zip(qv, k))
                     for k in keys]
                z = mpmath.fsum(mpmath.exp(x) for x in s)
                l = mpmath.log(z)
                lse[b, i, h] = float(l)
                w = [mpmath.exp(x - l) for x in s]
                for d in range(512):
                    out[b, i, h, d] = float(mpmath.fsum(wt * k[d] for wt, k in zip(w, keys)))
    return out, lse
