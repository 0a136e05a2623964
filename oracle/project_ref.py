"""Plain float64 oracle of the step after absorbed decode: the w_vc up-projection.

TEST INFRASTRUCTURE ONLY (see the package docstring for who may import it).

Absorbed decode attends in the 512-wide latent space: the values are c_kv,
and kv_b_proj's value half, w_vc, is applied after attention (page "Kimi K3
decode: DP16 vs DP2 x DCP8", section on the weight AllGather: kv_b_proj is
absorbed into w_kc / w_vc).  Under DCP the shards' partial (O, LSE) are first
merged by log-sum-exp (same page, section "MLA": dcp_lse_combine), and the
projection can run on the merged rows directly, so the merged latent O never
has to be stored:

    O[t, h]     = lse_combine over the parts (as lse_combine_ref)
    out[t, h, n] = sum_k O[t, h, k] * w_vc[h, k, n]        (k < 512, n < 128)

Reading where the pages are silent: w_vc maps the 512-wide latent to a
128-wide value head (v_head_dim = 128, the width w_kc maps from on the
query side).  A row whose parts are all empty (LSE = -inf) gives out = 0.
"""

from __future__ import annotations

import numpy as np

from .mla_ref import bf16_bits_to_f64, lse_combine_ref

D_V_HEAD = 128


def vc_project_ref(o, w_vc_t_bits) -> np.ndarray:
    """out[t, h, n] = sum_k o[t, h, k] * w_vc[h, k, n] in float64.

    o: [T, H, 512] float values; w_vc_t_bits: BF16 bits [H, 128, 512], each
    head's w_vc transposed (element (h, n, k) = w_vc[h, k, n]).
    """
    o = np.asarray(o, dtype=np.float64)
    wt = bf16_bits_to_f64(w_vc_t_bits)                   # [H, 128, 512]
    out = np.empty(o.shape[:2] + (wt.shape[1],), dtype=np.float64)
    for h in range(o.shape[1]):
        out[:, h, :] = o[:, h, :] @ wt[h].T
    return out


def lse_combine_project_ref(parts_o, parts_lse, w_vc_t_bits):
    """(out [T, H, 128], lse [T, H]) of parts [P, T, H, 512] / [P, T, H]."""
    o, lse = lse_combine_ref(parts_o, parts_lse)
    return vc_project_ref(o, w_vc_t_bits), lse
