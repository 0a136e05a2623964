"""Wave-quantisation arithmetic: the prior-art split rule and our plan's balance.

The page "Kimi K3 decode: DP16 vs DP2 x DCP8" (section "MLA") analyses a
decode kernel whose KV split is min(SMs // B // (2 q_len), 32) on a grid of
(2, B q_len, split) CTAs, one full-context scan per CTA.  With 148 SMs and 16
requests that is 160 CTAs: one full wave plus 12 CTAs in a second wave, so
the layer takes two wave times.  These helpers reproduce that arithmetic and
compute the same quantity for a plan made by mla_decode_plan.
"""

from __future__ import annotations

import math

import numpy as np


def prior_art_split(batch: int, q_len: int, sms: int, cap: int = 32) -> int:
    """The page's rule, floored at 1 (it prints split = 1 for B >= 8)."""
    return max(1, min(sms // batch // (q_len * 2), cap))


def prior_art_ctas(batch: int, q_len: int, sms: int) -> int:
    return 2 * batch * q_len * prior_art_split(batch, q_len, sms)


def waves(ctas: int, slots: int) -> int:
    """Whole waves needed to run `ctas` equal CTAs on `slots` concurrent slots."""
    return math.ceil(ctas / slots)


def prior_art_time(batch: int, q_len: int, sms: int, t_full_scan: float) -> float:
    """Modeled layer time: whole waves x the time one CTA needs for its KV share."""
    split = prior_art_split(batch, q_len, sms)
    return waves(prior_art_ctas(batch, q_len, sms), sms) * t_full_scan / split


def wave_rounded_time(batch: int, q_len: int, sms: int, t_full_scan: float) -> float:
    """The page's estimate if the split filled whole waves: time proportional to CTAs."""
    return t_full_scan * prior_art_ctas(batch, q_len, sms) / sms


def plan_wg_costs(plan, overhead_tokens: int = 128) -> np.ndarray:
    """Per-workgroup work of a plan in token-equivalents (tokens + per-unit overhead)."""
    wgb = plan.wg_begin()
    u = plan.units()
    cost = np.zeros(len(wgb) - 1)
    for x in range(len(wgb) - 1):
        seg = u[wgb[x]:wgb[x + 1]]
        cost[x] = float((seg[:, 3] - seg[:, 2]).sum() + overhead_tokens * len(seg))
    return cost


def plan_efficiency(plan, slots: int, overhead_tokens: int = 128) -> float:
    """Ideal / modeled makespan: total work spread over all slots vs the busiest slot."""
    cost = plan_wg_costs(plan, overhead_tokens)
    if cost.max() <= 0:
        return 1.0
    # Workgroups beyond `slots` would queue behind the first wave.
    per_slot = np.zeros(slots)
    for x, c in enumerate(cost):
        per_slot[x % slots] += c
    return float(cost.sum() / slots / per_slot.max())
