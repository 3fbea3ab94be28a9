"""Draft-depth choice (adaptive K) from measured step costs.

With per-slot acceptance a_K measured at depth K (the fraction of the K drafts
accepted), one step commits tau(K) = 1 + K a_K tokens on average -- the L4
table's identity in the jina-ocr-v1 blog ("Results") -- and costs t(K), the
draft passes plus the verify.  The best depth maximises tau(K) / t(K).  Host
policy only: it picks the K passed to the decode calls.
"""
from __future__ import annotations

from typing import Dict, Mapping


def expected_tokens(k: int, alpha: float) -> float:
    """Tokens committed per step at depth k with mean acceptance alpha (k = 0: 1)."""
    return 1.0 + k * alpha if k > 0 else 1.0


def choose_k(step_ms: Mapping[int, float], alpha: Mapping[int, float]) -> int:
    """The depth with the highest tokens per unit time; ties go to the smaller K.
    step_ms[k]: measured cost of one step at depth k; alpha[k]: acceptance at k
    (ignored for k = 0)."""
    best, best_rate = None, -1.0
    for k in sorted(step_ms):
        rate = expected_tokens(k, alpha.get(k, 0.0)) / step_ms[k]
        if rate > best_rate * (1 + 1e-12):
            best, best_rate = k, rate
    if best is None:
        raise ValueError("no step costs given")
    return best


def linear_step_costs(t_verify_ms: float, t_draft_pass_ms: float, k_max: int) -> Dict[int, float]:
    """Step cost model t(K) = t_verify + K t_draft_pass (the draft block runs K
    times; the verify pass grows little with K at batch 1)."""
    return {k: t_verify_ms + k * t_draft_pass_ms for k in range(k_max + 1)}
