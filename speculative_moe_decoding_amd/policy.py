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


class OnlineDepth:
    """Run-time choice of the draft depth, from what the decode itself shows.

    Acceptance: a step at depth k that accepts n drafts says that drafts 1..n
    were accepted and, if n < k, that draft n+1 was not.  Per draft position j
    the controller keeps those counts (a Beta(1, 1) prior) and estimates p_j,
    the chance that draft j is accepted once drafts 1..j-1 were; positions it
    has not seen take the last seen one's estimate.  Expected tokens per step
    at depth k: tau(k) = 1 + sum_{i<=k} prod_{j<=i} p_j (with p_j = alpha for
    every j this is the pages' geometric acceptance; the L4 table's tau = 1 +
    k alpha is its per-slot mean).  Cost: the measured time per step at each
    depth (exponential average); depths not yet timed take the line through
    the timed ones (t(k) = t_verify + k t_pass, the draft passes adding one
    pass each), or are timed first.  The choice maximises tau(k) / t(k); every
    `explore_every`-th call re-times the runner-up, so the costs stay current.
    Host policy only: it picks the K passed to the decode calls."""

    def __init__(self, k_max: int, k_min: int = 1, ema: float = 0.3, explore_every: int = 6):
        self.k_min, self.k_max, self.ema, self.explore_every = k_min, k_max, ema, explore_every
        self.acc = [1.0] * (k_max + 1)     # Beta pseudo-counts per draft position (index 1..k_max)
        self.rej = [1.0] * (k_max + 1)
        self.ms: Dict[int, float] = {}
        self.calls = 0

    def observe(self, k: int, accepted, ms_per_step: float) -> None:
        for n in accepted:
            n = int(n)
            for j in range(1, n + 1):
                self.acc[j] += 1.0
            if n < k:
                self.rej[n + 1] += 1.0
        old = self.ms.get(k)
        self.ms[k] = ms_per_step if old is None else (1 - self.ema) * old + self.ema * ms_per_step

    def p(self, j: int) -> float:
        return self.acc[j] / (self.acc[j] + self.rej[j])

    def tau(self, k: int) -> float:
        t, run = 1.0, 1.0
        for j in range(1, k + 1):
            run *= self.p(j)
            t += run
        return t

    def cost(self, k: int) -> float:
        if k in self.ms:
            return self.ms[k]
        ks = sorted(self.ms)
        if len(ks) >= 2:
            (k0, t0), (k1, t1) = (ks[0], self.ms[ks[0]]), (ks[-1], self.ms[ks[-1]])
            slope = (t1 - t0) / (k1 - k0)
            return t0 + (k - k0) * slope
        return float("nan")

    def choose(self) -> int:
        self.calls += 1
        untimed = [k for k in range(self.k_min, self.k_max + 1) if k not in self.ms]
        if len(self.ms) < 2 and untimed:          # time the two ends first, then interpolate
            return self.k_max if self.k_max in untimed else untimed[0]
        rates = sorted(((self.tau(k) / self.cost(k), -k) for k in range(self.k_min, self.k_max + 1)),
                       reverse=True)
        best = -rates[0][1]
        if self.explore_every and self.calls % self.explore_every == 0 and len(rates) > 1:
            return -rates[1][1]
        return best
