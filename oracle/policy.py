"""Block-size policy: the oracle's reading of how to pick the next cycle's block size.

TEST INFRASTRUCTURE (see ``oracle/dflash.py``).  The pages say only that a drafter
trained on 16-token blocks also drafts smaller blocks at inference ("DFlash"
technical summary, §4 ablations); which size to use per cycle is left open.  The
plainest reading that the rest supports: acceptance is a run of agreeing drafts
(summary §1, greedy verification), so take the per-position acceptance model —
every draft position is accepted with the same probability p once the ones before
it were — and pick the size that commits the most tokens per unit of time.

* distribution of the accept length tau at block size g:
      P(tau = t) = p^(t-1) (1 - p)  for 1 <= t < g,   P(tau = g) = p^(g-1)
* expected tokens per cycle E(g) = sum_t t P(tau = t) = (1 - p^g) / (1 - p)  (g when p = 1)
* estimate of p from recent cycles (t_i, g_i): maximum likelihood of the product of
  P(tau = t_i) over the cycles, with a Beta prior of weight w centred at p0 as
  pseudo-counts: p = (A + w p0) / (A + R + w), A = sum (t_i - 1), R = #{t_i < g_i}
* choice: argmax over the candidate sizes of E(g) / cost(g), ties to the smaller g.
"""
from __future__ import annotations

from typing import Dict, Sequence, Tuple


def tau_distribution(p: float, g: int) -> Dict[int, float]:
    """P(tau = t) for t = 1..g under the per-position acceptance model."""
    dist = {t: p ** (t - 1) * (1.0 - p) for t in range(1, g)}
    dist[g] = p ** (g - 1)
    return dist


def expected_tokens(p: float, g: int) -> float:
    """E(g), closed form of the geometric sum."""
    if p >= 1.0:
        return float(g)
    return (1.0 - p ** g) / (1.0 - p)


def estimate_accept(tau: Sequence[int], gamma_used: Sequence[int], prior_p: float,
                    prior_weight: float) -> float:
    a = sum(t - 1 for t in tau)
    r = sum(1 for t, g in zip(tau, gamma_used) if t < g)
    den = a + r + prior_weight
    return (a + prior_weight * prior_p) / den if den > 0 else prior_p


def choose_gamma(tau: Sequence[int], gamma_used: Sequence[int], cost_us: Sequence[float], gamma_min: int,
                 gamma_max: int, prior_p: float, prior_weight: float) -> Tuple[int, float]:
    p = estimate_accept(tau, gamma_used, prior_p, prior_weight)
    cands = [g for g in range(gamma_min, gamma_max + 1) if cost_us[g] > 0]
    best = max(cands, key=lambda g: (expected_tokens(p, g) / cost_us[g], -g))
    return best, p
