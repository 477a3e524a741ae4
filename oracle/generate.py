"""Plain CPU oracle for next-token choice and the generation loop.

TEST INFRASTRUCTURE ONLY (see oracle/smol.py): nothing on the product path may
import, call or run this module.

Sources: the generate methods of *Sualeh77 model.py* (section "7. Top-level
SmolLM2-135M Model Architecture": cached generation, temperature division, top-k,
top-p, multinomial draw, stop when every sequence emits the end id) and of
*abi96062 model.py* (SmolLM2Model.generate: greedy when the temperature is 0, top-k
clamped to the vocabulary, top-p applied only below 1, full recompute per step).

Readings taken where the pages leave a step open (each pinned in
tests/test_oracle_pins.py):

* greedy picks the lowest index among equal maxima (the behaviour of argmax);
* top-k compares logits: a token stays when its logit is >= the k-th largest, so
  ties at the threshold all stay;
* top-p orders tokens by logit, descending, equal logits by ascending index (a
  stable order; the pages' sort does not fix one), and keeps every token up to and
  including the first at which the cumulative probability exceeds p;
* the multinomial draw is the inverse CDF in vocabulary order with a uniform u
  supplied by the caller: the first index whose cumulative probability exceeds u.

Everything is float64. parity pinned: see tests/test_oracle_pins.py.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import numpy as np

from .smol import model_prefill


@dataclass
class Choice:
    token: int
    kept: Optional[np.ndarray]  # bool mask of the tokens the filters keep (None: greedy)
    p_margin: float  # distance of the top-p cut from flipping (inf when top-p is off)
    u_margin: float  # distance of u from the CDF steps around the chosen token (inf: greedy)


def top_k_keep(logits: np.ndarray, k: int) -> np.ndarray:
    """Tokens whose logit is >= the k-th largest (all tokens when k is 0 or >= V)."""
    V = logits.shape[0]
    if k <= 0 or k >= V:
        return np.ones(V, dtype=bool)
    kth = np.sort(logits)[V - k]
    return logits >= kth


def top_p_keep(logits: np.ndarray, weights: np.ndarray, keep: np.ndarray, p: float):
    """Nucleus filter over the kept tokens: (new keep mask, margin of the cut)."""
    if p >= 1.0:
        return keep, np.inf
    idx = np.nonzero(keep)[0]
    order = idx[np.lexsort((idx, -logits[idx]))]  # logit descending, then index ascending
    prob = weights[order] / weights[order].sum()
    cum = np.cumsum(prob)
    over = np.nonzero(cum > p)[0]
    s = int(over[0]) if over.size else len(order) - 1  # last kept position
    new = np.zeros_like(keep)
    new[order[: s + 1]] = True
    before = cum[s - 1] if s > 0 else 0.0
    margin = min(abs(cum[s] - p) if over.size else np.inf, abs(p - before) if s > 0 else np.inf)
    return new, margin


def next_token(logits, temperature: float, top_k: int = 0, top_p: float = 1.0, u: float = 0.0) -> Choice:
    """The next token from one row of logits (see the module docstring)."""
    l = np.asarray(logits, dtype=np.float64)
    if np.isnan(l).any():
        return Choice(-1, None, np.inf, np.inf)
    if temperature == 0:
        return Choice(int(np.argmax(l)), None, np.inf, np.inf)
    if not np.isfinite(l.max()):
        return Choice(-1, None, np.inf, np.inf)
    keep = top_k_keep(l, top_k)
    z = l / temperature
    weights = np.where(keep, np.exp(z - z.max()), 0.0)
    keep, p_margin = top_p_keep(l, weights, keep, top_p)
    weights = np.where(keep, weights, 0.0)
    cdf = np.cumsum(weights / weights.sum())
    j = int(np.searchsorted(cdf, u, side="right"))  # first index with cdf > u
    if j >= l.shape[0]:  # u at or above the total after rounding: the last kept token
        j = int(np.nonzero(keep)[0][-1])
    prev = cdf[j - 1] if j > 0 else 0.0
    u_margin = min(abs(cdf[j] - u), abs(u - prev))
    return Choice(j, keep, p_margin, u_margin)


def greedy_generate(prompt: np.ndarray, max_new: int, mw, cfg):
    """Greedy tokens [max_new, B] by full recompute (every step runs the whole
    sequence again, as abi96062 model.py's generate does), and the gap between the
    two largest logits at each step ([max_new, B]) to judge near-ties."""
    ids = np.asarray(prompt, dtype=np.int64)
    B = ids.shape[0]
    out = np.zeros((max_new, B), dtype=np.int64)
    gaps = np.zeros((max_new, B))
    for j in range(max_new):
        T = ids.shape[1]
        row = model_prefill(ids, mw, cfg, logit_rows=[b * T + T - 1 for b in range(B)])  # [B, V]
        for b in range(B):
            c = next_token(row[b], 0.0)
            out[j, b] = c.token
            top2 = np.sort(row[b])[-2:]
            gaps[j, b] = top2[1] - top2[0]
        ids = np.concatenate([ids, out[j][:, None]], axis=1)
    return out, gaps
