"""THE ORACLE's sampler -- test infrastructure only (see the package docstring).

One draw of the decode step's sampling exit, in fp64, with its stages in the sequence the "decode-ops" page
sets out ("Method"): temperature first, then the k-largest cut, then the probability-mass cut, then a
caller-supplied uniform chooses the token from what is left by its cumulative distribution; candidates rank by
logit, equal logits by the lower index first. The page gives the sequence and the tie rule; the
top-p cut and the inverse CDF are taken at their plainest readings (the HuggingFace warper rule the page
names as its reference):
  - top-p keeps a survivor while the probability mass of the survivors before it is below p, so the first
    survivor is always kept and the kept set is the shortest prefix whose mass reaches p;
  - the token is the first kept survivor whose cumulative renormalised probability exceeds u.
Temperature 0 is the greedy exit (the lowest index holding the maximum logit), as in the "forward pass"
page's generate loop. A NaN logit counts as -inf; when no survivor has finite mass the first survivor is
returned.
"""
from __future__ import annotations

import numpy as np


def sample_detail(logits, temperature: float, top_k: int, top_p: float, u: float) -> dict:
    """token, the survivor order, the number kept by top-p, and the cumulative probabilities over the kept."""
    z = np.asarray(logits, dtype=np.float64).copy()
    z[np.isnan(z)] = -np.inf
    n = z.size
    if temperature == 0.0:
        order = np.lexsort((np.arange(n), -z))
        return {"token": int(order[0]), "order": order[:1], "kept": 1, "cdf": np.array([1.0])}
    z = z / temperature
    order = np.lexsort((np.arange(n), -z))            # descending value, ties to the lower index
    k = n if top_k <= 0 or top_k >= n else top_k
    surv = order[:k]
    m = z[surv[0]]
    if not np.isfinite(m):
        return {"token": int(surv[0]), "order": surv, "kept": 1, "cdf": np.array([1.0])}
    w = np.exp(z[surv] - m)                           # -inf survivors weigh exactly 0
    prob = w / w.sum()
    before = np.concatenate(([0.0], np.cumsum(prob)[:-1]))
    kept = int(np.count_nonzero(before < top_p))
    q = w[:kept] / w[:kept].sum()
    cdf = np.cumsum(q)
    over = np.nonzero(cdf > u)[0]
    j = int(over[0]) if over.size else int(np.nonzero(q > 0)[0][-1])   # u past the rounded total: last with mass
    return {"token": int(surv[j]), "order": surv, "kept": kept, "cdf": cdf}


def sample(logits, temperature: float, top_k: int, top_p: float, u: float) -> int:
    return sample_detail(logits, temperature, top_k, top_p, u)["token"]
