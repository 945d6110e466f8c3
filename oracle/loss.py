"""Oracle for the loss aggregation over sequence shards.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Pinned by
``tests/test_oracle_rope_loss.py``.

What the pages fix ([ALST] "Integrarea cu Accelerate"): each rank computes
the loss on its part of the sequence, and the per-rank losses must be
combined weighted by each rank's number of valid tokens, padding tokens and
masked prompt tokens excluded; [ALST] "Cele mai bune practici și
recomandări", item 6, adds that balanced valid tokens per rank help this
aggregation.  The reading taken: the aggregated loss is the mean over every
valid token of the whole sequence,

  sum_r   = sum of token losses over rank r's valid tokens
  count_r = number of rank r's valid tokens
  loss    = (sum_r sum_r) / (sum_r count_r)

which is not the mean of the per-rank means when the counts differ.  With no
valid token at all the mean is undefined and the result is NaN.  Sums use
math.fsum (correctly rounded).
"""
from __future__ import annotations

import math

import numpy as np


def aggregate(token_loss, valid=None):
    """``token_loss`` ``[P][B][n/P]``, ``valid`` same shape (nonzero = counted)
    or None.  Returns ``(rank_sum [P], rank_count [P], loss)``."""
    tl = np.asarray(token_loss, dtype=np.float64)
    P = tl.shape[0]
    sums = np.zeros(P)
    counts = np.zeros(P, dtype=np.int64)
    for r in range(P):
        vals = tl[r].ravel()
        if valid is not None:
            vals = vals[np.asarray(valid[r]).ravel() != 0]
        sums[r] = math.fsum(vals.tolist())
        counts[r] = vals.size
    total = int(counts.sum())
    loss = math.fsum(sums.tolist()) / total if total > 0 else float("nan")
    return sums, counts, loss
