"""Oracle for the projections on either side of the exchanges.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Pinned by
``tests/test_oracle_proj.py``.

What the pages fix ([ALST] "Mecanismul de funcționare Ulysses", steps 2 and
6; [HFSUM] "Ulysses 序列平行化的原理"): each rank computes the query, key and
value projections of its own sequence shard before the first exchange, and
the output projection of its own shard after the second.  Readings taken
where they are silent: a projection is x @ W^T with W laid out
``[out features][in features]``; the fused QKV weight stacks the Hq query
heads, then the Hkv key heads, then the Hkv value heads, D features each;
the attention output of a token is its Hq heads concatenated in head order.

  qkv_proj_seq2head:  Y = x @ W^T per shard, split into Q, K, V, each run
                      through the first exchange (``exchange.seq2head``)
  head2seq_out_proj:  O head-sharded -> second exchange -> heads
                      concatenated per token -> @ W_o^T

Float64 throughout (NumPy matmul as the contraction step).
"""
from __future__ import annotations

import numpy as np

from .exchange import seq2head, head2seq


def qkv_proj_seq2head(x_seq, w, Hq: int, Hkv: int, D: int):
    """``x_seq`` ``[P][B][nl][hidden]``, ``w`` ``[(Hq + 2 Hkv) D][hidden]`` ->
    head-sharded ``(q [P][B][n][Hq/P][D], k, v [P][B][n][Hkv/P][D])``."""
    x = np.asarray(x_seq, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    P, B, nl, _ = x.shape
    if w.shape[0] != (Hq + 2 * Hkv) * D:
        raise ValueError("w must have (Hq + 2 Hkv) * D rows")
    y = x @ w.T                                                # [P][B][nl][(Hq + 2 Hkv) D]
    q = y[..., :Hq * D].reshape(P, B, nl, Hq, D)
    k = y[..., Hq * D:(Hq + Hkv) * D].reshape(P, B, nl, Hkv, D)
    v = y[..., (Hq + Hkv) * D:].reshape(P, B, nl, Hkv, D)
    return seq2head(q), seq2head(k), seq2head(v)


def head2seq_out_proj(o_heads, w_o):
    """``o_heads`` ``[P][B][n][Hq/P][D]`` (the attention output, head-sharded),
    ``w_o`` ``[hidden][Hq D]`` -> ``y`` ``[P][B][n/P][hidden]``."""
    o = head2seq(np.asarray(o_heads, dtype=np.float64))     # [P][B][nl][Hq][D]
    P, B, nl, Hq, D = o.shape
    return o.reshape(P, B, nl, Hq * D) @ np.asarray(w_o, dtype=np.float64).T
