"""Oracle for exact causal grouped-query softmax attention, forward and backward.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Pinned by
``tests/test_oracle_attention.py`` against brute force in pure Python,
hand-derived worked examples (``tests/golden/``), closed forms, finite
differences and a library routine on the CPU.

What is computed
----------------
After the first exchange each rank runs ordinary scaled-dot-product
attention over the full sequence for its heads ([ALST] section
"Mecanismul de funcționare Ulysses", step 4; [HFSUM] section
"Ulysses 序列平行化的原理").  Heads are independent ([ALST], same section,
closing paragraph), so the result is exactly that of unsharded attention.
The pages give no formula, so the oracle is the textbook definition, written
out per (batch b, query head h, query row t):

  allowed keys   K_t = { u : (u <= t if causal) and valid[b][u] }
  scores         s_u = scale * sum_c q[t][c] * k[u][c]           (u in K_t)
  softmax        m = max s_u,  w_u = exp(s_u - m),  L = sum w_u
  output         O[t] = sum_u (w_u / L) * v[u]
  logsumexp      LSE[t] = m + ln L                                (natural log)

computed in two passes over a materialised fp64 score row (no online
rescaling).  A row with no allowed key gets O = 0 and LSE = -inf.

The backward is the gradient of sum(O * dO) with respect to q, k, v,
evaluated with the oracle's own O and LSE:

  P[t][u]  = exp(s_tu - LSE[t]) on K_t, else 0
  dV[u]   += sum_t P[t][u] dO[t]
  dP[t][u] = dO[t] . v[u]
  Dl[t]    = dO[t] . O[t]
  dS[t][u] = P[t][u] * (dP[t][u] - Dl[t])
  dQ[t]    = scale * sum_u dS[t][u] k[u]
  dK[u]   += scale * sum_t dS[t][u] q[t]

Readings where the pages are silent (they do not mention grouped-query
attention, the mask or the backward at all): query head h reads KV head
floor(h / (Hq/Hkv)); the causal mask is on global positions with the
diagonal included; padding keys are excluded from every softmax, padding
query rows are computed like any other row.

Packed documents ([ALST] section "Integrarea cu Transformers Trainer și TRL
SFTTrainer" names the trainer's switch for variable sequence lengths, not
the mask it implies).  The reading taken: a packed sequence holds several
documents back to back and a token attends only to earlier tokens of its
own document.  The documents are given per token by ``doc_start[b][t]``,
the position of the first token of t's document (pad tokens after a
document belong to it), and the allowed set above gains one condition:

  K_t = { u : doc_start[b][t] <= u, (u <= t if causal) and valid[b][u] }

Every formula above is unchanged.  Nothing here assumes the documents are
contiguous or the array monotone: the condition is applied as written.

Layouts: q, o ``[B][n][Hq][D]``; k, v ``[B][n][Hkv][D]``; lse ``[B][Hq][n]``;
key_valid ``[B][n]`` (nonzero = valid) or None; doc_start ``[B][n]`` integer
or None.  All arithmetic is float64.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

try:  # keep one BLAS thread per worker so the pool scales and results are deterministic
    from threadpoolctl import threadpool_limits
except Exception:  # pragma: no cover
    threadpool_limits = None

DEFAULT_BLOCK = 256


def kv_head_of(h: int, Hq: int, Hkv: int) -> int:
    """KV head read by query head h: contiguous groups of Hq/Hkv query heads."""
    if Hq % Hkv != 0:
        raise ValueError(f"Hq={Hq} is not a multiple of Hkv={Hkv}")
    return h // (Hq // Hkv)


def allowed_mask(rows: np.ndarray, n_keys: int, causal: bool, valid_b, doc_b=None) -> np.ndarray:
    """Boolean [len(rows)][n_keys]: key u is allowed for query row t."""
    keys = np.arange(n_keys)
    if causal:
        m = keys[None, :] <= rows[:, None]
    else:
        m = np.ones((rows.size, n_keys), dtype=bool)
    if valid_b is not None:
        m = m & (np.asarray(valid_b[:n_keys]) != 0)[None, :]
    if doc_b is not None:
        m = m & (keys[None, :] >= np.asarray(doc_b, dtype=np.int64)[rows][:, None])
    return m


def _doc(doc_start, b):
    return None if doc_start is None else doc_start[b]


def _workers(workers):
    """Worker threads: every core of the process's affinity set by default
    (NumPy's matrix and elementwise kernels release the interpreter lock,
    and each worker runs one BLAS thread)."""
    if workers is not None:
        return max(1, int(workers))
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except Exception:  # pragma: no cover
        return 1


def _run(tasks, fn, workers):
    w = _workers(workers)
    ctx = threadpool_limits(limits=1) if threadpool_limits is not None else None
    try:
        if ctx is not None:
            ctx.__enter__()
        if w == 1 or len(tasks) <= 1:
            return [fn(t) for t in tasks]
        with ThreadPoolExecutor(max_workers=w) as ex:
            return list(ex.map(fn, tasks))
    finally:
        if ctx is not None:
            ctx.__exit__(None, None, None)


def _check(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B][n][H][D]")
    B, n, Hq, D = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[1] != n or k.shape[3] != D:
        raise ValueError("k and v must be [B][n][Hkv][D] matching q")
    Hkv = k.shape[2]
    if Hq % Hkv != 0:
        raise ValueError(f"Hq={Hq} is not a multiple of Hkv={Hkv}")
    return B, n, Hq, Hkv, D


def _head(x, b, h):
    """Contiguous float64 copy of one head's [n][D] slice."""
    return np.ascontiguousarray(x[b, :, h, :], dtype=np.float64)


def _softmax_rows(S: np.ndarray, allow: np.ndarray):
    """Two-pass softmax statistics of score rows under a mask.

    Returns (weights w = exp(s - m) masked to 0, row max m, row sum L)."""
    Sm = np.where(allow, S, -np.inf)
    m = Sm.max(axis=1)
    m_safe = np.where(np.isfinite(m), m, 0.0)
    w = np.where(allow, np.exp(Sm - m_safe[:, None]), 0.0)
    L = w.sum(axis=1)
    return w, m, L


def attn_fwd(q, k, v, scale: float, causal: bool = True, key_valid=None, rows=None,
             block: int = DEFAULT_BLOCK, workers=None, doc_start=None):
    """Forward attention.  Returns ``(O, LSE)`` in float64.

    ``rows``: optional sorted query-row indices; then ``O`` is
    ``[B][len(rows)][Hq][D]`` and ``LSE`` is ``[B][Hq][len(rows)]``.
    """
    B, n, Hq, Hkv, D = _check(q, k, v)
    rows = np.arange(n, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    R = rows.size
    O = np.zeros((B, R, Hq, D), dtype=np.float64)
    LSE = np.full((B, Hq, R), -np.inf, dtype=np.float64)

    tasks = [(b, h, r0) for b in range(B) for h in range(Hq) for r0 in range(0, R, block)]
    cache = {}

    def head_arrays(b, h):
        key = (b, h)
        if key not in cache:
            g = kv_head_of(h, Hq, Hkv)
            cache[key] = (_head(q, b, h), _head(k, b, g), _head(v, b, g))
        return cache[key]

    # build the per-head copies up front (serially) so the workers only read them
    for b in range(B):
        for h in range(Hq):
            head_arrays(b, h)

    def work(task):
        b, h, r0 = task
        qh, kh, vh = head_arrays(b, h)
        t = rows[r0:r0 + block]
        n_keys = int(t.max()) + 1 if causal else n
        allow = allowed_mask(t, n_keys, causal, None if key_valid is None else key_valid[b], _doc(doc_start, b))
        S = scale * (qh[t] @ kh[:n_keys].T)
        w, m, L = _softmax_rows(S, allow)
        with np.errstate(divide="ignore", invalid="ignore"):
            o = np.where(L[:, None] > 0, (w @ vh[:n_keys]) / L[:, None], 0.0)
            lse = np.where(L > 0, m + np.log(L), -np.inf)
        return task, o, lse

    for (b, h, r0), o, lse in _run(tasks, work, workers):
        O[b, r0:r0 + o.shape[0], h, :] = o
        LSE[b, h, r0:r0 + o.shape[0]] = lse
    return O, LSE


def attn_bwd(q, k, v, dout, scale: float, causal: bool = True, key_valid=None,
             block: int = DEFAULT_BLOCK, workers=None, doc_start=None):
    """Full backward.  Returns ``(dQ, dK, dV, O, LSE)`` in float64."""
    B, n, Hq, Hkv, D = _check(q, k, v)
    if dout.shape != q.shape:
        raise ValueError("dout must have q's shape")
    O, LSE = attn_fwd(q, k, v, scale, causal, key_valid, block=block, workers=workers, doc_start=doc_start)
    dQ = np.zeros((B, n, Hq, D), dtype=np.float64)
    dK = np.zeros((B, n, Hkv, D), dtype=np.float64)
    dV = np.zeros((B, n, Hkv, D), dtype=np.float64)

    tasks = [(b, h, r0) for b in range(B) for h in range(Hq) for r0 in range(0, n, block)]

    def work(task):
        b, h, r0 = task
        g = kv_head_of(h, Hq, Hkv)
        t = np.arange(r0, min(n, r0 + block))
        n_keys = int(t.max()) + 1 if causal else n
        qb = np.ascontiguousarray(q[b, t, h, :], dtype=np.float64)
        kb = np.ascontiguousarray(k[b, :n_keys, g, :], dtype=np.float64)
        vb = np.ascontiguousarray(v[b, :n_keys, g, :], dtype=np.float64)
        dob = np.ascontiguousarray(dout[b, t, h, :], dtype=np.float64)
        allow = allowed_mask(t, n_keys, causal, None if key_valid is None else key_valid[b], _doc(doc_start, b))
        S = scale * (qb @ kb.T)
        lse = LSE[b, h, t]
        lse_safe = np.where(np.isfinite(lse), lse, 0.0)
        Pm = np.where(allow, np.exp(np.where(allow, S, 0.0) - lse_safe[:, None]), 0.0)
        dv_part = Pm.T @ dob
        dP = dob @ vb.T
        Dl = np.sum(dob * O[b, t, h, :], axis=1)
        dS = Pm * (dP - Dl[:, None])
        dq = scale * (dS @ kb)
        dk_part = scale * (dS.T @ qb)
        return task, g, n_keys, dq, dk_part, dv_part

    results = _run(tasks, work, workers)
    # deterministic accumulation order: task order
    for (b, h, r0), g, n_keys, dq, dk_part, dv_part in results:
        dQ[b, r0:r0 + dq.shape[0], h, :] = dq
        dK[b, :n_keys, g, :] += dk_part
        dV[b, :n_keys, g, :] += dv_part
    return dQ, dK, dV, O, LSE


def attn_bwd_sampled(q, k, v, dout, scale: float, causal: bool = True, key_valid=None,
                     q_rows=None, k_rows=None, block: int = DEFAULT_BLOCK, workers=None, doc_start=None):
    """Backward at selected rows only.

    ``dQ`` at query rows ``q_rows`` (``[B][len(q_rows)][Hq][D]``) and ``dK``/``dV``
    at key rows ``k_rows`` (``[B][len(k_rows)][Hkv][D]``).  Key u's gradients
    need LSE and dO.O at every query row that may see u, so the forward is
    evaluated at rows [min(k_rows), n) (all rows when not causal).
    """
    B, n, Hq, Hkv, D = _check(q, k, v)
    g_size = Hq // Hkv
    q_rows = np.asarray([] if q_rows is None else q_rows, dtype=np.int64)
    k_rows = np.asarray([] if k_rows is None else k_rows, dtype=np.int64)
    dQ = np.zeros((B, q_rows.size, Hq, D))
    dK = np.zeros((B, k_rows.size, Hkv, D))
    dV = np.zeros((B, k_rows.size, Hkv, D))

    if q_rows.size:
        Oq, Lq = attn_fwd(q, k, v, scale, causal, key_valid, rows=q_rows, block=block, workers=workers,
                          doc_start=doc_start)
        tasks = [(b, h) for b in range(B) for h in range(Hq)]

        def work_q(task):
            b, h = task
            g = kv_head_of(h, Hq, Hkv)
            t = q_rows
            n_keys = int(t.max()) + 1 if causal else n
            kb = np.ascontiguousarray(k[b, :n_keys, g, :], dtype=np.float64)
            vb = np.ascontiguousarray(v[b, :n_keys, g, :], dtype=np.float64)
            qb = np.ascontiguousarray(q[b, t, h, :], dtype=np.float64)
            dob = np.ascontiguousarray(dout[b, t, h, :], dtype=np.float64)
            allow = allowed_mask(t, n_keys, causal, None if key_valid is None else key_valid[b], _doc(doc_start, b))
            S = scale * (qb @ kb.T)
            lse = Lq[b, h]
            lse_safe = np.where(np.isfinite(lse), lse, 0.0)
            Pm = np.where(allow, np.exp(np.where(allow, S, 0.0) - lse_safe[:, None]), 0.0)
            dP = dob @ vb.T
            Dl = np.sum(dob * Oq[b, :, h, :], axis=1)
            dS = Pm * (dP - Dl[:, None])
            return task, scale * (dS @ kb)

        for (b, h), dq in _run(tasks, work_q, workers):
            dQ[b, :, h, :] = dq

    if k_rows.size:
        r0 = int(k_rows.min()) if causal else 0
        t_all = np.arange(r0, n, dtype=np.int64)
        Ot, Lt = attn_fwd(q, k, v, scale, causal, key_valid, rows=t_all, block=block, workers=workers,
                          doc_start=doc_start)
        tasks = [(b, h) for b in range(B) for h in range(Hq)]

        def work_k(task):
            b, h = task
            g = kv_head_of(h, Hq, Hkv)
            qb = np.ascontiguousarray(q[b, t_all, h, :], dtype=np.float64)
            dob = np.ascontiguousarray(dout[b, t_all, h, :], dtype=np.float64)
            ku = np.ascontiguousarray(k[b, k_rows, g, :], dtype=np.float64)
            vu = np.ascontiguousarray(v[b, k_rows, g, :], dtype=np.float64)
            # allowed[t][u] for the sampled keys
            allow = np.ones((t_all.size, k_rows.size), dtype=bool)
            if causal:
                allow &= k_rows[None, :] <= t_all[:, None]
            if key_valid is not None:
                allow &= (np.asarray(key_valid[b])[k_rows] != 0)[None, :]
            if doc_start is not None:
                allow &= k_rows[None, :] >= np.asarray(doc_start[b], dtype=np.int64)[t_all][:, None]
            S = scale * (qb @ ku.T)                       # [t][u]
            lse = Lt[b, h]
            lse_safe = np.where(np.isfinite(lse), lse, 0.0)
            Pm = np.where(allow, np.exp(np.where(allow, S, 0.0) - lse_safe[:, None]), 0.0)
            dP = dob @ vu.T
            Dl = np.sum(dob * Ot[b, :, h, :], axis=1)
            dS = Pm * (dP - Dl[:, None])
            return task, g, scale * (dS.T @ qb), Pm.T @ dob

        for (b, h), g, dk, dv in _run(tasks, work_k, workers):
            dK[b, :, g, :] += dk
            dV[b, :, g, :] += dv
    _ = g_size
    return dQ, dK, dV


# --------------------------------------------------------------------------
# the whole path, sharded (page [ALST] "Mecanismul de funcționare Ulysses",
# steps 1, 3, 4, 5) -- used to pin "sharded path == unsharded attention"

def pipeline_fwd(q_seq, k_seq, v_seq, scale: float, causal: bool = True, key_valid=None,
                 block: int = DEFAULT_BLOCK, workers=None):
    """Sequence-sharded inputs ``[P][B][n/P][H][D]`` -> exchange -> per-rank
    attention -> exchange back.  Returns ``(O_seq [P][B][n/P][Hq][D],
    LSE per rank [P][B][Hq/P][n])``."""
    from .exchange import seq2head, head2seq
    P = q_seq.shape[0]
    qh, kh, vh = seq2head(q_seq), seq2head(k_seq), seq2head(v_seq)
    outs, lses = [], []
    for j in range(P):
        o, lse = attn_fwd(qh[j], kh[j], vh[j], scale, causal, key_valid, block=block, workers=workers)
        outs.append(o)
        lses.append(lse)
    return head2seq(np.stack(outs)), np.stack(lses)


def pipeline_bwd(q_seq, k_seq, v_seq, do_seq, scale: float, causal: bool = True, key_valid=None,
                 block: int = DEFAULT_BLOCK, workers=None):
    """Backward of the sharded path: the exchanges are permutations, so their
    adjoints are their inverses -- dO goes sequence->head, dQ/dK/dV go
    head->sequence.  Returns ``(dQ_seq, dK_seq, dV_seq)``."""
    from .exchange import seq2head, head2seq
    P = q_seq.shape[0]
    qh, kh, vh, doh = seq2head(q_seq), seq2head(k_seq), seq2head(v_seq), seq2head(do_seq)
    dqs, dks, dvs = [], [], []
    for j in range(P):
        dq, dk, dv, _, _ = attn_bwd(qh[j], kh[j], vh[j], doh[j], scale, causal, key_valid,
                                    block=block, workers=workers)
        dqs.append(dq)
        dks.append(dk)
        dvs.append(dv)
    return head2seq(np.stack(dqs)), head2seq(np.stack(dks)), head2seq(np.stack(dvs))
