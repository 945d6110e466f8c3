"""Write the oracle's expected values at sampled rows of the full-size
attention workloads, for the GPU parity tests.

    python tests/golden/make_sampled_goldens.py [64k] [96k]

The expected values come from ``oracle/`` alone, evaluated on the seeded
inputs of ``synth/`` (no GPU result is read or used).  At these sizes the
fp64 oracle needs minutes on the host's cores -- the dK/dV of the first keys
depend on the logsumexp and dO . O of every later row, so the whole forward
is evaluated -- which is why the values are computed once here and stored,
rather than on every GPU test run.

Per workload the file ``bwd_<name>_sampled.npz`` holds (float32 values,
plain arrays, no pickled objects):

* ``q_rows``: stratified query rows (``synth.stratified_rows``: first/last,
  tile edges +-1, rows spread over the first 512 positions, rows beside pad
  tokens, seeded picks);
* ``k_rows``: at least 64 key rows shared by every KV head: the first 512
  positions densely (where few rows see a key and the gradient is large),
  64/128-key tile edges, pad edges, the last keys, seeded picks;
* ``O`` ``[1][len(q_rows)][Hq][D]``, ``LSE`` ``[1][Hq][len(q_rows)]`` (natural
  log), ``dQ`` at ``q_rows``, ``dK`` and ``dV`` ``[1][len(k_rows)][Hkv][D]`` at
  ``k_rows``: the forward and the gradient of sum(O * dO) with respect to
  q, k, v (page "Paralelismul de Secvență Ulysses...", section "Mecanismul
  de funcționare Ulysses", step 4; the recompute from the logsumexp follows
  the same page, section "Provocarea antrenării cu secvențe lungi").
* ``seed_check``: the first 8 bf16 bit patterns of Q, K, V and dO, so a test
  can confirm it regenerated the same inputs.
"""
from __future__ import annotations

import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synth  # noqa: E402

# workload number -> file stem
WORKLOADS = {"64k": 3, "96k": 4}


def key_rows(gen, n, valid=None):
    """>= 64 stratified key rows: dense over the first 512 positions, tile
    edges, pad edges, the end, and seeded picks."""
    extra = set()
    for t in (0, 1, 2, 3, 31, 32, 33, 63, 64, 65, 95, 96, 127, 128, 129, 191, 192, 255, 256, 257,
              319, 320, 383, 384, 447, 448, 509, 510, 511, 512, 513):
        extra.add(t)
    for t in (n // 4, n // 2, 3 * n // 4):
        extra.update((t - 1, t))
    for t in (n - 129, n - 128, n - 65, n - 64, n - 2, n - 1):
        extra.add(t)
    if valid is not None:
        edges = np.nonzero(np.diff(valid.astype(np.int8)))[0]
        for e in edges[:8]:
            extra.update((int(e), int(e) + 1))
    return synth.sample_rows(gen, n, 32, extra)


def inputs(c):
    d = synth.local_attention_inputs(c, with_grad=True)
    valid = d["valid"]
    q_rows = synth.stratified_rows(d["row_gen"], d["n"], 40, None if valid is None else valid[0])
    k_rows = key_rows(d["row_gen"], d["n"], None if valid is None else valid[0])
    return d, q_rows, k_rows


def path(stem):
    return os.path.join(HERE, f"bwd_{stem}_sampled.npz")


def seed_check(d):
    return np.stack([d[x].reshape(-1)[:8].astype(np.uint16) for x in ("q", "k", "v", "do")])


def make(stem):
    c = WORKLOADS[stem]
    t0 = time.time()
    d, q_rows, k_rows = inputs(c)
    w = d["workload"]
    f64 = synth.bf16_bits_to_f64
    q, k, v, do = (f64(d[x]) for x in ("q", "k", "v", "do"))
    valid = d["valid"]
    print(f"[{stem}] n={d['n']} q_rows={q_rows.size} k_rows={k_rows.size}", flush=True)
    O, LSE = oracle.attn_fwd(q, k, v, w.scale, True, valid, rows=q_rows)
    print(f"[{stem}] forward rows done ({time.time() - t0:.0f} s)", flush=True)
    dQ, dK, dV = oracle.attn_bwd_sampled(q, k, v, do, w.scale, True, valid, q_rows=q_rows, k_rows=k_rows)
    print(f"[{stem}] sampled backward done ({time.time() - t0:.0f} s)", flush=True)
    np.savez_compressed(path(stem), q_rows=q_rows, k_rows=k_rows, O=O.astype(np.float32),
                        LSE=LSE.astype(np.float32), dQ=dQ.astype(np.float32), dK=dK.astype(np.float32),
                        dV=dV.astype(np.float32), seed_check=seed_check(d))
    print(f"[{stem}] wrote {path(stem)}: max|O| {np.abs(O).max():.3f} max|dQ| {np.abs(dQ).max():.3f} "
          f"max|dK| {np.abs(dK).max():.3f} max|dV| {np.abs(dV).max():.3f}", flush=True)


if __name__ == "__main__":
    for stem in (sys.argv[1:] or list(WORKLOADS)):
        make(stem)
