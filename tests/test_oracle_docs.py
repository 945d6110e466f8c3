"""Pins for the oracle's document-masked attention (CPU only).

A token attends only to earlier tokens of its own document; the documents
are given per token by ``doc_start`` (position of the document's first
token).  The oracle's masked path is checked against things other than
itself:
  * a hand-derived worked example (tests/golden/), exact;
  * separation: attention over the packed sequence equals ordinary causal
    attention run on each document alone (forward and all gradients), the
    defining property of the mask;
  * brute force in pure Python on tiny inputs, with the document membership
    written as document ids rather than start positions;
  * torch SDPA (CPU, float64) with the block-diagonal causal mask built from
    the document ids, and torch autograd for the gradients;
  * the sampled backward agrees with the full one on the same documents;
  * doc_start = 0 everywhere reduces to plain causal attention.
"""
import math

import numpy as np
import pytest
import torch

from oracle.attention import attn_fwd, attn_bwd, attn_bwd_sampled


def rnd(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


def starts_from_lengths(lengths):
    """Per-token document start for documents of the given lengths, in order."""
    out = []
    pos = 0
    for L in lengths:
        out += [pos] * L
        pos += L
    return np.array(out, dtype=np.int64)


def doc_ids_from_lengths(lengths):
    return np.concatenate([np.full(L, i) for i, L in enumerate(lengths)])


LAYOUTS = [
    [5, 1, 12, 3, 16],        # mixed, a one-token document
    [1, 1, 1, 1, 1, 1, 1],    # every token its own document
    [37],                     # one document: plain causal
    [20, 17],
]


def brute_docs_fwd(q, k, v, scale, doc_id, valid):
    """Pure-Python reference; membership by document id."""
    B, n, Hq, D = q.shape
    g = Hq // k.shape[2]
    O = np.zeros((B, n, Hq, D))
    L = np.full((B, Hq, n), -math.inf)
    for b in range(B):
        for h in range(Hq):
            kh = h // g
            for t in range(n):
                keys = [u for u in range(t + 1) if doc_id[b][u] == doc_id[b][t] and (valid is None or valid[b][u])]
                if not keys:
                    continue
                s = [scale * math.fsum(float(q[b, t, h, c]) * float(k[b, u, kh, c]) for c in range(D)) for u in keys]
                m = max(s)
                w = [math.exp(x - m) for x in s]
                tot = math.fsum(w)
                for c in range(D):
                    O[b, t, h, c] = math.fsum(wi * float(v[b, u, kh, c]) for wi, u in zip(w, keys)) / tot
                L[b, h, t] = m + math.log(tot)
    return O, L


def torch_docs_ref(q, k, v, dout, scale, doc_id, valid):
    B, n, Hq, D = q.shape
    tq = torch.tensor(q, dtype=torch.float64).permute(0, 2, 1, 3).contiguous().requires_grad_(True)
    tk = torch.tensor(k, dtype=torch.float64).permute(0, 2, 1, 3).contiguous().requires_grad_(True)
    tv = torch.tensor(v, dtype=torch.float64).permute(0, 2, 1, 3).contiguous().requires_grad_(True)
    ids = torch.tensor(np.asarray(doc_id))
    mask = torch.tril(torch.ones(n, n, dtype=torch.bool)).expand(B, n, n) & (ids[:, :, None] == ids[:, None, :])
    mask = mask[:, None].clone()
    if valid is not None:
        mask &= torch.tensor(np.asarray(valid) != 0)[:, None, None, :]
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=scale, enable_gqa=True)
    (o * torch.tensor(dout, dtype=torch.float64).permute(0, 2, 1, 3)).sum().backward()
    return {"o": o.detach().permute(0, 2, 1, 3).numpy(),
            "dq": tq.grad.permute(0, 2, 1, 3).numpy(),
            "dk": tk.grad.permute(0, 2, 1, 3).numpy(),
            "dv": tv.grad.permute(0, 2, 1, 3).numpy()}


# ------------------------------------------------------------- worked example
def test_worked_example_docs(golden):
    g = golden("worked_attention_docs_d1_n4.txt")
    shp = (1, 4, 1, 1)
    q, k, v, do = (np.array(g[x]).reshape(shp) for x in ("q", "k", "v", "dout"))
    ds = np.array(g["doc_start"]).reshape(1, 4)
    O, L = attn_fwd(q, k, v, g["scale"], True, doc_start=ds)
    np.testing.assert_allclose(O.ravel(), g["o"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(L.ravel(), g["lse"], rtol=0, atol=1e-14)
    dq, dk, dv, _, _ = attn_bwd(q, k, v, do, g["scale"], True, doc_start=ds)
    np.testing.assert_allclose(dq.ravel(), g["dq"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(dk.ravel(), g["dk"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(dv.ravel(), g["dv"], rtol=0, atol=1e-14)


# ----------------------------------------------------------------- separation
@pytest.mark.parametrize("lengths", LAYOUTS)
@pytest.mark.parametrize("masked", [False, True])
def test_packed_equals_documents_alone(lengths, masked):
    n, Hq, Hkv, D = sum(lengths), 4, 2, 5
    q, k, v, do = rnd(1, 1, n, Hq, D), rnd(2, 1, n, Hkv, D), rnd(3, 1, n, Hkv, D), rnd(4, 1, n, Hq, D)
    valid = None
    if masked:
        valid = (np.random.default_rng(5).random((1, n)) > 0.3).astype(np.uint8)
    ds = starts_from_lengths(lengths).reshape(1, n)
    dq, dk, dv, O, L = attn_bwd(q, k, v, do, 0.41, True, valid, block=8, doc_start=ds)
    pos = 0
    for Ld in lengths:
        sl = slice(pos, pos + Ld)
        vd = None if valid is None else valid[:, sl]
        dq1, dk1, dv1, O1, L1 = attn_bwd(q[:, sl], k[:, sl], v[:, sl], do[:, sl], 0.41, True, vd, block=8)
        np.testing.assert_allclose(O[:, sl], O1, rtol=0, atol=1e-12)
        np.testing.assert_array_equal(np.isneginf(L[:, :, sl]), np.isneginf(L1))
        fin = np.isfinite(L1)
        np.testing.assert_allclose(L[:, :, sl][fin], L1[fin], rtol=0, atol=1e-12)
        np.testing.assert_allclose(dq[:, sl], dq1, rtol=0, atol=1e-11)
        np.testing.assert_allclose(dk[:, sl], dk1, rtol=0, atol=1e-11)
        np.testing.assert_allclose(dv[:, sl], dv1, rtol=0, atol=1e-11)
        pos += Ld


# ---------------------------------------------------------------- brute force
@pytest.mark.parametrize("lengths,masked", [([3, 1, 5], False), ([2, 6, 1, 4], True), ([1] * 6, False)])
def test_docs_fwd_brute_force(lengths, masked):
    B, n, Hq, Hkv, D = 2, sum(lengths), 4, 2, 3
    q, k, v = rnd(11, B, n, Hq, D), rnd(12, B, n, Hkv, D), rnd(13, B, n, Hkv, D)
    valid = (np.random.default_rng(14).random((B, n)) > 0.3).astype(np.uint8) if masked else None
    # the second batch row packs the documents in reverse order
    ls = [lengths, lengths[::-1]]
    ds = np.stack([starts_from_lengths(x) for x in ls])
    ids = np.stack([doc_ids_from_lengths(x) for x in ls])
    O, L = attn_fwd(q, k, v, 0.6, True, valid, block=3, doc_start=ds)
    Ob, Lb = brute_docs_fwd(q, k, v, 0.6, ids, valid)
    np.testing.assert_allclose(O, Ob, rtol=0, atol=1e-13)
    np.testing.assert_array_equal(np.isneginf(L), np.isneginf(Lb))
    np.testing.assert_allclose(L[np.isfinite(Lb)], Lb[np.isfinite(Lb)], rtol=0, atol=1e-13)


# ------------------------------------------------------------ library routine
@pytest.mark.parametrize("masked", [False, True])
def test_docs_against_torch_sdpa(masked):
    lengths = [9, 1, 14, 4, 12]
    B, n, Hq, Hkv, D = 1, sum(lengths), 8, 2, 6
    q, k, v, do = rnd(21, B, n, Hq, D), rnd(22, B, n, Hkv, D), rnd(23, B, n, Hkv, D), rnd(24, B, n, Hq, D)
    valid = None
    if masked:
        valid = (np.random.default_rng(25).random((B, n)) > 0.25).astype(np.uint8)
        valid[0, np.cumsum([0] + lengths[:-1])] = 1     # every document's first token is real
    ds = starts_from_lengths(lengths).reshape(1, n)
    ref = torch_docs_ref(q, k, v, do, 0.3, doc_ids_from_lengths(lengths).reshape(1, n), valid)
    dq, dk, dv, O, _ = attn_bwd(q, k, v, do, 0.3, True, valid, block=7, doc_start=ds)
    np.testing.assert_allclose(O, ref["o"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(dq, ref["dq"], rtol=0, atol=1e-11)
    np.testing.assert_allclose(dk, ref["dk"], rtol=0, atol=1e-11)
    np.testing.assert_allclose(dv, ref["dv"], rtol=0, atol=1e-11)


# ------------------------------------------------------------------ consistency
def test_sampled_backward_matches_full_with_docs():
    lengths = [17, 3, 30, 1, 13]
    B, n, Hq, Hkv, D = 1, sum(lengths), 4, 1, 4
    q, k, v, do = rnd(31, B, n, Hq, D), rnd(32, B, n, Hkv, D), rnd(33, B, n, Hkv, D), rnd(34, B, n, Hq, D)
    valid = (np.random.default_rng(35).random((B, n)) > 0.2).astype(np.uint8)
    ds = starts_from_lengths(lengths).reshape(1, n)
    dq, dk, dv, _, _ = attn_bwd(q, k, v, do, 0.5, True, valid, block=16, doc_start=ds)
    qr = np.array([0, 5, 17, 19, 20, 21, 50, n - 1])
    kr = np.array([1, 16, 17, 20, 40, 51, 63])
    sq, sk, sv = attn_bwd_sampled(q, k, v, do, 0.5, True, valid, q_rows=qr, k_rows=kr, block=16, doc_start=ds)
    np.testing.assert_allclose(sq, dq[:, qr], rtol=0, atol=1e-12)
    np.testing.assert_allclose(sk, dk[:, kr], rtol=0, atol=1e-12)
    np.testing.assert_allclose(sv, dv[:, kr], rtol=0, atol=1e-12)


def test_zero_starts_are_plain_causal():
    B, n, Hq, Hkv, D = 2, 23, 2, 1, 3
    q, k, v, do = rnd(41, B, n, Hq, D), rnd(42, B, n, Hkv, D), rnd(43, B, n, Hkv, D), rnd(44, B, n, Hq, D)
    ds = np.zeros((B, n), dtype=np.int64)
    a = attn_bwd(q, k, v, do, 0.7, True, doc_start=ds)
    b = attn_bwd(q, k, v, do, 0.7, True)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)
