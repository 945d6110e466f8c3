"""Planted mistakes in the oracle (on the CPU) must trip at least one pin.

Each mutation replaces one helper of ``oracle.attention`` with a plausible
wrong version (an off-by-one mask, a wrong head mapping, a dropped mask in
the normaliser, a logsumexp without the row max, a wrong padding rule, a
document mask dropped, off by one or indexed by the key) and checks that
the independent references -- brute force, the worked example, torch SDPA --
then disagree with it.
"""
import math

import numpy as np
import pytest

import oracle.attention as oa
from tests.test_oracle_attention import brute_fwd, torch_ref, make_valid, rnd
from tests.test_oracle_docs import brute_docs_fwd, doc_ids_from_lengths, starts_from_lengths, torch_docs_ref


def _pins_fail(golden):
    """True when any of the independent references disagrees with the oracle."""
    try:
        g = golden("worked_attention_d1_n3.txt")
        q = np.array(g["q"]).reshape(1, 3, 1, 1)
        k = np.array(g["k"]).reshape(1, 3, 1, 1)
        v = np.array(g["v"]).reshape(1, 3, 1, 1)
        O, L = oa.attn_fwd(q, k, v, 1.0, True)
        if not (np.allclose(O.ravel(), g["o"], atol=1e-12) and np.allclose(L.ravel(), g["lse"], atol=1e-12)):
            return True
        n, Hq, Hkv, D = 12, 4, 2, 3
        q, k, v, do = rnd(1, 1, n, Hq, D), rnd(2, 1, n, Hkv, D), rnd(3, 1, n, Hkv, D), rnd(4, 1, n, Hq, D)
        valid = make_valid(5, 1, n)
        O, L = oa.attn_fwd(q, k, v, 0.5, True, valid)
        Ob, Lb = brute_fwd(q, k, v, 0.5, True, valid)
        if not (np.allclose(O, Ob, atol=1e-12) and np.allclose(L, Lb, atol=1e-12)):
            return True
        ref = torch_ref(q, k, v, do, 0.5, True, valid)
        dq, dk, dv, _, _ = oa.attn_bwd(q, k, v, do, 0.5, True, valid)
        if not (np.allclose(dq, ref["dq"], atol=1e-10) and np.allclose(dk, ref["dk"], atol=1e-10)
                and np.allclose(dv, ref["dv"], atol=1e-10)):
            return True
        # packed documents: brute force and torch SDPA with the block-diagonal causal mask
        lengths = [4, 1, 6, 3]
        n = sum(lengths)
        q, k, v, do = rnd(6, 1, n, Hq, D), rnd(7, 1, n, Hkv, D), rnd(8, 1, n, Hkv, D), rnd(9, 1, n, Hq, D)
        valid = make_valid(10, 1, n)
        ds = starts_from_lengths(lengths).reshape(1, n)
        ids = doc_ids_from_lengths(lengths).reshape(1, n)
        O, L = oa.attn_fwd(q, k, v, 0.5, True, valid, doc_start=ds)
        Ob, Lb = brute_docs_fwd(q, k, v, 0.5, ids, valid)
        if not (np.allclose(O, Ob, atol=1e-12) and np.array_equal(np.isneginf(L), np.isneginf(Lb))
                and np.allclose(L[np.isfinite(Lb)], Lb[np.isfinite(Lb)], atol=1e-12)):
            return True
        ref = torch_docs_ref(q, k, v, do, 0.5, ids, valid)
        dq, dk, dv, _, _ = oa.attn_bwd(q, k, v, do, 0.5, True, valid, doc_start=ds)
        return not (np.allclose(dq, ref["dq"], atol=1e-10) and np.allclose(dk, ref["dk"], atol=1e-10)
                    and np.allclose(dv, ref["dv"], atol=1e-10))
    except Exception:
        return True


def _docs(m, rows, n_keys, doc_b):
    """The correct document condition, for mutations that change something else."""
    if doc_b is None:
        return m
    return m & (np.arange(n_keys)[None, :] >= np.asarray(doc_b, dtype=np.int64)[rows][:, None])


def _mask_including_next(rows, n_keys, causal, valid_b, doc_b=None):
    keys = np.arange(n_keys)
    m = keys[None, :] <= rows[:, None] + 1 if causal else np.ones((rows.size, n_keys), bool)
    if valid_b is not None:
        m = m & (np.asarray(valid_b[:n_keys]) != 0)[None, :]
    return _docs(m, rows, n_keys, doc_b)


def _mask_ignoring_valid(rows, n_keys, causal, valid_b, doc_b=None):
    keys = np.arange(n_keys)
    m = keys[None, :] <= rows[:, None] if causal else np.ones((rows.size, n_keys), bool)
    return _docs(m, rows, n_keys, doc_b)


def _mask_query_padding(rows, n_keys, causal, valid_b, doc_b=None):
    """Wrong padding rule: masks the query's own validity instead of the key's."""
    keys = np.arange(n_keys)
    m = keys[None, :] <= rows[:, None] if causal else np.ones((rows.size, n_keys), bool)
    if valid_b is not None:
        m = m & (np.asarray(valid_b)[rows] != 0)[:, None]
    return _docs(m, rows, n_keys, doc_b)


def _mask_ignoring_documents(rows, n_keys, causal, valid_b, doc_b=None):
    return _orig_mask(rows, n_keys, causal, valid_b, None)


def _mask_document_start_excluded(rows, n_keys, causal, valid_b, doc_b=None):
    """Off by one at the document boundary: the document's first token is dropped."""
    m = _orig_mask(rows, n_keys, causal, valid_b, None)
    if doc_b is None:
        return m
    return m & (np.arange(n_keys)[None, :] > np.asarray(doc_b, dtype=np.int64)[rows][:, None])


def _mask_document_of_key(rows, n_keys, causal, valid_b, doc_b=None):
    """Transposed index: compares the row with the key's document start."""
    m = _orig_mask(rows, n_keys, causal, valid_b, None)
    if doc_b is None:
        return m
    return m & (rows[:, None] >= np.asarray(doc_b, dtype=np.int64)[:n_keys][None, :])


def _softmax_unmasked_sum(S, allow):
    Sm = np.where(allow, S, -np.inf)
    m = Sm.max(axis=1)
    w = np.where(allow, np.exp(Sm - m[:, None]), 0.0)
    L = np.exp(S - m[:, None]).sum(axis=1)          # normaliser forgets the mask
    return w, m, L


def _softmax_lse_drops_max(S, allow):
    w, m, L = _orig_softmax(S, allow)
    return w, np.zeros_like(m), L                    # logsumexp loses the row max


_orig_softmax = oa._softmax_rows
_orig_mask = oa.allowed_mask


MUTATIONS = {
    "gqa_modulo": ("kv_head_of", lambda h, Hq, Hkv: h % Hkv),
    "mask_off_by_one": ("allowed_mask", _mask_including_next),
    "mask_ignores_padding": ("allowed_mask", _mask_ignoring_valid),
    "mask_query_padding": ("allowed_mask", _mask_query_padding),
    "mask_ignores_documents": ("allowed_mask", _mask_ignoring_documents),
    "mask_drops_document_start": ("allowed_mask", _mask_document_start_excluded),
    "mask_document_of_key": ("allowed_mask", _mask_document_of_key),
    "normaliser_unmasked": ("_softmax_rows", _softmax_unmasked_sum),
    "lse_drops_max": ("_softmax_rows", _softmax_lse_drops_max),
}


def test_unmutated_oracle_passes(golden):
    assert not _pins_fail(golden)


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, golden, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(oa, attr, fn)
    assert _pins_fail(golden), f"planted mistake {name!r} went unnoticed"
