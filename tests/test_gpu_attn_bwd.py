"""GPU parity of the attention backward (dQ, dK, dV in float32) against the
fp64 oracle, max-abs 1e-2, on the same bf16-rounded inputs.

The oracle evaluates the backward with its own O and LSE; the GPU path uses
its forward's O and LSE, as a training step would.  With a float32 O the
bound is the plain 1e-2.  With a bfloat16 O, the row term Dl = dO . O
inherits O's storage rounding (at most 2^-8 |O| per element), which no
arithmetic can undo; those cases are checked at 1e-2 plus that rounding
propagated through dQ = scale * sum_u P (dP - Dl) k and dK = scale * sum_t
P (dP - Dl) q, computed elementwise from the oracle's O and LSE.
Full-size documents workload (n = 98304): dQ on stratified query rows and
dK/dV on key rows near the end of the sequence (where the oracle needs few
rows), plus exact properties at every key: padding keys get exactly zero
dK/dV.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import ulysses_sequence_parallelism_head_amd as U
from tests.gpu_helpers import say, bits_to_device, to_f64, to_host_f64, assert_close

pytestmark = pytest.mark.gpu


def _inputs(seed, n, Hq, Hkv, D, masked, B=1):
    g = synth.streams(seed)
    q = synth.normal_bf16(g[0], (B, n, Hq, D))
    k = synth.normal_bf16(g[1], (B, n, Hkv, D))
    v = synth.normal_bf16(g[2], (B, n, Hkv, D))
    do = synth.normal_bf16(g[3], (B, n, Hq, D))
    valid = None
    if masked:
        valid = np.stack([synth.document_valid(g[4], n, 4, max(1, n // 3))[0].reshape(n) for _ in range(B)])
    return q, k, v, do, valid


def o_rounding_bound(q, k, do, O, LSE, scale, causal, valid, block=256, doc_start=None):
    """Elementwise bound on the dQ / dK error caused by storing O in bfloat16."""
    B, n, Hq, D = q.shape
    Hkv = k.shape[2]
    g = Hq // Hkv
    bq = np.zeros((B, n, Hq, D))
    bk = np.zeros((B, n, Hkv, D))
    for b in range(B):
        for h in range(Hq):
            kv = h // g
            kh = k[b, :, kv, :]
            dD = np.sum(np.abs(do[b, :, h, :]) * (2.0 ** -8) * np.abs(O[b, :, h, :]), axis=1)   # [n]
            for r0 in range(0, n, block):
                t = np.arange(r0, min(n, r0 + block))
                allow = oracle.attention.allowed_mask(t, n, causal, None if valid is None else valid[b],
                                                      None if doc_start is None else doc_start[b])
                S = scale * (q[b, t, h, :] @ kh.T)
                lse = LSE[b, h, t]
                P = np.where(allow, np.exp(np.where(allow, S, 0.0) - np.where(np.isfinite(lse), lse, 0.0)[:, None]), 0.0)
                bq[b, t, h, :] = scale * dD[t][:, None] * (P @ np.abs(kh))
                bk[b, :, kv, :] += scale * (P * dD[t][:, None]).T @ np.abs(q[b, t, h, :])
    return bq, bk


def _gpu_fwd_bwd(q, k, v, do, valid, scale, causal, o_dtype):
    tq, tk, tv, tdo = bits_to_device(q), bits_to_device(k), bits_to_device(v), bits_to_device(do)
    tval = None if valid is None else torch.from_numpy(valid).to("cuda:0")
    o, lse = U.ulysses_attn_fwd(tq, tk, tv, tval, scale, causal, o_dtype=o_dtype)
    dq, dk, dv = U.ulysses_attn_bwd(tq, tk, tv, o, lse, tdo, tval, scale, causal)
    torch.cuda.synchronize()
    return to_host_f64(dq), to_host_f64(dk), to_host_f64(dv)


CASES = [
    # n, Hq, Hkv, D, causal, masked
    (1, 1, 1, 128, True, False),
    (33, 4, 1, 128, True, False),
    (130, 8, 2, 128, True, True),
    (200, 2, 2, 64, True, False),
    (257, 4, 4, 64, False, True),
    (1000, 8, 2, 128, True, False),
    (999, 6, 2, 128, True, True),     # g = 3
    (600, 16, 2, 128, True, False),   # g = 8
    (2048, 8, 2, 128, True, True),
]


@pytest.mark.parametrize("n,Hq,Hkv,D,causal,masked", CASES)
@pytest.mark.parametrize("o_dtype", [torch.float32, torch.bfloat16])
def test_bwd_small(n, Hq, Hkv, D, causal, masked, o_dtype):
    say(f"bwd n={n} Hq={Hq} Hkv={Hkv} D={D} causal={causal} masked={masked} o={o_dtype}")
    q, k, v, do, valid = _inputs(3 * n + Hq, n, Hq, Hkv, D, masked)
    scale = D ** -0.5
    dQ, dK, dV, O, L = oracle.attn_bwd(to_f64(q), to_f64(k), to_f64(v), to_f64(do), scale, causal, valid)
    dq, dk, dv = _gpu_fwd_bwd(q, k, v, do, valid, scale, causal, o_dtype)
    if o_dtype == torch.float32:
        assert_close("dQ", dq, dQ, 1e-2)
        assert_close("dK", dk, dK, 1e-2)
    else:
        bq, bk = o_rounding_bound(to_f64(q), to_f64(k), to_f64(do), O, L, scale, causal, valid)
        assert_close("dQ", dq, dQ, 1e-2 + bq)
        assert_close("dK", dk, dK, 1e-2 + bk)
    assert_close("dV", dv, dV, 1e-2)


@pytest.mark.parametrize("n,causal,masked", [(300, True, True), (520, True, False), (200, False, False)])
def test_bwd_batch2(n, causal, masked):
    """Two sequences in one call (an odd and an even number of 128-key
    blocks): each batch entry matches the oracle."""
    say(f"bwd B=2 n={n} causal={causal} masked={masked}")
    q, k, v, do, valid = _inputs(7 * n + 1, n, 8, 2, 128, masked, B=2)
    scale = 128 ** -0.5
    dQ, dK, dV, _, _ = oracle.attn_bwd(to_f64(q), to_f64(k), to_f64(v), to_f64(do), scale, causal, valid)
    dq, dk, dv = _gpu_fwd_bwd(q, k, v, do, valid, scale, causal, torch.float32)
    assert_close("dQ", dq, dQ, 1e-2)
    assert_close("dK", dk, dK, 1e-2)
    assert_close("dV", dv, dV, 1e-2)


def test_bwd_8k_docs_full():
    """The documents workload's shapes at n = 8192 (8q/2kv, d128, padding
    keys masked): every element of dQ, dK, dV."""
    say("bwd documents workload at n=8192, full")
    d = synth.local_attention_inputs(4, n=8192)
    w = d["workload"]
    valid = d["valid"]
    dQ, dK, dV, _, _ = oracle.attn_bwd(to_f64(d["q"]), to_f64(d["k"]), to_f64(d["v"]), to_f64(d["do"]),
                                       w.scale, True, valid)
    dq, dk, dv = _gpu_fwd_bwd(d["q"], d["k"], d["v"], d["do"], valid, w.scale, True, torch.float32)
    assert_close("dQ", dq, dQ, 1e-2)
    assert_close("dK", dk, dK, 1e-2)
    assert_close("dV", dv, dV, 1e-2)


def test_bwd_96k_docs_workload_sampled():
    """Workload 4 at full size (n = 98304): dQ on stratified rows, dK/dV on
    key rows in the last 1024 positions; zero dK/dV at every padding key."""
    say("bwd workload 4 (96K documents) sampled")
    d = synth.local_attention_inputs(4)
    w = d["workload"]
    valid = d["valid"]
    q_rows = synth.stratified_rows(d["row_gen"], w.n, 40, valid[0])
    k_rows = synth.sample_rows(d["row_gen"], w.n, 12, extra=(w.n - 1, w.n - 2, w.n - 1024))
    k_rows = k_rows[k_rows >= w.n - 1024]
    dq, dk, dv = _gpu_fwd_bwd(d["q"], d["k"], d["v"], d["do"], valid, w.scale, True, torch.float32)
    pad = valid[0] == 0
    assert np.all(dk[0, pad] == 0.0) and np.all(dv[0, pad] == 0.0)
    dQs, dKs, dVs = oracle.attn_bwd_sampled(to_f64(d["q"]), to_f64(d["k"]), to_f64(d["v"]), to_f64(d["do"]),
                                            w.scale, True, valid, q_rows=q_rows, k_rows=k_rows)
    assert_close("dQ rows", dq[:, q_rows], dQs, 1e-2)
    assert_close("dK rows", dk[:, k_rows], dKs, 1e-2)
    assert_close("dV rows", dv[:, k_rows], dVs, 1e-2)


def test_bwd_64k_workload_sampled():
    """Workload 3 at full size (n = 65536, 8q/2kv, d128, causal: the shapes
    bench.py times): dQ on stratified rows, dK/dV on key rows in the last
    1024 positions (where the oracle needs few rows)."""
    say("bwd workload 3 (64K) sampled")
    d = synth.local_attention_inputs(3, with_grad=True)
    w = d["workload"]
    q_rows = synth.stratified_rows(d["row_gen"], w.n, 40)
    # keys in the last 1024 positions: seeded picks, the ends and 64/128-key tile edges
    k_rows = (w.n - 1024) + synth.sample_rows(d["row_gen"], 1024, 12, extra=(0, 1, 511, 512, 895, 896, 959, 960,
                                                                            1022, 1023))
    dq, dk, dv = _gpu_fwd_bwd(d["q"], d["k"], d["v"], d["do"], None, w.scale, True, torch.float32)
    dQs, dKs, dVs = oracle.attn_bwd_sampled(to_f64(d["q"]), to_f64(d["k"]), to_f64(d["v"]), to_f64(d["do"]),
                                            w.scale, True, None, q_rows=q_rows, k_rows=k_rows)
    assert_close("dQ rows", dq[:, q_rows], dQs, 1e-2)
    assert_close("dK rows", dk[:, k_rows], dKs, 1e-2)
    assert_close("dV rows", dv[:, k_rows], dVs, 1e-2)


def test_bwd_deterministic():
    say("bwd determinism")
    q, k, v, do, valid = _inputs(77, 900, 8, 2, 128, True)
    a = _gpu_fwd_bwd(q, k, v, do, valid, 0.1, True, torch.bfloat16)
    b = _gpu_fwd_bwd(q, k, v, do, valid, 0.1, True, torch.bfloat16)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_bwd_pipeline_matches_unsharded():
    """Sharded path: seq2head(Q, K, V, dO) -> fwd/bwd per rank ->
    head2seq(dQ, dK, dV) equals the oracle's unsharded gradients (1e-2)."""
    say("bwd sharded pipeline P=4, n=1024, 32q/8kv")
    P, n, Hq, Hkv, D = 4, 1024, 32, 8, 128
    g = synth.streams(31)
    nl = n // P
    qs = synth.normal_bf16(g[0], (P, 1, nl, Hq, D))
    ks = synth.normal_bf16(g[1], (P, 1, nl, Hkv, D))
    vs = synth.normal_bf16(g[2], (P, 1, nl, Hkv, D))
    dos = synth.normal_bf16(g[3], (P, 1, nl, Hq, D))
    scale = D ** -0.5
    qh, kh, vh, doh = (U.ulysses_repack_seq2head(bits_to_device(x)) for x in (qs, ks, vs, dos))
    dqs, dks, dvs = [], [], []
    for j in range(P):
        o, lse = U.ulysses_attn_fwd(qh[j], kh[j], vh[j], None, scale, True, o_dtype=torch.float32)
        dq, dk, dv = U.ulysses_attn_bwd(qh[j], kh[j], vh[j], o, lse, doh[j], None, scale, True)
        dqs.append(dq)
        dks.append(dk)
        dvs.append(dv)
    dq_seq = U.ulysses_repack_head2seq(torch.stack(dqs))
    dk_seq = U.ulysses_repack_head2seq(torch.stack(dks))
    dv_seq = U.ulysses_repack_head2seq(torch.stack(dvs))
    torch.cuda.synchronize()
    dQ, dK, dV, _, _ = oracle.attn_bwd(to_f64(oracle.unshard(qs)), to_f64(oracle.unshard(ks)),
                                       to_f64(oracle.unshard(vs)), to_f64(oracle.unshard(dos)), scale, True)
    assert_close("dQ", oracle.unshard(to_host_f64(dq_seq)), dQ, 1e-2)
    assert_close("dK", oracle.unshard(to_host_f64(dk_seq)), dK, 1e-2)
    assert_close("dV", oracle.unshard(to_host_f64(dv_seq)), dV, 1e-2)


@pytest.mark.parametrize("docs", [False, True])
def test_bwd_padding_keys_extreme_values(docs):
    """Padding keys whose K and V rows are huge (scores far above every
    row's logsumexp, so an unmasked exp would overflow): the key-stationary
    pass leaves such keys unmasked and writes their dK/dV as zero, so every
    gradient must stay finite, padding keys must get exactly zero dK/dV and
    the rest must match the oracle, which never looks at padding keys."""
    n, Hq, Hkv, D = 300, 8, 2, 128
    say(f"bwd padding keys with extreme values, n={n}, documents={docs}")
    q, k, v, do, valid = _inputs(5150 + docs, n, Hq, Hkv, D, True)
    pad = valid[0] == 0
    assert pad.any() and (~pad).any()
    k = np.where(pad[None, :, None, None], np.uint16(0x4270), k)   # bf16 60.0 in every dim
    v = np.where(pad[None, :, None, None], np.uint16(0xC270), v)   # bf16 -60.0
    scale = D ** -0.5
    ds = None
    if docs:
        starts = np.array([0, 97, 98, 211])
        ds = np.zeros((1, n), np.int32)
        for s0 in starts:
            ds[0, s0:] = s0
    dQ, dK, dV, _, _ = oracle.attn_bwd(to_f64(q), to_f64(k), to_f64(v), to_f64(do), scale, True, valid,
                                       **({} if ds is None else {"doc_start": ds}))
    tq, tk, tv, tdo = bits_to_device(q), bits_to_device(k), bits_to_device(v), bits_to_device(do)
    tval = torch.from_numpy(valid).to("cuda:0")
    if docs:
        tds = torch.from_numpy(ds).to("cuda:0")
        o, lse = U.ulysses_attn_fwd_docs(tq, tk, tv, tds, tval, scale, o_dtype=torch.float32)
        dq, dk, dv = U.ulysses_attn_bwd_docs(tq, tk, tv, o, lse, tdo, tds, tval, scale)
    else:
        o, lse = U.ulysses_attn_fwd(tq, tk, tv, tval, scale, True, o_dtype=torch.float32)
        dq, dk, dv = U.ulysses_attn_bwd(tq, tk, tv, o, lse, tdo, tval, scale, True)
    torch.cuda.synchronize()
    dq, dk, dv = to_host_f64(dq), to_host_f64(dk), to_host_f64(dv)
    for name, x in (("dQ", dq), ("dK", dk), ("dV", dv)):
        assert np.all(np.isfinite(x)), f"{name}: non-finite value"
    assert np.all(dk[0, pad] == 0.0) and np.all(dv[0, pad] == 0.0)
    assert_close("dQ", dq, dQ, 1e-2)
    assert_close("dK", dk, dK, 1e-2)
    assert_close("dV", dv, dV, 1e-2)
