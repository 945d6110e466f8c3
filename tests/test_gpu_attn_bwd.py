"""GPU parity of the attention backward (dQ, dK, dV in float32) against the
fp64 oracle, max-abs 1e-2, on the same bf16-rounded inputs.

The oracle evaluates the backward with its own O and LSE; the GPU path uses
its forward's O and LSE, as a training step would, with O stored in bfloat16
(what the timed step does) or float32.  Both are held to the plain 1e-2.
(The row term Dl = dO . O would inherit a bf16 O's storage rounding; on the
rows where that matters -- rows that see few keys, where |O| is as large as
a V row -- the kernel recomputes Dl from the scores, see attn_bwd.hip.)
Full-size workloads (n = 65536 and the padded n = 98304): dQ at stratified
query rows and dK/dV at >= 64 stratified keys per KV head, the first 512
positions included, against expected values the oracle wrote once into
tests/golden/ (tests/golden/make_sampled_goldens.py); plus exact properties
at every key: padding keys get exactly zero dK/dV.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import ulysses_sequence_parallelism_head_amd as U
from tests.gpu_helpers import say, bits_to_device, to_f64, to_host_f64, assert_close, load_sampled_golden

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
    assert_close("dQ", dq, dQ, 1e-2)
    assert_close("dK", dk, dK, 1e-2)
    assert_close("dV", dv, dV, 1e-2)


@pytest.mark.parametrize("n,causal,masked", [(300, True, True), (520, True, False), (200, False, False)])
@pytest.mark.parametrize("o_dtype", [torch.float32, torch.bfloat16])
def test_bwd_batch2(n, causal, masked, o_dtype):
    """Two sequences in one call (an odd and an even number of 128-key
    blocks): each batch entry matches the oracle."""
    say(f"bwd B=2 n={n} causal={causal} masked={masked} o={o_dtype}")
    q, k, v, do, valid = _inputs(7 * n + 1, n, 8, 2, 128, masked, B=2)
    scale = 128 ** -0.5
    dQ, dK, dV, _, _ = oracle.attn_bwd(to_f64(q), to_f64(k), to_f64(v), to_f64(do), scale, causal, valid)
    dq, dk, dv = _gpu_fwd_bwd(q, k, v, do, valid, scale, causal, o_dtype)
    assert_close("dQ", dq, dQ, 1e-2)
    assert_close("dK", dk, dK, 1e-2)
    assert_close("dV", dv, dV, 1e-2)


@pytest.mark.parametrize("o_dtype", [torch.bfloat16, torch.float32])
def test_bwd_8k_docs_full(o_dtype):
    """The padded workload's shapes at n = 8192 (8q/2kv, d128, padding keys
    masked): every element of dQ, dK, dV."""
    say(f"bwd padded workload at n=8192, full, o={o_dtype}")
    d = synth.local_attention_inputs(4, n=8192)
    w = d["workload"]
    valid = d["valid"]
    dQ, dK, dV, _, _ = oracle.attn_bwd(to_f64(d["q"]), to_f64(d["k"]), to_f64(d["v"]), to_f64(d["do"]),
                                       w.scale, True, valid)
    dq, dk, dv = _gpu_fwd_bwd(d["q"], d["k"], d["v"], d["do"], valid, w.scale, True, o_dtype)
    assert_close("dQ", dq, dQ, 1e-2)
    assert_close("dK", dk, dK, 1e-2)
    assert_close("dV", dv, dV, 1e-2)


def _gpu_fwd_bwd_full(d, o_dtype):
    """Forward then backward on the device, as the timed step runs them;
    returns host copies of O (float64) and LSE besides the gradients."""
    tq, tk, tv, tdo = (bits_to_device(d[x]) for x in ("q", "k", "v", "do"))
    valid = d["valid"]
    tval = None if valid is None else torch.from_numpy(valid).to("cuda:0")
    w = d["workload"]
    o, lse = U.ulysses_attn_fwd(tq, tk, tv, tval, w.scale, True, o_dtype=o_dtype)
    dq, dk, dv = U.ulysses_attn_bwd(tq, tk, tv, o, lse, tdo, tval, w.scale, True)
    torch.cuda.synchronize()
    out = [to_host_f64(x) for x in (o, lse, dq, dk, dv)]
    del tq, tk, tv, tdo, o, lse, dq, dk, dv
    torch.cuda.empty_cache()
    return out


@pytest.mark.parametrize("stem,c", [("64k", 3), ("96k", 4)])
@pytest.mark.parametrize("o_dtype", [torch.bfloat16, torch.float32])
def test_bwd_full_size_sampled(stem, c, o_dtype):
    """The 64K workload (n = 65536, 8q/2kv, d128, causal: the step bench.py
    times) and the padded 96K workload (n = 98304): O and LSE at stratified
    rows, dQ at the same rows, dK/dV at >= 64 stratified keys per KV head
    including the first 512 positions, against the oracle's values stored
    in tests/golden/; every padding key's dK/dV exactly zero."""
    say(f"fwd+bwd full size {stem} (workload {c}) sampled, o={o_dtype}")
    d = synth.local_attention_inputs(c, with_grad=True)
    g = load_sampled_golden(stem, d)
    qr, kr = g["q_rows"], g["k_rows"]
    assert kr.size >= 64 and np.count_nonzero(kr < 512) >= 16
    o, lse, dq, dk, dv = _gpu_fwd_bwd_full(d, o_dtype)
    assert_close("O rows", o[:, qr], g["O"], 1e-2, bf16_out=o_dtype == torch.bfloat16)
    assert_close("LSE rows", lse[:, :, qr], g["LSE"], 1e-2)
    assert_close("dQ rows", dq[:, qr], g["dQ"], 1e-2)
    assert_close("dK keys", dk[:, kr], g["dK"], 1e-2)
    assert_close("dV keys", dv[:, kr], g["dV"], 1e-2)
    early = kr < 512
    assert_close("dK keys < 512", dk[:, kr[early]], g["dK"][:, early], 1e-2)
    if d["valid"] is not None:
        pad = d["valid"][0] == 0
        assert pad.any()
        assert np.all(dk[0, pad] == 0.0) and np.all(dv[0, pad] == 0.0)


@pytest.mark.parametrize("D,masked", [(128, False), (128, True), (64, False)])
def test_bwd_wide_dq_ragged(D, masked):
    """A causal backward long enough for the 8-wave dq workgroups (n = 4100,
    32q/8kv heads: 520 of them, the last 64-position block ragged), with a
    bf16 O: dQ at stratified rows and at the last 70 rows, dK/dV at 16 keys
    around the middle and at the last 64 keys, against the oracle."""
    n, Hq, Hkv = 4100, 32, 8
    say(f"bwd wide dq n={n} 32q/8kv d{D} masked={masked}")
    q, k, v, do, valid = _inputs(4100 + masked, n, Hq, Hkv, D, masked)
    g = synth.streams(77)
    q_rows = np.unique(np.concatenate([synth.stratified_rows(g[6], n, 16, None if valid is None else valid[0]),
                                       np.arange(n - 70, n)]))
    k_rows = np.unique(np.concatenate([np.arange(2040, 2056), np.arange(n - 64, n)]))
    scale = D ** -0.5
    dQ, dK, dV = oracle.attn_bwd_sampled(to_f64(q), to_f64(k), to_f64(v), to_f64(do), scale, True, valid,
                                         q_rows=q_rows, k_rows=k_rows)
    dq, dk, dv = _gpu_fwd_bwd(q, k, v, do, valid, scale, True, torch.bfloat16)
    assert_close("dQ rows", dq[:, q_rows], dQ, 1e-2)
    assert_close("dK keys", dk[:, k_rows], dK, 1e-2)
    assert_close("dV keys", dv[:, k_rows], dV, 1e-2)


def test_bwd_deterministic():
    say("bwd determinism")
    q, k, v, do, valid = _inputs(77, 900, 8, 2, 128, True)
    a = _gpu_fwd_bwd(q, k, v, do, valid, 0.1, True, torch.bfloat16)
    b = _gpu_fwd_bwd(q, k, v, do, valid, 0.1, True, torch.bfloat16)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


@pytest.mark.parametrize("o_dtype", [torch.bfloat16, torch.float32])
def test_bwd_pipeline_matches_unsharded(o_dtype):
    """Sharded path: seq2head(Q, K, V, dO) -> fwd/bwd per rank ->
    head2seq(dQ, dK, dV) equals the oracle's unsharded gradients (1e-2)."""
    say(f"bwd sharded pipeline P=4, n=1024, 32q/8kv, o={o_dtype}")
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
        o, lse = U.ulysses_attn_fwd(qh[j], kh[j], vh[j], None, scale, True, o_dtype=o_dtype)
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
