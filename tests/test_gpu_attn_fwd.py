"""GPU parity of the attention forward (O and logsumexp) against the fp64 oracle.

Tolerances (max-abs against the oracle on the same bf16-rounded inputs):
  * bf16 inputs, float32 O: 1e-2 on O and on LSE;
  * bf16 inputs, bf16 O: 1e-2 (the storage rounding is at most 2^-7 while
    |O| < 4); an element with |O| >= 4, where half a bf16 ulp alone exceeds
    that, gets its half-ulp plus the same 1e-2 - 2^-7 compute margin;
  * float32 inputs and O (fp32 path): 5e-5.
Shapes span several tiles with ragged tails, every GQA group size, both head
dims, causal and not, with and without a key-padding mask; the full-size
workloads are checked on rows the oracle computes one by one.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import ulysses_sequence_parallelism_head_amd as U
from tests.gpu_helpers import say, bits_to_device, f32_to_device, to_f64, to_host_f64, assert_close

pytestmark = pytest.mark.gpu


def _inputs(seed, n, Hq, Hkv, D, masked, dtype="bf16"):
    g = synth.streams(seed)
    if dtype == "bf16":
        q = synth.normal_bf16(g[0], (1, n, Hq, D))
        k = synth.normal_bf16(g[1], (1, n, Hkv, D))
        v = synth.normal_bf16(g[2], (1, n, Hkv, D))
    else:
        q = g[0].standard_normal((1, n, Hq, D), dtype=np.float32)
        k = g[1].standard_normal((1, n, Hkv, D), dtype=np.float32)
        v = g[2].standard_normal((1, n, Hkv, D), dtype=np.float32)
    valid = None
    if masked:
        valid, _ = synth.document_valid(g[4], n, 4, max(1, n // 3))
        valid = valid.reshape(1, n)
    return q, k, v, valid


def _dev(x):
    return bits_to_device(x) if x.dtype == np.uint16 else f32_to_device(x)


def _run(q, k, v, valid, scale, causal, o_dtype):
    tv = None if valid is None else torch.from_numpy(valid).to("cuda:0")
    o, lse = U.ulysses_attn_fwd(_dev(q), _dev(k), _dev(v), tv, scale, causal, o_dtype=o_dtype)
    torch.cuda.synchronize()
    return to_host_f64(o), to_host_f64(lse)


CASES = [
    # n, Hq, Hkv, D, causal, masked
    (1, 1, 1, 128, True, False),
    (17, 4, 1, 128, True, False),
    (64, 8, 2, 128, True, False),
    (100, 2, 2, 64, True, False),
    (257, 8, 2, 128, True, True),
    (300, 8, 1, 64, False, False),
    (1000, 8, 2, 128, True, False),
    (1000, 6, 2, 128, True, True),      # g = 3
    (777, 16, 2, 128, True, False),     # g = 8
    (2048, 4, 4, 128, False, True),
    (2049, 8, 2, 64, True, True),
]


@pytest.mark.parametrize("n,Hq,Hkv,D,causal,masked", CASES)
def test_fwd_bf16_small(n, Hq, Hkv, D, causal, masked):
    say(f"fwd bf16 n={n} Hq={Hq} Hkv={Hkv} D={D} causal={causal} masked={masked}")
    q, k, v, valid = _inputs(n + D + Hq, n, Hq, Hkv, D, masked)
    scale = D ** -0.5
    O, L = oracle.attn_fwd(to_f64(q), to_f64(k), to_f64(v), scale, causal, valid)
    o32, l32 = _run(q, k, v, valid, scale, causal, torch.float32)
    assert_close("O(f32 out)", o32, O, 1e-2)
    assert_close("LSE", l32, L, 1e-2)
    o16, l16 = _run(q, k, v, valid, scale, causal, torch.bfloat16)
    assert_close("O(bf16 out)", o16, O, 1e-2, bf16_out=True)
    assert np.array_equal(l16, l32)


@pytest.mark.parametrize("n,Hq,Hkv,D,causal,masked", [
    (256, 2, 2, 64, True, False), (300, 4, 2, 128, True, True), (97, 3, 1, 64, False, False),
    (1024, 8, 2, 128, True, False),
])
def test_fwd_f32(n, Hq, Hkv, D, causal, masked):
    say(f"fwd f32 n={n} Hq={Hq} Hkv={Hkv} D={D} causal={causal} masked={masked}")
    q, k, v, valid = _inputs(n + 1, n, Hq, Hkv, D, masked, dtype="f32")
    scale = 1.0 / 8.0
    O, L = oracle.attn_fwd(to_f64(q), to_f64(k), to_f64(v), scale, causal, valid)
    o, l = _run(q, k, v, valid, scale, causal, torch.float32)
    assert_close("O", o, O, 5e-5)
    assert_close("LSE", l, L, 5e-5)


def test_tiny_fp32_pipeline():
    """Workload 1: n=256, P=2, 4q=4kv heads, d64, fp32: sequence shards ->
    seq2head -> attention per rank -> head2seq, against the oracle's
    sharded pipeline and against unsharded attention (5e-5)."""
    say("tiny fp32 pipeline (workload 1)")
    d = synth.global_sharded_inputs(1)
    w = d["workload"]
    qs, ks, vs = d["q"], d["k"], d["v"]                   # [2][1][128][4][64] fp32
    qh = U.ulysses_repack_seq2head(f32_to_device(qs))
    kh = U.ulysses_repack_seq2head(f32_to_device(ks))
    vh = U.ulysses_repack_seq2head(f32_to_device(vs))
    outs = []
    for j in range(w.P):
        o, _ = U.ulysses_attn_fwd(qh[j], kh[j], vh[j], None, w.scale, True, o_dtype=torch.float32)
        outs.append(o)
    o_seq = U.ulysses_repack_head2seq(torch.stack(outs))
    torch.cuda.synchronize()
    ref_seq, _ = oracle.pipeline_fwd(qs.astype(np.float64), ks.astype(np.float64), vs.astype(np.float64), w.scale, True)
    assert_close("O_seq vs oracle pipeline", to_host_f64(o_seq), ref_seq, 5e-5)
    O, _ = oracle.attn_fwd(oracle.unshard(qs).astype(np.float64), oracle.unshard(ks).astype(np.float64),
                           oracle.unshard(vs).astype(np.float64), w.scale, True)
    assert_close("O_seq vs unsharded", oracle.unshard(to_host_f64(o_seq)), O, 5e-5)


def test_fwd_8k_workload_full():
    """Workload 2: n=8192, 8q/2kv, d128, bf16, causal -- every row."""
    say("fwd workload 2 (8K) full")
    d = synth.local_attention_inputs(2)
    w = d["workload"]
    O, L = oracle.attn_fwd(to_f64(d["q"]), to_f64(d["k"]), to_f64(d["v"]), w.scale, True)
    o32, l32 = _run(d["q"], d["k"], d["v"], None, w.scale, True, torch.float32)
    assert_close("O(f32 out)", o32, O, 1e-2)
    assert_close("LSE", l32, L, 1e-2)
    o16, _ = _run(d["q"], d["k"], d["v"], None, w.scale, True, torch.bfloat16)
    assert_close("O(bf16 out)", o16, O, 1e-2, bf16_out=True)


def _sampled(c, count):
    d = synth.local_attention_inputs(c)
    w = d["workload"]
    rows = synth.stratified_rows(d["row_gen"], w.n, count, d["valid"][0] if d["valid"] is not None else None)
    return d, w, rows


def test_fwd_64k_workload_sampled():
    """Workload 3: n=65536, 8q/2kv, d128, bf16, causal -- stratified rows."""
    say("fwd workload 3 (64K) sampled rows")
    d, w, rows = _sampled(3, 48)
    O, L = oracle.attn_fwd(to_f64(d["q"]), to_f64(d["k"]), to_f64(d["v"]), w.scale, True, rows=rows)
    o32, l32 = _run(d["q"], d["k"], d["v"], None, w.scale, True, torch.float32)
    assert_close("O(f32 out)", o32[:, rows], O, 1e-2)
    assert_close("LSE", l32[:, :, rows], L, 1e-2)
    o16, l16 = _run(d["q"], d["k"], d["v"], None, w.scale, True, torch.bfloat16)
    assert_close("O(bf16 out)", o16[:, rows], O, 1e-2, bf16_out=True)
    assert np.array_equal(l16, l32)


@pytest.mark.parametrize("masked", [False, True])
def test_fwd_wide_workgroups_ragged(masked):
    """A causal run long enough for the 8-wave workgroups (n = 16417: 514
    of them, with a ragged last block): stratified rows and every row of
    the last two blocks, against the oracle."""
    n, Hq, Hkv, D = 16417, 8, 2, 128
    say(f"fwd wide workgroups n={n} masked={masked}")
    q, k, v, valid = _inputs(16417 + masked, n, Hq, Hkv, D, masked)
    g = synth.streams(99)
    rows = np.unique(np.concatenate([synth.stratified_rows(g[6], n, 24, None if valid is None else valid[0]),
                                     np.arange(n - 100, n)]))
    scale = D ** -0.5
    O, L = oracle.attn_fwd(to_f64(q), to_f64(k), to_f64(v), scale, True, valid, rows=rows)
    o32, l32 = _run(q, k, v, valid, scale, True, torch.float32)
    assert_close("O(f32 out)", o32[:, rows], O, 1e-2)
    assert_close("LSE", l32[:, :, rows], L, 1e-2)
    o16, l16 = _run(q, k, v, valid, scale, True, torch.bfloat16)
    assert_close("O(bf16 out)", o16[:, rows], O, 1e-2, bf16_out=True)
    assert np.array_equal(l16, l32)


@pytest.mark.parametrize("masked", [False, True])
def test_fwd_noncausal_wide_ragged(masked):
    """A non-causal run long enough for the 8-wave workgroups (n = 16390,
    32q/8kv heads, d128: 2056 of them, the last block ragged): stratified
    rows and the last 70, against the oracle.  The scale 0.25 (scores of
    standard deviation 2.8) concentrates each row's softmax on a few dozen
    of its 16390 keys, so a tile left out or counted twice moves O and LSE
    well past the tolerance."""
    n, Hq, Hkv, D = 16390, 32, 8, 128
    say(f"fwd non-causal wide workgroups n={n} masked={masked}")
    q, k, v, valid = _inputs(16390 + masked, n, Hq, Hkv, D, masked)
    g = synth.streams(98)
    rows = np.unique(np.concatenate([synth.stratified_rows(g[6], n, 16, None if valid is None else valid[0]),
                                     np.arange(n - 70, n)]))
    scale = 0.25
    O, L = oracle.attn_fwd(to_f64(q), to_f64(k), to_f64(v), scale, False, valid, rows=rows)
    o32, l32 = _run(q, k, v, valid, scale, False, torch.float32)
    assert_close("O(f32 out)", o32[:, rows], O, 1e-2)
    assert_close("LSE", l32[:, :, rows], L, 1e-2)


def test_fwd_96k_docs_workload_sampled():
    """Workload 4 forward: n=98304 with packed documents (padding keys masked)."""
    say("fwd workload 4 (96K, documents) sampled rows")
    d, w, rows = _sampled(4, 48)
    valid = d["valid"]
    O, L = oracle.attn_fwd(to_f64(d["q"]), to_f64(d["k"]), to_f64(d["v"]), w.scale, True, valid, rows=rows)
    o16, l = _run(d["q"], d["k"], d["v"], valid, w.scale, True, torch.bfloat16)
    assert_close("O(bf16 out)", o16[:, rows], O, 1e-2, bf16_out=True)
    assert_close("LSE", l[:, :, rows], L, 1e-2)


def test_fwd_1m_workload_sampled():
    """Workload 5: n=1,048,576, one query head and one KV head, d128 -- 64
    seeded rows plus rows 0 and n-1."""
    say("fwd workload 5 (1M) sampled rows")
    d = synth.local_attention_inputs(5)
    w = d["workload"]
    rows = synth.sample_rows(d["row_gen"], w.n, 64, extra=(0, w.n - 1))
    O, L = oracle.attn_fwd(to_f64(d["q"]), to_f64(d["k"]), to_f64(d["v"]), w.scale, True, rows=rows, block=16)
    o16, l = _run(d["q"], d["k"], d["v"], None, w.scale, True, torch.bfloat16)
    assert_close("O(bf16 out)", o16[:, rows], O, 1e-2, bf16_out=True)
    assert_close("LSE", l[:, :, rows], L, 1e-2)


def test_fwd_masked_keys_inert_and_deterministic():
    """Perturbing padding keys leaves O and LSE bitwise unchanged; a repeat
    run is bitwise identical."""
    say("fwd masked-key perturbation + determinism")
    n = 1500
    q, k, v, valid = _inputs(5, n, 8, 2, 128, True)
    o1, l1 = _run(q, k, v, valid, 0.09, True, torch.bfloat16)
    o1b, l1b = _run(q, k, v, valid, 0.09, True, torch.bfloat16)
    assert np.array_equal(o1, o1b) and np.array_equal(l1, l1b)
    pad = valid[0] == 0
    k2, v2 = k.copy(), v.copy()
    g = synth.streams(55)
    k2[0, pad] = synth.normal_bf16(g[0], k2[0, pad].shape)
    v2[0, pad] = synth.normal_bf16(g[1], v2[0, pad].shape)
    o2, l2 = _run(q, k2, v2, valid, 0.09, True, torch.bfloat16)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_fwd_heads_independent():
    """All heads in one call equal one call per KV group, bitwise."""
    say("fwd heads independent")
    n = 700
    q, k, v, _ = _inputs(6, n, 8, 2, 128, False)
    o, l = _run(q, k, v, None, 0.1, True, torch.float32)
    for gi in range(2):
        og, lg = _run(np.ascontiguousarray(q[:, :, 4 * gi:4 * gi + 4]), np.ascontiguousarray(k[:, :, gi:gi + 1]),
                      np.ascontiguousarray(v[:, :, gi:gi + 1]), None, 0.1, True, torch.float32)
        assert np.array_equal(og, o[:, :, 4 * gi:4 * gi + 4]) and np.array_equal(lg, l[:, 4 * gi:4 * gi + 4])


def test_fwd_fully_masked_rows():
    """Rows whose every visible key is padding: O = 0, LSE = -inf."""
    say("fwd fully masked rows")
    n = 200
    q, k, v, _ = _inputs(8, n, 4, 1, 64, False)
    valid = np.ones((1, n), dtype=np.uint8)
    valid[0, :70] = 0
    o, l = _run(q, k, v, valid, 0.125, True, torch.float32)
    assert np.all(o[0, :70] == 0.0) and np.all(np.isneginf(l[0, :, :70]))
    O, L = oracle.attn_fwd(to_f64(q), to_f64(k), to_f64(v), 0.125, True, valid)
    assert_close("O", o, O, 1e-2)
    assert_close("LSE", l, L, 1e-2)
