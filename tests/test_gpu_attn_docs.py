"""GPU parity of document-masked causal attention (packed variable-length
documents: a token sees only earlier tokens of its own document) against
the fp64 oracle, forward and backward, on the same bf16-rounded inputs.

Tolerances are those of the plain attention tests: max-abs 1e-2 (a bf16 O
only widens it where |O| >= 4, by its own storage half-ulp; the gradients
keep 1e-2 with either O), 5e-5 for the fp32 path.

Layouts cover what the tile skipping and the lower mask must get right:
documents shorter than a tile, boundaries exactly on and next to tile and
workgroup edges, one-token documents, a single document (which must match
the plain causal kernels), padding keys inside documents, two
batch entries with different layouts, and a sliding window (a
non-decreasing per-row bound that is not a document split).  The full-size
documents workload (n = 98304) is checked on rows the oracle computes one
by one.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import ulysses_sequence_parallelism_head_amd as U
from tests.gpu_helpers import say, bits_to_device, f32_to_device, to_f64, to_host_f64, assert_close

pytestmark = pytest.mark.gpu


def starts_from_lengths(lengths):
    out = np.empty(sum(lengths), dtype=np.int32)
    pos = 0
    for L in lengths:
        out[pos:pos + L] = pos
        pos += L
    return out


def random_lengths(gen, n, mean):
    """Document lengths ~ U{1..2*mean-1} packed to exactly n tokens."""
    out, tot = [], 0
    while tot < n:
        L = min(int(gen.integers(1, 2 * mean)), n - tot)
        out.append(L)
        tot += L
    return out


def layout(name, n, seed):
    gen = np.random.default_rng(seed)
    if name == "one":                  # a single document: plain causal attention
        return np.zeros(n, dtype=np.int32)
    if name == "tokens":               # every token its own document
        return np.arange(n, dtype=np.int32)
    if name == "edges":                # boundaries on and next to tile/workgroup edges
        cuts = sorted({c for c in (31, 32, 33, 63, 64, 65, 127, 128, 129, 200, 255, 256, 257, 511, 512, 700)
                       if 0 < c < n})
        lengths = np.diff([0] + cuts + [n]).tolist()
        return starts_from_lengths(lengths)
    if name == "short":                # many documents shorter than a tile
        return starts_from_lengths(random_lengths(gen, n, 20))
    if name == "mixed":
        return starts_from_lengths(random_lengths(gen, n, max(2, n // 6)))
    if name == "window":               # sliding window of 100 keys
        return np.maximum(0, np.arange(n) - 99).astype(np.int32)
    raise ValueError(name)


def _inputs(seed, n, Hq, Hkv, D, masked, names, dtype="bf16"):
    """B = len(names) batch entries, entry b laid out by names[b]."""
    B = len(names)
    g = synth.streams(seed)
    if dtype == "bf16":
        draw = synth.normal_bf16
    else:
        def draw(gen, shape):
            return gen.standard_normal(shape, dtype=np.float32)
    q = draw(g[0], (B, n, Hq, D))
    k = draw(g[1], (B, n, Hkv, D))
    v = draw(g[2], (B, n, Hkv, D))
    do = draw(g[3], (B, n, Hq, D))
    ds = np.stack([layout(nm, n, seed + b) for b, nm in enumerate(names)])
    valid = None
    if masked:
        valid = (g[4].random((B, n)) > 0.2).astype(np.uint8)
    return q, k, v, do, ds, valid


def _dev(x):
    return bits_to_device(x) if x.dtype == np.uint16 else f32_to_device(x)


def _opt(x):
    return None if x is None else torch.from_numpy(np.ascontiguousarray(x)).to("cuda:0")


def _gpu(q, k, v, do, ds, valid, scale, o_dtype, backward=True):
    tq, tk, tv = _dev(q), _dev(k), _dev(v)
    tds, tval = _opt(ds), _opt(valid)
    o, lse = U.ulysses_attn_fwd_docs(tq, tk, tv, tds, tval, scale, o_dtype=o_dtype)
    out = {"o": o, "lse": lse}
    if backward:
        out["dq"], out["dk"], out["dv"] = U.ulysses_attn_bwd_docs(tq, tk, tv, o, lse, _dev(do), tds, tval, scale)
    torch.cuda.synchronize()
    return {key: to_host_f64(t) for key, t in out.items()}


FWD_CASES = [
    # n, Hq, Hkv, D, masked, layouts (one per batch entry)
    (1, 1, 1, 128, False, ("one",)),
    (77, 4, 1, 128, False, ("tokens",)),
    (300, 8, 2, 128, False, ("edges",)),
    (300, 8, 2, 128, True, ("short",)),
    (777, 8, 2, 128, True, ("mixed",)),
    (513, 2, 2, 64, False, ("edges",)),
    (640, 6, 2, 128, True, ("mixed",)),      # g = 3
    (900, 8, 1, 64, False, ("window",)),     # g = 8
    (1024, 8, 2, 128, True, ("mixed", "short")),
    (2500, 8, 2, 128, False, ("mixed",)),
]


@pytest.mark.parametrize("n,Hq,Hkv,D,masked,names", FWD_CASES)
@pytest.mark.parametrize("o_dtype", [torch.float32, torch.bfloat16])
def test_docs_fwd(n, Hq, Hkv, D, masked, names, o_dtype):
    say(f"docs fwd n={n} Hq={Hq} Hkv={Hkv} D={D} masked={masked} layouts={names} o={o_dtype}")
    q, k, v, _, ds, valid = _inputs(11 * n + Hq, n, Hq, Hkv, D, masked, names)
    scale = D ** -0.5
    O, L = oracle.attn_fwd(to_f64(q), to_f64(k), to_f64(v), scale, True, valid, doc_start=ds)
    got = _gpu(q, k, v, None, ds, valid, scale, o_dtype, backward=False)
    assert_close("O", got["o"], O, 1e-2, bf16_out=o_dtype == torch.bfloat16)
    assert_close("LSE", got["lse"], L, 1e-2)


@pytest.mark.parametrize("n,Hq,Hkv,D,masked,names", [(333, 4, 4, 64, True, ("mixed",)),
                                                     (260, 2, 1, 128, False, ("edges", "tokens"))])
def test_docs_fwd_f32(n, Hq, Hkv, D, masked, names):
    say(f"docs fwd fp32 n={n} Hq={Hq} Hkv={Hkv} D={D} layouts={names}")
    q, k, v, _, ds, valid = _inputs(5 * n + 3, n, Hq, Hkv, D, masked, names, dtype="f32")
    scale = D ** -0.5
    O, L = oracle.attn_fwd(to_f64(q), to_f64(k), to_f64(v), scale, True, valid, doc_start=ds)
    got = _gpu(q, k, v, None, ds, valid, scale, torch.float32, backward=False)
    assert_close("O", got["o"], O, 5e-5)
    assert_close("LSE", got["lse"], L, 5e-5)


BWD_CASES = [
    (1, 1, 1, 128, False, ("one",)),
    (130, 8, 2, 128, False, ("tokens",)),
    (300, 8, 2, 128, True, ("edges",)),
    (400, 8, 2, 128, True, ("short",)),
    (777, 8, 2, 128, True, ("mixed",)),
    (513, 2, 2, 64, False, ("edges",)),
    (640, 6, 2, 128, False, ("mixed",)),     # g = 3
    (900, 8, 1, 64, True, ("window",)),      # g = 8
    (1024, 8, 2, 128, True, ("mixed", "edges")),
    (2500, 8, 2, 128, False, ("mixed",)),
]


@pytest.mark.parametrize("n,Hq,Hkv,D,masked,names", BWD_CASES)
@pytest.mark.parametrize("o_dtype", [torch.float32, torch.bfloat16])
def test_docs_bwd(n, Hq, Hkv, D, masked, names, o_dtype):
    say(f"docs bwd n={n} Hq={Hq} Hkv={Hkv} D={D} masked={masked} layouts={names} o={o_dtype}")
    q, k, v, do, ds, valid = _inputs(13 * n + Hq, n, Hq, Hkv, D, masked, names)
    scale = D ** -0.5
    dQ, dK, dV, O, L = oracle.attn_bwd(to_f64(q), to_f64(k), to_f64(v), to_f64(do), scale, True, valid,
                                       doc_start=ds)
    got = _gpu(q, k, v, do, ds, valid, scale, o_dtype)
    assert_close("dQ", got["dq"], dQ, 1e-2)
    assert_close("dK", got["dk"], dK, 1e-2)
    assert_close("dV", got["dv"], dV, 1e-2)


def test_single_document_matches_causal_bitwise():
    """doc_start = 0 everywhere is plain causal attention: the document
    kernels must give the causal kernels' O, LSE and dQ bit for bit.  dK and
    dV sum the same terms, but the document kernel visits every key block's
    query tiles from the last down while the causal kernel visits half of
    them upwards, so those agree to float32 rounding of the sums.
    (n = 16400: long enough for the plain causal forward's shared-tile
    workgroups, whose arithmetic is the 4-wave kernel's; short plain causal
    runs split each block's keys between two wave groups and merge them,
    which rounds differently.)"""
    say("docs: one document == causal, bitwise")
    n, Hq, Hkv, D = 16400, 8, 2, 128
    q, k, v, do, ds, valid = _inputs(99, n, Hq, Hkv, D, True, ("one",))
    scale = D ** -0.5
    got = _gpu(q, k, v, do, ds, valid, scale, torch.bfloat16)
    tq, tk, tv, tval = _dev(q), _dev(k), _dev(v), _opt(valid)
    o, lse = U.ulysses_attn_fwd(tq, tk, tv, tval, scale, True, o_dtype=torch.bfloat16)
    dq, dk, dv = U.ulysses_attn_bwd(tq, tk, tv, o, lse, _dev(do), tval, scale, True)
    torch.cuda.synchronize()
    for name, ref in (("o", o), ("lse", lse), ("dq", dq)):
        assert np.array_equal(got[name], to_host_f64(ref)), name
    for name, ref in (("dk", dk), ("dv", dv)):
        r = to_host_f64(ref)
        assert np.max(np.abs(got[name] - r)) <= 1e-5 * max(1.0, float(np.max(np.abs(r)))), name


def test_documents_are_isolated():
    """Changing one document's K and V changes no other document's output
    or gradients (exact: the other documents' tiles are never combined
    with it)."""
    say("docs: isolation")
    n, Hq, Hkv, D = 1200, 8, 2, 128
    lengths = [300, 1, 250, 400, 249]
    ds = starts_from_lengths(lengths).reshape(1, n)
    g = synth.streams(5)
    q = synth.normal_bf16(g[0], (1, n, Hq, D))
    k = synth.normal_bf16(g[1], (1, n, Hkv, D))
    v = synth.normal_bf16(g[2], (1, n, Hkv, D))
    do = synth.normal_bf16(g[3], (1, n, Hq, D))
    a = _gpu(q, k, v, do, ds, None, 0.09, torch.float32)
    k2, v2 = k.copy(), v.copy()
    s, e = 301, 551                                    # the third document
    k2[:, s:e] = synth.normal_bf16(g[5], (1, e - s, Hkv, D))
    v2[:, s:e] = synth.normal_bf16(g[6], (1, e - s, Hkv, D))
    b = _gpu(q, k2, v2, do, ds, None, 0.09, torch.float32)
    other = np.r_[0:s, e:n]
    for name in ("o", "dq", "dk", "dv"):
        assert np.array_equal(a[name][:, other], b[name][:, other]), name
    assert np.array_equal(a["lse"][:, :, other], b["lse"][:, :, other])
    assert not np.array_equal(a["o"][:, s:e], b["o"][:, s:e])


def test_docs_96k_workload_sampled():
    """The documents workload at full size (n = 98304, 8q/2kv, d128, its
    packed documents and padding): O/LSE on stratified rows including every
    document's first rows, dQ on the same rows, dK/dV on keys of the last
    1024 positions; exact zeros of dK/dV at padding keys."""
    say("docs: 96K documents workload, sampled")
    d = synth.local_attention_inputs(4)
    w = d["workload"]
    valid, ds = d["valid"], d["doc_start"]
    starts = np.unique(ds[0])
    extra = [int(x) + o for x in starts for o in (0, 1, 63, 64, 600) if int(x) + o < w.n]
    rows = synth.sample_rows(d["row_gen"], w.n, 40, extra=extra)
    rows = np.unique(np.concatenate([rows, synth.stratified_rows(d["row_gen"], w.n, 16, valid[0])]))
    k_rows = synth.sample_rows(d["row_gen"], w.n, 12, extra=(w.n - 1, w.n - 2, w.n - 1024))
    k_rows = k_rows[k_rows >= w.n - 1024]
    runs = {}
    for o_dtype in (torch.bfloat16, torch.float32):
        got = _gpu(d["q"], d["k"], d["v"], d["do"], ds, valid, w.scale, o_dtype)
        pad = valid[0] == 0
        assert np.all(got["dk"][0, pad] == 0.0) and np.all(got["dv"][0, pad] == 0.0)
        runs[o_dtype] = {"o": got["o"][:, rows], "lse": got["lse"][:, :, rows], "dq": got["dq"][:, rows],
                         "dk": got["dk"][:, k_rows], "dv": got["dv"][:, k_rows]}
        del got
    qf, kf, vf, dof = to_f64(d["q"]), to_f64(d["k"]), to_f64(d["v"]), to_f64(d["do"])
    O, L = oracle.attn_fwd(qf, kf, vf, w.scale, True, valid, rows=rows, doc_start=ds)
    dQs, dKs, dVs = oracle.attn_bwd_sampled(qf, kf, vf, dof, w.scale, True, valid, q_rows=rows, k_rows=k_rows,
                                            doc_start=ds)
    for o_dtype, got in runs.items():
        say(f"  O stored as {o_dtype}")
        assert_close("O rows", got["o"], O, 1e-2, bf16_out=o_dtype == torch.bfloat16)
        assert_close("LSE rows", got["lse"], L, 1e-2)
        assert_close("dQ rows", got["dq"], dQs, 1e-2)
        assert_close("dK rows", got["dk"], dKs, 1e-2)
        assert_close("dV rows", got["dv"], dVs, 1e-2)


def test_docs_deterministic():
    say("docs determinism")
    q, k, v, do, ds, valid = _inputs(71, 1100, 8, 2, 128, True, ("mixed",))
    a = _gpu(q, k, v, do, ds, valid, 0.1, torch.bfloat16)
    b = _gpu(q, k, v, do, ds, valid, 0.1, torch.bfloat16)
    for key in a:
        assert np.array_equal(a[key], b[key]), key
