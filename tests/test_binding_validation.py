"""The Python binding checks every tensor's shape, dtype and device against
the leading tensor before it calls the library (no GPU needed).

The library receives raw pointers and derives every extent from q's shape
(or src's), so an undersized or differently typed buffer would be read or
written out of bounds on the device.  Here the library is replaced by a
stub that fails the test if any entry point is reached, the device check is
bypassed (CPU tensors stand in for device tensors), and each argument in
turn is given a wrong shape or dtype: every case must raise ValueError
before a call."""
import pytest
import torch

import ulysses_sequence_parallelism_head_amd as U


class _NoCall:
    def __getattr__(self, name):
        if name.startswith("ulysses_attn_bwd_workspace_bytes"):
            return lambda B, n, Hq, Hkv, D: 2 * B * n * Hq * 4
        def fail(*a, **k):
            raise AssertionError(f"library entry point {name} reached with an invalid argument")
        return fail


@pytest.fixture
def stub(monkeypatch):
    monkeypatch.setattr(U, "load_library", lambda *a, **k: _NoCall())
    monkeypatch.setattr(U, "_need_contig_cuda", lambda *ts: None)
    monkeypatch.setattr(U, "_stream", lambda dev: None)


B, n, Hq, Hkv, D = 1, 64, 8, 2, 128
bf, f32 = torch.bfloat16, torch.float32


def _good():
    return {
        "q": torch.zeros(B, n, Hq, D, dtype=bf), "k": torch.zeros(B, n, Hkv, D, dtype=bf),
        "v": torch.zeros(B, n, Hkv, D, dtype=bf), "o": torch.zeros(B, n, Hq, D, dtype=bf),
        "lse": torch.zeros(B, Hq, n, dtype=f32), "dout": torch.zeros(B, n, Hq, D, dtype=bf),
        "key_valid": torch.ones(B, n, dtype=torch.uint8), "doc_start": torch.zeros(B, n, dtype=torch.int32),
        "dq": torch.zeros(B, n, Hq, D, dtype=f32), "dk": torch.zeros(B, n, Hkv, D, dtype=f32),
        "dv": torch.zeros(B, n, Hkv, D, dtype=f32),
    }


BAD_BWD = [
    ("k", torch.zeros(B, n - 1, Hkv, D, dtype=bf)),
    ("k", torch.zeros(B, n, Hkv, D, dtype=f32)),
    ("v", torch.zeros(B, n, Hkv, D - 64, dtype=bf)),
    ("o", torch.zeros(B, n, Hq - 1, D, dtype=bf)),
    ("o", torch.zeros(B, n, Hq, D, dtype=torch.float16)),
    ("lse", torch.zeros(B, n, Hq, dtype=f32)),
    ("lse", torch.zeros(B, Hq, n, dtype=bf)),
    ("dout", torch.zeros(B, n, Hq, D // 2, dtype=bf)),
    ("dout", torch.zeros(B, n, Hq, D, dtype=f32)),
    ("key_valid", torch.ones(B, n, dtype=torch.int32)),
    ("key_valid", torch.ones(B, n + 1, dtype=torch.uint8)),
    ("doc_start", torch.zeros(B, n, dtype=torch.int64)),
    ("dq", torch.zeros(B, n, Hq, D, dtype=bf)),
    ("dq", torch.zeros(B, n // 2, Hq, D, dtype=f32)),
    ("dk", torch.zeros(B, n, Hq, D, dtype=f32)),
    ("dv", torch.zeros(B, n, Hkv, D, dtype=bf)),
]


@pytest.mark.parametrize("docs", [False, True])
@pytest.mark.parametrize("name,bad", BAD_BWD)
def test_bwd_rejects_before_call(stub, name, bad, docs):
    a = _good()
    a[name] = bad
    if name == "doc_start" and not docs:
        pytest.skip("doc_start is an argument of the documents entry point only")
    with pytest.raises(ValueError):
        if docs:
            U.ulysses_attn_bwd_docs(a["q"], a["k"], a["v"], a["o"], a["lse"], a["dout"], a["doc_start"],
                                    a["key_valid"], dq=a["dq"], dk=a["dk"], dv=a["dv"])
        else:
            U.ulysses_attn_bwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["dout"], a["key_valid"],
                               dq=a["dq"], dk=a["dk"], dv=a["dv"])


BAD_FWD = [
    ("k", torch.zeros(B, n, Hkv + 1, D, dtype=bf)),
    ("v", torch.zeros(B, n, Hkv, D, dtype=f32)),
    ("key_valid", torch.ones(n, dtype=torch.uint8)),
    ("out", torch.zeros(B, n, Hq, D - 1, dtype=bf)),
    ("out", torch.zeros(B, n, Hq, D, dtype=torch.float16)),
    ("lse", torch.zeros(B, Hq, n - 1, dtype=f32)),
    ("lse", torch.zeros(B, Hq, n, dtype=torch.float64)),
]


@pytest.mark.parametrize("name,bad", BAD_FWD)
def test_fwd_rejects_before_call(stub, name, bad):
    a = _good()
    a["out"], a["lse"] = a["o"], a["lse"]
    a[name] = bad
    with pytest.raises(ValueError):
        U.ulysses_attn_fwd(a["q"], a["k"], a["v"], a["key_valid"], out=a["out"], lse=a["lse"])
    with pytest.raises(ValueError):
        U.ulysses_attn_fwd_docs(a["q"], a["k"], a["v"], a["doc_start"], a["key_valid"], out=a["out"], lse=a["lse"])


def test_fwd_out_dtype_must_match_o_dtype(stub):
    a = _good()
    with pytest.raises(ValueError):
        U.ulysses_attn_fwd(a["q"], a["k"], a["v"], o_dtype=torch.float32, out=a["o"])   # o is bf16


def test_block_rejects_before_call(stub):
    a = _good()
    o32 = torch.zeros(B, n, Hq, D, dtype=f32)
    for bad in (("o", a["o"]), ("lse", torch.zeros(B, Hq, n + 1, dtype=f32)), ("v", a["dk"])):
        kw = {"o": o32, "lse": a["lse"], "v": a["v"]}
        kw[bad[0]] = bad[1]
        with pytest.raises(ValueError):
            U.ulysses_attn_fwd_block(a["q"], a["k"], kw["v"], kw["o"], kw["lse"], 0)


def test_repack_and_proj_outputs_checked(stub):
    x = torch.zeros(4, 1, 16, 8, 64, dtype=bf)
    with pytest.raises(ValueError):
        U.ulysses_repack_seq2head(x, out=torch.zeros(4, 1, 64, 2, 32, dtype=bf))
    with pytest.raises(ValueError):
        U.ulysses_repack_head2seq(torch.zeros(4, 1, 64, 2, 64, dtype=bf), out=torch.zeros(4, 1, 16, 8, 64, dtype=f32))
    xs = torch.zeros(4, 1, 16, 256, dtype=bf)
    w = torch.zeros((8 + 2 * 4) * 32, 256, dtype=bf)
    with pytest.raises(ValueError):
        U.ulysses_qkv_proj_seq2head(xs, w, 8, 4, 32, q=torch.zeros(4, 1, 64, 1, 32, dtype=bf))
    o = torch.zeros(4, 1, 64, 2, 32, dtype=bf)
    with pytest.raises(ValueError):
        U.ulysses_head2seq_out_proj(o, torch.zeros(256, 256, dtype=bf), y=torch.zeros(4, 1, 16, 128, dtype=bf))
    with pytest.raises(ValueError):
        U.ulysses_loss_aggregate(torch.zeros(4, 8, dtype=f32), rank_sum=torch.zeros(4, dtype=f32))


def test_good_arguments_reach_the_library(stub):
    """Control: with every argument right, the binding does call the library
    (the stub then fails the call)."""
    a = _good()
    with pytest.raises(AssertionError, match="ulysses_attn_bwd"):
        U.ulysses_attn_bwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["dout"], a["key_valid"],
                           dq=a["dq"], dk=a["dk"], dv=a["dv"])
    with pytest.raises(AssertionError, match="ulysses_attn_bwd_docs"):
        U.ulysses_attn_bwd_docs(a["q"], a["k"], a["v"], a["o"], a["lse"], a["dout"], a["doc_start"], a["key_valid"])
    with pytest.raises(AssertionError, match="ulysses_attn_fwd"):
        U.ulysses_attn_fwd(a["q"], a["k"], a["v"], a["key_valid"], out=a["o"], lse=a["lse"])
