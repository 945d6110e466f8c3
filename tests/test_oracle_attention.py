"""Pins for the oracle's attention forward/backward (CPU only).

The oracle is checked against things other than itself:
  * hand-derived worked examples (tests/golden/), exact;
  * brute force in pure Python (math.fsum / math.exp) on tiny inputs;
  * the library routine torch.nn.functional.scaled_dot_product_attention on
    the CPU in float64 (grouped-query, causal, boolean mask) and torch
    autograd for the gradients;
  * central finite differences of sum(O * dO);
  * closed forms (Q = 0, equal keys, one token, constant V, a dominant score);
  * invariants (convex combination, heads independent, grouped-query equals
    repeated-KV multi-head, masked keys inert, sharded path equals unsharded).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle.attention import attn_fwd, attn_bwd, attn_bwd_sampled, pipeline_fwd, pipeline_bwd


def rnd(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


# --------------------------------------------------------------------- helpers
def brute_fwd(q, k, v, scale, causal, valid):
    """Pure-Python reference, one row at a time."""
    B, n, Hq, D = q.shape
    Hkv = k.shape[2]
    g = Hq // Hkv
    O = np.zeros((B, n, Hq, D))
    L = np.full((B, Hq, n), -math.inf)
    for b in range(B):
        for h in range(Hq):
            kh = h // g
            for t in range(n):
                keys = [u for u in range(n) if (not causal or u <= t) and (valid is None or valid[b][u])]
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


def torch_ref(q, k, v, dout, scale, causal, valid):
    """torch CPU float64 SDPA + autograd; LSE via torch.logsumexp of masked scores."""
    B, n, Hq, D = q.shape
    tq = torch.tensor(q, dtype=torch.float64).permute(0, 2, 1, 3).contiguous().requires_grad_(True)
    tk = torch.tensor(k, dtype=torch.float64).permute(0, 2, 1, 3).contiguous().requires_grad_(True)
    tv = torch.tensor(v, dtype=torch.float64).permute(0, 2, 1, 3).contiguous().requires_grad_(True)
    mask = torch.ones(n, n, dtype=torch.bool)
    if causal:
        mask = torch.tril(mask)
    mask = mask.expand(B, 1, n, n).clone()
    if valid is not None:
        mask &= torch.tensor(np.asarray(valid) != 0)[:, None, None, :]
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=scale, enable_gqa=True)
    g = Hq // k.shape[2]
    kr = tk.detach().repeat_interleave(g, dim=1)
    s = scale * tq.detach() @ kr.transpose(-1, -2)
    lse = torch.logsumexp(s.masked_fill(~mask, -math.inf), dim=-1)
    out = {"o": o.detach().permute(0, 2, 1, 3).numpy(), "lse": lse.numpy()}
    if dout is not None:
        tdo = torch.tensor(dout, dtype=torch.float64).permute(0, 2, 1, 3)
        (o * tdo).sum().backward()
        out["dq"] = tq.grad.permute(0, 2, 1, 3).numpy()
        out["dk"] = tk.grad.permute(0, 2, 1, 3).numpy()
        out["dv"] = tv.grad.permute(0, 2, 1, 3).numpy()
    return out


def make_valid(seed, B, n, frac=0.3):
    v = (np.random.default_rng(seed).random((B, n)) > frac).astype(np.uint8)
    v[:, 0] = 1          # token 0 valid: every causal row has an allowed key
    return v


# ------------------------------------------------------------- worked examples
def test_worked_example_d1_n3(golden):
    g = golden("worked_attention_d1_n3.txt")
    q = np.array(g["q"]).reshape(1, 3, 1, 1)
    k = np.array(g["k"]).reshape(1, 3, 1, 1)
    v = np.array(g["v"]).reshape(1, 3, 1, 1)
    do = np.array(g["dout"]).reshape(1, 3, 1, 1)
    O, L = attn_fwd(q, k, v, g["scale"], causal=True)
    np.testing.assert_allclose(O.ravel(), g["o"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(L.ravel(), g["lse"], rtol=0, atol=1e-14)
    dq, dk, dv, _, _ = attn_bwd(q, k, v, do, g["scale"], causal=True)
    np.testing.assert_allclose(dq.ravel(), g["dq"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(dk.ravel(), g["dk"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(dv.ravel(), g["dv"], rtol=0, atol=1e-14)


def test_worked_example_gqa_mask(golden):
    g = golden("worked_attention_gqa_mask.txt")
    q = np.array(g["q"]).reshape(1, 3, 2, 1)
    k = np.array(g["k"]).reshape(1, 3, 1, 1)
    v = np.array(g["v"]).reshape(1, 3, 1, 1)
    valid = np.array(g["valid"], dtype=np.uint8).reshape(1, 3)
    O, L = attn_fwd(q, k, v, g["scale"], causal=True, key_valid=valid)
    np.testing.assert_allclose(O[0, :, :, 0], np.array(g["o"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(L[0], np.array(g["lse"]), rtol=0, atol=1e-14)


# ------------------------------------------------------------------ brute force
@pytest.mark.parametrize("n,Hq,Hkv,D,causal,masked", [
    (1, 1, 1, 3, True, False), (5, 2, 1, 4, True, False), (9, 4, 2, 3, True, True),
    (16, 2, 2, 5, True, False), (7, 3, 1, 2, False, True), (12, 4, 1, 8, True, True),
])
def test_fwd_brute_force(n, Hq, Hkv, D, causal, masked):
    B = 2
    q, k, v = rnd(1, B, n, Hq, D), rnd(2, B, n, Hkv, D), rnd(3, B, n, Hkv, D)
    valid = make_valid(4, B, n) if masked else None
    scale = 0.37
    O, L = attn_fwd(q, k, v, scale, causal, valid, block=4)
    Ob, Lb = brute_fwd(q, k, v, scale, causal, valid)
    np.testing.assert_allclose(O, Ob, rtol=0, atol=1e-13)
    np.testing.assert_allclose(L, Lb, rtol=0, atol=1e-13)


def test_fully_masked_row_convention():
    q, k, v = rnd(5, 1, 4, 1, 2), rnd(6, 1, 4, 1, 2), rnd(7, 1, 4, 1, 2)
    valid = np.array([[0, 0, 1, 1]], dtype=np.uint8)
    O, L = attn_fwd(q, k, v, 1.0, True, valid)
    assert np.all(O[0, :2] == 0.0) and np.all(np.isneginf(L[0, 0, :2]))
    Ob, Lb = brute_fwd(q, k, v, 1.0, True, valid)
    np.testing.assert_allclose(O[0, 2:], Ob[0, 2:], atol=1e-14)
    dq, dk, dv, _, _ = attn_bwd(q, k, v, rnd(8, 1, 4, 1, 2), 1.0, True, valid)
    assert np.all(dq[0, :2] == 0.0) and np.all(dk[0, :2] == 0.0) and np.all(dv[0, :2] == 0.0)


# ---------------------------------------------------------- library cross-check
@pytest.mark.parametrize("n,Hq,Hkv,D,causal,masked,scale", [
    (64, 4, 1, 16, True, False, 0.25), (200, 8, 2, 32, True, True, 1 / math.sqrt(32)),
    (96, 2, 2, 8, False, False, 0.5), (257, 4, 4, 64, True, False, 1 / 8),
])
def test_against_torch_sdpa(n, Hq, Hkv, D, causal, masked, scale):
    B = 1
    q, k, v, do = rnd(10, B, n, Hq, D), rnd(11, B, n, Hkv, D), rnd(12, B, n, Hkv, D), rnd(13, B, n, Hq, D)
    valid = make_valid(14, B, n) if masked else None
    ref = torch_ref(q, k, v, do, scale, causal, valid)
    dq, dk, dv, O, L = attn_bwd(q, k, v, do, scale, causal, valid, block=64)
    np.testing.assert_allclose(O, ref["o"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(L, ref["lse"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(dq, ref["dq"], rtol=0, atol=1e-11)
    np.testing.assert_allclose(dk, ref["dk"], rtol=0, atol=1e-11)
    np.testing.assert_allclose(dv, ref["dv"], rtol=0, atol=1e-11)


# ---------------------------------------------------------- finite differences
@pytest.mark.parametrize("n,Hq,Hkv,D,masked", [(6, 2, 1, 3, False), (8, 2, 2, 4, True), (5, 3, 1, 2, True)])
def test_bwd_finite_differences(n, Hq, Hkv, D, masked):
    B = 1
    q, k, v, do = rnd(20, B, n, Hq, D), rnd(21, B, n, Hkv, D), rnd(22, B, n, Hkv, D), rnd(23, B, n, Hq, D)
    valid = make_valid(24, B, n) if masked else None
    scale = 0.6

    def loss(qq, kk, vv):
        O, _ = attn_fwd(qq, kk, vv, scale, True, valid)
        return float(np.sum(O * do))

    dq, dk, dv, _, _ = attn_bwd(q, k, v, do, scale, True, valid)
    eps = 1e-6
    for arr, grad in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            old = arr[idx]
            arr[idx] = old + eps
            lp = loss(q, k, v)
            arr[idx] = old - eps
            lm = loss(q, k, v)
            arr[idx] = old
            num[idx] = (lp - lm) / (2 * eps)
        np.testing.assert_allclose(grad, num, rtol=0, atol=2e-8)


# ------------------------------------------------------------------ closed forms
def test_closed_form_zero_query():
    """Q = 0: uniform weights over allowed keys -> O_t = mean of allowed v,
    LSE_t = ln(#allowed); backward: dK = 0, dV_u = sum over rows t >= u of
    dO_t / (#allowed at t)."""
    n, D = 11, 4
    q = np.zeros((1, n, 2, D))
    k, v, do = rnd(30, 1, n, 1, D), rnd(31, 1, n, 1, D), rnd(32, 1, n, 2, D)
    valid = np.array([[1, 1, 0, 1, 1, 1, 0, 0, 1, 1, 1]], dtype=np.uint8)
    O, L = attn_fwd(q, k, v, 0.9, True, valid)
    dq, dk, dv, _, _ = attn_bwd(q, k, v, do, 0.9, True, valid)
    exp_dv = np.zeros((n, D))
    for t in range(n):
        keys = [u for u in range(t + 1) if valid[0, u]]
        for h in range(2):
            np.testing.assert_allclose(O[0, t, h], v[0, keys, 0].mean(axis=0), atol=1e-14)
            assert abs(L[0, h, t] - math.log(len(keys))) < 1e-14
        for u in keys:
            exp_dv[u] += (do[0, t, 0] + do[0, t, 1]) / len(keys)
    assert np.all(dk == 0.0)
    np.testing.assert_allclose(dv[0, :, 0], exp_dv, atol=1e-13)


def test_closed_form_equal_keys():
    n, D, s = 9, 3, 0.7
    q, v = rnd(33, 1, n, 1, D), rnd(34, 1, n, 1, D)
    kk = rnd(35, D)
    k = np.broadcast_to(kk, (1, n, 1, D)).copy()
    O, L = attn_fwd(q, k, v, s, True)
    for t in range(n):
        np.testing.assert_allclose(O[0, t, 0], v[0, :t + 1, 0].mean(axis=0), atol=1e-14)
        assert abs(L[0, 0, t] - (s * float(q[0, t, 0] @ kk) + math.log(t + 1))) < 1e-13


def test_closed_form_single_token():
    q, k, v = rnd(36, 1, 1, 3, 5), rnd(37, 1, 1, 1, 5), rnd(38, 1, 1, 1, 5)
    O, L = attn_fwd(q, k, v, 0.3, True)
    for h in range(3):
        np.testing.assert_array_equal(O[0, 0, h], v[0, 0, 0])
        assert abs(L[0, h, 0] - 0.3 * float(q[0, 0, h] @ k[0, 0, 0])) < 1e-14


def test_constant_v_and_dominant_score():
    n, D = 10, 4
    q, k = rnd(39, 1, n, 1, D), rnd(40, 1, n, 1, D)
    v = np.full((1, n, 1, D), 2.5)
    O, _ = attn_fwd(q, k, v, 0.5, True)
    np.testing.assert_allclose(O, 2.5, atol=1e-14)
    # key 3 aligned with a huge query: its weight dominates every row t >= 3
    k2 = k.copy()
    k2[0, 3, 0] = 50.0 * np.ones(D)
    q2 = np.ones((1, n, 1, D))
    v2 = rnd(41, 1, n, 1, D)
    O2, _ = attn_fwd(q2, k2, v2, 1.0, True)
    for t in range(3, n):
        np.testing.assert_allclose(O2[0, t, 0], v2[0, 3, 0], atol=1e-12)


# -------------------------------------------------------------------- invariants
def test_convex_combination_and_unit_mass():
    n, D = 40, 6
    q, k, v = rnd(42, 1, n, 2, D), rnd(43, 1, n, 1, D), rnd(44, 1, n, 1, D)
    valid = make_valid(45, 1, n)
    O, L = attn_fwd(q, k, v, 0.8, True, valid)
    for t in range(n):
        keys = [u for u in range(t + 1) if valid[0, u]]
        vv = v[0, keys, 0]
        for h in range(2):
            assert np.all(O[0, t, h] <= vv.max(axis=0) + 1e-12)
            assert np.all(O[0, t, h] >= vv.min(axis=0) - 1e-12)
            s = 0.8 * (k[0, keys, 0] @ q[0, t, h])
            assert abs(math.fsum(np.exp(s - L[0, h, t])) - 1.0) < 1e-13


def test_heads_independent_bitwise():
    n, D = 70, 8
    q, k, v, do = rnd(46, 1, n, 4, D), rnd(47, 1, n, 2, D), rnd(48, 1, n, 2, D), rnd(49, 1, n, 4, D)
    O, L = attn_fwd(q, k, v, 0.3, True, block=16)
    dq, dk, dv, _, _ = attn_bwd(q, k, v, do, 0.3, True, block=16)
    for g in range(2):
        sl = slice(2 * g, 2 * g + 2)
        Og, Lg = attn_fwd(q[:, :, sl], k[:, :, g:g + 1], v[:, :, g:g + 1], 0.3, True, block=16)
        assert np.array_equal(Og, O[:, :, sl]) and np.array_equal(Lg, L[:, sl])
        dqg, dkg, dvg, _, _ = attn_bwd(q[:, :, sl], k[:, :, g:g + 1], v[:, :, g:g + 1], do[:, :, sl], 0.3, True, block=16)
        assert np.array_equal(dqg, dq[:, :, sl])
        assert np.array_equal(dkg, dk[:, :, g:g + 1]) and np.array_equal(dvg, dv[:, :, g:g + 1])


def test_gqa_equals_repeated_kv_mha():
    n, D, g = 33, 5, 4
    q, k, v, do = rnd(50, 1, n, 8, D), rnd(51, 1, n, 2, D), rnd(52, 1, n, 2, D), rnd(53, 1, n, 8, D)
    kr, vr = np.repeat(k, g, axis=2), np.repeat(v, g, axis=2)
    O, L = attn_fwd(q, k, v, 0.4, True)
    Or, Lr = attn_fwd(q, kr, vr, 0.4, True)
    np.testing.assert_array_equal(O, Or)
    np.testing.assert_array_equal(L, Lr)
    dq, dk, dv, _, _ = attn_bwd(q, k, v, do, 0.4, True)
    dqr, dkr, dvr, _, _ = attn_bwd(q, kr, vr, do, 0.4, True)
    np.testing.assert_allclose(dq, dqr, atol=1e-13)
    np.testing.assert_allclose(dk, dkr.reshape(1, n, 2, g, D).sum(axis=3), atol=1e-13)
    np.testing.assert_allclose(dv, dvr.reshape(1, n, 2, g, D).sum(axis=3), atol=1e-13)


def test_masked_keys_inert():
    n, D = 50, 4
    q, k, v, do = rnd(54, 1, n, 2, D), rnd(55, 1, n, 1, D), rnd(56, 1, n, 1, D), rnd(57, 1, n, 2, D)
    valid = make_valid(58, 1, n, 0.4)
    O, L = attn_fwd(q, k, v, 0.5, True, valid)
    dq, dk, dv, _, _ = attn_bwd(q, k, v, do, 0.5, True, valid)
    pad = valid[0] == 0
    k2, v2 = k.copy(), v.copy()
    k2[0, pad] = 1e3 * rnd(59, int(pad.sum()), 1, D)
    v2[0, pad] = -7.0
    O2, L2 = attn_fwd(q, k2, v2, 0.5, True, valid)
    assert np.array_equal(O, O2) and np.array_equal(L, L2)
    dq2, dk2, dv2, _, _ = attn_bwd(q, k2, v2, do, 0.5, True, valid)
    assert np.array_equal(dq, dq2)
    assert np.all(dk[0, pad] == 0.0) and np.all(dv[0, pad] == 0.0)


# ---------------------------------------------------------------- sharded path
@pytest.mark.parametrize("P,nl,Hq,Hkv,D,masked", [(2, 16, 4, 4, 8, False), (4, 9, 8, 4, 4, True), (1, 20, 2, 1, 4, False)])
def test_pipeline_equals_unsharded_bitwise(P, nl, Hq, Hkv, D, masked):
    n = P * nl
    q, k, v, do = rnd(60, 1, n, Hq, D), rnd(61, 1, n, Hkv, D), rnd(62, 1, n, Hkv, D), rnd(63, 1, n, Hq, D)
    valid = make_valid(64, 1, n) if masked else None
    O_seq, L_ranks = pipeline_fwd(oracle.shard(q, P), oracle.shard(k, P), oracle.shard(v, P), 0.35, True, valid, block=8)
    O, L = attn_fwd(q, k, v, 0.35, True, valid, block=8)
    assert np.array_equal(oracle.unshard(O_seq), O)
    hp = Hq // P
    for j in range(P):
        assert np.array_equal(L_ranks[j], L[:, j * hp:(j + 1) * hp])
    dq_s, dk_s, dv_s = pipeline_bwd(oracle.shard(q, P), oracle.shard(k, P), oracle.shard(v, P), oracle.shard(do, P),
                                    0.35, True, valid, block=8)
    dq, dk, dv, _, _ = attn_bwd(q, k, v, do, 0.35, True, valid, block=8)
    assert np.array_equal(oracle.unshard(dq_s), dq)
    assert np.array_equal(oracle.unshard(dk_s), dk)
    assert np.array_equal(oracle.unshard(dv_s), dv)


# ---------------------------------------------------------------- sampled rows
def test_sampled_rows_match_full():
    n, D = 300, 8
    q, k, v, do = rnd(70, 1, n, 4, D), rnd(71, 1, n, 2, D), rnd(72, 1, n, 2, D), rnd(73, 1, n, 4, D)
    valid = make_valid(74, 1, n)
    rows = np.array([0, 1, 63, 64, 65, 150, 298, 299])
    O, L = attn_fwd(q, k, v, 0.3, True, valid, block=32)
    Os, Ls = attn_fwd(q, k, v, 0.3, True, valid, rows=rows, block=3)
    np.testing.assert_allclose(Os, O[:, rows], atol=1e-13)
    np.testing.assert_allclose(Ls, L[:, :, rows], atol=1e-13)
    dq, dk, dv, _, _ = attn_bwd(q, k, v, do, 0.3, True, valid, block=32)
    keys = np.array([3, 64, 200, 299])
    dqs, dks, dvs = attn_bwd_sampled(q, k, v, do, 0.3, True, valid, q_rows=rows, k_rows=keys)
    np.testing.assert_allclose(dqs, dq[:, rows], atol=1e-12)
    np.testing.assert_allclose(dks, dk[:, keys], atol=1e-12)
    np.testing.assert_allclose(dvs, dv[:, keys], atol=1e-12)
