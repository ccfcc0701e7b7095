"""Pins for the oracle's attention (O1) and split/combine (O2), against things
other than the oracle itself: exact brute force, a library routine, closed
forms and invariants.

Each pin is chosen so that a plausible slip in the oracle (a dropped term, a
stray factor on the QK product as chased in "CURRENT ISSUE: UMMA QK GEMM -- 4x
Scaling Bug", a wrong GQA head index, a wrong causal offset, a transposed
operand) makes at least one of them fail.
"""
import math
from fractions import Fraction

import mpmath
import numpy as np
import pytest
import torch

import oracle
from workloads import default_scale, make_qkv

mpmath.mp.dps = 50


def _bits(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def _exact(t):
    """bf16 tensor -> nested Fractions (exact)."""
    return np.vectorize(lambda x: Fraction(float(x)), otypes=[object])(t.float().numpy())


def brute_force(q, k, v, scale, causal):
    """Exact rational scores, 50-digit exponentials.  Independent of oracle.c."""
    B, Hq, Sq, D = q.shape
    _, Hkv, Sk, Dv = v.shape
    G = Hq // Hkv
    Q, K, V = _exact(q), _exact(k), _exact(v)
    sc = Fraction(float(np.float32(scale)))
    o = np.zeros((B, Hq, Sq, Dv))
    lse = np.zeros((B, Hq, Sq))
    for b in range(B):
        for h in range(Hq):
            kv = h // G
            for i in range(Sq):
                vis = [j for j in range(Sk) if (not causal) or j <= i + Sk - Sq]
                s = [sc * sum(Q[b, h, i, d] * K[b, kv, j, d] for d in range(D)) for j in vis]
                sm = [mpmath.mpf(x.numerator) / x.denominator for x in s]
                m = max(sm)
                w = [mpmath.exp(x - m) for x in sm]
                l = mpmath.fsum(w)
                for d in range(Dv):
                    num = mpmath.fsum(w[t] * mpmath.mpf(float(V[b, kv, vis[t], d]))
                                      for t in range(len(vis)))
                    o[b, h, i, d] = float(num / l)
                lse[b, h, i] = float(m + mpmath.log(l))
    return o, lse


def run_oracle(q, k, v, scale, causal, rows=None):
    B, Hq, Sq, D = q.shape
    _, Hkv, Sk, Dv = v.shape
    o, lse = oracle.attention(_bits(q), _bits(k), _bits(v), B=B, Hq=Hq, Hkv=Hkv, Sq=Sq, Sk=Sk,
                              D=D, Dv=Dv, scale=scale, causal=causal, rows=rows)
    if rows is None:
        return o.reshape(B, Hq, Sq, Dv), lse.reshape(B, Hq, Sq)
    return o, lse


TINY = [
    # B, Hq, Hkv, Sq, Sk, D, Dv, causal
    (1, 1, 1, 1, 1, 1, 1, False),
    (1, 1, 1, 3, 5, 2, 2, False),
    (2, 2, 1, 4, 7, 3, 5, False),   # GQA 2:1, Dv != D
    (1, 2, 2, 5, 5, 4, 4, True),    # causal, square
    (2, 2, 1, 3, 7, 5, 3, True),    # causal, Sq < Sk: bottom-right alignment
    (1, 2, 1, 7, 7, 2, 2, True),
]


@pytest.mark.parametrize("shape", TINY)
def test_brute_force_tiny(shape):
    B, Hq, Hkv, Sq, Sk, D, Dv, causal = shape
    q, k, v = make_qkv(B, Hq, Hkv, Sq, Sk, D, Dv, sigma=1.5, seed=sum(shape))
    scale = float(np.float32(default_scale(D) * 1.7))
    o_ref, lse_ref = brute_force(q, k, v, scale, causal)
    o, lse = run_oracle(q, k, v, scale, causal)
    np.testing.assert_allclose(o, o_ref, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse, lse_ref, rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("G", [1, 4])
def test_matches_torch_sdpa_float64(causal, G):
    """torch's own scaled_dot_product_attention in float64 on the CPU: an
    independent library routine (square Sq == Sk so its top-left causal mask
    coincides with the bottom-right one)."""
    B, Hkv, S, D = 2, 2, 37, 24
    Hq = Hkv * G
    q, k, v = make_qkv(B, Hq, Hkv, S, S, D, sigma=1.0, seed=11 + G)
    scale = default_scale(D)
    ke = k.double().repeat_interleave(G, dim=1)
    ve = v.double().repeat_interleave(G, dim=1)
    ref = torch.nn.functional.scaled_dot_product_attention(
        q.double(), ke, ve, is_causal=causal, scale=float(np.float32(scale)))
    o, lse = run_oracle(q, k, v, scale, causal)
    np.testing.assert_allclose(o, ref.numpy(), rtol=1e-12, atol=1e-12)
    s = (q.double() @ ke.transpose(-1, -2)) * float(np.float32(scale))
    if causal:
        s = s.masked_fill(torch.ones(S, S, dtype=torch.bool).triu(1), float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(s, -1).numpy(), rtol=1e-12, atol=1e-12)


def test_qk_is_the_exact_scalar_dot_product():
    """With a single key the LSE is the score itself: scale * <q, k>.  On
    integer inputs the dot product is an exact integer, and with a power-of-two
    scale so is every product -- no stray factor (the 4x of the QK page)."""
    rng = np.random.default_rng(5)
    for D in (1, 5, 16, 64):
        qi = rng.integers(-8, 9, size=(1, 3, 2, D))
        ki = rng.integers(-8, 9, size=(1, 3, 1, D))
        q = torch.tensor(qi, dtype=torch.bfloat16)
        k = torch.tensor(ki, dtype=torch.bfloat16)
        v = torch.ones((1, 3, 1, D), dtype=torch.bfloat16)
        o, lse = run_oracle(q, k, v, 0.25, False)
        expect = 0.25 * np.einsum("bhid,bhjd->bhi", qi, ki)
        assert np.array_equal(lse, expect.astype(np.float64))
        assert np.array_equal(o, np.ones_like(o))


def test_rows_of_p_sum_to_one():
    """V = 1 everywhere makes O_i = sum_j P_ij."""
    q, k, _ = make_qkv(2, 4, 2, 9, 33, 8, seed=3, sigma=2.0)
    v = torch.ones((2, 2, 33, 8), dtype=torch.bfloat16)
    for causal in (False, True):
        o, _ = run_oracle(q, k, v, 0.35, causal)
        assert np.max(np.abs(o - 1.0)) <= 1e-12


def test_identical_keys_give_mean_of_v():
    B, Hq, Hkv, Sq, Sk, D = 1, 2, 1, 6, 11, 8
    q, k, v = make_qkv(B, Hq, Hkv, Sq, Sk, D, seed=4)
    k = k[:, :, :1, :].expand(B, Hkv, Sk, D).contiguous()
    scale = default_scale(D)
    for causal in (False, True):
        o, lse = run_oracle(q, k, v, scale, causal)
        vv = v.double().numpy()
        for h in range(Hq):
            for i in range(Sq):
                n_vis = (i + Sk - Sq + 1) if causal else Sk
                mean = vv[0, 0, :n_vis].mean(axis=0)
                np.testing.assert_allclose(o[0, h, i], mean, rtol=0, atol=1e-13)
                s = float(np.float32(scale)) * float(
                    (q[0, h, i].double() * k[0, 0, 0].double()).sum())
                assert abs(lse[0, h, i] - (s + math.log(n_vis))) <= 1e-12


def test_one_hot_score_picks_that_row():
    Sk, D, jstar = 13, 16, 7
    q = torch.zeros((1, 1, 1, D), dtype=torch.bfloat16)
    q[0, 0, 0, 0] = 512.0
    k = torch.zeros((1, 1, Sk, D), dtype=torch.bfloat16)
    k[0, 0, jstar, 0] = 1.0
    _, _, v = make_qkv(1, 1, 1, 1, Sk, D, seed=9)
    o, lse = run_oracle(q, k, v, 0.125, False)   # score 64 against 0
    np.testing.assert_allclose(o[0, 0, 0], v[0, 0, jstar].double().numpy(), rtol=0, atol=1e-25)
    assert abs(lse[0, 0, 0] - 64.0) <= 1e-12


def test_zero_scores_and_single_key():
    B, Hq, Hkv, Sq, Sk, D = 1, 3, 3, 4, 9, 4
    _, k, v = make_qkv(B, Hq, Hkv, Sq, Sk, D, seed=7)
    q = torch.zeros((B, Hq, Sq, D), dtype=torch.bfloat16)
    o, lse = run_oracle(q, k, v, 0.5, False)
    np.testing.assert_allclose(o, np.broadcast_to(v.double().numpy().mean(axis=2, keepdims=True),
                                                  o.shape), atol=1e-14, rtol=0)
    np.testing.assert_allclose(lse, math.log(Sk), atol=1e-14, rtol=0)
    q, k, v = make_qkv(2, 2, 2, 3, 1, 8, seed=8)
    o, lse = run_oracle(q, k, v, 0.3, False)
    np.testing.assert_array_equal(o, np.broadcast_to(v.double().numpy(), o.shape))


def test_causal_row_equals_prefix_attention():
    B, H, S, D = 1, 2, 10, 8
    q, k, v = make_qkv(B, H, H, S, S, D, seed=12)
    o, lse = run_oracle(q, k, v, 0.4, True)
    for i in range(S):
        oi, li = run_oracle(q[:, :, i:i + 1].contiguous(), k[:, :, :i + 1].contiguous(),
                            v[:, :, :i + 1].contiguous(), 0.4, False)
        np.testing.assert_allclose(o[:, :, i], oi[:, :, 0], rtol=0, atol=1e-15)
        np.testing.assert_allclose(lse[:, :, i], li[:, :, 0], rtol=0, atol=1e-15)


def test_row_subset_matches_full_evaluation():
    q, k, v = make_qkv(2, 4, 2, 5, 17, 8, seed=13)
    o, lse = run_oracle(q, k, v, 0.3, True)
    rows = np.array([0, 3, 17, 39], dtype=np.int64)
    os_, ls_ = run_oracle(q, k, v, 0.3, True, rows=rows)
    np.testing.assert_array_equal(os_, o.reshape(-1, 8)[rows])
    np.testing.assert_array_equal(ls_, lse.reshape(-1)[rows])


@pytest.mark.parametrize("nsplit", [1, 2, 3, 7, 16])
def test_split_then_combine_equals_whole(nsplit):
    B, Hq, Hkv, Sq, Sk, D = 2, 4, 2, 3, 50, 8
    q, k, v = make_qkv(B, Hq, Hkv, Sq, Sk, D, seed=20 + nsplit)
    o, lse = run_oracle(q, k, v, 0.3, False)
    chunk = -(-Sk // nsplit)
    op, lp = oracle.attention_splits(_bits(q), _bits(k), _bits(v), B=B, Hq=Hq, Hkv=Hkv, Sq=Sq,
                                     Sk=Sk, D=D, scale=0.3, nsplit=nsplit, chunk=chunk)
    oc, lc = oracle.combine(op, lp)
    np.testing.assert_allclose(oc, o.reshape(-1, D), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lc, lse.reshape(-1), rtol=0, atol=1e-12)


def test_combine_with_empty_splits():
    """Splits past the end of the keys are empty (lse = -inf) and weigh 0."""
    B, Hq, Hkv, Sq, Sk, D = 1, 2, 1, 1, 5, 4
    q, k, v = make_qkv(B, Hq, Hkv, Sq, Sk, D, seed=30)
    op, lp = oracle.attention_splits(_bits(q), _bits(k), _bits(v), B=B, Hq=Hq, Hkv=Hkv, Sq=Sq,
                                     Sk=Sk, D=D, scale=0.5, nsplit=4, chunk=2)
    assert np.isneginf(lp[:, 3]).all() and (op[:, 3] == 0).all()
    oc, lc = oracle.combine(op, lp)
    o, lse = run_oracle(q, k, v, 0.5, False)
    np.testing.assert_allclose(oc, o.reshape(-1, D), rtol=0, atol=1e-13)
    np.testing.assert_allclose(lc, lse.reshape(-1), rtol=0, atol=1e-13)


def test_a_planted_mistake_is_caught():
    """Guard the guards: a stray factor 4 on the scores (the QK page's bug)
    must break the brute-force pin by far more than its tolerance."""
    q, k, v = make_qkv(1, 1, 1, 3, 5, 2, seed=2, sigma=1.5)
    o_ref, lse_ref = brute_force(q, k, v, 0.5, False)
    o_bad, lse_bad = run_oracle(q, k, v, 2.0, False)
    assert np.max(np.abs(lse_bad - lse_ref)) > 1e-3
