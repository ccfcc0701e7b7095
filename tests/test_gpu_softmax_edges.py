"""GPU parity of the online softmax with O rescale (item 5 of the feature list
on the page "NVFP4-1.1_RAW_CUDA_CPP_APPROACH.md": in-kernel softmax that
rescales the output accumulator across several KV tiles) on inputs built to
stress it, for the prefill kernel and for the split-KV decode (several splits
with a combine, and split groups that stream every split of a unit and combine
in the kernel).  Each output is compared with the fp64 oracle element by
element at the usual tolerances.

The cases:
  * one-hot score: q = c e0 with c * scale = 64, one key with k[0] = 1 and
    k[0] = 0 elsewhere, placed in the last tile of a range of more than 2000
    keys or deep inside a long split -- the running maximum jumps by 92 log2
    units late in the stream and every earlier contribution must vanish;
  * score ramps: the scores of a row rise linearly, 2 to 6 log2 units per 64
    keys depending on the row, and 7.9 and 8.1 units for two rows -- just
    under and just over the lazy-rescale slack of the kernels (8 log2 units),
    so rows of one wave rescale at different tiles;
  * identical keys (P uniform: O is the mean of the visible V rows);
  * Q = 0 (all scores 0: the same closed form);
  * scores of magnitude up to about 1000;
  * causal decode rows for which whole splits (all tiles of a split) are
    masked: with Sq = 4 and a last split holding only the last key, three of
    the four rows see no key of that split (lse_s = -inf, weight 0);
  * a few dominant keys: scores with a standard deviation of 3 or 4 (natural
    log units), so a handful of keys carry each row's softmax and the bf16
    rounding of P is most of the error -- the log-sum-exp must come from the
    sum of the unrounded p (from the bf16 P it was off by up to 2.6e-3).
"""
import numpy as np
import pytest
import torch

import decode_fmha_fwd_amd as F
from gpu_helpers import assert_parity, oracle_rows, poison_like, require_gpu
from workloads import default_scale

pytestmark = pytest.mark.gpu

LOG2E = 1.4426950408889634


def _gen(seed):
    return torch.Generator("cpu").manual_seed(seed)


def _bf16(t):
    return t.to(torch.bfloat16).contiguous()


def one_hot(B, Hq, Hkv, Sq, Sk, D, jstar, seed):
    g = _gen(seed)
    c = 64.0 / default_scale(D)  # c * scale = 64 (512 at D = 64: exact in bf16)
    q = torch.zeros((B, Hq, Sq, D))
    q[..., 0] = c
    k = torch.randn((B, Hkv, Sk, D), generator=g)
    k[..., 0] = 0.0
    k[:, :, jstar, 0] = 1.0
    v = torch.randn((B, Hkv, Sk, D), generator=g)
    return _bf16(q), _bf16(k), _bf16(v)


def ramp(B, Hq, Hkv, Sq, Sk, D, seed, base=4.0, kscale=1.0):
    """Row r of each head rises by base * alpha_r log2 units per 64 keys,
    alpha_r spread over [0.5, 1.5]; two rows per head get 7.9 and 8.1 units.
    kscale moves magnitude from the ramp column of K to that of Q (the same
    scores), so that K stays of order 1 where it also serves as V."""
    g = _gen(seed)
    scale = default_scale(D)
    rows = Hq * Sq
    alpha = torch.linspace(0.5, 1.5, rows)
    if rows >= 4:
        alpha[1] = 7.9 / base
        alpha[rows - 2] = 8.1 / base
    q = torch.randn((B, Hq, Sq, D), generator=g) * 0.1
    q[..., 0] = alpha.view(Hq, Sq) * kscale
    delta = base / (64.0 * scale * LOG2E)  # k[0] step per key for alpha = 1
    k = torch.randn((B, Hkv, Sk, D), generator=g)
    k[..., 0] = torch.arange(Sk, dtype=torch.float32) * (delta / kscale)
    v = torch.randn((B, Hkv, Sk, D), generator=g)
    return _bf16(q), _bf16(k), _bf16(v)


def identical_keys(B, Hq, Hkv, Sq, Sk, D, seed):
    g = _gen(seed)
    q = torch.randn((B, Hq, Sq, D), generator=g)
    k = torch.randn((B, Hkv, 1, D), generator=g).expand(B, Hkv, Sk, D)
    v = torch.randn((B, Hkv, Sk, D), generator=g)
    return _bf16(q), _bf16(k), _bf16(v)


def zero_q(B, Hq, Hkv, Sq, Sk, D, seed):
    g = _gen(seed)
    q = torch.zeros((B, Hq, Sq, D))
    k = torch.randn((B, Hkv, Sk, D), generator=g)
    v = torch.randn((B, Hkv, Sk, D), generator=g)
    return _bf16(q), _bf16(k), _bf16(v)


def large_scores(B, Hq, Hkv, Sq, Sk, D, seed):
    """Scores with a standard deviation of about 250 (maxima near 1000)."""
    g = _gen(seed)
    sig = (250.0 / (np.sqrt(D) * default_scale(D))) ** 0.5
    q = torch.randn((B, Hq, Sq, D), generator=g) * sig
    k = torch.randn((B, Hkv, Sk, D), generator=g) * sig
    v = torch.randn((B, Hkv, Sk, D), generator=g)
    return _bf16(q), _bf16(k), _bf16(v)


def run_fwd(q, k, v, causal):
    dev = require_gpu()
    B, Hq, Sq, D = q.shape
    _, Hkv, Sk, _ = k.shape
    qd = q.to(dev)
    o = poison_like(qd)
    lse = torch.full((B, Hq, Sq), float("nan"), dtype=torch.float32, device=dev)
    F.fmha_fwd(qd, k.to(dev), v.to(dev), o, lse, B, Hq, Hkv, Sq, Sk, D, default_scale(D), causal)
    torch.cuda.synchronize()
    return o, lse


def run_decode(q, k, v, causal, ns):
    dev = require_gpu()
    B, Hq, Sq, D = q.shape
    _, Hkv, Sk, _ = k.shape
    qd = q.to(dev)
    o = poison_like(qd)
    lse = torch.full((B, Hq, Sq), float("nan"), dtype=torch.float32, device=dev)
    nb = F.fmha_decode_splitkv_workspace_size(B, Hq, Hkv, Sq, Sk, D, ns)
    ws = torch.full((max(nb, 16),), 0xFF, dtype=torch.uint8, device=dev)
    F.fmha_decode_splitkv(qd, k.to(dev), v.to(dev), o, lse, B, Hq, Hkv, Sq, Sk, D,
                          default_scale(D), causal, ns, ws, nb)
    torch.cuda.synchronize()
    return o, lse


def few_dominant_keys(B, Hq, Hkv, Sq, Sk, D, seed, sd, Dv=None):
    """Q scaled so that the scores scale * q.k have standard deviation sd."""
    g = _gen(seed)
    sig = sd / (np.sqrt(D) * default_scale(D))
    q = torch.randn((B, Hq, Sq, D), generator=g) * sig
    k = torch.randn((B, Hkv, Sk, D), generator=g)
    v = torch.randn((B, Hkv, Sk, Dv or D), generator=g)
    return _bf16(q), _bf16(k), _bf16(v)


def check(q, k, v, causal, o, lse, what):
    o_ref, lse_ref = oracle_rows(q, k, v, default_scale(q.shape[-1]), causal)
    assert_parity(o, lse, o_ref, lse_ref, what=what)
    return o_ref, lse_ref


# ------------------------------------------------------------------ prefill

PREFILL_SHAPES = [
    # B, Hq, Hkv, S, D, causal
    (1, 2, 1, 2100, 64, False),
    (1, 2, 1, 2100, 64, True),
    (1, 2, 2, 2100, 128, False),
]


@pytest.mark.parametrize("shape", PREFILL_SHAPES)
@pytest.mark.parametrize("jstar", [2090, 1337])
def test_prefill_one_hot_score(shape, jstar):
    B, Hq, Hkv, S, D, causal = shape
    q, k, v = one_hot(B, Hq, Hkv, S, S, D, jstar, seed=jstar)
    o, lse = run_fwd(q, k, v, causal)
    o_ref, _ = check(q, k, v, causal, o, lse, f"one-hot key {jstar} {shape}")
    # rows that see the key pick out its V row (the rest see only zero scores)
    ref = v[0, 0, jstar].double().numpy()
    rows_seeing = jstar if causal else 0  # first row that sees jstar (j <= i when Sq = Sk)
    assert np.abs(o_ref.reshape(B, Hq, S, D)[0, 0, rows_seeing:] - ref).max() < 1e-12


@pytest.mark.parametrize("shape", PREFILL_SHAPES)
def test_prefill_score_ramp_across_the_rescale_slack(shape):
    B, Hq, Hkv, S, D, causal = shape
    q, k, v = ramp(B, Hq, Hkv, S, S, D, seed=5)
    o, lse = run_fwd(q, k, v, causal)
    check(q, k, v, causal, o, lse, f"ramp {shape}")


@pytest.mark.parametrize("make", [identical_keys, zero_q, large_scores])
@pytest.mark.parametrize("causal", [False, True])
def test_prefill_closed_form_and_large_inputs(make, causal):
    B, Hq, Hkv, S, D = 1, 4, 2, 700, 64
    q, k, v = make(B, Hq, Hkv, S, S, D, seed=11)
    o, lse = run_fwd(q, k, v, causal)
    o_ref, _ = check(q, k, v, causal, o, lse, f"{make.__name__} causal={causal}")
    if make is not large_scores:  # closed form: the mean of the visible V rows
        G = Hq // Hkv
        vv = v.double().numpy()
        for h in (0, Hq - 1):
            for i in (0, S // 2, S - 1):
                n = i + 1 if causal else S
                want = vv[0, h // G, :n].mean(axis=0)
                assert np.abs(o_ref.reshape(B, Hq, S, D)[0, h, i] - want).max() < 1e-12


# ------------------------------------------------------------------ split decode

DECODE_SHAPES = [
    # B, Hq, Hkv, Sk, D, num_splits: a few splits combined by the combine kernel,
    # and 512 (batch, KV head) units whose workgroups each stream all splits
    (2, 8, 2, 2100, 64, 4),
    (2, 8, 2, 2100, 128, 3),
    (64, 32, 8, 2100, 64, 8),
    (1, 64, 1, 2100, 512, 5),
]


@pytest.mark.parametrize("shape", DECODE_SHAPES)
@pytest.mark.parametrize("jstar", [2090, 1337])
def test_decode_one_hot_score(shape, jstar):
    B, Hq, Hkv, Sk, D, ns = shape
    q, k, v = one_hot(B, Hq, Hkv, 1, Sk, D, jstar, seed=jstar + 1)
    o, lse = run_decode(q, k, v, False, ns)
    o_ref, _ = check(q, k, v, False, o, lse, f"one-hot key {jstar} {shape}")
    assert np.abs(o_ref.reshape(B, Hq, D)[0, 0] - v[0, 0, jstar].double().numpy()).max() < 1e-12


@pytest.mark.parametrize("shape", DECODE_SHAPES)
def test_decode_score_ramp_across_the_rescale_slack(shape):
    B, Hq, Hkv, Sk, D, ns = shape
    q, k, v = ramp(B, Hq, Hkv, 1, Sk, D, seed=7)
    o, lse = run_decode(q, k, v, False, ns)
    check(q, k, v, False, o, lse, f"ramp {shape}")


@pytest.mark.parametrize("make", [identical_keys, zero_q, large_scores])
@pytest.mark.parametrize("shape", [DECODE_SHAPES[0], DECODE_SHAPES[2]])
def test_decode_closed_form_and_large_inputs(make, shape):
    B, Hq, Hkv, Sk, D, ns = shape
    q, k, v = make(B, Hq, Hkv, 1, Sk, D, seed=13)
    o, lse = run_decode(q, k, v, False, ns)
    o_ref, _ = check(q, k, v, False, o, lse, f"{make.__name__} {shape}")
    if make is not large_scores:
        want = v.double().numpy()[0, 0].mean(axis=0)
        assert np.abs(o_ref.reshape(B, Hq, D)[0, 0] - want).max() < 1e-12


@pytest.mark.parametrize("B,ns", [(2, 9), (256, 9)])
def test_decode_causal_rows_with_fully_masked_splits(B, ns):
    """Sq = 4, causal, Sk = 257 in splits of 32 keys: the last split holds key
    256 only, which only the last query row sees; for the other rows every
    tile of that split is masked.  B = 256 gives 512 units (split groups)."""
    Hq, Hkv, Sq, Sk, D = 8, 2, 4, 257, 64
    g = _gen(17)
    q = _bf16(torch.randn((B, Hq, Sq, D), generator=g))
    k = _bf16(torch.randn((B, Hkv, Sk, D), generator=g))
    v = _bf16(torch.randn((B, Hkv, Sk, D), generator=g))
    o, lse = run_decode(q, k, v, True, ns)
    check(q, k, v, True, o, lse, f"causal masked splits B={B}")


# ------------------------------------------------------------------ V inside the K rows

# B, Hq, Hkv, Sk, D, Dv, num_splits: V aliasing K at head dim 512, and V the
# first 512 columns of 576-wide K rows (64 query rows per KV head: the
# wide-head decode whose two waves per row group add their half-head-dim
# score partials before the softmax)
KVS_SHAPES = [
    (1, 64, 1, 2100, 512, 512, 5),
    (2, 64, 1, 2100, 576, 512, 3),
]


def run_decode_kvs(q, k, Dv, causal, ns):
    dev = require_gpu()
    B, Hq, Sq, D = q.shape
    _, Hkv, Sk, _ = k.shape
    qd, kd = q.to(dev), k.to(dev)
    o = torch.full((B, Hq, Sq, Dv), float("nan"), dtype=torch.bfloat16, device=dev)
    lse = torch.full((B, Hq, Sq), float("nan"), dtype=torch.float32, device=dev)
    nb = F.fmha_decode_splitkv_dv_workspace_size(B, Hq, Hkv, Sq, Sk, D, Dv, ns)
    ws = torch.full((max(nb, 16),), 0xFF, dtype=torch.uint8, device=dev)
    F.fmha_decode_splitkv_dv(qd, kd, kd, o, lse, B, Hq, Hkv, Sq, Sk, D, Dv, default_scale(D),
                             causal, ns, ws, nb)
    torch.cuda.synchronize()
    return o, lse


def check_kvs(q, k, Dv, causal, o, lse, what):
    return check(q, k, k[..., :Dv].contiguous(), causal, o, lse, what)


@pytest.mark.parametrize("shape", KVS_SHAPES)
@pytest.mark.parametrize("jstar", [2090, 1337])
def test_decode_v_in_k_one_hot_score(shape, jstar):
    B, Hq, Hkv, Sk, D, Dv, ns = shape
    q, k, _ = one_hot(B, Hq, Hkv, 1, Sk, D, jstar, seed=jstar + 2)
    o, lse = run_decode_kvs(q, k, Dv, False, ns)
    o_ref, _ = check_kvs(q, k, Dv, False, o, lse, f"V in K, one-hot key {jstar} {shape}")
    want = k[0, 0, jstar, :Dv].double().numpy()
    assert np.abs(o_ref.reshape(B, Hq, Dv)[0, 0] - want).max() < 1e-12


def ramp_small_k(B, Hq, Hkv, Sq, Sk, D, seed):
    return ramp(B, Hq, Hkv, Sq, Sk, D, seed, kscale=1024.0)


def large_scores_small_k(B, Hq, Hkv, Sq, Sk, D, seed):
    """The score distribution of large_scores with all the magnitude in Q
    (K, which is also V here, stays standard normal)."""
    g = _gen(seed)
    sig2 = 250.0 / (np.sqrt(D) * default_scale(D))
    q = torch.randn((B, Hq, Sq, D), generator=g) * sig2
    k = torch.randn((B, Hkv, Sk, D), generator=g)
    return _bf16(q), _bf16(k), None


@pytest.mark.parametrize("shape", KVS_SHAPES)
@pytest.mark.parametrize("make", [ramp_small_k, large_scores_small_k, zero_q])
def test_decode_v_in_k_ramp_large_and_closed_form(shape, make):
    B, Hq, Hkv, Sk, D, Dv, ns = shape
    q, k, _ = make(B, Hq, Hkv, 1, Sk, D, seed=19)
    o, lse = run_decode_kvs(q, k, Dv, False, ns)
    o_ref, _ = check_kvs(q, k, Dv, False, o, lse, f"V in K, {make.__name__} {shape}")
    if make is zero_q:  # all scores 0: the mean of the V rows
        want = k.double().numpy()[0, 0, :, :Dv].mean(axis=0)
        assert np.abs(o_ref.reshape(B, Hq, Dv)[0, 0] - want).max() < 1e-12


@pytest.mark.parametrize("D,Dv", [(512, 512), (576, 512)])
def test_decode_v_in_k_causal_fully_masked_splits(D, Dv):
    """Sq = 4 (64 rows per KV head with 16 heads), causal, Sk = 257 in splits
    of 32 keys: the last split holds key 256 only, which only the last query
    position sees."""
    B, Hq, Hkv, Sq, Sk = 2, 16, 1, 4, 257
    g = _gen(23)
    q = _bf16(torch.randn((B, Hq, Sq, D), generator=g))
    k = _bf16(torch.randn((B, Hkv, Sk, D), generator=g))
    o, lse = run_decode_kvs(q, k, Dv, True, 9)
    check_kvs(q, k, Dv, True, o, lse, f"V in K, causal masked splits D={D}")


# ------------------------------------------------------------------ few dominant keys

@pytest.mark.parametrize("sd", [3.0, 4.0])
@pytest.mark.parametrize("shape", [(2, 4, 4, 200, 64, True), (2, 4, 2, 300, 64, False),
                                   (1, 4, 4, 200, 128, True)])
def test_prefill_few_dominant_keys(shape, sd):
    B, Hq, Hkv, S, D, causal = shape
    q, k, v = few_dominant_keys(B, Hq, Hkv, S, S, D, seed=31, sd=sd)
    o, lse = run_fwd(q, k, v, causal)
    check(q, k, v, causal, o, lse, f"few dominant keys sd={sd} {shape}")


@pytest.mark.parametrize("sd", [3.0, 4.0])
@pytest.mark.parametrize("shape", [(4, 8, 2, 300, 64, 3), (4, 8, 8, 300, 128, 2),
                                   (2, 16, 1, 300, 512, 2)])
def test_decode_few_dominant_keys(shape, sd):
    B, Hq, Hkv, Sk, D, ns = shape
    q, k, v = few_dominant_keys(B, Hq, Hkv, 1, Sk, D, seed=37, sd=sd)
    o, lse = run_decode(q, k, v, False, ns)
    check(q, k, v, False, o, lse, f"few dominant keys sd={sd} {shape}")


@pytest.mark.parametrize("sd", [3.0, 4.0])
@pytest.mark.parametrize("shape", [(4, 64, 1, 40, 512, 512, 1), (4, 64, 1, 300, 512, 512, 2),
                                   (4, 64, 1, 300, 576, 512, 2)])
def test_decode_v_in_k_few_dominant_keys(shape, sd):
    B, Hq, Hkv, Sk, D, Dv, ns = shape
    q, k, _ = few_dominant_keys(B, Hq, Hkv, 1, Sk, D, seed=41, sd=sd)
    o, lse = run_decode_kvs(q, k, Dv, False, ns)
    check_kvs(q, k, Dv, False, o, lse, f"V in K, few dominant keys sd={sd} {shape}")
