"""GPU parity of the attention kernels (prefill fmha_fwd and split-KV decode
fmha_decode_splitkv) against the fp64 CPU oracle, through the C ABI.

Every test compares the whole output element by element -- the full-size
workloads too, in the same launch configuration the benchmark times -- except
the two long-sequence stress tests at the end, which check seeded row samples."""
import numpy as np
import pytest
import torch

import decode_fmha_fwd_amd as F
from gpu_helpers import assert_parity, bits, oracle_rows, poison_like, require_gpu
from workloads import WORKLOADS, default_scale, make_qkv, make_workload_inputs, sample_rows

pytestmark = pytest.mark.gpu


def run_fwd(q, k, v, scale, causal):
    dev = require_gpu()
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    B, Hq, Sq, D = q.shape
    _, Hkv, Sk, _ = k.shape
    o = poison_like(qd)
    lse = torch.full((B, Hq, Sq), float("nan"), dtype=torch.float32, device=dev)
    F.fmha_fwd(qd, kd, vd, o, lse, B, Hq, Hkv, Sq, Sk, D, scale, causal)
    torch.cuda.synchronize()
    return o, lse


def run_decode(q, k, v, scale, causal, num_splits, o_amax=None):
    dev = require_gpu()
    qd, kd = q.to(dev), k.to(dev)
    vd = kd if v is k else v.to(dev)  # V aliasing K stays one buffer
    B, Hq, Sq, D = q.shape
    _, Hkv, Sk, _ = k.shape
    o = poison_like(qd)
    lse = torch.full((B, Hq, Sq), float("nan"), dtype=torch.float32, device=dev)
    nb = F.fmha_decode_splitkv_workspace_size(B, Hq, Hkv, Sq, Sk, D, num_splits)
    ws = torch.full((max(nb, 16),), 0xFF, dtype=torch.uint8, device=dev)
    F.fmha_decode_splitkv(qd, kd, vd, o, lse, B, Hq, Hkv, Sq, Sk, D, scale, causal, num_splits,
                          ws, nb, o_amax)
    torch.cuda.synchronize()
    return o, lse


# ---------------------------------------------------------------- QK exactness

QK_CASES = [
    # decode, B, Hq, Hkv, Sq, Sk, D, Dv, v_is_k -- each the kernel the matching entry point
    # launches for that shape (prefill: 32-row waves on 32x32x16 MFMAs; decode: 16-row waves
    # on 16x16x32 MFMAs)
    (0, 1, 2, 1, 150, 200, 16, 16, False),
    (0, 1, 2, 1, 150, 200, 32, 32, False),
    (0, 1, 2, 1, 150, 200, 64, 64, False),
    (0, 2, 2, 2, 130, 190, 128, 128, False),
    (0, 1, 2, 1, 150, 200, 192, 128, False),
    (1, 2, 8, 2, 1, 300, 64, 64, False),      # 4 rows per KV head: one-wave workgroups
    (1, 1, 64, 2, 1, 300, 64, 64, False),     # 32 rows per KV head: four-wave workgroups
    (1, 2, 8, 2, 1, 300, 128, 128, False),
    (1, 1, 64, 2, 1, 300, 128, 128, False),
    (1, 1, 64, 1, 1, 200, 512, 512, False),   # two rings
    (1, 1, 64, 1, 1, 200, 512, 512, True),    # V aliasing K: one shared ring
    (1, 1, 64, 1, 1, 200, 576, 512, False),
    (1, 1, 64, 1, 1, 200, 576, 512, True),    # V the first 512 columns of the K rows
]


@pytest.mark.parametrize("case", QK_CASES)
def test_qk_scores_equal_exact_dot_product(case):
    """Integer inputs in [-8, 8]: every partial sum is an integer below 2^24, so
    the QK block of the attention kernel must give S = scale * <q, k> exactly --
    a stray factor (the 4x chased on the QK page) or a misplaced operand cannot
    pass.  The scores come from the production kernel's own QK block (copy ring,
    asm LDS reads, accumulation chains), stored before masking and softmax."""
    decode, B, Hq, Hkv, Sq, Sk, D, Dv, v_is_k = case
    dev = require_gpu()
    rng = np.random.default_rng(D + Sq + Sk + 7 * decode)
    qi = rng.integers(-8, 9, size=(B, Hq, Sq, D))
    ki = rng.integers(-8, 9, size=(B, Hkv, Sk, D))
    vi = rng.integers(-8, 9, size=(B, Hkv, Sk, Dv))
    q = torch.tensor(qi, dtype=torch.bfloat16, device=dev)
    k = torch.tensor(ki, dtype=torch.bfloat16, device=dev)
    v = k if v_is_k else torch.tensor(vi, dtype=torch.bfloat16, device=dev)
    G = Hq // Hkv
    dots = np.einsum("bhqd,bhkd->bhqk", qi, np.repeat(ki, G, axis=1)).astype(np.float64)
    for scale in (0.25, 0.125):
        s = torch.full((B * Hq * Sq, Sk), float("nan"), dtype=torch.float32, device=dev)
        F.fmha_debug_qk_scores(q, k, v, s, B, Hq, Hkv, Sq, Sk, D, Dv, scale, decode)
        torch.cuda.synchronize()
        got = s.cpu().numpy().astype(np.float64)
        np.testing.assert_array_equal(got, scale * dots.reshape(-1, Sk), err_msg=str(case))


# ---------------------------------------------------------------- prefill

def test_single_tile_d16_workload():
    w = WORKLOADS["single_tile_d16"]
    q, k, v = make_workload_inputs(w)
    o, lse = run_fwd(q, k, v, w.scale, w.causal)
    o_ref, lse_ref = oracle_rows(q, k, v, w.scale, w.causal)
    assert_parity(o, lse, o_ref, lse_ref, what=w.name)


FWD_CASES = [
    # B, Hq, Hkv, Sq, Sk, D, causal
    (1, 1, 1, 128, 128, 16, True),
    (2, 2, 2, 200, 200, 64, False),     # ragged: 200 = 3 x 64 + 8
    (2, 2, 2, 200, 200, 64, True),
    (1, 4, 2, 130, 333, 64, True),      # GQA, Sq < Sk (bottom-right causal)
    (1, 2, 1, 1, 77, 64, False),        # a single query row
    (1, 2, 2, 257, 257, 32, True),
    (1, 2, 2, 190, 300, 128, False),
    (1, 1, 1, 64, 1, 64, False),        # one key
    (3, 3, 1, 45, 45, 128, True),
    (1, 2, 1, 300, 100, 64, False),     # more queries than keys
    (2, 6, 3, 129, 129, 32, True),      # odd group size, one row past a 128-row block
    # head dim 64: several 128-row blocks, long key ranges
    (1, 2, 2, 600, 600, 64, True),      # three row blocks, the last ragged
    (2, 2, 2, 512, 512, 64, True),      # whole row blocks
    (1, 8, 2, 100, 100, 64, True),      # GQA: one row block spans four heads
    (1, 1, 1, 64, 1500, 64, False),     # 24 key tiles: the LDS ring wraps several times
    (1, 2, 1, 70, 1000, 64, True),      # few queries, long causal key range
]


@pytest.mark.parametrize("case", FWD_CASES)
def test_fwd_small_shapes(case):
    B, Hq, Hkv, Sq, Sk, D, causal = case
    q, k, v = make_qkv(B, Hq, Hkv, Sq, Sk, D, seed=sum(case))
    scale = default_scale(D)
    o, lse = run_fwd(q, k, v, scale, causal)
    o_ref, lse_ref = oracle_rows(q, k, v, scale, causal)
    assert_parity(o, lse, o_ref, lse_ref, what=str(case))


def test_prefill_causal_d64_workload():
    """B=4, H=16, S=2048, D=64, causal: all 131072 rows against the oracle."""
    w = WORKLOADS["prefill_causal_d64"]
    q, k, v = make_workload_inputs(w)
    o, lse = run_fwd(q, k, v, w.scale, w.causal)
    o_ref, lse_ref = oracle_rows(q, k, v, w.scale, w.causal)
    assert_parity(o, lse, o_ref, lse_ref, what=w.name)


@pytest.mark.parametrize("case", [
    # B, Hq, Hkv, S, causal: grids of two or more rounds of workgroup slots, where
    # each head-dim-64 workgroup takes a heavy and a light row block in turn
    (32, 16, 16, 384, True),    # 3 row blocks: one pair and one workgroup alone
    (32, 32, 8, 300, True),     # GQA: 1200 rows per KV head, blocks span heads, last ragged
    (32, 16, 16, 640, False),   # 5 row blocks, non-causal
])
def test_prefill_paired_row_blocks(case):
    """Every output row against the oracle when row blocks are paired."""
    B, Hq, Hkv, S, causal = case
    q, k, v = make_qkv(B, Hq, Hkv, S, S, 64, seed=S + Hkv)
    o, lse = run_fwd(q, k, v, default_scale(64), causal)
    o_ref, lse_ref = oracle_rows(q, k, v, default_scale(64), causal)
    assert_parity(o, lse, o_ref, lse_ref, what=str(case))


def test_fwd_is_deterministic():
    q, k, v = make_qkv(1, 2, 2, 300, 300, 64, seed=3)
    o1, l1 = run_fwd(q, k, v, 0.125, True)
    o2, l2 = run_fwd(q, k, v, 0.125, True)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


# ---------------------------------------------------------------- decode

DEC_CASES = [
    # B, Hq, Hkv, Sq, Sk, D, causal, num_splits
    (2, 8, 2, 1, 1000, 64, False, 1),
    (2, 8, 2, 1, 1000, 64, False, 3),
    (2, 8, 2, 1, 1000, 64, False, 16),
    (2, 8, 2, 1, 1000, 64, False, 0),
    (1, 64, 1, 1, 777, 512, False, 4),
    (1, 64, 1, 1, 300, 512, False, 1),
    (8, 64, 1, 1, 300, 512, False, 1),
    (2, 32, 2, 1, 500, 512, False, 3),  # two KV heads of 32 rows
    (3, 4, 4, 1, 513, 128, False, 1),
    (3, 4, 4, 1, 513, 128, False, 5),
    (2, 16, 2, 4, 390, 64, True, 2),    # small Sq > 1, causal bottom-right
    (2, 32, 1, 2, 129, 128, False, 2),  # 64 rows per KV head, 4 waves
    (1, 4, 1, 1, 1, 64, False, 1),      # one key
    (1, 2, 1, 1, 40, 64, False, 8),     # more splits than tiles: empty ranges
    (1, 4, 1, 1, 2400, 64, False, 75),  # more than 64 splits: the combine's second pass
    (1, 64, 1, 1, 4200, 512, False, 70),  # 66 effective splits at head dim 512
    (2, 6, 2, 1, 500, 64, False, 2),    # 3 rows per KV head
    (1, 128, 1, 1, 300, 64, False, 2),  # 128 rows per KV head: two 64-row workgroups
    (1, 128, 1, 1, 300, 512, False, 2),  # the same at head dim 512
    (2, 8, 8, 3, 200, 128, False, 2),   # Sq = 3 without a mask
]


@pytest.mark.parametrize("case", DEC_CASES)
def test_decode_small_shapes(case):
    B, Hq, Hkv, Sq, Sk, D, causal, ns = case
    q, k, v = make_qkv(B, Hq, Hkv, Sq, Sk, D, seed=sum(case), sigma=0.7)
    scale = default_scale(D)
    o, lse = run_decode(q, k, v, scale, causal, ns)
    o_ref, lse_ref = oracle_rows(q, k, v, scale, causal)
    assert_parity(o, lse, o_ref, lse_ref, what=str(case))


@pytest.mark.parametrize("name", ["decode_gqa_d64", "decode_mqa_d512", "decode_nvfp4_d128"])
def test_decode_workloads(name):
    """The full-size decode workloads, every output row against the oracle."""
    w = WORKLOADS[name]
    q, k, v = make_workload_inputs(w)
    o, lse = run_decode(q, k, v, w.scale, w.causal, w.num_splits)
    o_ref, lse_ref = oracle_rows(q, k, v, w.scale, w.causal)
    assert_parity(o, lse, o_ref, lse_ref, what=name)


VK_CASES = [
    # B, Hq, Hkv, Sq, Sk, D, causal, num_splits -- V is the same tensor as K
    (1, 64, 1, 1, 777, 512, False, 4),
    (1, 64, 1, 1, 300, 512, False, 1),
    (2, 32, 2, 1, 500, 512, False, 3),
    (1, 32, 1, 2, 400, 512, True, 2),
    (1, 8, 1, 16, 700, 512, True, 3),   # Sq = 16 causal: two 64-row blocks, several masked tiles
    (2, 8, 2, 1, 300, 64, False, 2),    # other head dims take the two-ring path
]


@pytest.mark.parametrize("case", VK_CASES)
def test_decode_v_aliasing_k(case):
    """V passed as the very K buffer (a shared latent): at head dim 512 the
    kernel streams each key row once and reads V^T from the K tile."""
    B, Hq, Hkv, Sq, Sk, D, causal, ns = case
    dev = require_gpu()
    q, k, _ = make_qkv(B, Hq, Hkv, Sq, Sk, D, seed=sum(case) + 1, sigma=0.7)
    scale = default_scale(D)
    qd, kd = q.to(dev), k.to(dev)
    o = poison_like(qd)
    lse = torch.full((B, Hq, Sq), float("nan"), dtype=torch.float32, device=dev)
    nb = F.fmha_decode_splitkv_workspace_size(B, Hq, Hkv, Sq, Sk, D, ns)
    ws = torch.full((max(nb, 16),), 0xFF, dtype=torch.uint8, device=dev)
    F.fmha_decode_splitkv(qd, kd, kd, o, lse, B, Hq, Hkv, Sq, Sk, D, scale, causal, ns, ws, nb)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle_rows(q, k, k, scale, causal)
    assert_parity(o, lse, o_ref, lse_ref, what=str(case))


def test_decode_v_is_k_workload():
    w = WORKLOADS["decode_mqa_d512_v_is_k"]
    q, k, v = make_workload_inputs(w)
    assert v is k
    o, lse = run_decode(q, k, v, w.scale, w.causal, w.num_splits)
    o_ref, lse_ref = oracle_rows(q, k, k, w.scale, w.causal)
    assert_parity(o, lse, o_ref, lse_ref, what=w.name)


def test_split_count_does_not_change_the_result():
    q, k, v = make_qkv(4, 8, 2, 1, 4096, 64, seed=5)
    outs = [run_decode(q, k, v, 0.125, False, ns) for ns in (1, 2, 7, 16)]
    base_o = outs[0][0].float()
    for o, lse in outs[1:]:
        assert (o.float() - base_o).abs().max().item() <= 1.6e-2
        assert (lse - outs[0][1]).abs().max().item() <= 1e-5


def test_decode_amax_fold():
    """o_amax receives max|O| of the bf16 O the call writes (the library clears
    it first), which is within the O tolerance of the oracle's max|O|."""
    dev = require_gpu()
    q, k, v = make_qkv(4, 16, 16, 1, 512, 128, seed=9)
    o_ref, _ = oracle_rows(q, k, v, default_scale(128), False)
    for ns in (1, 4):
        amax = torch.full((1,), 1e30, dtype=torch.float32, device=dev)  # stale value
        o, _ = run_decode(q, k, v, default_scale(128), False, ns, o_amax=amax)
        assert amax.item() == o.float().abs().max().item()
        assert abs(amax.item() - float(np.abs(o_ref).max())) <= 2e-2


@pytest.mark.parametrize("B,Hq,Hkv,Sq,Sk,D,causal,ns", [
    (64, 32, 8, 1, 1000, 64, False, 8),    # 1-wave workgroups, 8 splits of 128 keys, last ragged
    (64, 32, 8, 2, 1000, 64, True, 8),     # causal, two query rows
    (64, 32, 8, 1, 1000, 128, False, 8),
    (256, 64, 2, 1, 300, 64, False, 4),    # 32 rows per KV head: 4-wave workgroups
    (256, 48, 2, 1, 300, 64, False, 4),    # 24 rows: partials in LDS from two of four waves
    (256, 64, 2, 1, 300, 128, False, 3),
])
def test_split_groups_equal_one_workgroup_per_split(B, Hq, Hkv, Sq, Sk, D, causal, ns):
    """When the (batch, KV head) units alone give every CU two or more
    workgroups (here 512 units), one workgroup streams all splits of its unit
    and writes each split's partial: the arithmetic of one workgroup per
    split.  Batches of the grouped run must equal single-batch runs (too few
    units to group) bit for bit, and the oracle.  The 1-wave cases and the
    24-row case keep the partials in LDS (they fit beside the rings with every
    workgroup resident); the other 4-wave cases go through the workspace."""
    q, k, v = make_qkv(B, Hq, Hkv, Sq, Sk, D, seed=D + Sq + B)
    scale = default_scale(D)
    o, lse = run_decode(q, k, v, scale, causal, ns)
    for b in (0, B // 3, B - 1):
        o1, l1 = run_decode(q[b:b + 1], k[b:b + 1], v[b:b + 1], scale, causal, ns)
        assert torch.equal(o[b].view(torch.int16), o1[0].view(torch.int16)), b
        assert torch.equal(lse[b], l1[0]), b
    o_ref, lse_ref = oracle_rows(q, k, v, scale, causal)
    assert_parity(o, lse, o_ref, lse_ref, what=f"B={B} D={D} grouped splits")


# ---------------------------------------------------------------- long sequences

def test_decode_one_million_keys():
    """2^20 keys in 64 splits (256 MiB of K and V): key offsets past 2^26
    elements, split lengths of 16384 keys; checked against the oracle."""
    B, Hq, Hkv, Sq, Sk, D, ns = 1, 8, 1, 1, 1 << 20, 64, 64
    q, k, v = make_qkv(B, Hq, Hkv, Sq, Sk, D, seed=41)
    o, lse = run_decode(q, k, v, default_scale(D), False, ns)
    o_ref, lse_ref = oracle_rows(q, k, v, default_scale(D), False)
    assert_parity(o, lse, o_ref, lse_ref, what="1M keys")


def test_prefill_causal_32k():
    """One head, 32768 queries and keys, causal: 256 row blocks, the longest
    streaming 512 key tiles; sampled rows against the oracle."""
    B, H, S, D = 1, 1, 32768, 64
    q, k, v = make_qkv(B, H, H, S, S, D, seed=43)
    o, lse = run_fwd(q, k, v, default_scale(D), True)
    rows = sample_rows(S, 48, seed=47)
    o_ref, lse_ref = oracle_rows(q, k, v, default_scale(D), True, rows=rows)
    assert_parity(o, lse, o_ref, lse_ref, rows=rows, what="causal 32k")
