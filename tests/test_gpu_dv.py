"""GPU parity of the split-KV decode with a V/O head dim different from the
Q/K head dim (fmha_decode_splitkv_dv: D = 576, Dv = 512) against the fp64 CPU
oracle, through the C ABI.  V is either its own [B, Hkv, Sk, Dv] tensor or the
very K buffer, which makes V the first Dv columns of each K row; the oracle
always gets V as its own tensor."""
import pytest
import torch

import decode_fmha_fwd_amd as F
from gpu_helpers import assert_parity, oracle_rows, poison_like, require_gpu
from workloads import WORKLOADS, default_scale, make_qkv, make_workload_inputs, v_of

pytestmark = pytest.mark.gpu

D, DV = 576, 512


def run_decode_dv(q, k, v, dv, scale, causal, num_splits):
    """v is k: the K buffer is passed for V too (V inside the K rows)."""
    dev = require_gpu()
    qd, kd = q.to(dev), k.to(dev)
    vd = kd if v is k else v.to(dev)
    B, Hq, Sq, d = q.shape
    _, Hkv, Sk, _ = k.shape
    o = torch.full((B, Hq, Sq, dv), float("nan"), dtype=torch.bfloat16, device=dev)
    lse = torch.full((B, Hq, Sq), float("nan"), dtype=torch.float32, device=dev)
    nb = F.fmha_decode_splitkv_dv_workspace_size(B, Hq, Hkv, Sq, Sk, d, dv, num_splits)
    ws = torch.full((max(nb, 16),), 0xFF, dtype=torch.uint8, device=dev)
    F.fmha_decode_splitkv_dv(qd, kd, vd, o, lse, B, Hq, Hkv, Sq, Sk, d, dv, scale, causal,
                             num_splits, ws, nb)
    torch.cuda.synchronize()
    return o, lse


CASES = [
    # B, Hq, Hkv, Sq, Sk, causal, num_splits, v_in_k
    (1, 64, 1, 1, 777, False, 4, True),
    (1, 64, 1, 1, 300, False, 1, True),
    (2, 32, 2, 1, 500, False, 3, True),
    (1, 32, 1, 2, 400, True, 2, True),
    (2, 16, 1, 1, 1, False, 1, True),      # one key
    (1, 128, 1, 1, 2085, False, 0, True),  # two row blocks, heuristic splits, ragged tail
    (1, 64, 1, 1, 777, False, 4, False),
    (2, 32, 2, 1, 500, False, 1, False),
    (1, 32, 1, 2, 400, True, 2, False),
    (3, 8, 1, 1, 130, False, 2, False),    # 8 rows: a partly filled row block
    (2, 64, 4, 1, 1500, False, 0, True),   # 4 KV heads of 16 rows, heuristic splits
    (1, 16, 1, 3, 200, True, 2, False),    # three causal query rows (48 rows per KV head)
    (1, 8, 1, 16, 700, True, 3, True),     # Sq = 16 causal, V inside K: two row blocks, masked tiles
]


@pytest.mark.parametrize("case", CASES)
def test_decode_dv_small_shapes(case):
    B, Hq, Hkv, Sq, Sk, causal, ns, v_in_k = case
    q, k, v = make_qkv(B, Hq, Hkv, Sq, Sk, D, DV, seed=sum(case[:6]) + 7, sigma=0.5)
    scale = default_scale(D)
    o, lse = run_decode_dv(q, k, k if v_in_k else v, DV, scale, causal, ns)
    v_ref = v_of(k, DV) if v_in_k else v
    o_ref, lse_ref = oracle_rows(q, k, v_ref, scale, causal)
    assert_parity(o, lse, o_ref, lse_ref, what=str(case))


def test_decode_dv_uses_only_the_first_dv_columns():
    """With V inside the K rows, the 64 key dims past Dv take part in the
    scores but never in the output: changing them moves O only through P."""
    B, Hq, Hkv, Sq, Sk = 1, 16, 1, 1, 96
    q, k, _ = make_qkv(B, Hq, Hkv, Sq, Sk, D, DV, seed=21, sigma=0.5)
    q[..., DV:] = 0  # the extra key dims then do not move the scores either
    k2 = k.clone()
    k2[..., DV:] = torch.randn(k2[..., DV:].shape, generator=torch.Generator().manual_seed(5)).to(
        torch.bfloat16)
    scale = default_scale(D)
    o1, l1 = run_decode_dv(q, k, k, DV, scale, False, 2)
    o2, l2 = run_decode_dv(q, k2, k2, DV, scale, False, 2)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_decode_dv_workload():
    """The full-size 576/512 decode with V inside the K rows, every row."""
    w = WORKLOADS["decode_mqa_d576_dv512_v_in_k"]
    q, k, v = make_workload_inputs(w)
    assert v is k
    o, lse = run_decode_dv(q, k, k, w.Dv, w.scale, w.causal, w.num_splits)
    o_ref, lse_ref = oracle_rows(q, k, v_of(k, w.Dv), w.scale, w.causal)
    assert_parity(o, lse, o_ref, lse_ref, what=w.name)


def test_decode_dv_equal_dims_match_the_plain_decode():
    """fmha_decode_splitkv_dv with Dv == D is fmha_decode_splitkv, bit for bit."""
    B, Hq, Hkv, Sq, Sk, d = 2, 16, 4, 1, 700, 128
    q, k, v = make_qkv(B, Hq, Hkv, Sq, Sk, d, seed=3)
    o1, l1 = run_decode_dv(q, k, v, d, default_scale(d), False, 3)
    dev = require_gpu()
    o2, l2 = F.decode(q.to(dev), k.to(dev), v.to(dev), num_splits=3)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


# ---------------------------------------------------------------- prefill, Q/K 192, V/O 128

FWD_CASES = [
    # B, Hq, Hkv, Sq, Sk, causal
    (1, 2, 2, 200, 200, True),      # ragged: 200 = 3 x 64 + 8
    (2, 4, 2, 130, 333, True),      # GQA, Sq < Sk (bottom-right causal)
    (1, 2, 1, 77, 300, False),
    (1, 1, 1, 64, 1, False),        # one key
    (1, 2, 2, 600, 600, True),      # several 128-row blocks, the last ragged
    (1, 2, 1, 300, 100, False),     # more queries than keys
    (2, 6, 3, 129, 129, True),      # odd group size, one row past a 128-row block
]


def run_fwd_dv(q, k, v, scale, causal):
    dev = require_gpu()
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    B, Hq, Sq, d = q.shape
    _, Hkv, Sk, dv = v.shape
    o = torch.full((B, Hq, Sq, dv), float("nan"), dtype=torch.bfloat16, device=dev)
    lse = torch.full((B, Hq, Sq), float("nan"), dtype=torch.float32, device=dev)
    F.fmha_fwd_dv(qd, kd, vd, o, lse, B, Hq, Hkv, Sq, Sk, d, dv, scale, causal)
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("case", FWD_CASES)
def test_fwd_dv_small_shapes(case):
    B, Hq, Hkv, Sq, Sk, causal = case
    q, k, v = make_qkv(B, Hq, Hkv, Sq, Sk, 192, 128, seed=sum(case) + 3)
    scale = default_scale(192)
    o, lse = run_fwd_dv(q, k, v, scale, causal)
    o_ref, lse_ref = oracle_rows(q, k, v, scale, causal)
    assert_parity(o, lse, o_ref, lse_ref, what=str(case))


def test_fwd_dv_workload():
    """The full-size 192/128 causal prefill, every row."""
    w = WORKLOADS["prefill_causal_d192_dv128"]
    q, k, v = make_workload_inputs(w)
    o, lse = run_fwd_dv(q, k, v, w.scale, w.causal)
    o_ref, lse_ref = oracle_rows(q, k, v, w.scale, w.causal)
    assert_parity(o, lse, o_ref, lse_ref, what=w.name)
