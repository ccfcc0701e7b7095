"""GPU parity of the paged, variable-length split-KV decode (fmha_decode_paged)
through the C ABI.  K/V are drawn contiguous with the seeded generator,
scattered into a shuffled page pool whose unused slots are NaN (a read outside
a sequence would show), and each batch is compared with the fp64 oracle over
its own keys; with equal lengths the result must also equal the contiguous
decode bit for bit (same splits, same tile order)."""
import numpy as np
import pytest
import torch

import decode_fmha_fwd_amd as F
from gpu_helpers import assert_parity, oracle_rows, poison_like, require_gpu
from workloads import WORKLOADS, default_scale, make_qkv, make_workload_inputs, page_pool

pytestmark = pytest.mark.gpu


def run_paged(q, kc, vc, lens, table, page_size, num_pages, scale, causal, num_splits):
    dev = require_gpu()
    B, Hq, Sq, D = q.shape
    Hkv = kc.shape[1]
    max_pages = table.shape[1]
    qd = q.to(dev)
    o = poison_like(qd)
    lse = torch.full((B, Hq, Sq), float("nan"), dtype=torch.float32, device=dev)
    sl = torch.tensor(list(lens), dtype=torch.int32, device=dev)
    bt = torch.from_numpy(np.ascontiguousarray(table)).to(dev)
    nb = F.fmha_decode_splitkv_workspace_size(B, Hq, Hkv, Sq, max_pages * page_size, D,
                                              num_splits)
    ws = torch.full((max(nb, 16),), 0xFF, dtype=torch.uint8, device=dev)
    F.fmha_decode_paged(qd, kc.to(dev), vc.to(dev), o, lse, B, Hq, Hkv, Sq, sl, bt, max_pages,
                        page_size, num_pages, D, scale, causal, num_splits, ws, nb)
    torch.cuda.synchronize()
    return o, lse


def run_contiguous(q, k, v, scale, causal, num_splits):
    dev = require_gpu()
    B, Hq, Sq, D = q.shape
    _, Hkv, Sk, _ = k.shape
    qd = q.to(dev)
    o = poison_like(qd)
    lse = torch.full((B, Hq, Sq), float("nan"), dtype=torch.float32, device=dev)
    nb = F.fmha_decode_splitkv_workspace_size(B, Hq, Hkv, Sq, Sk, D, num_splits)
    ws = torch.full((max(nb, 16),), 0xFF, dtype=torch.uint8, device=dev)
    F.fmha_decode_splitkv(qd, k.to(dev), v.to(dev), o, lse, B, Hq, Hkv, Sq, Sk, D, scale, causal,
                          num_splits, ws, nb)
    torch.cuda.synchronize()
    return o, lse


PAGED_CASES = [
    # B, Hq, Hkv, Sq, D, page_size, lens, num_splits, causal
    (4, 8, 2, 1, 64, 64, (1, 64, 200, 1000), 0, False),     # ragged ends, one-key sequence
    (3, 8, 8, 1, 128, 128, (300, 0, 129), 4, False),        # an empty sequence, MHA
    (2, 64, 1, 1, 512, 64, (700, 33), 0, False),            # MQA at head dim 512
    (2, 8, 2, 3, 64, 256, (500, 3), 2, True),               # three query rows, causal
    (2, 4, 1, 2, 64, 64, (1, 130), 1, True),                # causal: row 0 of batch 0 sees no key
    (1, 4, 4, 1, 64, 64, (4096,), 16, False),               # 64 pages, 16 splits
    (2, 64, 8, 1, 64, 128, (2048, 1500), 0, False),         # GQA 8:1
    (3, 16, 4, 1, 128, 64, (77, 640, 1), 3, False),         # 4-wave tiles (64 keys) per page
]


@pytest.mark.parametrize("case", PAGED_CASES)
def test_paged_decode_matches_oracle(case):
    B, Hq, Hkv, Sq, D, P, lens, ns, causal = case
    S = max(max(lens), 1)
    q, k, v = make_qkv(B, Hq, Hkv, Sq, S, D, seed=7 + sum(lens))
    kc, vc, table, num_pages = page_pool(k, v, lens, P, seed=11)
    scale = default_scale(D)
    o, lse = run_paged(q, kc, vc, lens, table, P, num_pages, scale, causal, ns)
    for b, n in enumerate(lens):
        if n == 0:  # no keys: O = 0, LSE = -inf
            assert torch.equal(o[b].float().cpu(), torch.zeros(Hq, Sq, D))
            assert torch.isinf(lse[b]).all() and (lse[b] < 0).all()
            continue
        o_ref, lse_ref = oracle_rows(q[b:b + 1], k[b:b + 1, :, :n].contiguous(),
                                     v[b:b + 1, :, :n].contiguous(), scale, causal)
        assert_parity(o[b:b + 1], lse[b:b + 1], o_ref, lse_ref, what=f"{case} batch {b}")


@pytest.mark.parametrize("B,Hq,Hkv,D,P,S,ns", [
    (2, 32, 8, 64, 64, 1024, 4),
    (2, 16, 16, 128, 128, 768, 3),
    (2, 64, 1, 512, 256, 1024, 2),
])
def test_paged_equals_contiguous_bitwise(B, Hq, Hkv, D, P, S, ns):
    q, k, v = make_qkv(B, Hq, Hkv, 1, S, D, seed=5)
    kc, vc, table, num_pages = page_pool(k, v, [S] * B, P, seed=13)
    o1, l1 = run_paged(q, kc, vc, [S] * B, table, P, num_pages, default_scale(D), False, ns)
    o2, l2 = run_contiguous(q, k, v, default_scale(D), False, ns)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


def test_paged_gqa_decode_workload_equals_contiguous():
    # the GQA decode workload (B=64, 8 KV heads, 8192 keys, 16 splits) from a
    # shuffled pool of 64-key pages: bit-identical to the contiguous decode,
    # which the attention tests check against the oracle at this size
    w = WORKLOADS["decode_gqa_d64"]
    q, k, v = make_workload_inputs(w)
    kc, vc, table, num_pages = page_pool(k, v, [w.Sk] * w.B, 64, seed=17)
    o1, l1 = run_paged(q, kc, vc, [w.Sk] * w.B, table, 64, num_pages, w.scale, w.causal,
                       w.num_splits)
    del kc, vc
    o2, l2 = run_contiguous(q, k, v, w.scale, w.causal, w.num_splits)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
    o_ref, lse_ref = oracle_rows(q, k, v, w.scale, w.causal)  # and every row against the oracle
    assert_parity(o1, l1, o_ref, lse_ref, what="paged " + w.name)


def test_paged_split_groups_with_empty_splits():
    # 64 batches x 8 KV heads x 16 splits, lengths from 0 to 2048: whole
    # splits without keys (lse -inf, O 0 in the partials) next to full ones
    B, Hq, Hkv, D, P, ns = 64, 8, 8, 64, 64, 16
    lens = [int(x) for x in np.random.default_rng(3).integers(0, 2049, size=B)]
    lens[0], lens[1] = 0, 2048
    q, k, v = make_qkv(B, Hq, Hkv, 1, 2048, D, seed=19)
    kc, vc, table, num_pages = page_pool(k, v, lens, P, seed=23)
    scale = default_scale(D)
    o, lse = run_paged(q, kc, vc, lens, table, P, num_pages, scale, False, ns)
    for b, n in enumerate(lens):
        if n == 0:
            assert torch.equal(o[b].float().cpu(), torch.zeros(Hq, 1, D))
            assert torch.isinf(lse[b]).all() and (lse[b] < 0).all()
            continue
        o_ref, lse_ref = oracle_rows(q[b:b + 1], k[b:b + 1, :, :n].contiguous(),
                                     v[b:b + 1, :, :n].contiguous(), scale, False)
        assert_parity(o[b:b + 1], lse[b:b + 1], o_ref, lse_ref, what=f"batch {b} ({n} keys)")


@pytest.mark.parametrize("Sq,D,causal,ns", [(1, 64, False, 8), (2, 64, True, 8),
                                          (1, 128, False, 6)])
def test_paged_split_groups_equal_one_workgroup_per_split(Sq, D, causal, ns):
    # 64 batches x 8 KV heads (512 units: one workgroup streams all splits of
    # a unit) with lengths from 0 to 1500 against single-batch calls (8 units:
    # one workgroup per split), bit for bit, and the oracle
    B, Hq, Hkv, P = 64, 32, 8, 64
    lens = [int(x) for x in np.random.default_rng(D + Sq).integers(0, 1501, size=B)]
    lens[0], lens[1], lens[2] = 1500, 0, 1
    q, k, v = make_qkv(B, Hq, Hkv, Sq, 1500, D, seed=61 + D + Sq)
    kc, vc, table, num_pages = page_pool(k, v, lens, P, seed=67)
    scale = default_scale(D)
    o, lse = run_paged(q, kc, vc, lens, table, P, num_pages, scale, causal, ns)
    for b in (0, 1, 2, B // 2, B - 1):  # (causal, batch 2: query row 0 sees no key)
        o1, l1 = run_paged(q[b:b + 1], kc, vc, lens[b:b + 1], table[b:b + 1], P, num_pages,
                           scale, causal, ns)
        assert torch.equal(o[b].view(torch.int16), o1[0].view(torch.int16)), b
        assert torch.equal(lse[b], l1[0]), b
        if lens[b] >= Sq:
            o_ref, lse_ref = oracle_rows(q[b:b + 1], k[b:b + 1, :, :lens[b]].contiguous(),
                                         v[b:b + 1, :, :lens[b]].contiguous(), scale, causal)
            assert_parity(o[b:b + 1], lse[b:b + 1], o_ref, lse_ref,
                          what=f"batch {b} ({lens[b]} keys)")


def test_paged_one_million_keys():
    # 2^20 keys in 4096 shuffled 256-key pages: page ids and table slots in
    # the thousands, key offsets past 2^26 elements
    B, Hq, Hkv, D, P, S = 1, 4, 1, 64, 256, 1 << 20
    q, k, v = make_qkv(B, Hq, Hkv, 1, S, D, seed=53)
    kc, vc, table, num_pages = page_pool(k, v, [S], P, seed=59)
    scale = default_scale(D)
    o, lse = run_paged(q, kc, vc, [S], table, P, num_pages, scale, False, 32)
    o_ref, lse_ref = oracle_rows(q, k, v, scale, False)
    assert_parity(o, lse, o_ref, lse_ref, what="paged 1M keys")
