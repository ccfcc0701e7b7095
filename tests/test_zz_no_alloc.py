"""fmha_decode_splitkv_noalloc: the split-KV decode with its split partials in
the library's fixed scratch array instead of a caller workspace, called
through the C ABI.  Two calls in a row (the second smaller, with another head
dim, so it reads its partials from scratch that still holds the first call's)
must each equal fmha_decode_splitkv with a torch-allocated workspace bit for
bit, and the oracle at the parity tolerances; a request beyond the scratch
size is refused before anything runs."""
import ctypes

import pytest
import torch

import decode_fmha_fwd_amd as F
from gpu_helpers import assert_parity, oracle_rows, poison_like, require_gpu
from workloads import default_scale, make_qkv

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 64 << 20


def _with_workspace(qd, kd, vd, B, Hq, Hkv, Sq, Sk, D, causal, ns, amax):
    o = poison_like(qd)
    lse = torch.full((B, Hq, Sq), float("nan"), dtype=torch.float32, device=qd.device)
    nb = F.fmha_decode_splitkv_workspace_size(B, Hq, Hkv, Sq, Sk, D, ns)
    ws = torch.full((max(nb, 16),), 0xFF, dtype=torch.uint8, device=qd.device)
    F.fmha_decode_splitkv(qd, kd, vd, o, lse, B, Hq, Hkv, Sq, Sk, D, default_scale(D), causal,
                          ns, ws, nb, amax)
    return o, lse


def _noalloc(qd, kd, vd, B, Hq, Hkv, Sq, Sk, D, causal, ns, amax):
    """The entry point called through the C ABI (ctypes, device pointers)."""
    lib = F.load_library()
    o = poison_like(qd)
    lse = torch.full((B, Hq, Sq), float("nan"), dtype=torch.float32, device=qd.device)
    P = ctypes.c_void_p
    st = P(torch.cuda.current_stream(qd.device).cuda_stream)
    rc = lib.fmha_decode_splitkv_noalloc(
        P(qd.data_ptr()), P(kd.data_ptr()), P(vd.data_ptr()), P(o.data_ptr()),
        P(lse.data_ptr()), B, Hq, Hkv, Sq, Sk, D, default_scale(D), int(causal), ns,
        None if amax is None else P(amax.data_ptr()), st)
    assert rc == 0, lib.fmha_last_error().decode()
    return o, lse


CALLS = [
    # B, Hq, Hkv, Sq, Sk, D, causal, num_splits, amax -- the second call is the smaller one.
    # The first has 512 (batch, KV head) units: split groups that combine in the kernel;
    # the second goes through the combine kernel, which also folds max|O| into amax.
    (64, 32, 8, 1, 4096, 64, False, 16, False),
    (2, 8, 2, 2, 1000, 128, True, 3, True),
]


def test_noalloc_two_calls_match_the_workspace_entry_point():
    dev = require_gpu()
    for i, (B, Hq, Hkv, Sq, Sk, D, causal, ns, want_amax) in enumerate(CALLS):
        need = F.fmha_decode_splitkv_workspace_size(B, Hq, Hkv, Sq, Sk, D, ns)
        assert 0 < need <= SCRATCH_BYTES
        q, k, v = make_qkv(B, Hq, Hkv, Sq, Sk, D, seed=100 + i, sigma=0.8)
        qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
        a1 = torch.full((1,), 7.0, dtype=torch.float32, device=dev) if want_amax else None
        a2 = torch.full((1,), 7.0, dtype=torch.float32, device=dev) if want_amax else None
        o1, l1 = _noalloc(qd, kd, vd, B, Hq, Hkv, Sq, Sk, D, causal, ns, a1)
        o2, l2 = _with_workspace(qd, kd, vd, B, Hq, Hkv, Sq, Sk, D, causal, ns, a2)
        torch.cuda.synchronize()
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), f"call {i}: O"
        assert torch.equal(l1, l2), f"call {i}: LSE"
        if want_amax:
            assert torch.equal(a1, a2), f"call {i}: amax"
        o_ref, lse_ref = oracle_rows(q, k, v, default_scale(D), causal)
        assert_parity(o1, l1, o_ref, lse_ref, what=f"noalloc call {i}")


def test_noalloc_one_split_and_head_dim_512():
    dev = require_gpu()
    for (B, Hq, Hkv, Sk, D, ns) in [(1, 64, 1, 700, 512, 4), (3, 4, 4, 513, 128, 1)]:
        q, k, v = make_qkv(B, Hq, Hkv, 1, Sk, D, seed=D + ns, sigma=0.7)
        qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
        o1, l1 = _noalloc(qd, kd, vd, B, Hq, Hkv, 1, Sk, D, False, ns, None)
        o2, l2 = _with_workspace(qd, kd, vd, B, Hq, Hkv, 1, Sk, D, False, ns, None)
        torch.cuda.synchronize()
        assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


def test_noalloc_refuses_more_than_its_scratch():
    dev = require_gpu()
    B, Hq, Hkv, Sq, Sk, D, ns = 32, 64, 1, 1, 16384, 512, 32  # 128 MiB of partials
    assert F.fmha_decode_splitkv_workspace_size(B, Hq, Hkv, Sq, Sk, D, ns) > SCRATCH_BYTES
    q = torch.zeros((B, Hq, Sq, D), dtype=torch.bfloat16, device=dev)
    k = torch.zeros((1, 1, 1, D), dtype=torch.bfloat16, device=dev)  # never read
    o = torch.empty_like(q)
    lib = F.load_library()
    P = ctypes.c_void_p
    rc = lib.fmha_decode_splitkv_noalloc(P(q.data_ptr()), P(k.data_ptr()), P(k.data_ptr()),
                                         P(o.data_ptr()), None, B, Hq, Hkv, Sq, Sk, D, 0.04,
                                         0, ns, None, None)
    assert rc == 6 and b"scratch" in lib.fmha_last_error()
