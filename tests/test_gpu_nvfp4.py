"""GPU parity of the NVFP4 quantiser: bit-exact codes, block scales and global
scale against the oracle's step-by-step fp32 quantiser, including when both
are fed the oracle's own attention output (rounded to bf16) at the full
decode_nvfp4_d128 size."""
import json
import os

import numpy as np
import pytest
import torch

import decode_fmha_fwd_amd as F
import oracle
from gpu_helpers import bits, oracle_rows, require_gpu
from workloads import WORKLOADS, make_qkv, make_workload_inputs

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def gpu_quant(x_bits, rows, cols, amax_in=None):
    dev = require_gpu()
    x = torch.from_numpy(np.ascontiguousarray(x_bits).view(np.int16)).view(torch.bfloat16)
    x = x.reshape(rows, cols).to(dev)
    codes = torch.full((rows, cols // 2), 0xAA, dtype=torch.uint8, device=dev)
    scales = torch.full((rows, cols // 16), 0xAA, dtype=torch.uint8, device=dev)
    g = torch.full((1,), float("nan"), dtype=torch.float32, device=dev)
    nb = F.nvfp4_quantize_workspace_size(rows, cols)
    ws = torch.empty(nb, dtype=torch.uint8, device=dev)
    F.nvfp4_quantize(x, rows, cols, codes, scales, g, amax_in, ws, nb)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy(), g.cpu().numpy()[0]


def assert_bit_exact(x_bits, rows, cols):
    c, s, g = gpu_quant(x_bits, rows, cols)
    rc, rs, rg = oracle.nvfp4_quantize(x_bits, rows, cols)
    assert np.float32(g).view(np.uint32) == np.float32(rg).view(np.uint32)
    np.testing.assert_array_equal(s, rs)
    np.testing.assert_array_equal(c, rc)


def test_hand_worked_example():
    with open(os.path.join(GOLDEN, "nvfp4_hand_example.json")) as f:
        ex = json.load(f)
    x = torch.tensor(ex["x"], dtype=torch.float32).to(torch.bfloat16)
    c, s, g = gpu_quant(bits(x), ex["rows"], ex["cols"])
    assert g == ex["expected_global_scale"]
    np.testing.assert_array_equal(s, np.array(ex["expected_scales"], np.uint8))
    want = np.array([[int(h, 16) for h in row] for row in ex["expected_codes_hex"]], np.uint8)
    np.testing.assert_array_equal(c, want)


@pytest.mark.parametrize("sigma,seed", [(1.0, 0), (1e-3, 1), (300.0, 2), (1e-38, 3)])
def test_random_matrices_bit_exact(sigma, seed):
    rows, cols = 257, 128
    x = (torch.randn((rows, cols), generator=torch.Generator().manual_seed(seed)) * sigma)
    assert_bit_exact(bits(x.to(torch.bfloat16)), rows, cols)


def test_every_bf16_pattern_in_one_tensor():
    """All finite bf16 values (as 4096 rows of 16), so every element value
    meets the codecs; scales vary from block to block."""
    b = np.arange(65536, dtype=np.uint16)
    b = b[((b >> 7) & 0xFF) != 0xFF]  # drop inf/NaN
    b = np.concatenate([b, np.zeros((-b.size) % 16, np.uint16)])
    rng = np.random.default_rng(0)
    rng.shuffle(b)
    assert_bit_exact(b, b.size // 16, 16)


def test_zero_and_tie_blocks():
    x = np.zeros((4, 64), np.float32)
    x[1, :16] = [2688, 336, 112, 2240, 1120, 560, 784, 1568, -112, 0, 1, 2, 3, 4, 5, 6]
    x[2, 16:32] = 1e-30
    x[3, :] = -0.0
    assert_bit_exact(bits(torch.from_numpy(x).to(torch.bfloat16)), 4, 64)


def test_amax_in_path_matches():
    dev = require_gpu()
    x = torch.randn((64, 128), generator=torch.Generator().manual_seed(4)).to(torch.bfloat16)
    amax = torch.tensor([x.float().abs().max().item()], dtype=torch.float32, device=dev)
    a = gpu_quant(bits(x), 64, 128)
    b = gpu_quant(bits(x), 64, 128, amax_in=amax)
    for u, w in zip(a, b):
        np.testing.assert_array_equal(np.asarray(u), np.asarray(w))


def test_decode_nvfp4_workload_quantiser_fed_oracle_output():
    """The full decode_nvfp4_d128 output, computed by the oracle and rounded to
    bf16, quantised on the GPU and by the oracle: identical bits."""
    w = WORKLOADS["decode_nvfp4_d128"]
    q, k, v = make_workload_inputs(w)
    o_ref, _ = oracle_rows(q, k, v, w.scale, w.causal)
    o_bits = oracle.to_bf16_bits(o_ref)
    rows = w.B * w.Hq * w.Sq
    assert_bit_exact(o_bits, rows, w.Dv)


def test_decode_then_quantise_pipeline():
    """Decode with the amax folded in, then quantise with amax_in: equals
    quantising the same bf16 O from scratch."""
    dev = require_gpu()
    q, k, v = make_qkv(8, 16, 16, 1, 1024, 128, seed=6)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    amax = torch.zeros(1, dtype=torch.float32, device=dev)
    o, _ = F.decode(qd, kd, vd, num_splits=1, o_amax=amax)
    c1, s1, g1 = F.quantize_nvfp4(o, amax_in=amax)
    c2, s2, g2 = F.quantize_nvfp4(o)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2) and torch.equal(s1, s2) and torch.equal(g1, g2)
    rc, rs, rg = oracle.nvfp4_quantize(bits(o), o.numel() // 128, 128)
    np.testing.assert_array_equal(c1.cpu().numpy(), rc)
    np.testing.assert_array_equal(s1.cpu().numpy(), rs)


# ------------------------------------------- decode with the fused NVFP4 epilogue

def _decode_plain(q, k, v, scale, ns):
    dev = require_gpu()
    B, Hq, Sq, D = q.shape
    _, Hkv, Sk, _ = k.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=dev)
    nb = F.fmha_decode_splitkv_workspace_size(B, Hq, Hkv, Sq, Sk, D, ns)
    ws = torch.empty(max(nb, 16), dtype=torch.uint8, device=dev)
    F.fmha_decode_splitkv(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, scale, False, ns, ws, nb)
    return o, lse


def _decode_fused(q, k, v, scale, ns, g, want_o):
    dev = require_gpu()
    B, Hq, Sq, D = q.shape
    _, Hkv, Sk, _ = k.shape
    rows = B * Hq * Sq
    o = torch.full_like(q, float("nan")) if want_o else None
    lse = torch.full((B, Hq, Sq), float("nan"), dtype=torch.float32, device=dev)
    codes = torch.full((rows, D // 2), 0xAA, dtype=torch.uint8, device=dev)
    scales = torch.full((rows, D // 16), 0xAA, dtype=torch.uint8, device=dev)
    nb = F.fmha_decode_splitkv_workspace_size(B, Hq, Hkv, Sq, Sk, D, ns)
    ws = torch.empty(max(nb, 16), dtype=torch.uint8, device=dev)
    gd = torch.tensor([g], dtype=torch.float32, device=dev)
    F.fmha_decode_splitkv_nvfp4(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, scale, False, ns, ws, nb,
                                gd, codes, scales)
    torch.cuda.synchronize()
    return o, lse, codes.cpu().numpy(), scales.cpu().numpy()


FUSED_CASES = [
    # B, Hq, Hkv, Sk, D, num_splits  (Sq = 1)
    (2, 4, 4, 300, 128, 1),      # no split: the attention kernel's epilogue encodes
    (2, 8, 2, 1000, 64, 5),      # split: the combine kernel encodes
    (1, 64, 1, 700, 512, 3),
    (3, 16, 16, 257, 128, 2),
    (64, 32, 8, 1000, 64, 8),    # 512 (batch, KV head) units: split groups, then the combine encodes
]


@pytest.mark.parametrize("case", FUSED_CASES)
@pytest.mark.parametrize("g_mode", ["tensor", "fixed"])
def test_fused_nvfp4_epilogue_bit_exact(case, g_mode):
    """Codes and scales of the fused epilogue equal the oracle's per-block
    recipe applied to the decode's own bf16 output with the same global scale
    (the output and LSE are unchanged by the fusion)."""
    B, Hq, Hkv, Sk, D, ns = case
    dev = require_gpu()
    q, k, v = (t.to(dev) for t in make_qkv(B, Hq, Hkv, 1, Sk, D, seed=sum(case), sigma=0.8))
    scale = float(np.float32(1.0 / np.sqrt(D)))
    o_ref, lse_ref = _decode_plain(q, k, v, scale, ns)
    torch.cuda.synchronize()
    rows = B * Hq
    o_bits = bits(o_ref.cpu()).reshape(rows, D)
    if g_mode == "tensor":
        amax = np.float32(np.abs(o_ref.float().cpu().numpy()).max())
        g = np.float32(amax / np.float32(2688.0))
    else:
        g = np.float32(0.0007)
    want_c, want_s = oracle.nvfp4_quantize_with_scale(o_bits, rows, D, g)
    for want_o in (True, False):
        o, lse, c, s = _decode_fused(q, k, v, scale, ns, float(g), want_o)
        np.testing.assert_array_equal(s, want_s)
        np.testing.assert_array_equal(c, want_c)
        assert torch.equal(lse, lse_ref)
        if want_o:
            assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16))
