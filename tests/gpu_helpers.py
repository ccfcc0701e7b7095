"""Shared helpers of the GPU parity tests: device checks, the parity bar, and
oracle calls on the same seeded inputs."""
import numpy as np
import pytest
import torch

import oracle

# Parity bar on O (bf16 output against the unrounded fp64 oracle) and LSE.
O_MAX_ABS = 2e-2
O_MEAN_ABS = 2e-3
LSE_MAX_ABS = 1e-3


def require_gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU")
    import decode_fmha_fwd_amd as F
    F.load_library()
    return torch.device("cuda:0")


def bits(t):
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def oracle_rows(q, k, v, scale, causal, rows=None, nthreads=0):
    B, Hq, Sq, D = q.shape
    _, Hkv, Sk, Dv = v.shape
    return oracle.attention(bits(q), bits(k), bits(v), B=B, Hq=Hq, Hkv=Hkv, Sq=Sq, Sk=Sk, D=D,
                            Dv=Dv, scale=scale, causal=causal, rows=rows, nthreads=nthreads)


def assert_parity(o_gpu, lse_gpu, o_ref, lse_ref, rows=None, what=""):
    """o_gpu: bf16 GPU tensor [B, H, S, D]; lse_gpu fp32 [B, H, S] or None;
    o_ref [nrows, D] fp64; lse_ref [nrows]; rows: flat row ids of the reference
    rows (None = all)."""
    D = o_gpu.shape[-1]
    og = o_gpu.detach().float().cpu().numpy().astype(np.float64).reshape(-1, D)
    if rows is not None:
        og = og[rows]
    assert np.isfinite(og).all(), f"{what}: non-finite output (unwritten or NaN)"
    err = np.abs(og - o_ref)
    mx, mean = float(err.max()), float(err.mean())
    assert mx <= O_MAX_ABS and mean <= O_MEAN_ABS, f"{what}: O max {mx:.3e} mean {mean:.3e}"
    if lse_gpu is not None:
        lg = lse_gpu.detach().cpu().numpy().astype(np.float64).reshape(-1)
        if rows is not None:
            lg = lg[rows]
        # a row that sees no key has lse = -inf on both sides
        same_inf = np.isinf(lg) & np.isinf(lse_ref) & (np.sign(lg) == np.sign(lse_ref))
        with np.errstate(invalid="ignore"):
            lerr = float(np.where(same_inf, 0.0, np.abs(lg - lse_ref)).max())
        assert lerr <= LSE_MAX_ABS, f"{what}: LSE max {lerr:.3e}"
    return mx, mean


def poison_like(t):
    """A same-shaped output buffer pre-filled with NaN, so unwritten elements show."""
    out = torch.empty_like(t)
    out.fill_(float("nan"))
    return out
