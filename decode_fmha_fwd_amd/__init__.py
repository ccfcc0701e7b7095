"""Python binding of libfmha.so: fused multi-head attention forward, split-KV
decode with a log-sum-exp combine, and an NVFP4 output quantiser, as
hand-written HIP kernels for MI355X (gfx950).

The functions named like the C ABI (``fmha_fwd``, ``fmha_decode_splitkv``,
``nvfp4_quantize``, ...) only marshal arguments: they take torch tensors that
already live on the GPU, pass their device pointers and torch's current HIP
stream to the library, and raise ``FmhaError`` on a non-zero status.  Every
step of the computation runs in the library's kernels; PyTorch only provides
device memory and the stream.  There is no fallback: if ``libfmha.so`` is
missing or cannot be loaded, every call raises.

Convenience wrappers ``fwd``, ``decode`` and ``quantize_nvfp4`` allocate the
outputs (and the decode workspace) with torch and call the entry points.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfmha.so")

STATUS = {0: "FMHA_OK", 1: "FMHA_ERR_NULL", 2: "FMHA_ERR_SHAPE", 3: "FMHA_ERR_HEAD_DIM",
          4: "FMHA_ERR_GQA", 5: "FMHA_ERR_ALIGN", 6: "FMHA_ERR_WORKSPACE", 7: "FMHA_ERR_HIP",
          8: "FMHA_ERR_ARG"}

# name -> (restype, argtypes)
_P, _I, _LL, _F, _SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_longlong, ctypes.c_float, ctypes.c_size_t
SIGNATURES = {
    "fmha_fwd": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _P]),
    "fmha_fwd_dv": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _I, _P]),
    "fmha_decode_splitkv_workspace_size": (_SZ, [_I, _I, _I, _I, _I, _I, _I]),
    "fmha_decode_splitkv": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _I, _P, _SZ,
                                 _P, _P]),
    "fmha_decode_splitkv_nvfp4": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _I, _P,
                                       _SZ, _P, _P, _P, _P]),
    "fmha_decode_paged": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _P, _P, _I, _I, _I, _I, _F,
                               _I, _I, _P, _SZ, _P]),
    "fmha_decode_splitkv_noalloc": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _F, _I, _I,
                                         _P, _P]),
    "fmha_decode_default_splits": (_I, [_I, _I, _I, _I, _I, _I]),
    "fmha_decode_splitkv_dv_workspace_size": (_SZ, [_I, _I, _I, _I, _I, _I, _I, _I]),
    "fmha_decode_splitkv_dv": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _I, _I,
                                    _P, _SZ, _P]),
    "nvfp4_quantize_workspace_size": (_SZ, [_LL, _I]),
    "nvfp4_quantize": (_I, [_P, _LL, _I, _P, _P, _P, _P, _P, _SZ, _P]),
    "fmha_debug_qk_scores": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _F, _I, _P]),
    "fmha_status_string": (ctypes.c_char_p, [_I]),
    "fmha_last_error": (ctypes.c_char_p, []),
}


class FmhaError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str):
        super().__init__(f"{fn} -> {STATUS.get(status, status)}: {detail}")
        self.status = status


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libfmha.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise FmhaError("load_library", -1,
                            f"{path} not found; build it with `python -m decode_fmha_fwd_amd.build`")
        lib = ctypes.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _check(fn: str, status: int):
    if status != 0:
        detail = load_library().fmha_last_error().decode()
        raise FmhaError(fn, status, detail)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device=None) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need_gpu_bf16(name, t):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != torch.bfloat16:
        raise ValueError(f"{name} must be bfloat16")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


# ---------------------------------------------------------------- C ABI names

def fmha_fwd(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, scale, causal, stream=None):
    lib = load_library()
    st = stream if stream is not None else _stream(q.device)
    _check("fmha_fwd", lib.fmha_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv,
                                    Sq, Sk, D, float(scale), int(causal), st))


def fmha_fwd_dv(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, Dv, scale, causal, stream=None):
    lib = load_library()
    st = stream if stream is not None else _stream(q.device)
    _check("fmha_fwd_dv", lib.fmha_fwd_dv(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq,
                                          Hkv, Sq, Sk, D, Dv, float(scale), int(causal), st))


def fmha_decode_splitkv_workspace_size(B, Hq, Hkv, Sq, Sk, D, num_splits) -> int:
    return load_library().fmha_decode_splitkv_workspace_size(B, Hq, Hkv, Sq, Sk, D, num_splits)


def fmha_decode_default_splits(B, Hq, Hkv, Sq, Sk, D) -> int:
    return load_library().fmha_decode_default_splits(B, Hq, Hkv, Sq, Sk, D)


def fmha_decode_splitkv(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, scale, causal, num_splits,
                        workspace, workspace_bytes, o_amax=None, stream=None):
    lib = load_library()
    st = stream if stream is not None else _stream(q.device)
    _check("fmha_decode_splitkv",
           lib.fmha_decode_splitkv(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, Sq,
                                   Sk, D, float(scale), int(causal), int(num_splits),
                                   _ptr(workspace), int(workspace_bytes), _ptr(o_amax), st))


def fmha_decode_splitkv_noalloc(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, scale, causal,
                                num_splits, o_amax=None, stream=None):
    lib = load_library()
    st = stream if stream is not None else _stream(q.device)
    _check("fmha_decode_splitkv_noalloc",
           lib.fmha_decode_splitkv_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq,
                                           Hkv, Sq, Sk, D, float(scale), int(causal),
                                           int(num_splits), _ptr(o_amax), st))


def fmha_decode_splitkv_dv_workspace_size(B, Hq, Hkv, Sq, Sk, D, Dv, num_splits) -> int:
    return load_library().fmha_decode_splitkv_dv_workspace_size(B, Hq, Hkv, Sq, Sk, D, Dv,
                                                                num_splits)


def fmha_decode_splitkv_dv(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, Dv, scale, causal, num_splits,
                           workspace, workspace_bytes, stream=None):
    lib = load_library()
    st = stream if stream is not None else _stream(q.device)
    _check("fmha_decode_splitkv_dv",
           lib.fmha_decode_splitkv_dv(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv,
                                      Sq, Sk, D, Dv, float(scale), int(causal), int(num_splits),
                                      _ptr(workspace), int(workspace_bytes), st))


def fmha_decode_splitkv_nvfp4(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, scale, causal, num_splits,
                              workspace, workspace_bytes, global_scale, codes, scales,
                              stream=None):
    lib = load_library()
    st = stream if stream is not None else _stream(q.device)
    _check("fmha_decode_splitkv_nvfp4",
           lib.fmha_decode_splitkv_nvfp4(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq,
                                         Hkv, Sq, Sk, D, float(scale), int(causal),
                                         int(num_splits), _ptr(workspace), int(workspace_bytes),
                                         _ptr(global_scale), _ptr(codes), _ptr(scales), st))


def fmha_decode_paged(q, k_cache, v_cache, o, lse, B, Hq, Hkv, Sq, seqlens_k, block_table,
                      max_pages_per_seq, page_size, num_pages, D, scale, causal, num_splits,
                      workspace, workspace_bytes, stream=None):
    lib = load_library()
    st = stream if stream is not None else _stream(q.device)
    _check("fmha_decode_paged",
           lib.fmha_decode_paged(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(o), _ptr(lse), B, Hq,
                                 Hkv, Sq, _ptr(seqlens_k), _ptr(block_table),
                                 int(max_pages_per_seq), int(page_size), int(num_pages), D,
                                 float(scale), int(causal), int(num_splits), _ptr(workspace),
                                 int(workspace_bytes), st))


def nvfp4_quantize_workspace_size(rows, cols) -> int:
    return load_library().nvfp4_quantize_workspace_size(rows, cols)


def nvfp4_quantize(x, rows, cols, codes, scales, global_scale, amax_in=None, workspace=None,
                   workspace_bytes=0, stream=None):
    lib = load_library()
    st = stream if stream is not None else _stream(x.device)
    _check("nvfp4_quantize",
           lib.nvfp4_quantize(_ptr(x), rows, cols, _ptr(codes), _ptr(scales), _ptr(global_scale),
                              _ptr(amax_in), _ptr(workspace), int(workspace_bytes), st))


def fmha_debug_qk_scores(q, k, v, s_out, B, Hq, Hkv, Sq, Sk, D, Dv, scale, decode, stream=None):
    lib = load_library()
    st = stream if stream is not None else _stream(q.device)
    _check("fmha_debug_qk_scores",
           lib.fmha_debug_qk_scores(_ptr(q), _ptr(k), _ptr(v), _ptr(s_out), B, Hq, Hkv, Sq, Sk, D,
                                    Dv, float(scale), int(decode), st))


# ---------------------------------------------------------------- conveniences

def fwd(q, k, v, *, causal=False, scale=None, want_lse=True):
    """Attention forward on [B, H, S, D] bf16 GPU tensors (V may have its own
    head dim) -> (o bf16 [B, Hq, Sq, Dv], lse fp32 or None)."""
    for n, t in (("q", q), ("k", k), ("v", v)):
        _need_gpu_bf16(n, t)
    B, Hq, Sq, D = q.shape
    _, Hkv, Sk, _ = k.shape
    Dv = v.shape[-1]
    scale = (1.0 / D ** 0.5) if scale is None else scale
    o = torch.empty((B, Hq, Sq, Dv), dtype=torch.bfloat16, device=q.device)
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device) if want_lse else None
    if Dv == D:
        fmha_fwd(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, scale, causal)
    else:
        fmha_fwd_dv(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, Dv, scale, causal)
    return o, lse


class DecodeWorkspace:
    """Reusable split-KV workspace, grown on demand (allocated by torch)."""

    def __init__(self):
        self.buf = None

    def get(self, nbytes, device):
        if nbytes == 0:
            return None
        if self.buf is None or self.buf.numel() < nbytes or self.buf.device != torch.device(device):
            self.buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
        return self.buf


def decode(q, k, v, *, num_splits=0, causal=False, scale=None, workspace=None, o_amax=None,
           want_lse=True):
    """Split-KV decode on [B, H, S, D] bf16 GPU tensors -> (o bf16, lse fp32 or None)."""
    for n, t in (("q", q), ("k", k), ("v", v)):
        _need_gpu_bf16(n, t)
    B, Hq, Sq, D = q.shape
    _, Hkv, Sk, _ = k.shape
    scale = (1.0 / D ** 0.5) if scale is None else scale
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device) if want_lse else None
    nbytes = fmha_decode_splitkv_workspace_size(B, Hq, Hkv, Sq, Sk, D, num_splits)
    ws = (workspace or DecodeWorkspace()).get(nbytes, q.device)
    fmha_decode_splitkv(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, scale, causal, num_splits, ws,
                        nbytes, o_amax)
    return o, lse


def decode_dv(q, k, v, dv, *, num_splits=0, causal=False, scale=None, workspace=None,
              want_lse=True):
    """Split-KV decode with V/O head dim ``dv`` (Q/K: q.shape[-1]) -> (o [B, Hq, Sq, dv],
    lse).  ``v`` is a [B, Hkv, Sk, dv] tensor, or ``k`` itself, which makes V the
    first ``dv`` columns of the K rows."""
    for n, t in (("q", q), ("k", k), ("v", v)):
        _need_gpu_bf16(n, t)
    B, Hq, Sq, D = q.shape
    _, Hkv, Sk, _ = k.shape
    scale = (1.0 / D ** 0.5) if scale is None else scale
    o = torch.empty((B, Hq, Sq, dv), dtype=torch.bfloat16, device=q.device)
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device) if want_lse else None
    nbytes = fmha_decode_splitkv_dv_workspace_size(B, Hq, Hkv, Sq, Sk, D, dv, num_splits)
    ws = (workspace or DecodeWorkspace()).get(nbytes, q.device)
    fmha_decode_splitkv_dv(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, dv, scale, causal, num_splits,
                           ws, nbytes)
    return o, lse


def quantize_nvfp4(x, amax_in=None):
    """NVFP4 quantisation of a bf16 GPU tensor viewed as [rows, last_dim] ->
    (codes uint8 [rows, cols/2], scales uint8 [rows, cols/16], global_scale fp32 [1])."""
    _need_gpu_bf16("x", x)
    cols = x.shape[-1]
    rows = x.numel() // cols
    codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=x.device)
    scales = torch.empty((rows, cols // 16), dtype=torch.uint8, device=x.device)
    g = torch.empty((1,), dtype=torch.float32, device=x.device)
    nbytes = nvfp4_quantize_workspace_size(rows, cols)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=x.device) if amax_in is None else None
    nvfp4_quantize(x, rows, cols, codes, scales, g, amax_in, ws, nbytes if ws is not None else 0)
    return codes, scales, g
