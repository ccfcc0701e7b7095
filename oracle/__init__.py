"""CPU oracle for the fused attention forward / split-KV decode path and its
NVFP4 output quantiser.

TEST INFRASTRUCTURE ONLY: the test-suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The HIP product path never imports
this package, and this package never imports the product.  The arithmetic
lives in ``oracle.c`` (fp64 attention, fp32 step-by-step quantiser); this file
only marshals numpy arrays into it.

Inputs are bf16 tensors handed over as their raw 16-bit patterns
(``numpy.uint16``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

GCC_CMD = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
           "-shared", _SRC, "-o", _LIB, "-lm"]


def build() -> str:
    """Compile liboracle.so with gcc (fp contraction off, no fast-math)."""
    subprocess.run(GCC_CMD, check=True)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32, i64, f64 = ctypes.c_int, ctypes.c_longlong, ctypes.c_double
        L.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_to_double.restype = f64
        L.oracle_double_to_bf16.argtypes = [f64]
        L.oracle_double_to_bf16.restype = ctypes.c_uint16
        L.oracle_attention.argtypes = [P, P, P, i32, i32, i32, i32, i32, i32, i32, f64, i32,
                                       i64, P, P, P, i32]
        L.oracle_attention_splits.argtypes = [P, P, P, i32, i32, i32, i32, i32, i32, i32, f64,
                                              i32, i32, i32, P, P, i32]
        L.oracle_combine.argtypes = [P, P, i64, i32, i32, P, P]
        L.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_value.restype = f64
        L.oracle_e4m3_encode.argtypes = [ctypes.c_float]
        L.oracle_e4m3_encode.restype = ctypes.c_uint8
        L.oracle_e2m1_value.argtypes = [ctypes.c_uint8]
        L.oracle_e2m1_value.restype = f64
        L.oracle_e2m1_encode.argtypes = [ctypes.c_float]
        L.oracle_e2m1_encode.restype = ctypes.c_uint8
        L.oracle_nvfp4_quantize.argtypes = [P, i64, i32, P, P, P]
        L.oracle_nvfp4_quantize_with_scale.argtypes = [P, i64, i32, ctypes.c_float, P, P]
        L.oracle_double_to_bf16_array.argtypes = [P, i64, P]
        L.oracle_bf16_to_double_array.argtypes = [P, i64, P]
        L.oracle_e4m3_encode_array.argtypes = [P, i64, P]
        L.oracle_e2m1_encode_array.argtypes = [P, i64, P]
        for f in ("oracle_double_to_bf16_array", "oracle_bf16_to_double_array",
                  "oracle_e4m3_encode_array", "oracle_e2m1_encode_array"):
            getattr(L, f).restype = None
        L.oracle_num_threads.argtypes = []
        L.oracle_num_threads.restype = i32
        for f in ("oracle_attention", "oracle_attention_splits", "oracle_combine",
                  "oracle_nvfp4_quantize", "oracle_nvfp4_quantize_with_scale"):
            getattr(L, f).restype = i32
        _lib = L
    return _lib


def _u16(a) -> np.ndarray:
    """Raw bf16 bit patterns as a contiguous uint16 array (accepts torch bf16 CPU
    tensors or uint16/int16 numpy arrays)."""
    if hasattr(a, "dtype") and str(a.dtype) == "torch.bfloat16":
        import torch
        a = a.detach().to("cpu").contiguous().view(torch.int16).numpy()
    a = np.ascontiguousarray(a)
    if a.dtype == np.int16:
        a = a.view(np.uint16)
    if a.dtype != np.uint16:
        raise TypeError("expected raw bf16 bits (uint16) or a torch.bfloat16 tensor")
    return a


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def attention(q, k, v, *, B, Hq, Hkv, Sq, Sk, D, Dv=None, scale, causal=False,
              rows=None, nthreads=0):
    """O1: plain softmax attention in fp64.  Returns (o[nrows, Dv], lse[nrows]).

    ``rows`` (optional) selects flat row ids ``(b*Hq + h)*Sq + i``; without it
    every row is evaluated and o reshapes to [B, Hq, Sq, Dv]."""
    Dv = D if Dv is None else Dv
    qa, ka, va = _u16(q), _u16(k), _u16(v)
    assert qa.size == B * Hq * Sq * D and ka.size == B * Hkv * Sk * D
    assert va.size == B * Hkv * Sk * Dv
    if rows is None:
        n, rp = B * Hq * Sq, None
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        n, rp = rows.size, _ptr(rows)
    o = np.empty((n, Dv), np.float64)
    lse = np.empty((n,), np.float64)
    rc = lib().oracle_attention(_ptr(qa), _ptr(ka), _ptr(va), B, Hq, Hkv, Sq, Sk, D, Dv,
                                float(scale), int(bool(causal)), n, rp, _ptr(o), _ptr(lse),
                                int(nthreads))
    if rc:
        raise ValueError(f"oracle_attention failed with code {rc}")
    return o, lse


def attention_splits(q, k, v, *, B, Hq, Hkv, Sq, Sk, D, Dv=None, scale, causal=False,
                     nsplit, chunk, nthreads=0):
    """O2, first half: per-split outputs and log-sum-exps over key ranges
    [s*chunk, (s+1)*chunk).  Returns (o_part[rows, nsplit, Dv], lse_part[rows, nsplit])."""
    Dv = D if Dv is None else Dv
    qa, ka, va = _u16(q), _u16(k), _u16(v)
    n = B * Hq * Sq
    op = np.empty((n, nsplit, Dv), np.float64)
    lp = np.empty((n, nsplit), np.float64)
    rc = lib().oracle_attention_splits(_ptr(qa), _ptr(ka), _ptr(va), B, Hq, Hkv, Sq, Sk, D,
                                       Dv, float(scale), int(bool(causal)), nsplit, chunk,
                                       _ptr(op), _ptr(lp), int(nthreads))
    if rc:
        raise ValueError(f"oracle_attention_splits failed with code {rc}")
    return op, lp


def combine(o_part, lse_part):
    """O2, second half: log-sum-exp combine of split results."""
    op = np.ascontiguousarray(o_part, dtype=np.float64)
    lp = np.ascontiguousarray(lse_part, dtype=np.float64)
    n, ns, dv = op.shape
    o = np.empty((n, dv), np.float64)
    lse = np.empty((n,), np.float64)
    rc = lib().oracle_combine(_ptr(op), _ptr(lp), n, ns, dv, _ptr(o), _ptr(lse))
    if rc:
        raise ValueError(f"oracle_combine failed with code {rc}")
    return o, lse


def to_bf16_bits(x) -> np.ndarray:
    """Round fp64 values to bf16 (one RNE rounding); returns uint16 bits."""
    xa = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(xa.shape, np.uint16)
    lib().oracle_double_to_bf16_array(_ptr(xa), xa.size, _ptr(out))
    return out


def bf16_bits_to_f64(h) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp64."""
    ha = _u16(h)
    out = np.empty(ha.shape, np.float64)
    lib().oracle_bf16_to_double_array(_ptr(ha), ha.size, _ptr(out))
    return out


def e4m3_encode_array(x) -> np.ndarray:
    xa = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(xa.shape, np.uint8)
    lib().oracle_e4m3_encode_array(_ptr(xa), xa.size, _ptr(out))
    return out


def e2m1_encode_array(x) -> np.ndarray:
    xa = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(xa.shape, np.uint8)
    lib().oracle_e2m1_encode_array(_ptr(xa), xa.size, _ptr(out))
    return out


def nvfp4_quantize(x_bits, rows, cols):
    """O3: NVFP4 quantiser on a bf16 matrix.  Returns (codes[rows, cols/2] u8,
    scales[rows, cols/16] u8, global_scale float32)."""
    xa = _u16(x_bits)
    assert xa.size == rows * cols
    codes = np.empty((rows, cols // 2), np.uint8)
    scales = np.empty((rows, cols // 16), np.uint8)
    g = np.zeros((1,), np.float32)
    rc = lib().oracle_nvfp4_quantize(_ptr(xa), rows, cols, _ptr(codes), _ptr(scales), _ptr(g))
    if rc:
        raise ValueError(f"oracle_nvfp4_quantize failed with code {rc}")
    return codes, scales, g[0]


def nvfp4_quantize_with_scale(x_bits, rows, cols, g):
    """O3 per-block recipe for a given global scale g (float32).  Returns
    (codes[rows, cols/2] u8, scales[rows, cols/16] u8)."""
    xa = _u16(x_bits)
    assert xa.size == rows * cols
    codes = np.empty((rows, cols // 2), np.uint8)
    scales = np.empty((rows, cols // 16), np.uint8)
    rc = lib().oracle_nvfp4_quantize_with_scale(_ptr(xa), rows, cols, float(np.float32(g)),
                                                _ptr(codes), _ptr(scales))
    if rc:
        raise ValueError(f"oracle_nvfp4_quantize_with_scale failed with code {rc}")
    return codes, scales


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return lib().oracle_num_threads()


def e4m3_value(c: int) -> float:
    return lib().oracle_e4m3_value(c)


def e4m3_encode(x: float) -> int:
    return lib().oracle_e4m3_encode(x)


def e2m1_value(c: int) -> float:
    return lib().oracle_e2m1_value(c)


def e2m1_encode(x: float) -> int:
    return lib().oracle_e2m1_encode(x)
