"""Seeded synthetic inputs and the named workloads.

This module holds none of the attention arithmetic: it only draws inputs.
Both the HIP path's tests/benchmark and the CPU oracle take their inputs from
here, so the two sides always see the same bits.

Recipe: ``g = torch.Generator('cpu').manual_seed(seed)``; Q, then K, then V,
each drawn as ``torch.randn(shape, generator=g, dtype=float32) * sigma`` and
rounded to bf16 (round-to-nearest-even, torch's cast).  Shapes are BHSD,
row-major: Q [B, Hq, Sq, D], K [B, Hkv, Sk, D], V [B, Hkv, Sk, Dv].
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "fwd" (prefill), "decode" (split-KV), "decode_nvfp4",
                         # "decode_nvfp4_fused", "decode_paged", "decode_dv" and
                         # "fwd_dv" (Dv != D)
    B: int
    Hq: int
    Hkv: int
    Sq: int
    Sk: int
    D: int
    Dv: int
    sigma: float
    seed: int
    causal: bool
    num_splits: int = 0  # decode only; 0 = the library's heuristic
    v_is_k: bool = False  # V is the same tensor as K (a shared latent)
    page_size: int = 0    # decode_paged: keys per page of the K/V cache
    note: str = ""

    @property
    def scale(self) -> float:
        return default_scale(self.D)

    def shapes(self):
        return ((self.B, self.Hq, self.Sq, self.D), (self.B, self.Hkv, self.Sk, self.D),
                (self.B, self.Hkv, self.Sk, self.Dv))

    def visible_pairs_per_head(self) -> int:
        """Number of (query, key) pairs that take part, per (b, h)."""
        if not self.causal:
            return self.Sq * self.Sk
        return sum(min(self.Sk, i + 1 + self.Sk - self.Sq) for i in range(self.Sq))

    def flops(self) -> int:
        """Algorithmic FLOPs: 2*D per score for QK^T plus 2*Dv per score for PV."""
        return 2 * (self.D + self.Dv) * self.B * self.Hq * self.visible_pairs_per_head()

    def bytes(self) -> int:
        """Algorithmic HBM bytes: Q, K and V read once, O (bf16) and LSE (fp32)
        written once; the NVFP4 workload adds the codes, scales and the global
        scale."""
        q = self.B * self.Hq * self.Sq * self.D
        kv = self.B * self.Hkv * self.Sk * (self.D if self.v_is_k else self.D + self.Dv)
        o = self.B * self.Hq * self.Sq * self.Dv
        n = 2 * (q + kv + o) + 4 * self.B * self.Hq * self.Sq
        if self.kind == "decode_nvfp4":
            n += o // 2 + o // 16 + 4
        elif self.kind == "decode_nvfp4_fused":  # codes and scales instead of O; g read
            n += o // 2 + o // 16 + 4 - 2 * o
        elif self.kind == "decode_paged":  # the block table and the key counts
            n += 4 * self.B * (-(-self.Sk // self.page_size) + 1)
        return n

    def kv_bytes(self) -> int:
        return 2 * self.B * self.Hkv * self.Sk * (self.D if self.v_is_k else self.D + self.Dv)


def default_scale(D: int) -> float:
    """fp32 round-to-nearest of 1/sqrt(D), computed in double."""
    return float(np.float32(1.0 / math.sqrt(D)))


WORKLOADS = {
    w.name: w
    for w in [
        Workload("single_tile_d16", "fwd", 1, 1, 1, 128, 128, 16, 16, 1.0, 0, False,
                 note="one 128x128 score tile, head dim 16"),
        Workload("prefill_causal_d64", "fwd", 4, 16, 16, 2048, 2048, 64, 64, 1.0, 1, True,
                 note="causal prefill, 128x128 tiles"),
        Workload("decode_gqa_d64", "decode", 64, 32, 8, 1, 8192, 64, 64, 1.0, 2, False,
                 num_splits=16, note="GQA 4:1 decode, 16 KV splits"),
        Workload("decode_mqa_d512", "decode", 32, 64, 1, 1, 16384, 512, 512, 0.5, 3, False,
                 note="all 64 query heads share one KV head, head dim 512"),
        Workload("decode_nvfp4_d128", "decode_nvfp4", 128, 16, 16, 1, 4096, 128, 128, 1.0, 4,
                 False, num_splits=1, note="MHA decode, O quantised to NVFP4"),
        Workload("decode_nvfp4_d128_fused", "decode_nvfp4_fused", 128, 16, 16, 1, 4096, 128, 128,
                 1.0, 4, False, num_splits=1,
                 note="the same decode with NVFP4 encoded in its epilogue for a global scale "
                      "held from an earlier step; no bf16 O written"),
        Workload("decode_gqa_d64_paged", "decode_paged", 64, 32, 8, 1, 8192, 64, 64, 1.0, 2,
                 False, num_splits=16, page_size=64,
                 note="the GQA decode reading K/V through a block table from a shuffled pool "
                      "of 64-key pages"),
        Workload("decode_mqa_d512_v_is_k", "decode", 32, 64, 1, 1, 16384, 512, 512, 0.5, 3, False,
                 v_is_k=True,
                 note="the wide-head decode with V the same tensor as K (a shared latent): "
                      "each key row is streamed once"),
        Workload("prefill_causal_d192_dv128", "fwd_dv", 4, 16, 16, 2048, 2048, 192, 128, 1.0, 6,
                 True, note="causal prefill with Q/K head dim 192 and V/O head dim 128"),
        Workload("decode_mqa_d576_dv512_v_in_k", "decode_dv", 32, 64, 1, 1, 16384, 576, 512, 0.5,
                 5, False, v_is_k=True,
                 note="the wide-head decode with Q/K head dim 576 and V the first 512 columns "
                      "of each K row (a 512-wide latent plus 64 more key dims)"),
    ]
}


def make_qkv(B, Hq, Hkv, Sq, Sk, D, Dv=None, *, sigma=1.0, seed=0):
    """Q, K, V as contiguous bf16 CPU tensors drawn from one seeded generator."""
    Dv = D if Dv is None else Dv
    g = torch.Generator("cpu").manual_seed(int(seed))
    out = []
    for shape in ((B, Hq, Sq, D), (B, Hkv, Sk, D), (B, Hkv, Sk, Dv)):
        t = torch.randn(shape, generator=g, dtype=torch.float32)
        if sigma != 1.0:
            t.mul_(sigma)
        out.append(t.to(torch.bfloat16).contiguous())
        del t
    return tuple(out)


def page_pool(k, v, lens, page_size, *, seed, spare_pages=2):
    """A paged KV cache holding the first lens[b] keys of batch b of the
    contiguous K/V [B, Hkv, S, D] (bf16, CPU): pools [num_pages, Hkv,
    page_size, D] whose pages sit in a seeded random order, the block table
    [B, max_pages] (int32, unused entries -1) and num_pages.  Slots that hold
    no key (past a sequence's end, and the spare pages) are NaN, so a read
    outside a sequence shows in the output."""
    B, Hkv, S, D = k.shape
    need = [-(-int(n) // page_size) for n in lens]
    max_pages = max(max(need), 1)
    num_pages = sum(need) + spare_pages
    perm = np.random.default_rng(seed).permutation(num_pages)
    pools = [torch.empty((num_pages, Hkv, page_size, D), dtype=torch.bfloat16) for _ in range(2)]
    for pool in pools:
        pool.view(torch.int16).fill_(0x7FC0)  # bf16 quiet NaN
    table = np.full((B, max_pages), -1, np.int32)
    nxt = 0
    for b in range(B):
        n = int(lens[b])
        if need[b] == 0:
            continue
        pids = perm[nxt:nxt + need[b]]
        nxt += need[b]
        table[b, :need[b]] = pids
        for src, pool in zip((k, v), pools):
            rows = torch.empty((Hkv, need[b] * page_size, D), dtype=torch.bfloat16)
            rows.view(torch.int16).fill_(0x7FC0)
            rows[:, :n] = src[b, :, :n]
            pool[torch.from_numpy(pids.astype(np.int64))] = (
                rows.view(Hkv, need[b], page_size, D).permute(1, 0, 2, 3))
    return pools[0], pools[1], table, num_pages


def make_workload_inputs(w: Workload):
    """(q, k, v); with v_is_k, v is k itself (V = the first Dv columns of each K row)."""
    q, k, v = make_qkv(w.B, w.Hq, w.Hkv, w.Sq, w.Sk, w.D, w.Dv, sigma=w.sigma, seed=w.seed)
    return (q, k, k) if w.v_is_k else (q, k, v)


def v_of(k, dv):
    """V as its own contiguous tensor when V is the first dv columns of the K
    rows (for a caller that needs V apart, such as the oracle)."""
    return k if k.shape[-1] == dv else k[..., :dv].contiguous()


def sample_rows(total: int, n: int, seed: int = 1234) -> np.ndarray:
    """A seeded, sorted sample of flat row ids (always including the first and
    last row), for checking full-size outputs one row at a time."""
    rng = np.random.default_rng(seed)
    n = min(n, total)
    pick = rng.choice(total, size=n, replace=False)
    pick[0] = 0
    if n > 1:
        pick[1] = total - 1
    return np.unique(pick).astype(np.int64)
