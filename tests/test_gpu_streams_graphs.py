"""The entry points on a caller's stream and inside a captured HIP graph.

Every entry point launches on the stream it is given and on nothing else, so
a graph captured on torch's capture stream holds the whole call (split
kernels, combine, the library's amax clear and fold, quantiser).  The replays are checked
bit for bit against the same calls made eagerly on the same inputs, with new
inputs written between replays, and the first replay against the oracle."""
import ctypes

import numpy as np
import pytest
import torch

from gpu_helpers import assert_parity, oracle_rows, require_gpu

pytestmark = pytest.mark.gpu


def _randn(shape, g, dev, sigma=1.0):
    return (torch.randn(shape, generator=g) * sigma).to(torch.bfloat16).to(dev)


class _Calls:
    """Static buffers and one step of calls: a GQA decode with 16 splits (all
    splits of a (batch, KV head) in one workgroup), an MHA decode at head dim
    128 folding max|O| into a caller-held amax and quantising O with it, and a
    causal prefill whose output is quantised with the library's own amax."""

    def __init__(self, dev, g):
        import decode_fmha_fwd_amd as F
        self.F = F
        # GQA decode, head dim 64
        self.a = dict(B=64, Hq=32, Hkv=8, Sq=1, Sk=1024, D=64, ns=16)
        a = self.a
        self.qa = _randn((a["B"], a["Hq"], 1, a["D"]), g, dev)
        self.ka = _randn((a["B"], a["Hkv"], a["Sk"], a["D"]), g, dev)
        self.va = _randn((a["B"], a["Hkv"], a["Sk"], a["D"]), g, dev)
        self.oa = torch.empty_like(self.qa)
        self.la = torch.empty((a["B"], a["Hq"], 1), dtype=torch.float32, device=dev)
        self.nba = F.fmha_decode_splitkv_workspace_size(a["B"], a["Hq"], a["Hkv"], 1, a["Sk"],
                                                        a["D"], a["ns"])
        self.wsa = torch.empty(self.nba, dtype=torch.uint8, device=dev)
        # MHA decode, head dim 128, default splits, amax fold + NVFP4 of O
        self.b = dict(B=4, Hq=16, Hkv=16, Sq=1, Sk=2000, D=128)
        b = self.b
        self.qb = _randn((b["B"], b["Hq"], 1, b["D"]), g, dev)
        self.kb = _randn((b["B"], b["Hkv"], b["Sk"], b["D"]), g, dev)
        self.vb = _randn((b["B"], b["Hkv"], b["Sk"], b["D"]), g, dev)
        self.ob = torch.empty_like(self.qb)
        self.lb = torch.empty((b["B"], b["Hq"], 1), dtype=torch.float32, device=dev)
        self.nbb = F.fmha_decode_splitkv_workspace_size(b["B"], b["Hq"], b["Hkv"], 1, b["Sk"],
                                                        b["D"], 0)
        self.wsb = torch.empty(max(self.nbb, 16), dtype=torch.uint8, device=dev)
        self.amax = torch.empty(1, dtype=torch.float32, device=dev)
        rows_b = b["B"] * b["Hq"]
        self.cb = torch.empty((rows_b, b["D"] // 2), dtype=torch.uint8, device=dev)
        self.sb = torch.empty((rows_b, b["D"] // 16), dtype=torch.uint8, device=dev)
        self.gb = torch.empty(1, dtype=torch.float32, device=dev)
        # causal prefill, head dim 64, quantised with the library's own amax
        self.c = dict(B=1, H=4, S=700, D=64)
        c = self.c
        self.qc = _randn((c["B"], c["H"], c["S"], c["D"]), g, dev)
        self.kc = _randn((c["B"], c["H"], c["S"], c["D"]), g, dev)
        self.vc = _randn((c["B"], c["H"], c["S"], c["D"]), g, dev)
        self.oc = torch.empty_like(self.qc)
        self.lc = torch.empty((c["B"], c["H"], c["S"]), dtype=torch.float32, device=dev)
        rows_c = c["B"] * c["H"] * c["S"]
        self.cc = torch.empty((rows_c, c["D"] // 2), dtype=torch.uint8, device=dev)
        self.sc = torch.empty((rows_c, c["D"] // 16), dtype=torch.uint8, device=dev)
        self.gc = torch.empty(1, dtype=torch.float32, device=dev)
        self.nbc = F.nvfp4_quantize_workspace_size(rows_c, c["D"])
        self.wsc = torch.empty(max(self.nbc, 16), dtype=torch.uint8, device=dev)

    def outputs(self):
        return [self.oa, self.la, self.ob, self.lb, self.amax, self.cb, self.sb, self.gb,
                self.oc, self.lc, self.cc, self.sc, self.gc]

    def poison(self):
        for t in self.outputs():
            if t.dtype == torch.uint8:
                t.fill_(0xAA)
            else:
                t.fill_(float("nan"))

    def new_inputs(self, g):
        for t in (self.qa, self.qb, self.qc, self.kc):
            t.copy_(_randn(tuple(t.shape), g, t.device))

    def step(self, stream=None):
        F, a, b, c = self.F, self.a, self.b, self.c
        F.fmha_decode_splitkv(self.qa, self.ka, self.va, self.oa, self.la, a["B"], a["Hq"],
                              a["Hkv"], 1, a["Sk"], a["D"], a["D"] ** -0.5, 0, a["ns"], self.wsa,
                              self.nba, None, stream=stream)
        F.fmha_decode_splitkv(self.qb, self.kb, self.vb, self.ob, self.lb, b["B"], b["Hq"],
                              b["Hkv"], 1, b["Sk"], b["D"], b["D"] ** -0.5, 0, 0, self.wsb,
                              self.nbb, self.amax, stream=stream)
        F.nvfp4_quantize(self.ob, b["B"] * b["Hq"], b["D"], self.cb, self.sb, self.gb, self.amax,
                         None, 0, stream=stream)
        F.fmha_fwd(self.qc, self.kc, self.vc, self.oc, self.lc, c["B"], c["H"], c["H"], c["S"],
                   c["S"], c["D"], c["D"] ** -0.5, 1, stream=stream)
        F.nvfp4_quantize(self.oc, c["B"] * c["H"] * c["S"], c["D"], self.cc, self.sc, self.gc,
                         None, self.wsc, self.nbc, stream=stream)

    def snapshot(self):
        return [t.detach().cpu().clone() for t in self.outputs()]


def _same_bits(x, y, what):
    xb = x.contiguous().view(torch.uint8).numpy()
    yb = y.contiguous().view(torch.uint8).numpy()
    n = int((xb != yb).sum())
    assert n == 0, f"{what}: {n} bytes differ"


def _check_oracle(calls):
    a, c = calls.a, calls.c
    rows = np.random.default_rng(7).choice(a["B"] * a["Hq"], 256, replace=False)
    o_ref, l_ref = oracle_rows(calls.qa, calls.ka, calls.va, a["D"] ** -0.5, False, rows=rows)
    assert_parity(calls.oa, calls.la, o_ref, l_ref, rows=rows, what="graph GQA decode")
    rows = np.random.default_rng(8).choice(c["B"] * c["H"] * c["S"], 256, replace=False)
    o_ref, l_ref = oracle_rows(calls.qc, calls.kc, calls.vc, c["D"] ** -0.5, True, rows=rows)
    assert_parity(calls.oc, calls.lc, o_ref, l_ref, rows=rows, what="graph causal prefill")


def test_calls_on_a_side_stream_match_the_default_stream():
    dev = require_gpu()
    g = torch.Generator().manual_seed(21)
    calls = _Calls(dev, g)
    calls.poison()
    calls.step()
    torch.cuda.synchronize()
    ref = calls.snapshot()
    calls.poison()
    torch.cuda.synchronize()
    side = torch.cuda.Stream(device=dev)  # default priority
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        calls.poison()  # ordered before the calls on the side stream only
        calls.step(stream=ctypes.c_void_p(side.cuda_stream))
    side.synchronize()
    for i, (x, y) in enumerate(zip(ref, calls.snapshot())):
        _same_bits(x, y, f"output {i}")


def test_graph_replays_match_eager_calls():
    dev = require_gpu()
    g = torch.Generator().manual_seed(22)
    calls = _Calls(dev, g)
    # warm-up on a side stream, as torch asks before a capture
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        calls.step()
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls.step()
    torch.cuda.synchronize()
    for rep in range(3):
        calls.new_inputs(g)
        calls.poison()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        replayed = calls.snapshot()
        if rep == 0:
            _check_oracle(calls)
        calls.poison()
        calls.step()
        torch.cuda.synchronize()
        for i, (x, y) in enumerate(zip(replayed, calls.snapshot())):
            _same_bits(x, y, f"replay {rep}, output {i}")
