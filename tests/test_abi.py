"""Host-side checks of the C ABI (no GPU needed, nothing is launched): the
library loads, exports every function include/fmha.h declares, and rejects bad
arguments with the documented status before any launch."""
import ctypes
import os
import re

import pytest

import decode_fmha_fwd_amd as F

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "fmha.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*[A-Za-z_][\w\s\*]*?\b(\w+)\s*\(", src, flags=re.M)))


def test_library_exports_every_declared_symbol():
    lib = F.load_library()
    names = declared_functions()
    assert {"fmha_fwd", "fmha_decode_splitkv", "nvfp4_quantize"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert set(F.SIGNATURES) == set(names)


def test_status_strings():
    lib = F.load_library()
    for s in range(9):
        assert lib.fmha_status_string(s)
    assert lib.fmha_status_string(99) == b"unknown status"


FAKE = 0x100000  # aligned, never dereferenced: every case below fails validation first


def call_fwd(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None, B=1, Hq=1, Hkv=1, Sq=4, Sk=4, D=64,
             scale=0.125, causal=0):
    return F.load_library().fmha_fwd(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, scale, causal, None)


def call_dec(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None, B=1, Hq=4, Hkv=1, Sq=1, Sk=1024, D=64,
             scale=0.125, causal=0, ns=4, ws=None, wsb=0, amax=None):
    return F.load_library().fmha_decode_splitkv(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, scale,
                                                causal, ns, ws, wsb, amax, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), 1), (dict(o=None), 1),
    (dict(B=0), 2), (dict(Sk=0), 2), (dict(Sq=5, Sk=4, causal=1), 2),
    (dict(D=48), 3), (dict(D=512), 3),
    (dict(Hq=3, Hkv=2), 4),
    (dict(q=FAKE + 8), 5), (dict(lse=FAKE + 4), 5),
    (dict(scale=0.0), 8), (dict(scale=float("nan")), 8), (dict(causal=2), 8),
])
def test_fwd_validation(kw, status):
    assert call_fwd(**kw) == status
    assert F.load_library().fmha_last_error()


@pytest.mark.parametrize("kw,status", [
    (dict(k=None), 1), (dict(Hq=6, Hkv=4), 4), (dict(D=16), 3), (dict(D=256), 3),
    (dict(ns=-1), 8), (dict(ns=2000), 8), (dict(v=FAKE + 2), 5),
    (dict(ns=4, ws=None, wsb=0), 6), (dict(ns=4, ws=FAKE, wsb=16), 6),
    (dict(ns=4, ws=FAKE + 8, wsb=1 << 30), 5), (dict(amax=FAKE + 1), 5),
])
def test_decode_validation(kw, status):
    assert call_dec(**kw) == status


def call_dec_dv(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None, B=1, Hq=4, Hkv=1, Sq=1, Sk=1024, D=576,
                Dv=512, scale=0.125, causal=0, ns=4, ws=None, wsb=0):
    return F.load_library().fmha_decode_splitkv_dv(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, Dv,
                                                   scale, causal, ns, ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(Dv=256), 3), (dict(D=512, Dv=576), 3), (dict(D=128, Dv=64), 3), (dict(Dv=576), 3),
    (dict(D=64, Dv=512), 3),
    (dict(k=None), 1), (dict(o=None), 1), (dict(Hq=6, Hkv=4), 4), (dict(v=FAKE + 2), 5),
    (dict(ns=4, ws=None, wsb=0), 6), (dict(ns=4, ws=FAKE, wsb=1024), 6), (dict(ns=-1), 8),
    (dict(Sq=2, Sk=1, causal=1), 2),
])
def test_decode_dv_validation(kw, status):
    assert call_dec_dv(**kw) == status
    assert F.load_library().fmha_last_error()


def test_decode_576_needs_the_dv_entry_point():
    assert call_dec(D=576) == 3
    lib = F.load_library()
    assert lib.fmha_decode_splitkv_nvfp4(FAKE, FAKE, FAKE, FAKE, None, 1, 4, 1, 1, 1024, 576,
                                         0.125, 0, 1, None, 0, FAKE, FAKE, FAKE, None) == 3
    assert call_paged(D=576) == 3


def test_dv_workspace_formula():
    rows, ns, dv = 32 * 64, 8, 512
    want = -(-rows * ns * dv * 4 // 256) * 256 + -(-rows * ns * 4 // 256) * 256
    assert F.fmha_decode_splitkv_dv_workspace_size(32, 64, 1, 1, 16384, 576, 512, 8) == want
    assert F.fmha_decode_splitkv_dv_workspace_size(32, 64, 1, 1, 16384, 576, 576, 8) == 0
    assert F.fmha_decode_splitkv_dv_workspace_size(32, 64, 1, 1, 16384, 576, 512, 1) == 0
    # equal dims: the plain decode's formula
    assert (F.fmha_decode_splitkv_dv_workspace_size(64, 32, 8, 1, 8192, 64, 64, 16) ==
            F.fmha_decode_splitkv_workspace_size(64, 32, 8, 1, 8192, 64, 16))


def call_fwd_dv(q=FAKE, k=FAKE, v=2 * FAKE, o=FAKE, lse=None, B=1, Hq=1, Hkv=1, Sq=4, Sk=4, D=192,
                Dv=128, scale=0.125, causal=0):
    return F.load_library().fmha_fwd_dv(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, D, Dv, scale, causal,
                                        None)


@pytest.mark.parametrize("kw,status", [
    (dict(Dv=64), 3), (dict(D=128, Dv=192), 3), (dict(D=64, Dv=128), 3), (dict(Dv=192), 3),
    (dict(D=576, Dv=512), 3), (dict(v=None), 1), (dict(Hq=3, Hkv=2), 4), (dict(o=FAKE + 4), 5),
    (dict(Sq=5, Sk=4, causal=1), 2), (dict(scale=-1.0), 8),
])
def test_fwd_dv_validation(kw, status):
    assert call_fwd_dv(**kw) == status
    assert F.load_library().fmha_last_error()


def test_fwd_dv_rejects_v_inside_k():
    assert call_fwd_dv(k=FAKE, v=FAKE) == 8
    assert b"decode only" in F.load_library().fmha_last_error()


def test_fwd_192_needs_the_dv_entry_point():
    assert call_fwd(D=192) == 3


def call_paged(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=None, B=2, Hq=4, Hkv=1, Sq=1, sl=FAKE, bt=FAKE,
               mp=8, ps=64, npages=16, D=64, scale=0.125, causal=0, ns=4, ws=None, wsb=0):
    return F.load_library().fmha_decode_paged(q, k, v, o, lse, B, Hq, Hkv, Sq, sl, bt, mp, ps,
                                              npages, D, scale, causal, ns, ws, wsb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(sl=None), 1), (dict(bt=None), 1), (dict(k=None), 1), (dict(o=None), 1),
    (dict(sl=FAKE + 2), 5), (dict(bt=FAKE + 1), 5), (dict(k=FAKE + 8), 5),
    (dict(ps=32), 8), (dict(ps=96), 8), (dict(ps=1 << 25), 8), (dict(mp=0), 8),
    (dict(npages=0), 8), (dict(mp=1 << 20, ps=1 << 12), 8),
    (dict(D=16), 3), (dict(Hq=6, Hkv=4), 4),
    (dict(Sq=600, causal=1), 2),          # causal needs Sq <= max_pages * page_size (512)
    (dict(ns=4, ws=None, wsb=0), 6),      # 4 splits of 512 keys need a workspace
])
def test_paged_decode_validation(kw, status):
    assert call_paged(**kw) == status
    assert F.load_library().fmha_last_error()


def test_workspace_formula():
    # rows * splits * (D + 1) floats, each section rounded up to 256 bytes
    rows, ns, D = 64 * 32, 16, 64
    want = -(-rows * ns * D * 4 // 256) * 256 + -(-rows * ns * 4 // 256) * 256
    assert F.fmha_decode_splitkv_workspace_size(64, 32, 8, 1, 8192, 64, 16) == want
    assert F.fmha_decode_splitkv_workspace_size(64, 32, 8, 1, 8192, 64, 1) == 0
    assert F.fmha_decode_splitkv_workspace_size(64, 32, 8, 1, 8192, 48, 4) == 0
    assert F.fmha_decode_splitkv_workspace_size(64, 32, 7, 1, 8192, 64, 4) == 0


def test_default_splits_heuristic():
    ns = F.fmha_decode_default_splits
    for args in [(64, 32, 8, 1, 8192, 64), (32, 64, 1, 1, 16384, 512), (128, 16, 16, 1, 4096, 128),
                 (1, 1, 1, 1, 100, 64)]:
        n = ns(*args)
        assert 1 <= n <= 1024 and (n & (n - 1)) == 0
    assert ns(1, 1, 1, 1, 100, 64) == 1            # too short to split
    assert ns(32, 64, 1, 1, 16384, 512) >= 8       # 32 (batch, KV head) units need splitting


def test_nvfp4_validation():
    lib = F.load_library()
    q = lib.nvfp4_quantize
    assert q(None, 4, 16, FAKE, FAKE, FAKE, None, FAKE, 256, None) == 1
    assert q(FAKE, 4, 24, FAKE, FAKE, FAKE, None, FAKE, 256, None) == 2
    assert q(FAKE, 0, 16, FAKE, FAKE, FAKE, None, FAKE, 256, None) == 2
    assert q(FAKE + 2, 4, 16, FAKE, FAKE, FAKE, None, FAKE, 256, None) == 5
    assert q(FAKE, 4, 16, FAKE, FAKE, FAKE, None, None, 0, None) == 6
    assert lib.nvfp4_quantize_workspace_size(4, 16) >= 4


def test_debug_scores_validation():
    lib = F.load_library()
    d = lib.fmha_debug_qk_scores

    def call(q=FAKE, k=FAKE, v=FAKE, s=FAKE, B=1, Hq=4, Hkv=1, Sq=4, Sk=64, D=64, Dv=64,
             scale=0.125, decode=0):
        return d(q, k, v, s, B, Hq, Hkv, Sq, Sk, D, Dv, scale, decode, None)

    assert call(s=None) == 1
    assert call(q=None) == 1
    assert call(Sk=0) == 2
    assert call(B=1 << 12, Hq=1 << 12, Sk=1 << 8) == 2   # s_out past 2^31 elements
    assert call(D=512, Dv=512) == 3                       # no 512 prefill
    assert call(D=16, Dv=16, decode=1) == 3               # no 16 decode
    assert call(D=576, Dv=512) == 3                       # 576/512 is decode only
    assert call(D=192, Dv=128, decode=1) == 3             # 192/128 is prefill only
    assert call(Hq=3, Hkv=2) == 4
    assert call(s=FAKE + 4) == 5
    assert call(decode=2) == 8
    assert call(D=192, Dv=128, v=FAKE) == 8               # V inside K: decode only


def test_noalloc_validation_before_any_device_call():
    """The no-allocation decode checks everything on the host, including that
    its partials fit the fixed 64 MiB scratch, before touching the device."""
    lib = F.load_library()
    d = lib.fmha_decode_splitkv_noalloc

    def call(q=FAKE, o=FAKE, B=32, Hq=64, Hkv=1, Sq=1, Sk=16384, D=512, ns=8, scale=0.04):
        return d(q, FAKE, FAKE, o, None, B, Hq, Hkv, Sq, Sk, D, scale, 0, ns, None, None)

    assert call(q=None) == 1
    assert call(B=0) == 2
    assert call(D=576) == 3 and call(D=16) == 3
    assert call(Hq=3, Hkv=2) == 4
    assert call(o=FAKE + 2) == 5
    assert call(ns=-1) == 8 and call(ns=1025) == 8
    assert call(ns=32) == 6   # 128 MiB of partials
    assert b"64" in lib.fmha_last_error() or b"67108864" in lib.fmha_last_error()


def test_library_has_no_undefined_symbols_of_its_own():
    """Every kernel launched from host code has its host stub defined (a
    missing stub only shows when the library is loaded for a call)."""
    import shutil
    import subprocess
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm not available")
    out = subprocess.run([nm, "-C", "--undefined-only", F.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    own = [ln for ln in out.splitlines() if "fmha" in ln]
    assert not own, own
