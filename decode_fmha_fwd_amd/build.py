"""Build libfmha.so (hand-written HIP kernels for gfx950 behind a C ABI) in-tree.

    python -m decode_fmha_fwd_amd.build

compiles every ``csrc/*.hip`` with hipcc for ``--offload-arch=gfx950`` and links
them into ``decode_fmha_fwd_amd/libfmha.so``.  Packed-fp32 instructions are
turned off for all device code; the NVFP4 translation unit additionally keeps
fp contraction off, correctly rounded fp32 division and fp32 denormals,
because it decides integer codes; the prefill kernels keep MFMA accumulators
in ordinary VGPRs.

The attention translation units issue some LDS reads from inline asm; their
device assembly (a device-only ``-S`` compile with the same flags, run beside
the object compile) is checked by ``asm_check`` before the library is linked,
so a build in which register allocation touched such a read's result before
its wait fails here instead of computing with stale data.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

try:
    from . import asm_check
except ImportError:  # run as a script
    import asm_check

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libfmha.so")
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wno-unused-command-line-argument"]
PER_FILE = {
    # prefill keeps MFMA accumulators in ordinary VGPRs (no AGPR round trips
    # around the softmax); decode at head dim 512 needs the AGPR file for O
    "fmha_prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
    # test-only score stores: the flags of the prefill and decode units
    # (accumulators in VGPRs would change the decode's register budget, so
    # the debug unit keeps the decode's default; the prefill's QK block
    # compiles to the same instructions either way)
    "fmha_debug.hip": ["-fhip-fp32-correctly-rounded-divide-sqrt",
                       "-fno-gpu-flush-denormals-to-zero"],
    # the decode epilogues can encode NVFP4: the same fp32 semantics as nvfp4.hip
    "fmha_decode.hip": ["-fhip-fp32-correctly-rounded-divide-sqrt",
                        "-fno-gpu-flush-denormals-to-zero"],
    "fmha_decode_paged.hip": ["-fhip-fp32-correctly-rounded-divide-sqrt",
                              "-fno-gpu-flush-denormals-to-zero"],
    "nvfp4.hip": ["-ffp-contract=off", "-fhip-fp32-correctly-rounded-divide-sqrt",
                  "-fno-gpu-flush-denormals-to-zero"],
}
SOURCES = ["fmha_api.hip", "fmha_prefill.hip", "fmha_decode.hip", "fmha_decode_paged.hip",
           "fmha_decode_wide.hip", "fmha_debug.hip", "nvfp4.hip"]
ASM_CHECKED = {"fmha_prefill.hip", "fmha_decode.hip", "fmha_decode_paged.hip",
               "fmha_decode_wide.hip", "fmha_debug.hip"}


def hipcc() -> str:
    h = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(h):
        raise RuntimeError("hipcc not found: the HIP library cannot be built")
    return h


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, src.replace(".hip", ".o"))
    cmd = [hipcc(), *COMMON, *PER_FILE.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def _check_asm(src: str) -> None:
    """Device assembly of `src` (a device-only compile with the same flags),
    checked for inline-asm LDS read hazards."""
    asm = os.path.join(BUILD, src.replace(".hip", f"-{ARCH}.s"))
    cmd = [hipcc(), *COMMON, *PER_FILE.get(src, []), "--cuda-device-only", "-S",
           os.path.join(CSRC, src), "-o", asm]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc (device assembly) failed for {src}:\n{r.stderr}")
    rep = asm_check.check_file(asm)
    if rep.problems:
        raise RuntimeError(f"{src}: inline-asm LDS read hazard(s):\n" + "\n".join(rep.problems[:10]))
    os.remove(asm)


def build(verbose: bool = False) -> str:
    """Compile all kernels and link libfmha.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES) + len(ASM_CHECKED)) as ex:
        checks = [ex.submit(_check_asm, src) for src in sorted(ASM_CHECKED)]
        objs = list(ex.map(_compile, SOURCES))
        for c in checks:
            c.result()
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
