"""Build libfa.so (gfx950 code objects + the C ABI host code) in-tree with hipcc.

    python -m io_aware_exact_24_amd.build

Each source compiles to an object in _build/ (in parallel), then they link
into io_aware_exact_24_amd/libfa.so.  Packed fp32 VALU instructions are turned
off for the device code (-target-feature -packed-fp32-ops).
"""

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libfa.so")
BUILD = os.path.join(ROOT, "_build")

SOURCES = ["fa_fwd.hip", "fa_bwd_dkdv.hip", "fa_bwd_dq.hip", "fa_bwd.hip", "fa_generic.hip",
           "fa_api.cpp"]
# The dK/dV kernel keeps its long-lived accumulators in AccVGPRs through inline
# assembly; every other MFMA must write ordinary VGPRs, which the VALU reads.
_VGPR_FORM = ["-mllvm", "--amdgpu-mfma-vgpr-form"]
EXTRA = {"fa_bwd_dkdv.hip": _VGPR_FORM, "fa_bwd_dq.hip": _VGPR_FORM}

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# The tile loops index register arrays (operand rings, accumulators) by the
# loop counter and must unroll completely; a long body (the dropout variants
# draw Philox numbers inside it) would otherwise pass LLVM's size limit for
# "#pragma unroll", leave the loop rolled and turn every such index into a
# chain of selects.
COMMON = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-mllvm", "-pragma-unroll-threshold=1000000",
    "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"),
]


def _compile(src):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    lang = ["-x", "hip"]
    cmd = [HIPCC] + COMMON + EXTRA.get(src, []) + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    # hipcc's host pass warns that it does not know the device-only feature flag
    noise = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    return obj, "\n".join(noise)


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        results = list(ex.map(_compile, SOURCES))
    for (obj, msg), src in zip(results, SOURCES):
        if verbose and msg:
            print(f"[{src}]\n{msg}", file=sys.stderr)
    tmp = OUT + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + [o for o, _ in results]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
