"""Build libcpattn.so (HIP, gfx950 only) in-tree.

    python -m kv_context_parallelism_amd.build [--asm]

Each csrc/*.hip file is compiled by hipcc for gfx950 and the objects are
linked into kv_context_parallelism_amd/libcpattn.so.  Packed-FP32 VALU ops
are disabled for all device code.  ``--asm`` also keeps the device assembly
under _build/ for inspection.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build", "cpattn")
LIB = os.path.join(PKG, "libcpattn.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]

# Per-file additions.  prefill.hip: every accumulator of the kernel (outputs,
# scores) must stay in arch VGPRs, where the online-softmax rescale can update
# them in place; the default heuristic puts MFMA accumulators in AGPRs and then
# copies all of them to VGPRs and back on every tile.  (decode_mla.hip issues
# its MFMAs from asm with explicit register classes -- output accumulators in
# AGPRs, score accumulators in VGPRs -- and keeps the default.)
FILE_FLAGS = {
    "prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def _compile(src: str, asm: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC, *CFLAGS, *FILE_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    if asm:
        cmd[1:1] = ["-save-temps=obj"]
    r = subprocess.run(cmd, capture_output=True, text=True, cwd=BUILD)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    err = "\n".join(ln for ln in r.stderr.splitlines()
                    if "packed-fp32-ops" not in ln and ln.strip())
    if err:
        print(err, file=sys.stderr)
    return obj


def build(asm: bool = False, verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, asm), srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources")
    return LIB


if __name__ == "__main__":
    build(asm="--asm" in sys.argv)
