"""Build the HIP library libmoe_mi355x.so in-tree (gfx950 only).

    python -m mixture_experts_layer_scan_amd.build

Each .hip file is compiled to an object under _build/ in parallel, then linked
with hipcc.  Packed FP32 instructions are disabled for device code.
"""
from __future__ import annotations

import concurrent.futures
import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(PKG, "libmoe_mi355x.so")
BUILD_DIR = os.path.join(ROOT, "_build")
ARCH = "gfx950"

SOURCES = ["api.hip", "route.hip", "permute.hip", "gemm.hip", "decode_gemm.hip", "finalize.hip",
           "quant.hip"]

DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]

# A kernel whose registers spill beyond this many bytes of scratch per lane
# fails the build: a spill that size inside a k-loop costs tens of times the
# kernel's time (the tiles that keep a few spilled registers stay below it).
MAX_SCRATCH_BYTES = 128


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found (ROCm is required to build the MoE library)")
    return path


def _scratch_use(lines) -> dict:
    """Scratch bytes per lane of each kernel, from the compiler's resource
    usage remarks (a "Function Name" line, then its "ScratchSize" line)."""
    use, fn = {}, None
    for l in lines:
        if "Function Name:" in l:
            fn = l.split("Function Name:", 1)[1].split("[-Rpass")[0].strip()
        elif "ScratchSize [bytes/lane]:" in l and fn is not None:
            use[fn] = int(l.split("ScratchSize [bytes/lane]:", 1)[1].split("[-Rpass")[0])
    return use


def _compile(src: str, obj: str, extra) -> None:
    cmd = [hipcc(), "-x", "hip", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
           "-I", INCLUDE, "-Wall", "-Wno-unused-function", *DEVICE_FLAGS,
           "-Rpass-analysis=kernel-resource-usage", *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    lines = (r.stderr or "").splitlines()
    spills = {f: b for f, b in _scratch_use(lines).items() if b > MAX_SCRATCH_BYTES}
    if spills:
        raise RuntimeError(f"{src}: kernels spill more than {MAX_SCRATCH_BYTES} bytes of scratch "
                           f"per lane: " + ", ".join(f"{f} ({b})" for f, b in sorted(spills.items())))
    # drop the remarks with their source excerpts, and the host pass's note
    # on the device-only feature flag
    msgs, in_remark = [], False
    for l in lines:
        if "-Rpass-analysis=kernel-resource-usage" in l:
            in_remark = True
        elif in_remark and re.match(r"^\s*(\d+\s*)?\|", l):
            pass
        elif "'-packed-fp32-ops' is not a recognized feature" not in l:
            in_remark = False
            msgs.append(l)
    if msgs:
        sys.stderr.write("\n".join(msgs) + "\n")


def build(extra_flags=None, out: str = OUT) -> str:
    """Compile every HIP source for gfx950 and link ``out``.  Always rebuilds."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    extra = list(extra_flags or [])
    objs = []
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        futs = []
        for s in SOURCES:
            obj = os.path.join(BUILD_DIR, os.path.splitext(s)[0] + ".o")
            objs.append(obj)
            futs.append(ex.submit(_compile, os.path.join(CSRC, s), obj, extra))
        for f in futs:
            f.result()
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(sys.argv[1:]))
