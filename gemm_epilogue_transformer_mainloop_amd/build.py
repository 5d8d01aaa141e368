"""Build libcoda.so (gfx950) in-tree with hipcc.

    python -m gemm_epilogue_transformer_mainloop_amd.build

The library is rebuilt on every call.  Packed-fp32 VALU instructions are
disabled for the device code; the host pass warns that it does not know the
feature, which is harmless.

The compiler's per-kernel resource report (VGPRs, AGPRs, scratch bytes per
lane) is written to libcoda.resources.json beside the library, and the build
fails if any kernel uses scratch memory: a spilling GEMM kernel is slow, and
under this much register pressure the register allocator has been seen to
drop an accumulator copy in a spilling epilogue (wrong results, no error).
"""

from __future__ import annotations

import json
import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libcoda.so")
RESOURCES = os.path.join(HERE, "libcoda.resources.json")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["coda_api.hip", "coda_unfused.hip"]

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-Rpass-analysis=kernel-resource-usage",
]

_REMARK = re.compile(r"remark:\s+(Function Name|VGPRs|AGPRs|ScratchSize \[bytes/lane\]|Occupancy \[waves/SIMD\]|"
                     r"VGPRs Spill|LDS Size \[bytes/block\]): (\S+)")


def parse_resources(text: str) -> dict:
    """Per-kernel register, scratch, LDS and occupancy figures from the resource remarks."""
    out, cur = {}, None
    keys = {"VGPRs": "vgprs", "AGPRs": "agprs", "ScratchSize [bytes/lane]": "scratch",
            "Occupancy [waves/SIMD]": "occupancy", "VGPRs Spill": "vgpr_spill",
            "LDS Size [bytes/block]": "lds"}
    for m in _REMARK.finditer(text):
        k, v = m.group(1), m.group(2)
        if k == "Function Name":
            cur = out.setdefault(v, {})
        elif cur is not None:
            cur[keys[k]] = int(v)
    return out


def build(verbose: bool = False, occ2: bool = False, out: str = None) -> str:
    """Build the library.  occ2=True builds the variant whose forward and
    data-gradient calls use two workgroups per CU (coda_mainloop_occ2.hpp)
    into `out` (default libcoda_occ2.so); the default library does not use it."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES if os.path.exists(os.path.join(CSRC, s))]
    lib = out or (os.path.join(HERE, "libcoda_occ2.so") if occ2 else LIB)
    tmp = lib + ".tmp"
    cmd = [HIPCC] + FLAGS + (["-DCODA_OCC2=1"] if occ2 else []) + srcs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed ({res.returncode})")
    text = res.stdout + res.stderr
    errs = [l for l in text.splitlines()
            if "error" in l.lower() and "packed-fp32-ops" not in l]
    if errs:
        sys.stderr.write("\n".join(errs) + "\n")
    resources = parse_resources(text)
    spills = {k: v["scratch"] for k, v in resources.items() if v.get("scratch", 0) > 0}
    if spills:
        os.remove(tmp)
        raise RuntimeError(f"kernels use scratch memory (register spills): {spills}")
    if not occ2:
        with open(RESOURCES, "w") as f:
            json.dump(resources, f, indent=1, sort_keys=True)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True, occ2="--occ2" in sys.argv[1:]))
