"""Build libcoda.so (gfx950) in-tree with hipcc.

    python -m gemm_epilogue_transformer_mainloop_amd.build
    python -m gemm_epilogue_transformer_mainloop_amd.build --timeline   # libcoda_timeline.so

The library is rebuilt on every call: each translation unit is compiled to an
object in parallel (one hipcc per source), then the objects are linked.
Packed-fp32 VALU instructions are disabled for the device code; the host pass
warns that it does not know the feature, which is harmless.

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
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libcoda.so")
TIMELINE_LIB = os.path.join(HERE, "libcoda_timeline.so")
RESOURCES = os.path.join(HERE, "libcoda.resources.json")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["coda_aux.hip", "coda_fwd.hip", "coda_pair.hip", "coda_bwd.hip", "coda_ce.hip", "coda_unfused.hip",
           "coda_probe.hip", "coda_ln.hip"]
OBJDIR = os.path.join(HERE, "_build")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
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


def _compile(src: str, obj: str, extra: list, verbose: bool) -> str:
    cmd = [HIPCC] + FLAGS + extra + ["-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed on {os.path.basename(src)} ({res.returncode})")
    return res.stdout + res.stderr


def build(verbose: bool = False, out: str = None, extra: list = None, jobs: int = None,
          timeline: bool = False) -> str:
    """Build the library (default: libcoda.so beside this file) and return its
    path.  timeline=True builds libcoda_timeline.so instead: the same kernels
    with the per-wave tile timeline compiled in (CODA_TIMELINE=1)."""
    extra = list(extra or [])
    if timeline:
        extra.append("-DCODA_TIMELINE=1")
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    lib = out or (TIMELINE_LIB if timeline else LIB)
    objdir = OBJDIR + ("_timeline" if timeline else "")
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, os.path.basename(s).replace(".hip", ".o")) for s in srcs]
    jobs = jobs or min(len(srcs), max(1, len(os.sched_getaffinity(0))))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        texts = list(ex.map(lambda a: _compile(a[0], a[1], extra, verbose), zip(srcs, objs)))
    text = "\n".join(texts)
    errs = [l for l in text.splitlines()
            if "error" in l.lower() and "packed-fp32-ops" not in l]
    if errs:
        sys.stderr.write("\n".join(errs) + "\n")
    resources = parse_resources(text)
    spills = {k: v["scratch"] for k, v in resources.items() if v.get("scratch", 0) > 0}
    if spills:
        raise RuntimeError(f"kernels use scratch memory (register spills): {spills}")
    tmp = lib + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC"] + objs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"link failed ({res.returncode})")
    if out is None and not timeline:
        with open(RESOURCES, "w") as f:
            json.dump(resources, f, indent=1, sort_keys=True)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose=True, timeline="--timeline" in sys.argv[1:]))
