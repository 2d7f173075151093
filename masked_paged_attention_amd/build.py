"""Builds libmpa.so (the C ABI of include/mpa.h) for gfx950 with hipcc, in-tree.

    python -m masked_paged_attention_amd.build      # or build_library() from Python

Sources are compiled in parallel into masked_paged_attention_amd/_build/ and
linked into masked_paged_attention_amd/lib/libmpa.so.  Every call recompiles.
The compiler's per-kernel register and scratch figures of the device code are
kept in _build/kernel_resources.json.
"""

import concurrent.futures
import json
import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIBDIR = os.path.join(PKG, "lib")
LIB = os.path.join(LIBDIR, "libmpa.so")

SOURCES = ["api.cpp", "planner.cpp", "prefill_fwd.hip", "mla_decode.hip", "lse_merge.hip", "static_scratch.hip"]
ARCH = "gfx950"


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else (shutil.which("hipcc") or "hipcc")


def common_flags():
    # Packed fp32 VALU ops are disabled for all device code.
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
            "-Wno-unused-command-line-argument"]


RESOURCES = os.path.join(BUILD, "kernel_resources.json")
_RU = re.compile(r"remark:\s+(Function Name|VGPRs|AGPRs|ScratchSize \[bytes/lane\]): (\S+)")


def _resources(text):
    """Per-kernel register and scratch use from the compiler's resource remarks."""
    out, name = {}, None
    for key, val in _RU.findall(text):
        if key == "Function Name":
            name = val
            out[name] = {}
        elif name is not None:
            out[name][{"VGPRs": "vgpr", "AGPRs": "agpr"}.get(key, "scratch")] = int(val)
    return out


def _compile(src):
    out = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + common_flags() + ["-c", os.path.join(CSRC, src), "-o", out]
    if src.endswith(".cpp"):
        cmd.insert(1, "-x")
        cmd.insert(2, "hip")
    else:
        cmd.append("-Rpass-analysis=kernel-resource-usage")
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(line for line in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in line and "remark:" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{errs}")
    return out, _resources(r.stderr)


def build_library(verbose=True):
    os.makedirs(BUILD, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        done = list(ex.map(_compile, SOURCES))
    objs = [o for o, _ in done]
    resources = {k: v for _, ru in done for k, v in ru.items()}
    with open(RESOURCES, "w") as f:
        json.dump(resources, f, indent=1, sort_keys=True)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build_library()
    sys.exit(0)
