"""Build libpkv.so: the C ABI, the host core and the gfx950 kernels.

Every source is compiled with hipcc for gfx950 only; host-only C++ files go
through the same driver.  Objects land in ``_build/`` next to this file and
the library in this package directory, so it travels with the source tree.
"""

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libpkv.so")

SOURCES = [
    "host/pool.cpp",
    "host/plan.cpp",
    "host/radix.cpp",
    "host/tree.cpp",
    "capi.hip",
    "kernels/append.hip",
    "kernels/commit.hip",
    "kernels/attn.hip",
    "kernels/wide.hip",
    "kernels/path.hip",
    "kernels/merge.hip",
    "kernels/quant.hip",
    "kernels/probe.hip",
]

ARCH = "gfx950"


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def _flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-Wall", "-Wno-unused-result",
        # packed fp32 VALU ops stay off in device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # MFMA accumulators in VGPRs: the online-softmax rescale works on them
        # with VALU ops, so AGPR copies would cost a move per element per step
        "-mllvm", "-amdgpu-mfma-vgpr-form",
        # leading kernel arguments arrive in SGPRs at wave start
        "-mllvm", "-amdgpu-kernarg-preload-count=16",
        f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
    ]


def _compile(src):
    obj = os.path.join(BUILD, src.replace("/", "_") + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [hipcc()] + _flags() + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n{r.stdout}\n{r.stderr}")
    return obj, r.stderr


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        results = list(ex.map(_compile, SOURCES))
    objs = [o for o, _ in results]
    if verbose:
        for (_, err), src in zip(results, SOURCES):
            noise = [l for l in err.splitlines() if "packed-fp32-ops" not in l]
            if noise:
                print(f"[{src}]\n" + "\n".join(noise), file=sys.stderr)
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
