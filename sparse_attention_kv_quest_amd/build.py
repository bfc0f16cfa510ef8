"""Builds libse.so (all HIP sources of csrc/) for gfx950, in place.

Run as `python -m sparse_attention_kv_quest_amd.build`.  Each source is
compiled to an object in _build/ (in parallel), then linked into
sparse_attention_kv_quest_amd/libse.so.
"""
import concurrent.futures as cf
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
ROOT = os.path.dirname(HERE)
OUT = os.path.join(HERE, "libse.so")
BUILD = os.path.join(ROOT, "_build")
ARCH = os.environ.get("SE_OFFLOAD_ARCH", "gfx950")

FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-I" + os.path.join(ROOT, "include"),
    # packed fp32 VALU forms stay off in every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in VGPRs: without this the compiler parks the SnapKV scoring passes'
    # score tiles in AGPRs and copies each one back (one v_accvgpr_read per element)
    # before the exps; no kernel of the library needs the AGPR file for capacity
    "-mllvm", "-amdgpu-mfma-vgpr-form",
]


def _compile(src):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = ["hipcc", *FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in (r.stderr or "").splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    return obj, err


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(min(8, len(srcs))) as ex:
        results = list(ex.map(_compile, srcs))
    for obj, err in results:
        if err.strip() and verbose:
            print(err, file=sys.stderr)
    tmp = OUT + ".tmp"
    cmd = ["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *[o for o, _ in results]]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stderr)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
