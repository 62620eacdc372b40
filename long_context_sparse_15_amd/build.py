"""Build libcsa.so (the HIP kernels and the C ABI) for gfx950 with hipcc, in-tree.

Usage: python -m long_context_sparse_15_amd.build   (or __graft_entry__.build()).
Objects go to _build/ at the repository root; the library to the package directory.
"""
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libcsa.so")
BUILD = os.path.join(ROOT, "_build")
SOURCES = ["api.hip", "index.hip", "topk.hip", "mqa.hip", "mqa_hb.hip", "compress.hip", "proj.hip",
           "profile.hip",
           "blocks.hip"]

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # no packed fp32 math (v_pk_*_f32) anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + os.path.join(ROOT, "include"),
]
# Per-file flags.  The indexer's MFMA results feed VALU epilogues directly, so they are produced
# in VGPRs; the sliced attention kernels keep their accumulators in VGPRs too, one register pool.
# The head-block kernel (mqa_hb.hip) is built the same way for its logits and writes its output
# MFMAs out with accumulation-register operands (256 output accumulators a wave).
FILE_FLAGS = {"index.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
              "topk.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
              "mqa.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
              "mqa_hb.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if r.returncode != 0:
        raise RuntimeError("command failed: %s\n%s" % (" ".join(cmd), out))
    return out


def build(jobs=8, verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    objs = []
    cmds = []
    for s in SOURCES:
        o = os.path.join(BUILD, s.replace(".hip", ".o"))
        objs.append(o)
        cmds.append([HIPCC] + FLAGS + FILE_FLAGS.get(s, []) + ["-c", os.path.join(SRC, s), "-o", o])
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        for out in ex.map(_run, cmds):
            if verbose and out.strip():
                print(out)
    tmp = OUT + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
