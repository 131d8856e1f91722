"""Build libbsa.so (host C++ and gfx950 HIP kernels) in the package directory.

    python -m dynamic_block_sparse_bsa_amd.build  [--jobs N]

Every translation unit is compiled with hipcc for gfx950 only.  The built-in
plan table (tables/gfx950_v2.txt) is embedded into the library as a string.
"""

import argparse
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libbsa.so")
TABLE = os.path.join(HERE, "tables", "gfx950_v2.txt")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = [
    "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-result", "-Wno-unused-value",
    f"--offload-arch={ARCH}",
    # packed FP32 arithmetic is kept off for every HIP translation unit
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(HERE, "..", "include"),
]
SOURCES = ["api.cpp", "catalog.cpp", "plan_kernels.hip", "merge_kernel.hip", "attn_kernels.hip",
           "static_scratch.hip"]
# MFMA accumulators in VGPRs: the softmax reads every score, and AGPR operands
# would need a v_accvgpr_read per element.
EXTRA = {"attn_kernels.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def write_table_inc():
    text = open(TABLE).read() if os.path.exists(TABLE) else ""
    inc = os.path.join(CSRC, "table_builtin.inc")
    body = 'R"BSATABLE(' + text + ')BSATABLE"\n'
    if not os.path.exists(inc) or open(inc).read() != body:
        with open(inc, "w") as f:
            f.write(body)


def compile_one(src):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC] + COMMON + EXTRA.get(src, []) + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(ln for ln in (r.stdout + r.stderr).splitlines()
                     if "packed-fp32-ops" not in ln)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {src}\n{' '.join(cmd)}\n{msgs}")
    return obj, msgs


def build(jobs=8, verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    write_table_inc()
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(compile_one, SOURCES))
    objs = [o for o, _ in results]
    if verbose:
        for _, m in results:
            if m.strip():
                print(m)
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=8)
    ap.add_argument("-v", action="store_true")
    a = ap.parse_args()
    print(build(a.jobs, a.v))
    sys.exit(0)
