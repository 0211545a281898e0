"""Build the gfx950 HIP library in-tree: lib/libsparse_attn.so.

    python -m long_context_sparse_block_amd.build [--verbose]

Every source under csrc/ is compiled with hipcc for gfx950 (one object per
file, in parallel) and linked into one shared library next to this file
(with zlib, which the host-side literal-flag function uses).
"""

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(HERE, "_build")
LIBDIR = os.path.join(HERE, "lib")
LIBNAME = "libsparse_attn.so"
SOURCES = ["host_common.hip", "mask_build.hip", "bsa_fwd.hip", "offset_fwd.hip", "bwd.hip", "literal_flags.cpp"]
ARCH = "gfx950"


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def compile_flags():
    return [f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
            # packed fp32 VALU ops stay disabled on this target
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # MFMA accumulators in plain VGPRs: no copies between register files
            "-mllvm", "-amdgpu-mfma-vgpr-form=1",
            "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
            "-I", INCLUDE, "-I", CSRC]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(line for line in r.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, flush=True)


def build(verbose=False, jobs=None):
    """Compile every source and link the library; returns the library path."""
    os.makedirs(OBJDIR, exist_ok=True)
    os.makedirs(LIBDIR, exist_ok=True)
    cc = hipcc()
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
        objs.append(obj)
        cmds.append([cc] + compile_flags() + ["-c", os.path.join(CSRC, src), "-o", obj])
    jobs = jobs or min(len(cmds), os.cpu_count() or 1, 8)
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    lib = os.path.join(LIBDIR, LIBNAME)
    tmp = lib + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs + ["-lz"], verbose)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    path = build(verbose="--verbose" in sys.argv)
    print(path)
