"""Build the gfx950 HIP library libbitlinear.so in-tree with hipcc.

Every call compiles from source (no caching).  The object files are built in
parallel, then linked into bit_gemv_bitlinear_amd/libbitlinear.so.
"""
import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libbitlinear.so")
SOURCES = ["abi.hip", "pack.hip", "quant.hip", "gemv.hip", "gemv_local.hip", "gemv_group.hip",
           "gemv_norm.hip", "gemv_lut.hip", "gemm_band.hip", "gemm_mfma.hip", "gemm_prefill.hip",
           "ternarize.hip"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wextra",
    "-Wno-unused-parameter",
    # IEEE fp32 division for the activation scale 127 / amax
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    # no packed-fp32 instructions (v_pk_*_f32) anywhere
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]
LDFLAGS = ["-shared", "-fPIC", f"--offload-arch={ARCH}", "-Wl,-rpath,/opt/rocm/lib"]
# Per-source additions.  gemv.hip: the first 14 dwords of every kernel's
# arguments (all that the GEMV needs before its first weight load) arrive
# preloaded in SGPRs, so no wavefront waits on a kernel-argument load before
# issuing its loads (same box: 13824 x 2560 int8 3.36 -> 3.31 us, 2560 x 2560
# 2.57 -> 2.48 us).  The code object keeps a prologue that loads them the
# usual way, for firmware that does not preload.
SOURCE_FLAGS = {"gemv.hip": ["-mllvm", "-amdgpu-kernarg-preload-count=14"]}


def flags_for(src):
    """hipcc flags for one source file under csrc/."""
    return [*FLAGS, *SOURCE_FLAGS.get(src, [])]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(line for line in r.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in line)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if out.strip() and verbose:
        print(out, flush=True)


def build(verbose: bool = False) -> str:
    with tempfile.TemporaryDirectory(prefix="bl_build_") as tmp:
        objs = []
        cmds = []
        for src in SOURCES:
            obj = os.path.join(tmp, src.replace(".hip", ".o"))
            objs.append(obj)
            cmds.append([HIPCC, *flags_for(src), "-c", os.path.join(CSRC, src), "-o", obj])
        with ThreadPoolExecutor(max_workers=min(len(cmds), 8)) as ex:
            list(ex.map(lambda c: _run(c, verbose), cmds))
        out_tmp = LIB + ".tmp"
        _run([HIPCC, *LDFLAGS, *objs, "-o", out_tmp], verbose)
        os.replace(out_tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
