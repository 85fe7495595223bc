"""Build libsparse_ffn.so (the C-ABI library with the gfx950 HIP kernels) in place.

``python -m activation_sparse_transformer_amd.build`` compiles every source under
``csrc/`` with hipcc for gfx950 (one process per source, in parallel) and links them into
``activation_sparse_transformer_amd/libsparse_ffn.so``.  Packed-fp32 instructions are
disabled for device code.
"""
import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libsparse_ffn.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-result"]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith(".hip") or f.endswith(".cpp"))


def build(verbose: bool = False, extra=(), out: str = OUT) -> str:
    """Compile every source with ``extra`` flags added and link the library into ``out``."""
    srcs = sources()
    tmpdir = tempfile.mkdtemp(prefix="sffn_build_")
    try:
        objs = [os.path.join(tmpdir, os.path.basename(f) + ".o") for f in srcs]
        cmds = [[HIPCC, *FLAGS, *extra, "-c", f, "-o", o] for f, o in zip(srcs, objs)]

        def compile_one(cmd):
            if verbose:
                print(" ".join(cmd), flush=True)
            subprocess.check_call(cmd)

        jobs = max(1, min(len(cmds), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
        with ThreadPoolExecutor(jobs) as ex:
            list(ex.map(compile_one, cmds))
        tmp = out + ".tmp"
        link = [HIPCC, f"--offload-arch={ARCH}", "-fPIC", "-shared", *objs, "-o", tmp]
        if verbose:
            print(" ".join(link), flush=True)
        subprocess.check_call(link)
        os.replace(tmp, out)
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
    return out


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
