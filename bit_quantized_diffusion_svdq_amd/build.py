"""Build libsvdq.so (the gfx950 HIP kernels and the C ABI) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libsvdq.so")
SOURCES = ["api.hip", "act_quant.hip", "gemm_w4a4.hip", "gemv_w4a16.hip", "probe.hip", "offline.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 VALU forms are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def _filter(text: str) -> str:
    # The feature flag is meant for the device pass; the host pass also sees
    # it and prints a notice that it does not know it (one line per source),
    # which carries no information: drop exactly that line.
    return "".join(l for l in text.splitlines(keepends=True)
                   if "'-packed-fp32-ops' is not a recognized feature" not in l)


def build(verbose: bool = False) -> str:
    """Compile every HIP source (in parallel, one hipcc per source) and link
    them into bit_quantized_diffusion_svdq_amd/libsvdq.so."""
    import concurrent.futures
    import tempfile

    compile_flags = [f for f in HIPCC_FLAGS if f != "-shared"]
    with tempfile.TemporaryDirectory(prefix="svdq_build_") as tmpdir:
        def compile_one(src):
            obj = os.path.join(tmpdir, src + ".o")
            cmd = [hipcc()] + compile_flags + ["-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            r = subprocess.run(cmd, capture_output=True, text=True)
            return obj, r.returncode, _filter(r.stdout + r.stderr)

        jobs = max(1, min(len(SOURCES), os.cpu_count() or 1, 16))
        with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
            results = list(ex.map(compile_one, SOURCES))
        failed = False
        for (obj, rc, out), src in zip(results, SOURCES):
            if out.strip() and (rc != 0 or verbose):
                sys.stderr.write(out)
            failed |= rc != 0
        if failed:
            raise RuntimeError("hipcc failed building libsvdq.so")
        tmp = LIB + ".tmp"
        cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC"] + [r[0] for r in results] + ["-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            sys.stderr.write(_filter(r.stdout + r.stderr))
            raise RuntimeError("linking libsvdq.so failed")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
