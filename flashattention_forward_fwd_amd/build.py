"""Build libfa2.so (the HIP kernels and their C ABI) in-tree for gfx950.

    python -m flashattention_forward_fwd_amd.build

Every HIP source is compiled with packed-fp32 instructions disabled
(-Xclang -target-feature -Xclang -packed-fp32-ops); hipcc's host pass warns that
it does not know that feature, which is harmless.
"""
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libfa2.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]
NOISE = "'-packed-fp32-ops' is not a recognized feature for this target (ignoring feature)"


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if NOISE not in ln]
    return res.returncode, msgs


def build(verbose: bool = False) -> str:
    """Compile every HIP source (one hipcc process each, in parallel) and link them
    into libfa2.so next to this file; return its path."""
    from concurrent.futures import ThreadPoolExecutor

    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tag = "%d" % os.getpid()
    objs = [os.path.join(CSRC, os.path.basename(src) + ".o" + tag) for src in sources()]
    jobs = max(1, min(len(objs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    try:
        with ThreadPoolExecutor(jobs) as pool:
            results = list(pool.map(
                lambda so: _run([hipcc] + HIPCC_FLAGS + ["-I", INCLUDE, "-I", CSRC, "-c", so[0], "-o", so[1]],
                                verbose), zip(sources(), objs)))
        for rc, msgs in results:
            if rc != 0:
                sys.stderr.write("\n".join(msgs) + "\n")
                raise RuntimeError("hipcc failed compiling a libfa2.so source (exit %d)" % rc)
            if verbose and msgs:
                print("\n".join(msgs))
        tmp = LIB + ".tmp" + tag
        rc, msgs = _run([hipcc, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs, verbose)
        if rc != 0:
            sys.stderr.write("\n".join(msgs) + "\n")
            raise RuntimeError("hipcc failed linking libfa2.so (exit %d)" % rc)
        os.replace(tmp, LIB)
    finally:
        for o in objs:
            if os.path.exists(o):
                os.remove(o)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
