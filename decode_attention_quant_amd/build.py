"""Build the HIP libraries in place (gfx950).

    python -m decode_attention_quant_amd.build

Every source in csrc/ is compiled by hipcc for gfx950 and linked into
libkvq.so next to this file; probe/ (streaming kernels that calibrate
measurements, not part of the kvq ABI) becomes libkvq_probe.so.  Packed fp32
VALU instructions are turned off (``-packed-fp32-ops``); fp32 denormals and
IEEE division stay at the HIP defaults, which the bit-exact encoders rely on.
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libkvq.so")
PROBE_SRC = os.path.join(HERE, "probe")
PROBE_LIB = os.path.join(HERE, "libkvq_probe.so")
ARCH = os.environ.get("KVQ_OFFLOAD_ARCH", "gfx950")


def sources(folder=CSRC):
    return sorted(os.path.join(folder, f) for f in os.listdir(folder) if f.endswith(".hip"))


def hipcc():
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def build(verbose=False, jobs=8):
    """Compile and link libkvq.so and libkvq_probe.so; returns libkvq.so's path."""
    _build_lib(sources(CSRC), LIB, verbose, jobs)
    _build_lib(sources(PROBE_SRC), PROBE_LIB, verbose, jobs)
    return LIB


def _build_lib(srcs, lib, verbose, jobs):
    """Compile each source to an object under _build/, then link ``lib``."""
    objdir = os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    common = [
        "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-unused-command-line-argument",
        "-I" + os.path.join(HERE, "..", "include"), "-I" + CSRC,
    ]
    procs, objs = [], []
    for src in srcs:
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        objs.append(obj)
        cmd = [hipcc()] + common + ["-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        while len([p for _, p in procs if p.poll() is None]) >= jobs:
            procs[0][1].wait()
    failed = []
    for src, p in procs:
        out = p.communicate()[0].decode(errors="replace")
        if p.returncode != 0:
            failed.append((src, out))
        elif verbose and out.strip():
            print(out)
    if failed:
        for src, out in failed:
            sys.stderr.write("---- %s\n%s\n" % (src, out))
        raise RuntimeError("hipcc failed for %s" % ", ".join(os.path.basename(s) for s, _ in failed))
    tmp = lib + ".tmp"
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
