"""Build the gfx950 SPICY-KV library in-tree: coarse_grained_decode_amd/libspicy.so.

    python -m coarse_grained_decode_amd.build

Each source compiles to its own object (in parallel), then hipcc links them
into the shared library.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libspicy.so")
# the benchmark's streaming-read reference, a library of its own
PROBE_LIB = os.path.join(PKG, "libspicy_probe.so")
PROBE_SOURCE = "readprobe.hip"
OBJDIR = os.path.join(PKG, "_build")
# (source, object, extra flags): coarsen.hip builds once per (element type,
# head dim) so that its kernels compile in parallel
UNITS = [("api.hip", "api", []), ("decode.hip", "decode", []), ("policy.hip", "policy", []),
         ("merge.hip", "merge", []), ("compact.hip", "compact", [])] + [("coarsen.hip", f"coarsen{i}", [f"-DSPICY_COARSEN_PART={i}"])
                                         for i in range(4)]
SOURCES = sorted({src for src, _, _ in UNITS})   # the library's sources
HEADERS = ["launch.h", "spicy_device.h"]
ARCH = os.environ.get("SPICY_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def flags():
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            # packed fp32 VALU forms are kept out of the generated code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def compile_command(src: str, obj: str, extra=()):
    return [hipcc(), *flags(), *extra, "-c", os.path.join(CSRC, src), "-o", obj]


def link_command(objs, out: str = LIB):
    return [hipcc(), f"--offload-arch={ARCH}", "-fPIC", "-shared", *objs, "-o", out]


def build(verbose: bool = True, jobs: int | None = None) -> str:
    os.makedirs(OBJDIR, exist_ok=True)
    objs = [os.path.join(OBJDIR, name + ".o") for _, name, _ in UNITS]
    cmds = [compile_command(src, o, extra) for (src, _, extra), o in zip(UNITS, objs)]
    if verbose:
        for c in cmds:
            print(" ".join(c), flush=True)

    def run(c):
        return subprocess.run(c, capture_output=True, text=True)

    probe_obj = os.path.join(OBJDIR, "readprobe.o")
    cmds.append(compile_command(PROBE_SOURCE, probe_obj))
    jobs = jobs or min(len(cmds), max(1, os.cpu_count() or 1))
    with ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(run, cmds))
    for c, r in zip(cmds, results):
        err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
        if err.strip() and (verbose or r.returncode != 0):
            print(err, file=sys.stderr, flush=True)
        if r.returncode != 0:
            raise subprocess.CalledProcessError(r.returncode, c)
    for out, ob in ((LIB, objs), (PROBE_LIB, [probe_obj])):
        tmp = out + ".tmp"
        lcmd = link_command(ob, tmp)
        if verbose:
            print(" ".join(lcmd), flush=True)
        subprocess.run(lcmd, check=True)
        os.replace(tmp, out)
    return LIB


def stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    deps = [os.path.join(CSRC, f) for f in SOURCES + HEADERS] + [os.path.join(ROOT, "include", "spicy.h")]
    if not os.path.exists(PROBE_LIB) or os.path.getmtime(os.path.join(CSRC, PROBE_SOURCE)) > os.path.getmtime(PROBE_LIB):
        return True
    return any(os.path.getmtime(p) > t for p in deps)


if __name__ == "__main__":
    build()
    sys.exit(0)
