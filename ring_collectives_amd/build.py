"""Build libring_collectives.so (the HIP kernels and the C ABI) for gfx950.

    python -m ring_collectives_amd.build

hipcc cross-compiles for gfx950 without a GPU.  The library is written next
to this file so it travels with the source tree.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
SOURCES = ["ring_api.hip", "ring_kernels.hip", "gemm_rs.hip", "ag_gemm.hip", "tp_mlp.hip"]
LIB = os.path.join(HERE, "libring_collectives.so")
ARCH = os.environ.get("RING_OFFLOAD_ARCH", "gfx950")

FLAGS = [
    "-O3", "-std=c++17", "-fPIC",
    "--offload-arch=" + ARCH,
    "-ffp-contract=off",                       # no fused multiply-add rewrites
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
]
LINK_FLAGS = ["-shared", "-fPIC", "--offload-arch=" + ARCH]
HOST_NOTE = "'-packed-fp32-ops' is not a recognized feature for this target (ignoring feature)"


def _run(cmd, verbose):
    """Run one hipcc command; returns (returncode, the lines it printed minus
    the host-pass notes described below, how many notes were dropped)."""
    # The packed-fp32 switch is meant for the gfx950 device pass; the driver
    # cannot forward a -Xclang pair to that pass alone (-Xarch_device takes
    # no option with a separate argument), so the x86 host pass sees it too
    # and prints a note per translation unit that it ignores the feature.
    # Those notes, and only those, are dropped; everything else the compiler
    # prints is passed on.
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    lines = res.stdout.splitlines()
    kept = [ln for ln in lines if HOST_NOTE not in ln]
    return res.returncode, kept, len(lines) - len(kept)


def build(verbose: bool = False) -> str:
    """Compile every source to an object (in parallel), then link the
    shared library next to this file."""
    from concurrent.futures import ThreadPoolExecutor
    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)
    inc = ["-I", os.path.join(ROOT, "include"), "-I", CSRC]
    jobs = []
    for s in SOURCES:
        obj = os.path.join(objdir, s.replace(".hip", ".o"))
        jobs.append((obj, ["hipcc", *FLAGS, "-c", *inc, os.path.join(CSRC, s), "-o", obj]))
    with ThreadPoolExecutor(len(jobs)) as ex:
        results = list(ex.map(lambda j: _run(j[1], verbose), jobs))
    dropped = 0
    failed = False
    for (obj, cmd), (rc, kept, nd) in zip(jobs, results):
        for ln in kept:
            print(ln, flush=True)
        dropped += nd
        if rc != 0:
            failed = True
            print("build: %s failed (%d)" % (os.path.basename(obj), rc), flush=True)
    if failed:
        raise subprocess.CalledProcessError(1, "hipcc")
    tmp = LIB + ".tmp%d" % os.getpid()
    rc, kept, nd = _run(["hipcc", *LINK_FLAGS, *[j[0] for j in jobs], "-o", tmp], verbose)
    for ln in kept:
        print(ln, flush=True)
    if rc != 0:
        raise subprocess.CalledProcessError(rc, "hipcc (link)")
    if verbose and dropped + nd:
        print("(%d host-pass notes about the device-only packed-fp32 switch not shown)" % (dropped + nd),
              flush=True)
    # A kernel template the host pass failed to instantiate leaves no error,
    # only an object without it and a library whose launch stubs refer to an
    # undefined symbol; refuse such a library here rather than at load time.
    und = subprocess.run(["nm", "-D", "--undefined-only", tmp], stdout=subprocess.PIPE, text=True).stdout
    missing = [ln.split()[-1] for ln in und.splitlines() if ln.split() and ln.split()[-1].startswith("_ZN5ringc")]
    if missing:
        os.remove(tmp)
        raise RuntimeError("build: the library leaves its own symbols undefined: %s" % ", ".join(missing))
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
