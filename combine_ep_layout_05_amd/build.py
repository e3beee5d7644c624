"""Builds libep_mi355x.so, the HIP library behind include/ep.h, for gfx950.

hipcc, -O3, one shared object from every .hip file under csrc/.  Device code
is compiled without FP contraction (every fused multiply-add is written as
one) and without packed-fp32 instructions.
"""
import glob
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libep_mi355x.so")
ARCH = os.environ.get("EP_OFFLOAD_ARCH", "gfx950")

FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off", "-mcode-object-version=5",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wl,-soname,libep_mi355x.so",
    "-I", os.path.join(ROOT, "include"),
]


LOOP = os.path.join(HERE, "ep_loop")     # native serving-loop timer over the C ABI
CEILINGS = os.path.join(HERE, "ep_ceilings")   # native HBM read/write/copy rate probe


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(verbose: bool = False, extra_flags=()) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["hipcc", *FLAGS, *extra_flags, *sources(), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature and says so; that is harmless
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + msg)
    if verbose and msg.strip():
        print(msg)
    os.replace(tmp, LIB)
    # the native loop timer links the library just built (host code only)
    tmp = LOOP + ".tmp%d" % os.getpid()
    cmd = ["hipcc", "-O2", "-std=c++17", "-I", os.path.join(ROOT, "include"),
           os.path.join(CSRC, "ep_loop.cpp"), "-L", HERE, "-lep_mi355x",
           "-Wl,-rpath,$ORIGIN", "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed on ep_loop.cpp:\n" + r.stdout + r.stderr)
    os.replace(tmp, LOOP)
    # the ceilings probe: its own kernels, same code-generation flags, no library
    tmp = CEILINGS + ".tmp%d" % os.getpid()
    cmd = ["hipcc", "-x", "hip", *[f for f in FLAGS if f not in ("-fPIC", "-shared")
                                   and not f.startswith("-Wl,-soname")],
           os.path.join(CSRC, "ep_ceilings.cpp"), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
        raise RuntimeError("hipcc failed on ep_ceilings.cpp:\n" + msg)
    os.replace(tmp, CEILINGS)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))


# sources each kernel family is compiled from (shared headers included)
KERNEL_SOURCES = {
    "layout": ["layout.hip", "ep_device.h"],
    "dispatch": ["dispatch.hip", "ep_numerics.h", "ep_device.h"],
    "layout_dispatch": ["dispatch.hip", "ep_numerics.h", "ep_device.h"],
    "combine": ["combine.hip", "ep_numerics.h", "ep_device.h"],
}


def source_digest(kernel=None) -> str:
    """sha256 of the HIP sources a kernel is built from (all sources when
    kernel is None), the code-generation flags and, for dispatch and combine,
    the tuned launch-geometry rules, with comments and whitespace removed: it
    changes when the compiled code or its launch can change, not when a
    comment does.  Recorded next to rocprofv3 counter readings so that a
    reading is only reused for the kernel code it was taken from."""
    import hashlib
    import re
    h = hashlib.sha256()
    h.update(" ".join(f for f in FLAGS if f.startswith(("-O", "--offload", "-f", "-m", "-std"))).encode())
    if kernel is None:
        files = sorted(sources() + glob.glob(os.path.join(CSRC, "*.h")))
    else:
        files = [os.path.join(CSRC, n) for n in KERNEL_SOURCES[kernel]]
    if kernel in ("dispatch", "combine"):
        # the launch geometry the bench takes from the tuned rules
        files = files + [os.path.join(HERE, "tuned_geometry.json")]
    for p in files:
        if not os.path.exists(p):
            continue
        text = open(p).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        text = re.sub(r"\s+", " ", text)
        h.update(os.path.basename(p).encode() + b"\0" + text.encode())
    return h.hexdigest()
