"""Build libp3d.so (HIP, gfx950) in-tree next to this file.

hipcc cross-compiles for gfx950 without a GPU. Flags:
  -ffp-contract=off   no implicit multiply-add fusion: the projection and the
                      source-index mapping round once per written operation,
                      which keeps pixel indices and masks reproducible; fused
                      multiply-adds appear only where the code calls fmaf.
  -Xclang -target-feature -Xclang -packed-fp32-ops
                      no packed binary32 VALU instructions.
"""
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libp3d.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-command-line-argument",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def build(out=LIB, extra=(), jobs=8, verbose=False, objdir=None, link_extra=()):
    """Compile every HIP source and link the shared library; returns its path.
    extra: more compile flags (later flags win, e.g. another -O level);
    objdir: where the objects go (default _build/ next to this file)."""
    objdir = objdir or os.path.join(HERE, "_build")
    os.makedirs(objdir, exist_ok=True)
    procs, objs = [], []
    for src in sources():
        obj = os.path.join(objdir, os.path.basename(src) + ".o")
        cmd = [HIPCC, *FLAGS, *extra, "-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd))
        procs.append((src, subprocess.Popen(cmd, stderr=subprocess.PIPE, text=True)))
        objs.append(obj)
        if len(procs) >= jobs:
            _wait(procs.pop(0))
    for p in procs:
        _wait(p)
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *link_extra, *objs,
                    "-o", tmp], check=True)
    os.replace(tmp, out)
    return out


def _wait(item):
    src, p = item
    _, err = p.communicate()
    lines = [l for l in (err or "").splitlines() if "packed-fp32-ops" not in l]
    if p.returncode != 0:
        sys.stderr.write("\n".join(lines) + "\n")
        raise RuntimeError("hipcc failed on %s" % src)
    if lines:
        sys.stderr.write("\n".join(lines) + "\n")


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
