"""Build libmoe.so for gfx950 in-tree with hipcc (no GPU needed: hipcc cross-compiles).

    python -m mixture_experts_ffn_moerouter_amd.build [--jobs N]

Every HIP source under csrc/ is compiled to an object in csrc/_build/, in parallel, and
linked into mixture_experts_ffn_moerouter_amd/libmoe.so; the measurement probes under
probes/ (include/moe_probes.h) are linked into libmoe_probes.so the same way. Packed-FP32 instructions are
turned off for device code (-packed-fp32-ops): the compiler still emits scalar FP32.
"""
import argparse
import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(CSRC, "_build")
LIB = os.path.join(PKG, "libmoe.so")
PROBES = os.path.join(PKG, "probes")
PROBE_LIB = os.path.join(PKG, "libmoe_probes.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++20", "-fPIC", "-Wall",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I" + os.path.join(os.path.dirname(PKG), "include")]


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the device feature flag; that warning is harmless
    out = "\n".join(l for l in p.stdout.splitlines()
                    if "packed-fp32-ops" not in l and "not a recognized feature" not in l)
    return p.returncode, out


def _compile_and_link(srcs, objdir, lib, jobs, verbose):
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, os.path.basename(s)[:-4] + ".o") for s in srcs]
    cmds = [[HIPCC, *FLAGS, "-c", s, "-o", o] for s, o in zip(srcs, objs)]
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(_run, cmds))
    failed = False
    for cmd, (rc, out) in zip(cmds, results):
        if out.strip() and (rc or verbose):
            print(out, file=sys.stderr)
        if rc:
            print("FAILED: " + " ".join(cmd), file=sys.stderr)
            failed = True
    name = os.path.basename(lib)
    if failed:
        raise RuntimeError(name + ": compilation failed")
    tmp = lib + ".tmp"
    rc, out = _run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs])
    if rc:
        print(out, file=sys.stderr)
        raise RuntimeError(name + ": link failed")
    os.replace(tmp, lib)


def build(jobs: int = 8, verbose: bool = False) -> str:
    _compile_and_link(sorted(glob.glob(os.path.join(CSRC, "*.hip"))), BUILD, LIB, jobs,
                      verbose)
    _compile_and_link(sorted(glob.glob(os.path.join(PROBES, "*.hip"))),
                      os.path.join(PROBES, "_build"), PROBE_LIB, jobs, verbose)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=8)
    ap.add_argument("-v", action="store_true")
    a = ap.parse_args()
    print(build(a.jobs, a.v))
