"""Build the native libraries of the package in-tree.

* ``libcsa2.so``        -- the HIP library behind include/csa2.h (hipcc, gfx950).
* ``libcsa2_synth.so``  -- the seeded synthetic-input generator (gcc).
* ``libcsa2_probe.so``  -- the row-gather rate probe behind ``bench.py
  --gather-probe`` (a measurement aid, not part of the ABI).
"""
import concurrent.futures as cf
import glob
import os
import subprocess
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

HIP_LIB = os.path.join(PKG, "libcsa2.so")
SYNTH_LIB = os.path.join(PKG, "libcsa2_synth.so")
PROBE_LIB = os.path.join(PKG, "libcsa2_probe.so")

def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)


def build_synth(verbose: bool = False) -> str:
    src = os.path.join(PKG, "synth_c", "csa2_synth.c")
    _run(["gcc", "-O2", "-std=c99", "-D_DEFAULT_SOURCE", "-ffp-contract=off", "-fopenmp", "-fPIC",
          "-shared", "-Wall", "-Wextra", "-o", SYNTH_LIB + ".tmp", src, "-lm"], verbose)
    os.replace(SYNTH_LIB + ".tmp", SYNTH_LIB)
    return SYNTH_LIB


def _hip_flags(src):
    flags = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
             # packed-fp32 instructions are kept out of every kernel
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             # matrix-core accumulators in ordinary VGPRs, so the register
             # allocator can use the accumulation registers for staged rows
             "-mllvm", "-amdgpu-mfma-vgpr-form",
             "-Wall", "-Wno-unused-result", "-I", os.path.join(ROOT, "include")]
    return flags


def build_hip(verbose: bool = False) -> str:
    srcs = sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")))
    if not srcs:
        raise RuntimeError("no HIP sources under csrc/")
    with tempfile.TemporaryDirectory(prefix="csa2_build_") as tmp:
        objs = [os.path.join(tmp, os.path.basename(s) + ".o") for s in srcs]
        jobs = min(len(srcs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1)))
        with cf.ThreadPoolExecutor(max_workers=max(jobs, 1)) as ex:
            futs = [ex.submit(_run, [HIPCC] + _hip_flags(s) + ["-c", s, "-o", o], verbose) for s, o in zip(srcs, objs)]
            for f in futs:
                f.result()
        _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", HIP_LIB + ".tmp"] + objs, verbose)
    os.replace(HIP_LIB + ".tmp", HIP_LIB)
    return HIP_LIB


def build_probe(verbose: bool = False) -> str:
    src = os.path.join(PKG, "probe", "gather_rate.hip")
    _run([HIPCC] + _hip_flags(src) + ["-shared", "-o", PROBE_LIB + ".tmp", src], verbose)
    os.replace(PROBE_LIB + ".tmp", PROBE_LIB)
    return PROBE_LIB


def build_all(verbose: bool = False):
    return build_synth(verbose), build_hip(verbose), build_probe(verbose)


if __name__ == "__main__":
    build_all(verbose=True)
