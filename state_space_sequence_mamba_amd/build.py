"""Build libssd.so (the gfx950 SSD kernels and their C ABI) in-tree with hipcc.

    python -m state_space_sequence_mamba_amd.build        # or build() from Python

Each .hip file is compiled to an object in _build/ (in parallel), then linked into
state_space_sequence_mamba_amd/libssd.so (and the measurement-only libssd_peak.so).  Always
recompiles.
"""
import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libssd.so")

SOURCES = ["ssd_api.hip", "chunk_state.hip", "chunk_state_seg.hip", "state_passing.hip", "chunk_scan.hip",
           "chunk_scan_group.hip",
           "ssd_step.hip", "conv1d.hip", "ssd_bwd.hip", "gated_norm.hip"]
# measurement only (bench.py --peak-probe): register-resident MFMA loops, a library of its own
PEAK_SOURCES = ["peak_probe.hip"]
LIB_PEAK = os.path.join(PKG, "libssd_peak.so")
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # no packed-fp32 instructions (v_pk_fma_f32 and friends) anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libssd.so)")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature and says so; that line is noise
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    return err


def build(verbose=False, jobs=None):
    os.makedirs(BUILD, exist_ok=True)
    cc = hipcc()
    cmds = []
    for src in SOURCES + PEAK_SOURCES:
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        cmds.append([cc, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    jobs = jobs or min(len(cmds), os.cpu_count() or 4, 8)
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        for cmd, err in zip(cmds, ex.map(_run, cmds)):
            if verbose or err.strip():
                print(" ".join(os.path.basename(c) for c in cmd[-3:]), err, file=sys.stderr)
    for lib, srcs in ((LIB, SOURCES), (LIB_PEAK, PEAK_SOURCES)):
        objs = [os.path.join(BUILD, os.path.splitext(src)[0] + ".o") for src in srcs]
        tmp = lib + ".tmp"
        _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
        os.replace(tmp, lib)
    return LIB


# Host code built with AddressSanitizer (device code unchanged), for the CPU tests of the C ABI's
# host logic: loaded by a Python process that preloads the clang ASan runtime.
ASAN_DIR = os.path.join(BUILD, "asan")
LIB_ASAN = os.path.join(ASAN_DIR, "libssd_asan.so")
ASAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]


def asan_runtime():
    """The clang ASan runtime matching hipcc's host compiler (None if not installed)."""
    root = os.path.join(os.path.dirname(os.path.dirname(hipcc())), "llvm", "lib", "clang")
    if not os.path.isdir(root):
        return None
    for ver in sorted(os.listdir(root), reverse=True):
        cand = os.path.join(root, ver, "lib", "linux", "libclang_rt.asan-x86_64.so")
        if os.path.exists(cand):
            return cand
    return None


def build_asan(force=False, jobs=None):
    """Build (or reuse, when newer than every source and header) the host-sanitized library."""
    os.makedirs(ASAN_DIR, exist_ok=True)
    deps = [os.path.join(CSRC, f) for f in os.listdir(CSRC)] + [os.path.join(INCLUDE, f) for f in os.listdir(INCLUDE)]
    if not force and os.path.exists(LIB_ASAN) and os.path.getmtime(LIB_ASAN) > max(map(os.path.getmtime, deps)):
        return LIB_ASAN
    cc = hipcc()
    cmds = [[cc, *FLAGS, *ASAN_FLAGS, "-c", os.path.join(CSRC, src), "-o",
             os.path.join(ASAN_DIR, os.path.splitext(src)[0] + ".o")] for src in SOURCES]
    jobs = jobs or min(len(cmds), os.cpu_count() or 4, 8)
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        list(ex.map(_run, cmds))
    objs = [c[-1] for c in cmds]
    tmp = LIB_ASAN + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address", "-shared-libasan",
          "-o", tmp, *objs])
    os.replace(tmp, LIB_ASAN)
    return LIB_ASAN


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
