"""Build libcf.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Each translation unit under csrc/ is compiled in parallel into _build/ and
linked into cnn_cosmology_volumes_amd/libcf.so (in-tree, next to this file).
"""
import concurrent.futures
import glob
import os
import shutil
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libcf.so")
ARCH = "gfx950"


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build libcf.so)")


COMMON = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
    # packed fp32 instructions are disabled for every kernel in this library
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in VGPRs rather than AGPRs: saves the AGPR-to-VGPR copies
    # of accumulators that feed VALU epilogues (no other kernel changes)
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wno-unused-result",
]


# Per-file code generation options, chosen by measurement (A/B of whole
# library builds on the GPU): LLVM's max-ILP machine scheduler makes the pool
# kernels faster and other kernels slower, so it is applied per file.
PER_FILE = {
    "k_pool.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"],
}


def _compile(src: str, obj: str) -> str:
    extra = PER_FILE.get(os.path.basename(src), [])
    cmd = [hipcc()] + COMMON + extra + ["-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr))
    return obj


PROBE_SRC = os.path.join(HERE, "probe", "mfma_peak.hip")
PROBE_LIB = os.path.join(HERE, "libcfprobe.so")


def build_probe() -> str:
    """The matrix-core throughput probe used by bench.py --mfma-peak (a
    library of its own, not linked into libcf.so)."""
    tmp = PROBE_LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc()] + COMMON + ["-shared", PROBE_SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("probe build failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr))
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


def build(jobs: int = 0) -> str:
    """Compile every csrc/*.hip and link libcf.so; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    objs = [os.path.join(BUILD, os.path.basename(s)[:-4] + ".o") for s in srcs]
    jobs = jobs or min(len(srcs), max(1, (os.cpu_count() or 4)))
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(_compile, srcs, objs))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr))
    os.replace(tmp, LIB)
    build_probe()
    return LIB


if __name__ == "__main__":
    print(build())
