"""Build step for the HIP library: compiles every ``csrc/*.hip`` source for
gfx950 into ``bit_quantized_mat_amd/libbqm.so`` (in-tree, so the built
library travels with the source tree)."""
import concurrent.futures
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libbqm.so")
# calibration kernels used only by bench.py (empty dispatch, streaming read)
PROBE_SRC = os.path.join(HERE, "probes", "probes.hip")
PROBE_LIB = os.path.join(HERE, "libbqm_probes.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    # no packed-fp32 instructions anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # every fp32 operation rounds once, as written; fused multiply-adds only
    # where the source calls fmaf (HIP's default would also fuse a product
    # with its fp16 conversion, rounding once instead of twice)
    "-ffp-contract=off",
    "-Wall", "-Wno-unused-function",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


OBJ_DIR = os.path.join(HERE, "_build")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.run(cmd, check=True)


def _compile(srcs, out, verbose):
    """Each source to its own object (in parallel: every translation unit
    holds its own kernels and launchers), then one shared library."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    inc = ["-I", os.path.join(HERE, "..", "include")]
    objs = [os.path.join(OBJ_DIR, os.path.basename(s) + ".%d.o" % os.getpid()) for s in srcs]
    jobs = max(1, min(len(srcs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        list(ex.map(lambda so: _run([HIPCC, *FLAGS, *inc, "-c", so[0], "-o", so[1]], verbose),
                    zip(srcs, objs)))
    tmp = out + ".tmp%d" % os.getpid()
    try:
        _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp], verbose)
        os.replace(tmp, out)
    finally:
        for o in objs:
            if os.path.exists(o):
                os.remove(o)


def build(verbose: bool = False) -> str:
    """Compile the library and the benchmark's probe library (always
    recompiles); returns the library path."""
    _compile(sources(), LIB, verbose)
    _compile([PROBE_SRC], PROBE_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
