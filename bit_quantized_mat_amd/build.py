"""Build step for the HIP library: compiles every ``csrc/*.hip`` source for
gfx950 into ``bit_quantized_mat_amd/libbqm.so`` (in-tree, so the built
library travels with the source tree)."""
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
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-fvisibility=hidden",
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


def _compile(srcs, out, verbose):
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, "-I", os.path.join(HERE, "..", "include"), *srcs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """Compile the library and the benchmark's probe library (always
    recompiles); returns the library path."""
    _compile(sources(), LIB, verbose)
    _compile([PROBE_SRC], PROBE_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
