"""Build libmoe.so in-tree for gfx950 with hipcc (cross-compiles without a GPU)."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmoe.so")
SOURCES = ["route.hip", "permute.hip", "grouped_gemm.hip", "combine.hip", "quant.hip", "api.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # keep the compiler from forming packed fp32 instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


# The same library with its host code (argument checks, workspace carve,
# launch sequence) under AddressSanitizer and UndefinedBehaviorSanitizer, for
# the CPU tests of the C ABI; the device code is compiled as for LIB.
HOSTSAN_LIB = os.path.join(HERE, "libmoe_hostsan.so")
HOSTSAN_FLAGS = [
    "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-omit-frame-pointer", "-shared-libsan", "-g",
]


def asan_runtime() -> str:
    """Path of the clang AddressSanitizer runtime that HOSTSAN_LIB links."""
    import glob
    hits = sorted(glob.glob(os.path.join(os.path.dirname(os.path.dirname(HIPCC)), "llvm", "lib", "clang", "*",
                                         "lib", "linux", "libclang_rt.asan-x86_64.so")))
    if not hits:
        raise RuntimeError("clang AddressSanitizer runtime not found under the ROCm LLVM")
    return hits[-1]


# The bounds-checked build of the kernels (include/moe_debug.h).
DEBUG_LIB = os.path.join(HERE, "libmoe_debug.so")

# The load-only streaming probes (csrc/stream_probe.hip), a library of their
# own that the layer never loads; bench.py --stream-probe times them.
PROBE_LIB = os.path.join(HERE, "libmoe_probe.so")
PROBE_SOURCES = ["stream_probe.hip"]


def build(verbose: bool = False, hostsan: bool = False, debug: bool = False, probe: bool = False) -> str:
    """Compile every HIP source into mixture_experts_router_amd/libmoe.so
    (hostsan: into libmoe_hostsan.so with sanitised host code; debug: into
    libmoe_debug.so with the kernels' bounds checks; probe: the streaming
    probes into libmoe_probe.so)."""
    out = PROBE_LIB if probe else (HOSTSAN_LIB if hostsan else (DEBUG_LIB if debug else LIB))
    tmp = out + ".tmp"
    extra = (HOSTSAN_FLAGS if hostsan else []) + (["-DMOE_DEBUG"] if debug else [])
    srcs = PROBE_SOURCES if probe else SOURCES
    cmd = [HIPCC, *FLAGS, *extra, "-o", tmp] + [os.path.join(CSRC, s) for s in srcs]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{msgs}")
    if verbose and msgs.strip():
        print(msgs, flush=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
