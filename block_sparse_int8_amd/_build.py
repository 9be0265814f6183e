"""Compiles the gfx950 HIP kernels and the C ABI into libsparse_attn.so (in-tree)."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libsparse_attn.so")
SOURCES = ["abi.hip", "quantize.hip", "route.hip", "fwd.hip"]
# measurement probes for bench.py --peaks (matrix-core and HBM ceilings); not
# part of the attention library
PROBE_LIB = os.path.join(HERE, "libsa_probe.so")
PROBE_SOURCES = ["probe.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # fused multiply-adds only where the source writes them
    "-ffp-contract=off",
    # no packed fp32 instructions in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def _hipcc(sources, out, verbose, extra=()):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    cmd = [hipcc, *HIPCC_FLAGS, *extra, "-I", os.path.join(HERE, "..", "include"),
           *[os.path.join(CSRC, s) for s in sources], "-o", out + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "packed-fp32-ops"
    err = "\n".join(l for l in r.stderr.splitlines() if noise not in l)
    if r.returncode != 0:
        sys.stderr.write(err + "\n")
        raise RuntimeError("hipcc failed")
    if verbose and err.strip():
        print(err)
    os.replace(out + ".tmp", out)
    return out


def build(verbose: bool = False, extra=()) -> str:
    _hipcc(PROBE_SOURCES, PROBE_LIB, verbose, extra)
    return _hipcc(SOURCES, LIB, verbose, extra)


if __name__ == "__main__":
    print(build(verbose=True))
