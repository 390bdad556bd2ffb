"""Build libmla_dcp.so in-tree with hipcc for gfx950."""

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libmla_dcp.so")
SOURCES = [os.path.join(PKG, "csrc", "api.hip"), os.path.join(PKG, "csrc", "host.cpp")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # packed fp32 VALU ops stay off: plain float code is compiled to scalar
    # v_fma/v_add/v_mul only
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


# the bench's streaming-read reference (not part of the decode library)
PROBE_LIB = os.path.join(PKG, "libmla_hbm_probe.so")
PROBE_SOURCES = [os.path.join(PKG, "csrc", "hbm_probe.hip")]


def _compile(lib, sources, verbose):
    tmp = lib + ".tmp"
    cmd = [HIPCC] + FLAGS + ["-o", tmp] + sources
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed building {os.path.basename(lib)}")
    if verbose:
        sys.stdout.write(res.stderr)
    os.replace(tmp, lib)


def build(verbose=False):
    """Compile libmla_dcp.so (every decode-library source) and the bench's
    libmla_hbm_probe.so in-tree."""
    _compile(LIB, SOURCES, verbose)
    _compile(PROBE_LIB, PROBE_SOURCES, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
