"""Build libqli.so for gfx950 with hipcc (in-tree, no JIT cache)."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libqli.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = [os.path.join(CSRC, "qli_api.cpp"), os.path.join(CSRC, "qli_kernels.hip"),
           os.path.join(CSRC, "qli_quant.hip"), os.path.join(CSRC, "qli_attn.hip")]
# the ceiling probes (measurement only) are a library of their own
PROBE_SOURCES = [os.path.join(CSRC, "qli_probe.hip")]
PROBE_OUT = os.path.join(HERE, "libqli_probe.so")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # one IEEE rounding per golden step: no fused multiply-add contraction
    "-ffp-contract=off",
    # no packed FP32 instructions anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _compile(sources, out, verbose):
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, *sources, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    if verbose:
        print(r.stderr)
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """Compile the indexer into quantized_top_indexer_amd/libqli.so and the
    ceiling probes into libqli_probe.so."""
    _compile(SOURCES, OUT, verbose)
    _compile(PROBE_SOURCES, PROBE_OUT, verbose)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
