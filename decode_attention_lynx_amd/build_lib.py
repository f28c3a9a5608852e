"""Build liblynx.so in place with hipcc for gfx950 (python -m decode_attention_lynx_amd.build_lib)."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
SOURCES = ["csrc/lynx_abi.hip", "csrc/lynx_codec.hip", "csrc/lynx_attn.hip", "csrc/lynx_verify.hip"]
OUT = os.path.join(PKG, "liblynx.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall",
         # no packed-FP32 instructions anywhere in the device code
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


PROBE_SOURCES = ["csrc/hbm_probe.hip"]
PROBE_OUT = os.path.join(PKG, "libhbmprobe.so")


def _hipcc(sources, out, verbose):
    tmp = out + ".tmp"
    cmd = [HIPCC, *FLAGS, "-o", tmp, *[os.path.join(PKG, s) for s in sources]]
    r = subprocess.run(cmd, cwd=PKG, capture_output=True, text=True)
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{' '.join(cmd)}\n{msgs}")
    if verbose and msgs.strip():
        print(msgs, file=sys.stderr)
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """liblynx.so (the Lynx path) and libhbmprobe.so (the benchmark's HBM reference kernels)."""
    _hipcc(SOURCES, OUT, verbose)
    _hipcc(PROBE_SOURCES, PROBE_OUT, verbose)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
