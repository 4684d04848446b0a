"""Build libse_hbmread.so, the plain streaming-read kernel that bench.py
measures the decode step against, in-tree with the library's hipcc flags.
It is measurement equipment beside bench.py, not part of the library.

Run as ``python -m stream_read.build`` or call ``build_probe()``.
"""
from __future__ import annotations

import os
import subprocess

from sparse_kv_long_amd.build import ARCH, COMMON, HIPCC

HERE = os.path.dirname(os.path.abspath(__file__))
PROBE_SRC = os.path.join(HERE, "hbm_read.hip")
PROBE_LIB = os.path.join(HERE, "libse_hbmread.so")


def build_probe() -> str:
    tmp = PROBE_LIB + ".tmp"
    cmd = [HIPCC, "-x", "hip", f"--offload-arch={ARCH}", *COMMON, "-shared", "-o", tmp, PROBE_SRC]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed on " + PROBE_SRC + ":\n" + r.stdout + r.stderr)
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


if __name__ == "__main__":
    print(build_probe())
