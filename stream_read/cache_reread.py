"""Read rate of a buffer read again and again, by size: up to the 256 MB
Infinity Cache the data comes from the cache, beyond it from HBM.  The
SnapKV vote passes read every key twice; this is what a second read out of
the cache could gain.

Run on one GPU as ``python -m stream_read.cache_reread``; prints one JSON
line per size (the best of two grid sizes, median of 10 event-timed calls
after 3 untimed ones, no flush between calls)."""
from __future__ import annotations

import ctypes
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))


def main() -> None:
    import numpy as np
    import torch

    from bench import timed_calls
    from stream_read.build import PROBE_LIB
    if not os.path.exists(PROBE_LIB):
        raise RuntimeError(f"{PROBE_LIB} is missing: build it first (python -m stream_read.build)")
    h = ctypes.CDLL(PROBE_LIB)
    for name in ("se_hbm_read", "se_cache_reread"):
        fn = getattr(h, name)
        fn.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
        fn.restype = ctypes.c_int
    buf = torch.ones((1 << 30) // 4, dtype=torch.float32, device="cuda")
    sink = torch.zeros((1,), dtype=torch.int32, device="cuda")
    for mib in (32, 64, 128, 192, 256, 384, 1024):
        nbytes = mib << 20
        for name in ("se_cache_reread", "se_hbm_read"):
            fn = getattr(h, name)
            best = 0.0
            for blocks in (2048, 8192):
                def read(i):
                    rc = fn(buf.data_ptr(), nbytes, blocks, sink.data_ptr(), torch.cuda.current_stream().cuda_stream)
                    if rc != 0:
                        raise RuntimeError(f"{name} failed: {rc}")
                ms, _ = timed_calls(read, 10, 3, None)
                best = max(best, nbytes / (float(np.median(ms)) * 1e-3) / 1e9)
            print(json.dumps({"read": name, "MiB": mib, "GBps": round(best)}), flush=True)


if __name__ == "__main__":
    main()
