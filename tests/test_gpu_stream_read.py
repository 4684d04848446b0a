"""The streaming-read yardstick that bench.py reports the decode step against,
and its cache re-read twin, read every 16-byte chunk of their buffer: each
lane folds what it reads into one XOR and stores only if that equals a fixed
constant, so a zero buffer with one planted chunk that folds to the constant
is stored from, wherever the chunk sits and whatever the grid, only if that
chunk is read."""
import ctypes

import pytest
import torch

from gpu_util import DEV, announce

pytestmark = pytest.mark.gpu

MAGIC_I32 = 0x9E3779B9 - (1 << 32)  # the kernel's constant as a signed 32-bit word


def _read_fn(name):
    from stream_read.build import PROBE_LIB
    h = ctypes.CDLL(PROBE_LIB)
    f = getattr(h, name)
    f.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    f.restype = ctypes.c_int
    return f


@pytest.mark.parametrize("name", ["se_hbm_read", "se_cache_reread"])
@pytest.mark.parametrize("blocks", [1, 7, 1024, 65536])
@pytest.mark.parametrize("nbytes", [16, 4096 + 48, (3 << 20) + 16 * 5])
def test_every_chunk_is_read(name, blocks, nbytes):
    announce(f"{name} {nbytes} B, {blocks} blocks")
    f = _read_fn(name)
    nchunk = nbytes // 16
    g = torch.Generator()
    g.manual_seed(nbytes * 131 + blocks)
    spots = sorted({0, nchunk - 1, nchunk // 2, *torch.randint(0, nchunk, (3,), generator=g).tolist()})
    buf = torch.zeros((nchunk, 4), dtype=torch.int32, device=DEV)
    out = torch.zeros((1,), dtype=torch.int32, device=DEV)
    stream = torch.cuda.current_stream().cuda_stream
    for c in spots:
        buf.zero_()
        buf[c, 1] = MAGIC_I32
        out.zero_()
        assert f(buf.data_ptr(), nbytes, blocks, out.data_ptr(), stream) == 0
        torch.cuda.synchronize()
        assert out.item() == MAGIC_I32, f"chunk {c} of {nchunk} not read with {blocks} blocks"
    # and with nothing planted nothing is stored
    buf.zero_()
    out.zero_()
    assert f(buf.data_ptr(), nbytes, blocks, out.data_ptr(), stream) == 0
    torch.cuda.synchronize()
    assert out.item() == 0
