"""The benchmark's pattern-ceiling helper (libdlceiling, csrc/dl_ceiling.hip):
the step kernel's access pattern on the state with nothing else, a read pass
or an in-place read and rewrite.  On the CPU: the library loads, exports its
two calls and rejects bad arguments before any HIP call.  On the GPU: a read
pass changes nothing (its one store is never taken), and a rewrite pass leaves
the state bit for bit as it was, so neither can disturb what bench.py times
around it."""
import ctypes
import math
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "recurrent_state_update_amd", "libdlceiling.so")


def _lib():
    lib = ctypes.CDLL(LIB)
    lib.dlc_sink_floats.argtypes = [ctypes.c_int] * 3
    lib.dlc_sink_floats.restype = ctypes.c_long
    lib.dlc_tile_pass.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_void_p, ctypes.c_float, ctypes.c_void_p]
    lib.dlc_tile_pass.restype = ctypes.c_int
    return lib


def test_ceiling_helper_validates_before_any_launch():
    lib = _lib()
    assert lib.dlc_sink_floats(2048, 128, 128) == 2048 * 128
    assert lib.dlc_sink_floats(8192, 64, 64) == 8192 * 64
    assert lib.dlc_sink_floats(0, 128, 128) == 0
    assert lib.dlc_sink_floats(4, 32, 128) == 0       # only d_k, d_v in {64, 128}
    S, SINK = 0x7f0000000000, 0x7f0010000000           # fake addresses, never dereferenced
    nan = float("nan")
    assert lib.dlc_tile_pass(None, 4, 128, 128, 0, SINK, nan, None) == -1
    assert lib.dlc_tile_pass(S, 4, 128, 128, 0, None, nan, None) == -1
    assert lib.dlc_tile_pass(S, 4, 16, 128, 0, SINK, nan, None) == -1
    assert lib.dlc_tile_pass(S + 4, 4, 128, 128, 0, SINK, nan, None) == -1   # 16-byte alignment
    assert lib.dlc_tile_pass(S, 4, 128, 128, 1, SINK + 8, nan, None) == -1
    assert lib.dlc_tile_pass(S, 1 << 17, 128, 128, 0, SINK, nan, None) == -1  # 2^31 elements


@pytest.mark.gpu
@pytest.mark.skipif(not __import__("torch").cuda.is_available(), reason="no GPU")
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (128, 64), (64, 128)])
def test_ceiling_passes_change_nothing(dk, dv):
    import torch
    lib = _lib()
    BH = 300  # several workgroups per CU's share, not a multiple of anything
    S = torch.randn(BH * dk * dv, device="cuda")
    ref = S.clone()
    sink = torch.full((lib.dlc_sink_floats(BH, dk, dv),), 7.0, device="cuda")
    sp = torch.cuda.current_stream().cuda_stream
    for write in (0, 1, 0, 1):
        assert lib.dlc_tile_pass(S.data_ptr(), BH, dk, dv, write, sink.data_ptr(), math.nan, sp) == 0
    torch.cuda.synchronize()
    assert torch.equal(S, ref)
    assert bool((sink == 7.0).all())
