"""The MFMA-rate calibration kernel (measurement support for bench.py) does the
work its header states: with all-ones operands every thread's sum is the
closed form 16 accumulator elements x 4 accumulators x (K per MFMA) x 4 x iters."""
import ctypes

import pytest
import torch

import sparse_attention_indexer_lightning_amd as sa

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _fn():
    f = sa.lib().idxc_calib_mfma_rate
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                  ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    return f


@pytest.mark.parametrize("kind,one,K", [(0, 0x38, 64), (1, 0x3F80, 16)])   # fp8 e4m3 1.0; bf16 1.0
def test_calib_closed_form(kind, one, K):
    f = _fn()
    if kind == 0:
        a = torch.full((4096,), one, dtype=torch.uint8, device=DEV)
    else:
        a = torch.full((2048,), one, dtype=torch.int16, device=DEV)
    blocks, iters = 3, 2
    out = torch.full((blocks * 256,), -1.0, dtype=torch.float32, device=DEV)
    s = torch.cuda.current_stream()
    nbytes = a.numel() * a.element_size()
    assert f(kind, a.data_ptr(), nbytes, a.data_ptr(), nbytes, iters, blocks, out.data_ptr(), s.cuda_stream) == 0
    torch.cuda.synchronize()
    want = 16 * 4 * K * 4 * iters
    assert torch.all(out == want), (out.min().item(), out.max().item(), want)
    z = torch.zeros_like(a)
    assert f(kind, z.data_ptr(), nbytes, z.data_ptr(), nbytes, iters, blocks, out.data_ptr(), s.cuda_stream) == 0
    torch.cuda.synchronize()
    assert torch.all(out == 0)
