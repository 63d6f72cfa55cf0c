"""The calibration kernels (measurement support for bench.py) do the work their
header states.  MFMA rate: with all-ones operands every thread's sum is the
closed form 16 accumulator elements x 4 accumulators x (K per MFMA) x 4 x iters.
Gather rate: the XOR over all threads of their outputs equals the XOR of every
32-bit word of the rows the index set names (skipped entries excluded),
computed here with numpy from the same rows."""
import ctypes

import numpy as np
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


def _gather_fn():
    f = sa.lib().idxc_calib_gather_rate
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_longlong, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                  ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    return f


@pytest.mark.parametrize("row_bytes,nq,rows_per_seq,k,blocks", [(1152, 3, 1000, 77, 5), (128, 2, 300, 64, 1),
                                                                (2048, 1, 50, 13, 64), (1152, 4, 4096, 2048, 37)])
def test_calib_gather_closed_form(row_bytes, nq, rows_per_seq, k, blocks):
    f = _gather_fn()
    g = np.random.default_rng(row_bytes + nq + k)
    words = g.integers(0, 2 ** 32, size=(nq * rows_per_seq, row_bytes // 4), dtype=np.uint64).astype(np.uint32)
    t = g.integers(-2, rows_per_seq + 3, size=(nq, k)).astype(np.int32)   # a few entries outside the rows
    t[0, 0] = -1
    t[-1, -1] = rows_per_seq
    want = np.uint32(0)
    for b in range(nq):
        for j in range(k):
            ix = int(t[b, j])
            if 0 <= ix < rows_per_seq:
                want ^= np.bitwise_xor.reduce(words[b * rows_per_seq + ix])
    rows = torch.from_numpy(words.view(np.int32)).to(DEV)
    td = torch.from_numpy(t).to(DEV)
    out = torch.full((blocks * 256,), -1, dtype=torch.int32, device=DEV)
    s = torch.cuda.current_stream()
    assert f(rows.data_ptr(), row_bytes, rows_per_seq, td.data_ptr(), nq, k, blocks, out.data_ptr(),
             s.cuda_stream) == 0
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    assert got == want, (hex(int(got)), hex(int(want)))
