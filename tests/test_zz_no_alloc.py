"""The allocation-free device pack (bitnet_pack_weights_static) against the
device pack it mirrors (bitnet_pack_weights with BITNET_MEM_DEVICE), through
the C ABI: two calls in a row, the second on a smaller input, must each give
the same packed bytes, scales, segment means and zero counts as the
allocating entry point -- so nothing left in the shared fixed array by the
first call leaks into the second.  A non-finite weight is reported, and the
next call is clean again."""
import ctypes

import numpy as np
import pytest
import torch

import ternary_weight_bitlinear_amd as tw
from ternary_weight_bitlinear_amd import _lib
from ternary_weight_bitlinear_amd import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _call(static: bool, W: torch.Tensor, segments):
    N, K = W.shape
    Kp = tw.padded_k(K)
    packed = torch.full((N, Kp // 4), 0xAA, dtype=torch.uint8, device=DEV)
    w_scale = torch.full((N,), float("nan"), device=DEV)
    segs = (ctypes.c_int64 * len(segments))(*segments)
    seg_mean = (ctypes.c_float * len(segments))()
    zeros = (ctypes.c_int64 * len(segments))()
    stream = torch.cuda.current_stream().cuda_stream
    dt = _lib.BF16 if W.dtype == torch.bfloat16 else _lib.F32
    L = _lib.lib()
    if static:
        st = L.bitnet_pack_weights_static(stream, W.data_ptr(), dt, N, K, W.stride(0), segs, len(segments),
                                          packed.data_ptr(), w_scale.data_ptr(), seg_mean, zeros)
    else:
        st = L.bitnet_pack_weights(_lib.MEM_DEVICE, stream, W.data_ptr(), dt, N, K, W.stride(0), segs,
                                   len(segments), packed.data_ptr(), w_scale.data_ptr(), seg_mean, zeros)
    return st, packed.cpu(), w_scale.cpu(), np.array(seg_mean[:], dtype=np.float32), np.array(zeros[:])


def _same(a, b):
    assert a[0] == _lib.OK and b[0] == _lib.OK, (a[0], b[0], _lib.lib().bitnet_last_error())
    assert torch.equal(a[1], b[1])
    assert torch.equal(a[2].view(torch.int32), b[2].view(torch.int32))
    assert np.array_equal(a[3].view(np.uint32), b[3].view(np.uint32))
    assert np.array_equal(a[4], b[4])


def test_static_pack_matches_device_pack_twice():
    print("[case] static pack: 13824 x 2560 fused gate|up, then 640 x 1152", flush=True)
    big = wl.weight_for(wl.WORKLOADS["c5"], 0, device=DEV)                     # two 6912-row segments
    _same(_call(True, big, [6912, 6912]), _call(False, big, [6912, 6912]))
    small = wl.draw_weight((640, 1152), seed=17, dist="laplace", device=DEV)
    _same(_call(True, small, [640]), _call(False, small, [640]))
    torch.cuda.synchronize()


def test_static_pack_reports_non_finite_then_recovers():
    print("[case] static pack: non-finite weight, then a clean call", flush=True)
    W = wl.draw_weight((96, 320), seed=5, device=DEV).float()
    W[40, 7] = float("inf")
    st = _call(True, W, [32, 64])[0]
    assert st == _lib.ERR_NONFINITE
    W2 = wl.draw_weight((96, 320), seed=6, device=DEV)[:, :304]                  # strided rows, fewer columns
    _same(_call(True, W2, [32, 32, 32]), _call(False, W2, [32, 32, 32]))
    torch.cuda.synchronize()
