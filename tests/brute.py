"""Independent fp64 brute force of y = linear(ActQuant(x), WeightQuant(W)).

Written from the formulas on "BitVLA -- 1.58-bit Vision-Language-Action on Core
AI", s1 (WeightQuant = round(W*s).clamp(-1,1)/s with s = 1/mean|W|; ActQuant =
round(x*127/max|x|).clamp(-128,127)/(127/max|x|)), in vectorised numpy and
without the integer path: the dequantised operands are multiplied in fp64.
Only the rounding decisions are taken in fp32, the precision the library
takes them in.  Used on tiny shapes only.
"""
import math

import numpy as np


def act_quant_dequant(x: np.ndarray):
    """x fp32 [M, K] -> (dequantised activations fp64, int codes, sa fp32)."""
    amax = np.abs(x).max(axis=1).astype(np.float32)
    safe = np.where(amax > 0, amax, np.float32(1))
    sa = np.float32(127) / safe
    q = np.clip(np.rint(x * sa[:, None]), -128, 127)
    q = np.where(amax[:, None] > 0, q, 0)
    return q / sa.astype(np.float64)[:, None], q.astype(np.int8), sa


def weight_quant_dequant(W: np.ndarray):
    """W fp32 [N, K], one tensor -> (dequantised weights fp64, codes, s fp32)."""
    mean = np.float32(math.fsum(np.abs(W.astype(np.float64)).ravel()) / W.size)
    s = np.float32(1) / mean
    t = np.clip(np.rint(W * s), -1, 1)
    return t / np.float64(s), t.astype(np.int8), s


def linear(x: np.ndarray, W: np.ndarray):
    """Returns (Y fp64 [M, N], error bound [M, N], q, t).

    The bound covers the fp32 epilogue and the difference between the two
    equivalent ways of writing the scales (1/sa vs amax/127, 1/s vs mean):
    a few fp32 ulps of sum |q*t| / (sa*s), plus a tiny absolute floor.
    """
    xd, q, sa = act_quant_dequant(x)
    Wd, t, s = weight_quant_dequant(W)
    Y = xd @ Wd.T
    mag = (np.abs(q).astype(np.float64) @ np.abs(t).astype(np.float64).T)
    bound = 1e-6 * mag / (sa.astype(np.float64)[:, None] * np.float64(s)) + 1e-30
    return Y, bound, q, t
