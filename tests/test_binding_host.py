"""The Python binding rejects tensors whose shape, dtype, layout or device does
not match what the C ABI will read or write, before any call into the library
(run on the CPU: every check fires before a kernel could be launched)."""
import pytest
import torch

import ternary_weight_bitlinear_amd as tw

M, N, K = 3, 40, 144
KP = 256


def weight():
    return tw.PackedWeight(torch.zeros((N, KP // 4), dtype=torch.uint8), torch.ones(N), N, K,
                           torch.ones(1), torch.zeros(1, dtype=torch.int64))


def quantised(m=M):
    return (torch.zeros((m, KP), dtype=torch.int8), torch.ones(m), torch.zeros(m, dtype=torch.int32))


def test_linear_rejects_bad_q_and_scales():
    w = weight()
    q, a, r = quantised()
    bad = [
        (q.to(torch.int16), a, r), (q[:, :KP - 16], a, r), (torch.zeros((M, 2 * KP), dtype=torch.int8)[:, ::2], a, r),
        (q, a[:2], r), (q, a.double(), r), (q, a, r.long()), (q, a, r[:1]),
        (torch.zeros((M, KP), dtype=torch.int8).t().contiguous().t(), a, r),
    ]
    for args in bad:
        with pytest.raises(ValueError):
            tw.linear(*args, w)


def test_linear_rejects_bad_output():
    w = weight()
    q, a, r = quantised()
    for out in (torch.empty((M - 1, N)), torch.empty((M, N - 1)), torch.empty((M, N + 3))[:, 1::1][:, :N - 1],
                torch.empty((N, M)).t(), torch.empty(M * N)):
        with pytest.raises(ValueError):
            tw.linear(q, a, r, w, out=out)
    with pytest.raises(TypeError):
        tw.linear(q, a, r, w, out=torch.empty((M, N), dtype=torch.float16))


def test_linear_rejects_bad_weight_buffers():
    q, a, r = quantised()
    w = weight()
    w.packed = w.packed[:, :-1]
    with pytest.raises(ValueError):
        tw.linear(q, a, r, w)
    w = weight()
    w.w_scale = w.w_scale[:-1]
    with pytest.raises(ValueError):
        tw.linear(q, a, r, w)


def test_checked_arguments_must_live_on_the_gpu():
    """Shapes all correct, but host tensors: refused before the library is called."""
    w = weight()
    q, a, r = quantised()
    with pytest.raises(ValueError, match="CUDA"):
        tw.linear(q, a, r, w)
    with pytest.raises(ValueError, match="CUDA"):
        tw.act_quant(torch.zeros((M, K), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="CUDA"):
        tw.bitlinear(torch.zeros((M, K), dtype=torch.bfloat16), w)


def test_linear_blocked_rejects_bad_arguments():
    nb = -(-K // 256)
    wb = tw.BlockPackedWeight(torch.zeros((N, KP // 4), dtype=torch.uint8), torch.ones((nb, N)), N, K)
    q, a, _ = quantised()
    with pytest.raises(ValueError):
        tw.linear_blocked(q, a[:1], wb)
    with pytest.raises(ValueError):
        tw.linear_blocked(q, a, wb, out=torch.empty((M - 1, N)))
    wb.block_scale = torch.ones((nb + 1, N))
    with pytest.raises(ValueError):
        tw.linear_blocked(q, a, wb)


def test_bitlinear_rejects_bad_workspace_and_output():
    w = weight()
    x = torch.zeros((M, K), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        tw.bitlinear(x, w, workspace=quantised(M - 1))
    with pytest.raises(ValueError):
        tw.bitlinear(x, w, workspace=(torch.zeros((M, KP), dtype=torch.uint8),) + quantised()[1:])
    with pytest.raises(ValueError):
        tw.bitlinear(x, w, out=torch.empty((M, N - 1)))
    with pytest.raises(ValueError):
        tw.rmsnorm_bitlinear(x, torch.ones(K), w, out=torch.empty((M + 1, N)))
    with pytest.raises(ValueError):
        tw.linear_a16(x, w, out=torch.empty((M, 2 * N))[:, ::2])


def test_grouped_rejects_mixed_dtypes_and_bad_outputs():
    w = weight()
    x = torch.zeros((1, K), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        tw.GroupedBitLinear([(x, w, torch.empty((1, N))), (x.float(), w, torch.empty((1, N)))])
    with pytest.raises(ValueError):
        tw.GroupedBitLinear([(x, w, torch.empty((1, N))), (x, w, torch.empty((1, N), dtype=torch.bfloat16))])
    with pytest.raises(ValueError):
        tw.GroupedBitLinear([(x, w, torch.empty((N, 1)).t())])
