"""Parity of the per-256-block weight-scale variant (HIP path, through the C
ABI) with the CPU oracle's readings R15 and R16.

Bar: packed bytes and block scales bit-exact; y bit-exact for fp32 (the fp32
operation order is fixed by the definition, block by block) and for bf16.
Weights get a different spread in every row and, in some cases, all-zero
blocks, so every block has its own scale; K covers partial last blocks
(1152, 4304, 400) and padded K (4304 -> Kp 4352).
"""
import numpy as np
import pytest
import torch

import ternary_weight_bitlinear_amd as tw
from ternary_weight_bitlinear_amd import _lib
from ternary_weight_bitlinear_amd import workloads as wl

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[case] {request.node.nodeid}", flush=True)
    yield
    torch.cuda.synchronize()


def bits(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def blocked_case(seed, M, N, K, zero_blocks=False):
    x = wl.draw_activation((M, K), seed=seed, dist="normal_outliers")
    W = wl.draw_weight((N, K), seed=seed + 1).float()
    W = W * torch.linspace(0.5, 3.0, N).unsqueeze(1)                  # a different spread per row
    W[:, : min(K, 256)] *= 4.0                                        # and per block
    if zero_blocks:
        W[::3, 256: min(K, 512)] = 0.0
    return x, W.to(torch.bfloat16)


CASES = [(1, 300, 1152, False), (5, 257, 4304, True), (17, 130, 2560, False), (130, 257, 6912, True),
         (300, 200, 400, False), (256, 512, 2560, True), (64, 33, 8192, False)]


@pytest.mark.parametrize("M,N,K,zero_blocks", CASES)
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_blocked_linear(orc, M, N, K, zero_blocks, out):
    x, W = blocked_case(M * 131 + N * 7 + K, M, N, K, zero_blocks)
    ref = orc.linear_blocked(bits(x), bits(W), out=out)
    pw = tw.pack_blocked(W.to(DEV))
    assert np.array_equal(pw.packed.cpu().numpy(), ref["packed"])
    assert np.array_equal(pw.block_scale.cpu().numpy().view(np.uint32), ref["block_scale"].view(np.uint32))
    q, a, _ = tw.act_quant(x.to(DEV))
    assert np.array_equal(q.cpu().numpy(), ref["q"])
    y = tw.linear_blocked(q, a, pw, out_dtype=torch.float32 if out == "f32" else torch.bfloat16)
    yd = bits(y)
    if out == "f32":
        rel = np.abs(yd.astype(np.float64) - ref["y"]) / np.maximum(np.abs(ref["y"].astype(np.float64)), 1e-30)
        assert np.all((rel <= 1e-5) | (yd == ref["y"])), float(rel.max())
        assert np.array_equal(yd.view(np.uint32), ref["y"].view(np.uint32))
    else:
        assert np.array_equal(yd, ref["y"])


def test_blocked_strided_output_and_fp32_weights(orc):
    M, N, K = 40, 150, 1152
    x, W = blocked_case(5, M, N, K)
    W32 = W.float() * 1.001                                           # fp32 weights, not bf16 values
    ref = orc.linear_blocked(bits(x), W32.numpy())
    pw = tw.pack_blocked(W32.to(DEV))
    assert np.array_equal(pw.packed.cpu().numpy(), ref["packed"])
    q, a, _ = tw.act_quant(x.to(DEV))
    ybuf = torch.full((M, N + 10), float("nan"), device=DEV)
    tw.linear_blocked(q, a, pw, out=ybuf[:, :N])
    assert np.array_equal(bits(ybuf[:, :N]).view(np.uint32), ref["y"].view(np.uint32))
    assert torch.isnan(ybuf[:, N:]).all()


def test_blocked_rejects_non_finite():
    W = torch.zeros((8, 512), dtype=torch.bfloat16, device=DEV)
    W[3, 300] = float("inf")
    with pytest.raises(RuntimeError):
        tw.pack_blocked(W)
    assert b"finite" in _lib.lib().bitnet_last_error()


@pytest.mark.parametrize("proj", [0, 1, 2])
def test_blocked_full_size(orc, proj):
    """The benchmarked shapes (BitNet-b1.58-2B prefill, M = 4096: gate|up,
    down, q|k|v) with block-scaled weights, in the launch the bench times,
    every output against the oracle."""
    w5 = wl.WORKLOADS["c5"]
    p = w5.projections[proj]
    W = wl.weight_for(w5, proj, device=DEV)
    x = wl.activation_for(w5, proj, device=DEV)
    pb = tw.pack_blocked(W)
    q, a, _ = tw.act_quant(x)
    y = tw.linear_blocked(q, a, pb, out_dtype=torch.bfloat16)
    print(f"[case] blocked c5 {p.name} M={w5.M} N={p.N} K={p.K}", flush=True)
    ref = orc.linear_blocked(bits(x), bits(W), out="bf16")
    assert np.array_equal(pb.packed.cpu().numpy(), ref["packed"])
    assert np.array_equal(pb.block_scale.cpu().numpy().view(np.uint32), ref["block_scale"].view(np.uint32))
    assert np.array_equal(bits(y), ref["y"])
