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


@pytest.mark.parametrize("M,N,K", [(1, 2560, 2560), (1, 640, 6912), (1, 13824, 2560), (2, 257, 400), (3, 130, 8192),
                                   (16, 100, 2048), (1, 33, 16), (4, 2560, 6912)])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_blocked_decode(orc, M, N, K, out):
    """Decode sizes (M <= 16) of the block-scaled linear run on the streaming
    kernel: bit-exact against the oracle, incl. a partial last block (K = 400),
    27 blocks (K = 6912), the largest K (8192), ragged N and N < 64."""
    x, W = blocked_case(M * 17 + N + K, M, N, K, zero_blocks=(K > 512))
    ref = orc.linear_blocked(bits(x), bits(W), out=out)
    pw = tw.pack_blocked(W.to(DEV))
    q, a, _ = tw.act_quant(x.to(DEV))
    ybuf = torch.full((M, N + 8), float("nan"), device=DEV,
                      dtype=torch.float32 if out == "f32" else torch.bfloat16)
    y = tw.linear_blocked(q, a, pw, out=ybuf[:, :N])
    assert np.array_equal(bits(y).view(np.uint32 if out == "f32" else np.uint16),
                          ref["y"].view(np.uint32) if out == "f32" else ref["y"])
    assert torch.isnan(ybuf[:, N:].float()).all()


@pytest.mark.parametrize("M", [1, 4])
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_blocked_grouped(orc, M, out):
    """A decoder layer's projections (and a few ragged ones) with block-scaled
    weights in one grouped launch, tokens quantised in the launch; every output
    bit-exact against the oracle, on two launches of the same plan."""
    shapes = [(2560, 2560), (640, 2560), (640, 2560), (2560, 2560), (6912, 2560), (6912, 2560), (2560, 6912),
              (130, 1152), (33, 400)]
    dt = torch.float32 if out == "f32" else torch.bfloat16
    items, refs = [], []
    for i, (N, K) in enumerate(shapes):
        x, W = blocked_case(700 + i, M, N, K, zero_blocks=(i % 3 == 0 and K > 512))
        refs.append(orc.linear_blocked(bits(x), bits(W), out=out)["y"])
        items.append((x.to(DEV), tw.pack_blocked(W.to(DEV)), torch.full((M, N), float("nan"), device=DEV, dtype=dt)))
    group = tw.GroupedBitLinear(items)
    assert group.kernel == "stream-blocked"
    for rep in range(2):
        for _, _, y in items:
            y.fill_(float("nan"))
        group()
        torch.cuda.synchronize()
        for j, ((_, _, y), ref) in enumerate(zip(items, refs)):
            got = bits(y)
            assert np.array_equal(got.view(np.uint32) if out == "f32" else got,
                                  ref.view(np.uint32) if out == "f32" else ref), (rep, j)


def test_blocked_grouped_decode_30_layers(orc):
    """The BitNet-b1.58-2B-shaped decode stream (30 layers x 7 projections,
    M = 1) with per-256-block weight scales in one grouped launch, every output
    against the oracle."""
    from concurrent.futures import ThreadPoolExecutor
    w = wl.WORKLOADS["c2"]
    items, host = [], []
    for layer in range(w.layers):
        for i, p in enumerate(w.projections):
            W = wl.weight_for(w, i, layer=layer, device=DEV)
            x = wl.activation_for(w, i, layer=layer, device=DEV)
            items.append((x, tw.pack_blocked(W), torch.full((1, p.N), float("nan"), device=DEV)))
            host.append((bits(W), bits(x)))
            del W
    group = tw.GroupedBitLinear(items)
    print(f"[case] blocked c2 grouped 210 items, kernel {group.kernel}", flush=True)
    group()
    torch.cuda.synchronize()
    with ThreadPoolExecutor(max_workers=16) as pool:
        refs = list(pool.map(lambda hw: orc.linear_blocked(hw[1], hw[0])["y"], host))
    for j, ((_, _, y), ref) in enumerate(zip(items, refs)):
        assert np.array_equal(bits(y).view(np.uint32), ref.view(np.uint32)), j
