"""Parity at the full workload sizes, in the launch configurations the
benchmark times, element by element against the oracle.

c1, c3, c4, c5: each projection through bitnet_bitlinear_forward (ActQuant,
then the decode kernel or the GEMM), as the prefill leg of the benchmark runs
it.  The packed bytes, w_scale, the zero counts, q, a_scale and q_rowsum are
compared in full; every int32 acc is compared with the oracle's integer dot
(threaded over output rows on the host) and every y with the oracle's
epilogue, bit for bit (fp32 and bf16).

c2: the benchmark's headline launch -- all 30 layers x 7 projections (210
items, M = 1) in one grouped launch -- with every output compared with the
oracle, plus the per-projection calls of three layers.
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import ternary_weight_bitlinear_amd as tw
from ternary_weight_bitlinear_amd import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda"
THREADS = max(1, min(16, os.cpu_count() or 1))


def bits(t):
    t = t.detach().cpu().contiguous()
    return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()


def u32(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def check_projection(orc, W, x, segments, out_dtype=torch.float32):
    M, K = x.shape
    pw = tw.pack(W, segments)
    t, ws, sm, zc = orc.weight_quant(bits(W), segments)
    assert np.array_equal(pw.packed.cpu().numpy(), orc.pack(t))
    assert np.array_equal(u32(pw.w_scale.cpu().numpy()), u32(ws))
    assert np.array_equal(u32(pw.seg_mean.numpy()), u32(sm))
    assert np.array_equal(pw.zero_count.numpy(), zc)

    q = torch.empty((M, tw.padded_k(K)), dtype=torch.int8, device=DEV)
    a = torch.empty(M, dtype=torch.float32, device=DEV)
    r = torch.empty(M, dtype=torch.int32, device=DEV)
    y = tw.bitlinear(x, pw, out_dtype=out_dtype, workspace=(q, a, r))
    qo, ao, ro = orc.act_quant(bits(x))
    assert np.array_equal(q.cpu().numpy(), qo)
    assert np.array_equal(u32(a.cpu().numpy()), u32(ao))
    assert np.array_equal(r.cpu().numpy(), ro)

    acc_o = orc.int_dot(qo, t, nthreads=THREADS)
    yo = orc.epilogue(acc_o, ao, ws, "bf16" if out_dtype == torch.bfloat16 else "f32")
    if out_dtype == torch.bfloat16:
        assert np.array_equal(bits(y), yo)
    else:
        assert np.array_equal(u32(y.cpu().numpy()), u32(yo))
    # the same launch again with the exact int32 sums written out
    _, acc = tw.linear(q, a, r, pw, out_dtype=out_dtype, acc_debug=True)
    assert np.array_equal(acc.cpu().numpy(), acc_o)
    del pw, q, y, acc


@pytest.mark.parametrize("cfg", ["c1", "c3", "c4", "c5"])
def test_workload_full_size(orc, cfg):
    w = wl.WORKLOADS[cfg]
    for i, p in enumerate(w.projections):
        out_dtype = torch.bfloat16 if cfg in ("c3", "c4", "c5") and i % 2 == 0 else torch.float32
        print(f"[case] {cfg} {p.name} M={w.M} N={p.N} K={p.K} out={out_dtype}", flush=True)
        W = wl.weight_for(w, i, device=DEV)
        x = wl.activation_for(w, i, device=DEV)
        check_projection(orc, W, x, p.segments or None, out_dtype)
        torch.cuda.synchronize()


@pytest.mark.parametrize("layer", [0, 15, 29])
def test_decode_layers(orc, layer):
    """Per-projection single calls (the decode kernels a caller without a plan uses)."""
    w = wl.WORKLOADS["c2"]
    for i, p in enumerate(w.projections):
        print(f"[case] c2 layer {layer} {p.name} N={p.N} K={p.K}", flush=True)
        W = wl.weight_for(w, i, layer=layer, device=DEV)
        x = wl.activation_for(w, i, layer=layer, device=DEV)
        check_projection(orc, W, x, None)
        torch.cuda.synchronize()


def test_decode_grouped_210_items(orc):
    """The benchmark's headline launch: 30 layers x 7 projections at M = 1 in one
    grouped launch (weights packed on the device, fp32 outputs), every output
    against the oracle."""
    w = wl.WORKLOADS["c2"]
    items, host = [], []
    for layer in range(w.layers):
        for i, p in enumerate(w.projections):
            W = wl.weight_for(w, i, layer=layer, device=DEV)
            x = wl.activation_for(w, i, layer=layer, device=DEV)
            y = torch.full((1, p.N), float("nan"), device=DEV)
            items.append((x, tw.pack(W), y))
            host.append((bits(W), bits(x)))
            del W
    group = tw.GroupedBitLinear(items)
    print(f"[case] c2 grouped 210 items, kernel {group.kernel}", flush=True)
    assert group.kernel == "stream"
    group()
    torch.cuda.synchronize()
    ys = [y.cpu().numpy() for _, _, y in items]

    def reference(hw):
        Wb, xb = hw
        t, ws, _, _ = orc.weight_quant(Wb)
        q, a, _ = orc.act_quant(xb)
        return orc.epilogue(orc.int_dot(q, t), a, ws)

    with ThreadPoolExecutor(max_workers=THREADS) as pool:     # the oracle's calls release the GIL
        refs = list(pool.map(reference, host))
    for j, (yh, yo) in enumerate(zip(ys, refs)):
        assert np.array_equal(u32(yh), u32(yo)), f"item {j} (layer {j // 7}, {w.projections[j % 7].name})"
    # a second launch over the same plan gives the same bits
    for _, _, y in items:
        y.fill_(float("nan"))
    group()
    torch.cuda.synchronize()
    for j, (_, _, y) in enumerate(items):
        assert np.array_equal(u32(y.cpu().numpy()), u32(refs[j])), f"item {j}, second launch"
