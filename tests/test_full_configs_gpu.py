"""Parity at the full workload sizes, in the launch configuration the benchmark
times (bitnet_bitlinear_forward per projection).

For each projection: the packed bytes, w_scale and q are compared in full with
the oracle; the int32 acc and y are compared on sampled outputs (random pairs,
two whole token rows, two whole output columns) which the oracle computes one
by one; and on every element y must equal fp32(acc) * fp32(a_scale * w_scale)
and acc must respect |acc| <= 127 * K.
"""
import numpy as np
import pytest
import torch

import ternary_weight_bitlinear_amd as tw
from ternary_weight_bitlinear_amd import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda"


def bits(t):
    t = t.detach().cpu().contiguous()
    return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()


def u32(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def check_projection(orc, W, x, segments, rng, out_dtype=torch.float32):
    M, K = x.shape
    N = W.shape[0]
    pw = tw.pack(W, segments)
    t, ws, sm, zc = orc.weight_quant(bits(W), segments)
    assert np.array_equal(pw.packed.cpu().numpy(), orc.pack(t))
    assert np.array_equal(u32(pw.w_scale.cpu().numpy()), u32(ws))
    assert np.array_equal(pw.zero_count.numpy(), zc)

    q = torch.empty((M, tw.padded_k(K)), dtype=torch.int8, device=DEV)
    a = torch.empty(M, dtype=torch.float32, device=DEV)
    r = torch.empty(M, dtype=torch.int32, device=DEV)
    y = tw.bitlinear(x, pw, out_dtype=out_dtype, workspace=(q, a, r))
    qo, ao, ro = orc.act_quant(bits(x))
    assert np.array_equal(q.cpu().numpy(), qo)
    assert np.array_equal(u32(a.cpu().numpy()), u32(ao))
    assert np.array_equal(r.cpu().numpy(), ro)

    _, acc = tw.linear(q, a, r, pw, out_dtype=out_dtype, acc_debug=True)
    assert int(acc.abs().max()) <= 127 * K
    # epilogue property at every element (torch fp32 ops are single IEEE roundings)
    f = a[:, None] * pw.w_scale[None, :]
    expect = acc.float() * f
    if out_dtype == torch.bfloat16:
        assert torch.equal(y, expect.to(torch.bfloat16))
    else:
        assert torch.equal(y.view(torch.int32), expect.view(torch.int32))

    # sampled outputs against the oracle
    mi = np.concatenate([rng.integers(0, M, 256), np.repeat(rng.integers(0, M, 2), N),
                         np.tile(np.arange(M), 2)])
    ni = np.concatenate([rng.integers(0, N, 256), np.tile(np.arange(N), 2),
                         np.repeat(rng.integers(0, N, 2), M)])
    acc_o = orc.int_dot_pairs(qo, t, mi, ni)
    acc_h = acc.cpu().numpy()[mi, ni]
    assert np.array_equal(acc_h, acc_o)
    yo = np.array([orc.dequant_one(int(c), float(ao[m]), float(ws[n])) for c, m, n in
                   zip(acc_o[:256], mi[:256], ni[:256])], dtype=np.float32)
    yh = y.float().cpu().numpy()[mi[:256], ni[:256]]
    if out_dtype == torch.bfloat16:
        assert np.array_equal(bits(y)[mi[:256], ni[:256]], orc.bf16_from_f32(yo))
    else:
        assert np.array_equal(u32(yh), u32(yo))
    del pw, q, y, acc


@pytest.mark.parametrize("cfg", ["c1", "c3", "c4", "c5"])
def test_workload_full_size(orc, cfg):
    w = wl.WORKLOADS[cfg]
    rng = np.random.default_rng(w.index)
    for i, p in enumerate(w.projections):
        print(f"[case] {cfg} {p.name} M={w.M} N={p.N} K={p.K}", flush=True)
        W = wl.weight_for(w, i, device=DEV)
        x = wl.activation_for(w, i, device=DEV)
        check_projection(orc, W, x, p.segments or None, rng,
                         out_dtype=torch.bfloat16 if cfg in ("c3", "c4") and i % 2 else torch.float32)
        torch.cuda.synchronize()


@pytest.mark.parametrize("layer", [0, 15, 29])
def test_decode_layers(orc, layer):
    w = wl.WORKLOADS["c2"]
    rng = np.random.default_rng(layer)
    for i, p in enumerate(w.projections):
        print(f"[case] c2 layer {layer} {p.name} N={p.N} K={p.K}", flush=True)
        W = wl.weight_for(w, i, layer=layer, device=DEV)
        x = wl.activation_for(w, i, layer=layer, device=DEV)
        check_projection(orc, W, x, None, rng)
        torch.cuda.synchronize()
