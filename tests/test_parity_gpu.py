"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Bar: packed bytes, codes, w_scale, q, a_scale, q_rowsum and the int32 acc are
bit-exact; fp32 y is within 1e-5 relative of the oracle (the operation order is
the same, so it is expected and checked to be bit-exact as well); bf16 y is
bit-exact.  Inputs come from the seeded generators in
ternary_weight_bitlinear_amd.workloads; the oracle sees the same bytes.
"""
import numpy as np
import pytest
import torch

import ternary_weight_bitlinear_amd as tw
from ternary_weight_bitlinear_amd import _lib
from ternary_weight_bitlinear_amd import workloads as wl

pytestmark = pytest.mark.gpu

DEV = "cuda"


def bits(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def f32bits(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def check_y(y_dev: torch.Tensor, y_orc: np.ndarray):
    if y_dev.dtype == torch.bfloat16:
        assert np.array_equal(bits(y_dev), y_orc)
        return
    y = y_dev.cpu().numpy()
    rel = np.abs(y.astype(np.float64) - y_orc) / np.maximum(np.abs(y_orc.astype(np.float64)), 1e-30)
    assert np.all((rel <= 1e-5) | (y == y_orc)), float(rel.max())
    assert np.array_equal(f32bits(y), f32bits(y_orc))     # same op order: bit-exact


@pytest.fixture(autouse=True)
def _announce(request):
    print(f"\n[case] {request.node.nodeid}", flush=True)
    yield
    torch.cuda.synchronize()


# ------------------------------------------------------------------ ActQuant

@pytest.mark.parametrize("M,K,dist", [
    (1, 16, "normal"), (1, 2560, "normal_outliers"), (3, 144, "normal"), (17, 1152, "normal"),
    (64, 4304, "student_t_channels"), (5, 6912, "normal"), (2, 20480, "normal"), (300, 1024, "normal"),
    (4, 8192, "normal_outliers"), (3, 8208, "normal"),   # last K of the per-token workgroup kernel, first past it
])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_act_quant(orc, M, K, dist, dtype):
    x = wl.draw_activation((M, K), seed=M * 7 + K, dist=dist)
    xd = x.to(DEV).to(dtype)
    q, a, r = tw.act_quant(xd)
    xo = bits(x) if dtype == torch.bfloat16 else x.float().numpy()
    qo, ao, ro = orc.act_quant(xo)
    assert np.array_equal(q.cpu().numpy(), qo)
    assert np.array_equal(f32bits(a.cpu().numpy()), f32bits(ao))
    assert np.array_equal(r.cpu().numpy(), ro)


def test_act_quant_strided_zero_and_extreme_tokens(orc):
    K = 272
    base = wl.draw_activation((6, K + 40), seed=99).to(DEV)
    base[1].zero_()                                  # all-zero token
    base[2] *= 2.0 ** 100                            # huge values
    base[3] *= 2.0 ** -100                           # tiny values
    base[4, 3] = 254.0                               # exact ties (amax = 254)
    base[4, :3] = torch.tensor([1.0, 3.0, 5.0])
    base[4, 4:] = 0
    x = base[:, :K]                                  # ldx = K + 40, rows not 16-byte aligned
    q, a, r = tw.act_quant(x)
    qo, ao, ro = orc.act_quant(bits(x))
    assert np.array_equal(q.cpu().numpy(), qo)
    assert np.array_equal(f32bits(a.cpu().numpy()), f32bits(ao))
    assert np.array_equal(r.cpu().numpy(), ro)
    assert a[1].item() == 0 and not q[1].any()


def test_act_quant_long_rows_strided_zero_and_extreme_tokens(orc):
    """Rows long enough for one workgroup per token (4096 < K <= 8192), not
    16-byte aligned, with an all-zero token, huge and tiny values and exact ties."""
    K = 4112
    base = wl.draw_activation((6, K + 40), seed=98).to(DEV)
    base[1].zero_()
    base[2] *= 2.0 ** 100
    base[3] *= 2.0 ** -100
    base[4, 3] = 254.0
    base[4, :3] = torch.tensor([1.0, 3.0, 5.0])
    base[4, 4:] = 0
    base[5, :] = base[5, :] / base[5, :].abs().max() * 2.0 ** -122   # zero token by the fp32 edge
    x = base[:, :K]
    q, a, r = tw.act_quant(x)
    qo, ao, ro = orc.act_quant(bits(x))
    assert np.array_equal(q.cpu().numpy(), qo)
    assert np.array_equal(f32bits(a.cpu().numpy()), f32bits(ao))
    assert np.array_equal(r.cpu().numpy(), ro)
    assert a[1].item() == 0 and not q[1].any() and a[5].item() == 0


def test_tokens_at_the_fp32_scale_edge(orc):
    """R5 at the edge of fp32: a token whose largest magnitude is 2^-122 (127/amax
    overflows fp32) quantises as a zero token, one at 2^-121 as any other; every
    quantiser -- ActQuant, RMSNorm -> ActQuant, the fused single-call decode
    kernels and a grouped launch's batched quantiser -- agrees with the oracle."""
    K = 2560
    base = wl.draw_activation((4, K), seed=77).float()
    x = base.clone()
    x[1] = base[1] / base[1].abs().max() * 2.0 ** -122
    x[2] = base[2] / base[2].abs().max() * 2.0 ** -121
    x = x.to(torch.bfloat16)
    xd = x.to(DEV)
    q, a, r = tw.act_quant(xd)
    qo, ao, ro = orc.act_quant(bits(x))
    assert np.array_equal(q.cpu().numpy(), qo)
    assert np.array_equal(f32bits(a.cpu().numpy()), f32bits(ao))
    assert np.array_equal(r.cpu().numpy(), ro)
    assert ao[1] == 0 and not qo[1].any() and ao[2] > 0 and qo[2].any()
    g = torch.ones(K, dtype=torch.bfloat16)
    qn, an, rn = tw.rmsnorm_act_quant(xd, g.to(DEV), 1e-6)
    qno, ano, rno = orc.rms_act_quant(bits(x), bits(g), 1e-6)
    assert np.array_equal(qn.cpu().numpy(), qno) and np.array_equal(rn.cpu().numpy(), rno)
    assert np.allclose(an.cpu().numpy(), ano, rtol=1e-5, atol=0) and ano[1] == 0
    for N in (640, 13824):                   # split-K and streaming single calls
        W = wl.draw_weight((N, K), seed=78)
        ref = orc.linear(bits(x), bits(W))
        check_y(tw.bitlinear(xd, tw.pack(W.to(DEV))), ref["y"])
    items, refs = [], []
    for i in range(4):                       # one token per problem: the batched quantiser
        W = wl.draw_weight((2560, K), seed=80 + i)
        items.append((xd[i:i + 1], tw.pack(W.to(DEV)), torch.full((1, 2560), float("nan"), device=DEV)))
        refs.append(orc.linear(bits(x[i:i + 1]), bits(W))["y"])
    group = tw.GroupedBitLinear(items)
    group()
    torch.cuda.synchronize()
    for (_, _, y), ref in zip(items, refs):
        check_y(y, ref)


# -------------------------------------------------------------------- packer

@pytest.mark.parametrize("N,K,segments,dist", [
    (1, 16, None, "normal"), (5, 144, None, "normal"), (33, 1152, (11, 11, 11), "normal"),
    (640, 2560, None, "normal"), (4304, 1152, None, "normal"), (1152, 4304, None, "laplace"),
    (3840, 2560, (2560, 640, 640), "normal"), (70, 6912, (35, 35), "laplace"),
])
def test_device_pack(orc, N, K, segments, dist):
    W = wl.draw_weight((N, K), seed=N + K, dist=dist)
    if segments:
        scales = torch.cat([torch.full((rr, 1), 3.0 ** i) for i, rr in enumerate(segments)])
        W = (W.float() * scales).to(torch.bfloat16)
    pw = tw.pack(W.to(DEV), segments)
    t, ws, sm, zc = orc.weight_quant(bits(W), segments)
    assert np.array_equal(pw.packed.cpu().numpy(), orc.pack(t))
    assert np.array_equal(f32bits(pw.w_scale.cpu().numpy()), f32bits(ws))
    assert np.array_equal(f32bits(pw.seg_mean.numpy()), f32bits(sm))
    assert np.array_equal(pw.zero_count.numpy(), zc)
    # the host packer of the library gives the same bytes
    ph = tw.pack(W, segments)
    assert torch.equal(ph.packed, pw.packed.cpu())


def test_device_pack_fp32_strided_and_degenerate(orc):
    W = wl.draw_weight((48, 320), seed=3).float().to(DEV)[:, :304]
    pw = tw.pack(W)
    t, ws, _, _ = orc.weight_quant(W.cpu().contiguous().numpy())
    assert np.array_equal(pw.packed.cpu().numpy(), orc.pack(t))
    assert np.array_equal(f32bits(pw.w_scale.cpu().numpy()), f32bits(ws))
    Z = torch.zeros((20, 64), dtype=torch.bfloat16, device=DEV)
    pz = tw.pack(Z)
    assert torch.all(pz.packed == 0x55) and torch.all(pz.w_scale == 0)


def test_device_pack_rejects_non_finite():
    W = wl.draw_weight((9, 64), seed=4).to(DEV)
    W[5, 60] = float("nan")
    with pytest.raises(tw.BitnetError) as e:
        tw.pack(W)
    assert e.value.status == _lib.ERR_NONFINITE


# ------------------------------------------------------ RMSNorm -> ActQuant

def _norm_weight(K: int, seed: int, dtype) -> torch.Tensor:
    g = 1.0 + 0.2 * wl.draw_activation((1, K), seed=seed).float()[0]
    return g.to(dtype)


def _check_scale(a_dev: torch.Tensor, a_orc: np.ndarray):
    """a_scale: the codes decide nothing here; the fp64 sums differ only in order, so
    the fp32 result is expected bit-exact and must be within 1e-5 relative."""
    a = a_dev.cpu().numpy()
    rel = np.abs(a.astype(np.float64) - a_orc) / np.maximum(np.abs(a_orc.astype(np.float64)), 1e-30)
    assert np.all((rel <= 1e-5) | (a == a_orc)), float(rel.max())


def check_y_tol(y_dev: torch.Tensor, y_orc: np.ndarray, rel_tol: float = 1e-5):
    y = y_dev.cpu().numpy().astype(np.float64)
    rel = np.abs(y - y_orc) / np.maximum(np.abs(y_orc.astype(np.float64)), 1e-30)
    assert np.all((rel <= rel_tol) | (y == y_orc)), float(rel.max())


# The kernels evaluate silu(gate) * up with their own fp32 steps (exp from a
# two-part split of t * log2(e), the hardware exp2 and an exact 2^n scaling,
# then a reciprocal: within 4.3 fp32 ulps of the true silu(a) * u); the oracle
# evaluates the definition in fp64 and rounds once.  Policy for the gated input:
#   * a code may differ by one only where the oracle's value before rounding,
#     v = fp32(h * g) * fp32(127 / amax) (exact product), lies within GATE_WINDOW
#     of a .5 tie.  GATE_WINDOW: h differs by <= 4.5 * 2^-23 relative, then z,
#     amax, sa and v add one rounding each (<= 13 * 2^-23 relative in all), and
#     |v| <= 127, so |dv| <= 127 * 13 * 2^-23 < 2e-4;
#   * every other code is equal, and q_rowsum is the sum of the kernel's codes;
#   * a_scale is within 1e-5 relative (it moves by ~1e-6 at most);
#   * y is within 1e-5 relative plus one a_scale * w_scale step per code of the
#     token inside the window (|t| <= 1, so each such code moves acc by <= 1).
GATE_WINDOW = 2e-4


def gated_reference(orc, gate_np, up_np, g_np, eps):
    """Oracle q, a_scale, q_rowsum for RMSNorm(silu(gate) * up) and the window mask."""
    h = orc.swiglu(gate_np, up_np)
    qo, ao, ro = orc.rms_act_quant(h, g_np, eps)
    gv = g_np if g_np.dtype == np.float32 else (g_np.astype(np.uint32) << 16).view(np.float32)
    z = (h * gv[None, :]).astype(np.float32)
    amax = np.abs(z).max(axis=1)
    sa = np.where(amax > 0, np.float32(127) / np.where(amax > 0, amax, np.float32(1)), np.float32(0))
    v = z.astype(np.float64) * sa.astype(np.float64)[:, None]
    window = np.abs(np.abs(v - np.trunc(v)) - 0.5) <= GATE_WINDOW
    win = np.zeros_like(qo, dtype=bool)
    win[:, :h.shape[1]] = window
    return qo, ao, ro, win


def check_gated_codes(q_dev, a_dev, r_dev, qo, ao, ro, win):
    q = q_dev.cpu().numpy()
    d = q.astype(np.int32) - qo.astype(np.int32)
    assert np.all(d[~win] == 0), int(np.count_nonzero(d[~win]))
    assert np.all(np.abs(d[win]) <= 1)
    assert np.array_equal(r_dev.cpu().numpy(), q.astype(np.int64).sum(axis=1).astype(np.int32))
    _check_scale(a_dev, ao)


def check_y_gated(y_dev, y_orc, a_o, ws_o, win):
    """y against the oracle under the gated-input policy (see GATE_WINDOW)."""
    y = y_dev.float().cpu().numpy().astype(np.float64)
    steps = win.sum(axis=1).astype(np.float64)[:, None] * (a_o.astype(np.float64)[:, None] *
                                                            ws_o.astype(np.float64)[None, :])
    err = np.abs(y - y_orc.astype(np.float64))
    assert np.all(err <= 1e-5 * np.abs(y_orc.astype(np.float64)) + steps * (1 + 1e-5)), float(err.max())


@pytest.mark.parametrize("M,K,dist", [
    (1, 16, "normal"), (1, 2560, "normal_outliers"), (3, 1152, "normal"), (17, 4304, "student_t_channels"),
    (5, 6912, "normal"), (2, 20480, "normal"), (64, 1024, "normal_outliers"),
])
@pytest.mark.parametrize("x_dtype,g_dtype", [(torch.bfloat16, torch.bfloat16), (torch.float32, torch.float32),
                                             (torch.bfloat16, torch.float32)])
def test_rmsnorm_act_quant(orc, M, K, dist, x_dtype, g_dtype):
    x = wl.draw_activation((M, K), seed=M * 13 + K, dist=dist)
    if M > 2:
        x[1] = 0                                   # an all-zero token
        x[2] *= 1e-5                               # eps dominates
    g = _norm_weight(K, K + 1, g_dtype)
    xd = x.to(DEV).to(x_dtype)
    q, a, r = tw.rmsnorm_act_quant(xd, g.to(DEV), 1e-6)
    xo = bits(x.to(x_dtype)) if x_dtype == torch.bfloat16 else x.float().numpy()
    go = bits(g) if g_dtype == torch.bfloat16 else g.numpy()
    qo, ao, ro = orc.rms_act_quant(xo, go, 1e-6)
    assert np.array_equal(q.cpu().numpy(), qo)
    assert np.array_equal(r.cpu().numpy(), ro)
    _check_scale(a, ao)


@pytest.mark.parametrize("M,K", [(1, 6912), (4, 2048), (9, 16), (2, 20480), (3, 8192)])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_gated_rmsnorm_act_quant(orc, M, K, dtype):
    """The down projection's input: silu(gate) * up, then RMSNorm and ActQuant;
    gate and up are strided views of one [M, 2K] buffer (the fused gate|up output).
    Held to the oracle's fp64 silu under the gated-input policy (GATE_WINDOW)."""
    gu = (wl.draw_activation((M, 2 * K), seed=K + M, dist="normal").float() * 3).to(dtype)
    g = _norm_weight(K, K + 7, torch.bfloat16)
    gud = gu.to(DEV)
    q, a, r = tw.rmsnorm_act_quant(gud[:, :K], g.to(DEV), 1e-6, up=gud[:, K:])
    if dtype == torch.bfloat16:
        go, uo = bits(gu[:, :K].contiguous()), bits(gu[:, K:].contiguous())
    else:
        go, uo = gu[:, :K].contiguous().numpy(), gu[:, K:].contiguous().numpy()
    qo, ao, ro, win = gated_reference(orc, go, uo, bits(g), 1e-6)
    check_gated_codes(q, a, r, qo, ao, ro, win)


def test_rmsnorm_strided_unaligned_and_eps_zero(orc):
    """x rows at an odd fp32 stride (the unaligned load path), eps = 0, fp32 weight."""
    M, K = 6, 1152
    base = wl.draw_activation((M, K + 3), seed=77).float()
    x = base.to(DEV)[:, 1:K + 1]
    g = _norm_weight(K, 5, torch.float32)
    q, a, r = tw.rmsnorm_act_quant(x, g.to(DEV), 0.0)
    qo, ao, ro = orc.rms_act_quant(base[:, 1:K + 1].contiguous().numpy(), g.numpy(), 0.0)
    assert np.array_equal(q.cpu().numpy(), qo)
    assert np.array_equal(r.cpu().numpy(), ro)
    _check_scale(a, ao)


@pytest.mark.parametrize("K", [2560, 6912])
def test_rmsnorm_unaligned_norm_weight(orc, K):
    """Aligned token rows with a norm weight that is not 16-byte aligned (a view
    one element into its buffer): every input then takes element loads."""
    M = 5
    x = wl.draw_activation((M, K), seed=K + 3, dist="normal_outliers")
    g = _norm_weight(K, K + 11, torch.bfloat16)
    gbuf = torch.empty(K + 1, dtype=torch.bfloat16, device=DEV)
    gbuf[1:] = g.to(DEV)
    q, a, r = tw.rmsnorm_act_quant(x.to(DEV), gbuf[1:], 1e-6)
    qo, ao, ro = orc.rms_act_quant(bits(x), bits(g), 1e-6)
    assert np.array_equal(q.cpu().numpy(), qo)
    assert np.array_equal(r.cpu().numpy(), ro)
    _check_scale(a, ao)


def test_rmsnorm_then_linear(orc):
    """Normalised, quantised tokens through the decode and GEMM paths against the
    oracle's integer dot and epilogue on its own codes."""
    for M, N, K in ((1, 640, 2560), (40, 257, 1152)):
        x, W = wl.random_case(2100 + M, M, N, K, x_dist="normal_outliers")
        g = _norm_weight(K, 9, torch.bfloat16)
        pw = tw.pack(W.to(DEV))
        q, a, r = tw.rmsnorm_act_quant(x.to(DEV), g.to(DEV), 1e-6)
        y, acc = tw.linear(q, a, r, pw, acc_debug=True)
        qo, ao, _ = orc.rms_act_quant(bits(x), bits(g), 1e-6)
        t, ws, _, _ = orc.weight_quant(bits(W))
        acc_o = orc.int_dot(qo, t)
        assert np.array_equal(acc.cpu().numpy(), acc_o)
        check_y_tol(y, orc.epilogue(acc_o, ao, ws))


@pytest.mark.parametrize("M,N,K,gated", [
    (1, 640, 2560, False), (3, 257, 1152, False), (16, 100, 2048, False),    # split-K decode kernel
    (1, 13824, 2560, False), (2, 8200, 4096, False),                          # streaming decode kernel
    (1, 2560, 6912, True), (1, 5120, 6912, True), (4, 96, 2048, True),       # down projection inputs
    (17, 130, 1152, False), (20, 64, 2048, True),                            # ActQuant launch + GEMM
])
def test_rmsnorm_bitlinear(orc, M, N, K, gated):
    """Input norm fused into the decode kernels' token prologue (or a separate
    launch for larger M) against the oracle: codes and sums bit-exact, a_scale
    and y within 1e-5 relative; gated inputs under the GATE_WINDOW policy."""
    x, W = wl.random_case(3100 + M * 7 + N, M, N, K, x_dist="normal_outliers")
    g = _norm_weight(K, K + 11, torch.bfloat16)
    pw = tw.pack(W.to(DEV))
    xd = x.to(DEV)
    up = wl.draw_activation((M, K), seed=N + 5).to(DEV) if gated else None
    ws = (torch.empty((M, tw.padded_k(K)), dtype=torch.int8, device=DEV),
          torch.empty(M, dtype=torch.float32, device=DEV), torch.empty(M, dtype=torch.int32, device=DEV))
    y = tw.rmsnorm_bitlinear(xd, g.to(DEV), pw, 1e-6, up=up, workspace=ws)
    t, wsc, _, _ = orc.weight_quant(bits(W))
    if gated:
        qo, ao, ro, win = gated_reference(orc, bits(x), bits(up), bits(g), 1e-6)
        check_gated_codes(ws[0], ws[1], ws[2], qo, ao, ro, win)
        # y is the epilogue of the kernel's own codes, and within the policy of the oracle's
        qk, ak = ws[0].cpu().numpy(), ws[1].cpu().numpy()
        assert np.array_equal(f32bits(y.cpu().numpy()), f32bits(orc.epilogue(orc.int_dot(qk, t), ak, wsc)))
        check_y_gated(y, orc.epilogue(orc.int_dot(qo, t), ao, wsc), ao, wsc, win)
    else:
        qo, ao, ro = orc.rms_act_quant(bits(x), bits(g), 1e-6)
        assert np.array_equal(ws[0].cpu().numpy(), qo)
        assert np.array_equal(ws[2].cpu().numpy(), ro)
        _check_scale(ws[1], ao)
        check_y_tol(y, orc.epilogue(orc.int_dot(qo, t), ao, wsc))


@pytest.mark.parametrize("kernel", ["stream", "persistent"])
def test_grouped_rmsnorm(orc, kernel, monkeypatch):
    """A layer's projections with their input norms in one grouped launch: plain,
    normalised and gated (down) inputs mixed, on both grouped kernels."""
    if kernel == "persistent":
        monkeypatch.setenv("BITNET_GROUP_KERNEL", "persistent")
    else:
        monkeypatch.delenv("BITNET_GROUP_KERNEL", raising=False)
    shapes = [(2560, 2560, "norm"), (640, 2560, "norm"), (640, 2560, None), (2560, 2560, "norm"),
              (6912, 2560, "norm"), (6912, 2560, "norm"), (2560, 6912, "gated"), (130, 1152, "gated")]
    items, norms, refs = [], [], []
    for i, (N, K, kind) in enumerate(shapes):
        x, W = wl.random_case(4100 + i, 1, N, K, x_dist="normal_outliers")
        pw = tw.pack(W.to(DEV))
        y = torch.full((1, N), float("nan"), device=DEV)
        items.append((x.to(DEV), pw, y))
        t, wsc, _, _ = orc.weight_quant(bits(W))
        if kind is None:
            norms.append(None)
            qo, ao, _ = orc.act_quant(bits(x))
        else:
            g = _norm_weight(K, 50 + i, torch.bfloat16 if i % 2 else torch.float32)
            up = wl.draw_activation((1, K), seed=60 + i).to(DEV) if kind == "gated" else None
            norms.append((g.to(DEV), up, 1e-6))
            go = bits(g) if g.dtype == torch.bfloat16 else g.numpy()
            if kind == "gated":
                qo, ao, _, win = gated_reference(orc, bits(x), bits(up), go, 1e-6)
                refs.append((orc.epilogue(orc.int_dot(qo, t), ao, wsc), ao, wsc, win))
                continue
            qo, ao, _ = orc.rms_act_quant(bits(x), go, 1e-6)
        refs.append((orc.epilogue(orc.int_dot(qo, t), ao, wsc), None, None, None))
    group = tw.GroupedBitLinear(items, norms)
    assert group.kernel == kernel
    for rep in range(2):
        for _, _, y in items:
            y.fill_(float("nan"))
        group()
        torch.cuda.synchronize()
        for (_, _, y), (ref, ao, wsc, win) in zip(items, refs):
            if win is None:
                check_y_tol(y, ref)
            else:
                check_y_gated(y, ref, ao, wsc, win)


# ------------------------------------------------------------------- I2_S

@pytest.mark.parametrize("N,K", [(24, 48), (2560, 2560), (3, 4352), (6912, 2560), (640, 6912)])
@pytest.mark.parametrize("order", ["strided", "consecutive"])
def test_i2s_device(orc, N, K, order):
    """Device export of a packed weight equals the oracle's I2_S bytes; device import
    of them gives back the layout-v1 bytes and the scale, and the imported weight
    runs through linear to the oracle's outputs."""
    W = wl.draw_weight((N, K), seed=N + 7 * K, dist="normal")
    pw = tw.pack(W.to(DEV))
    t, ws, _, _ = orc.weight_quant(bits(W))
    s = np.float32(1) / ws[0]
    buf = tw.i2s_export(pw, order)
    assert np.array_equal(buf.cpu().numpy(), orc.i2s_pack(t, s, order))
    back = tw.i2s_import(buf, N, K, order)
    assert torch.equal(back.packed, pw.packed)
    assert np.array_equal(f32bits(back.w_scale.cpu().numpy()), f32bits(np.full(N, np.float32(1) / s)))
    if N <= 2560:
        x = wl.draw_activation((2, K), seed=N)
        y = tw.bitlinear(x.to(DEV), back)
        qo, ao, _ = orc.act_quant(bits(x))
        check_y(y, orc.epilogue(orc.int_dot(qo, t), ao, np.full(N, np.float32(1) / s)))


def test_i2s_device_rejects_bad_fields():
    W = wl.draw_weight((8, 64), seed=2).to(DEV)
    buf = tw.i2s_export(tw.pack(W))
    buf[3] = 0xFF
    with pytest.raises(tw.BitnetError, match="holds 3"):
        tw.i2s_import(buf, 8, 64)
    buf = tw.i2s_export(tw.pack(W))
    buf[-4:] = 0                                         # scale +0
    with pytest.raises(tw.BitnetError, match="not positive"):
        tw.i2s_import(buf, 8, 64)
    two = tw.pack((W.float() * torch.tensor([[1.0]] * 4 + [[3.0]] * 4, device=DEV)).to(torch.bfloat16), (4, 4))
    with pytest.raises(tw.BitnetError, match="differs between rows"):
        tw.i2s_export(two)


# --------------------------------------------------------------- W1.58A16

@pytest.mark.parametrize("M,N,K", [(1, 640, 2560), (3, 257, 1152), (16, 100, 2048), (1, 2560, 6912),
                                   (20, 130, 1152), (1, 1, 16), (2, 4352, 4304),
                                   (1, 13824, 2560), (4, 6912, 6912), (16, 8192, 4096)])
@pytest.mark.parametrize("out", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("xdt", [torch.bfloat16, torch.float16])
def test_linear_a16(orc, M, N, K, out, xdt):
    """bf16 or fp16 activations x ternary weights against the oracle's fp64 value,
    within the bound the header states for an fp32 sum in the hardware's order;
    the last three shapes are the largest decode-size calls (8.4-11.9 MB of
    packed weights, up to 16 tokens)."""
    x, W = wl.random_case(5100 + M * 3 + N, M, N, K, x_dist="normal_outliers")
    x = x.to(xdt)
    pw = tw.pack(W.to(DEV))
    base = torch.zeros((M, K + 8), dtype=xdt, device=DEV)
    base[:, :K] = x.to(DEV)
    y = tw.linear_a16(base[:, :K], pw, out_dtype=out)          # ldx = K + 8: strided rows
    t, ws, _, _ = orc.weight_quant(bits(W))
    ye, mag = orc.linear_a16(a16_bits(x), t, ws)
    tol = ws.astype(np.float64)[None, :] * (K / 32 + 64) * 2.0 ** -24 * mag
    got = y.float().cpu().numpy().astype(np.float64)
    if out == torch.bfloat16:
        tol = tol + np.abs(ye) * 2.0 ** -8
    else:
        tol = tol + np.abs(ye) * 2.0 ** -24
    err = np.abs(got - ye)
    assert np.all(err <= tol), float((err / np.maximum(tol, 1e-300)).max())


def a16_bits(x: torch.Tensor) -> np.ndarray:
    """Activations for the oracle's W1.58A16 reference: bf16 bit patterns, or float16."""
    x = x.detach().cpu().contiguous()
    return x.numpy() if x.dtype == torch.float16 else bits(x)


def _check_a16(orc, y, x, W):
    """y against the oracle's fp64 value of w_scale * (x . t), within the bound
    bitnet_linear_a16 states for an fp32 sum in the hardware's order."""
    K = x.shape[1]
    t, ws, _, _ = orc.weight_quant(bits(W))
    ye, mag = orc.linear_a16(a16_bits(x), t, ws)
    tol = ws.astype(np.float64)[None, :] * (K / 32 + 64) * 2.0 ** -24 * mag
    tol = tol + np.abs(ye) * (2.0 ** -8 if y.dtype == torch.bfloat16 else 2.0 ** -24)
    err = np.abs(y.float().cpu().numpy().astype(np.float64) - ye)
    assert np.all(err <= tol), float((err / np.maximum(tol, 1e-300)).max())


@pytest.mark.parametrize("M,shapes,y_dtype", [
    (1, "group", torch.float32), (1, "group", torch.bfloat16), (3, "group", torch.float32),
    (4, "small", torch.bfloat16), (16, "tiny", torch.float32)])
@pytest.mark.parametrize("xdt", [torch.bfloat16, torch.float16])
def test_grouped_a16(orc, M, shapes, y_dtype, xdt):
    """The W1.58A16 group (bf16 or fp16 x kept unquantised) in one streaming launch:
    ragged N, K not a multiple of 128, one-tile problems; each launch of the
    reused plan within the oracle bound."""
    sh = {"group": GROUP_SHAPES, "small": [(640, 1024), (100, 512), (64, 256), (130, 1152)],
          "tiny": [(100, 512), (64, 256), (33, 128)]}[shapes]
    items, cases = [], []
    for i, (N, K) in enumerate(sh):
        x, W = wl.random_case(5300 + 17 * M + i, M, N, K, x_dist="normal_outliers")
        x = x.to(xdt)
        pw = tw.pack(W.to(DEV))
        items.append((x.to(DEV), pw, torch.full((M, N), float("nan"), device=DEV, dtype=y_dtype)))
        cases.append((x, W))
    group = tw.GroupedBitLinear(items, a16=True)
    assert group.kernel == "stream-a16"
    for rep in range(2):
        for _, _, y in items:
            y.fill_(float("nan"))
        group()
        torch.cuda.synchronize()
        for (_, _, y), (x, W) in zip(items, cases):
            _check_a16(orc, y, x, W)


def test_grouped_a16_decoder_layers(orc):
    """Two BitNet-2B-shaped decoder layers (14 projections) as one W1.58A16
    launch: workgroup shares span several projections."""
    shapes = [(2560, 2560), (640, 2560), (640, 2560), (2560, 2560), (6912, 2560), (6912, 2560), (2560, 6912)] * 2
    items, cases = [], []
    for i, (N, K) in enumerate(shapes):
        x, W = wl.random_case(5500 + i, 1, N, K, x_dist="normal_outliers")
        pw = tw.pack(W.to(DEV))
        items.append((x.to(DEV), pw, torch.full((1, N), float("nan"), device=DEV)))
        cases.append((x, W))
    group = tw.GroupedBitLinear(items, a16=True)
    group()
    torch.cuda.synchronize()
    for (_, _, y), (x, W) in zip(items, cases):
        _check_a16(orc, y, x, W)


def test_grouped_a16_rejects_what_does_not_fit():
    """16 bf16 token rows of K = 6912 (221 KB) exceed a workgroup's LDS: the plan
    says so; fp32 activations are refused before any plan is made."""
    x = torch.zeros((16, 6912), dtype=torch.bfloat16, device=DEV)
    pw = tw.pack(torch.ones((64, 6912), dtype=torch.bfloat16, device=DEV))
    with pytest.raises(tw.BitnetError) as e:
        tw.GroupedBitLinear([(x, pw, torch.empty((16, 64), device=DEV))], a16=True)
    assert e.value.status == _lib.ERR_UNSUPPORTED
    with pytest.raises(ValueError):
        tw.GroupedBitLinear([(x.float(), pw, torch.empty((16, 64), device=DEV))], a16=True)


def test_linear_a16_rejects_fp32_activations():
    x = torch.zeros((1, 64), device=DEV)
    pw = tw.pack(torch.ones((8, 64), dtype=torch.bfloat16, device=DEV))
    with pytest.raises(tw.BitnetError) as e:
        tw.linear_a16(x, pw)
    assert e.value.status == _lib.ERR_UNSUPPORTED


# -------------------------------------------------------------------- linear

LINEAR_CASES = [
    # decode kernel (M <= 16)
    (1, 1, 16), (1, 16, 128), (1, 33, 144), (1, 640, 2560), (2, 257, 1152), (5, 130, 4304),
    (8, 64, 6912), (16, 100, 2048), (1, 4304, 1152),
    # single calls of 8 MB or more packed bytes: the streaming decode kernel
    (1, 13824, 2560), (3, 8200, 4096),
    # GEMM (M > 16)
    (17, 16, 16), (33, 130, 144), (130, 257, 1152), (300, 200, 4304), (257, 129, 6912), (512, 640, 2560),
]


@pytest.mark.parametrize("M,N,K", LINEAR_CASES)
@pytest.mark.parametrize("out", ["f32", "bf16"])
def test_linear(orc, M, N, K, out):
    x, W = wl.random_case(M * 131 + N * 7 + K, M, N, K, x_dist="normal_outliers")
    ref = orc.linear(bits(x), bits(W), out=out)
    pw = tw.pack(W.to(DEV))
    q, a, r = tw.act_quant(x.to(DEV))
    dt = torch.float32 if out == "f32" else torch.bfloat16
    check_y(tw.linear(q, a, r, pw, out_dtype=dt), ref["y"])          # the launch the benchmark times
    y, acc = tw.linear(q, a, r, pw, out_dtype=dt, acc_debug=True)    # and with the exact sums written out
    assert np.array_equal(pw.packed.cpu().numpy(), ref["packed"])
    assert np.array_equal(q.cpu().numpy(), ref["q"])
    assert np.array_equal(acc.cpu().numpy(), ref["acc"])
    check_y(y, ref["y"])


_TILE_REFS = {}


def _tile_case(orc, M, N, K):
    """Inputs and oracle results of one GEMM tile case, computed once per shape."""
    if (M, N, K) not in _TILE_REFS:
        x, W = wl.random_case(M * 31 + N * 3 + K, M, N, K, x_dist="normal_outliers")
        ref = orc.linear(bits(x), bits(W), out="f32")
        ref["y_bf16"] = orc.epilogue(ref["acc"], ref["a_scale"], ref["w_scale"], "bf16")
        _TILE_REFS[(M, N, K)] = (x, W, ref)
    return _TILE_REFS[(M, N, K)]


@pytest.mark.parametrize("M,N,K", [(17, 16, 16), (130, 257, 1152), (300, 200, 4304), (257, 129, 6912),
                                   (384, 512, 2560), (520, 1100, 2560)])
@pytest.mark.parametrize("kernel", ["dma", "regs"])
@pytest.mark.parametrize("tile", ["small", "wide", "tiny"])
@pytest.mark.parametrize("epilogue", ["lds", "direct"])
@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_linear_each_gemm_tile(orc, kernel, tile, epilogue, out, M, N, K, monkeypatch):
    """Every GEMM tile (128x128, 128x256 and 64x64, forced) of both kernels
    (LDS-DMA and register-staged loads), with the LDS-staged and the direct
    epilogue of the LDS-DMA kernel, gives the oracle's exact sums and outputs
    on ragged M, N and padded K, bf16 and fp32."""
    if (kernel == "regs" or tile == "tiny") and epilogue == "lds":
        pytest.skip("the LDS-staged epilogue belongs to the LDS-DMA kernel")
    if kernel == "regs" and tile == "tiny":
        pytest.skip("the 64x64 tile has one kernel")
    monkeypatch.setenv("BITNET_GEMM_TILE", tile)
    monkeypatch.setenv("BITNET_GEMM_KERNEL", kernel)
    if epilogue == "direct":
        monkeypatch.setenv("BITNET_GEMM_EPILOGUE", "direct")
    else:
        monkeypatch.delenv("BITNET_GEMM_EPILOGUE", raising=False)
    x, W, ref = _tile_case(orc, M, N, K)
    dt = torch.bfloat16 if out == "bf16" else torch.float32
    want = ref["y_bf16"] if out == "bf16" else ref["y"]
    pw = tw.pack(W.to(DEV))
    q, a, r = tw.act_quant(x.to(DEV))
    check_y(tw.linear(q, a, r, pw, out_dtype=dt), want)
    y, acc = tw.linear(q, a, r, pw, out_dtype=dt, acc_debug=True)
    assert np.array_equal(acc.cpu().numpy(), ref["acc"])
    check_y(y, want)


@pytest.mark.parametrize("pad", [0, 3, 4, 8])
@pytest.mark.parametrize("out", ["bf16", "f32"])
@pytest.mark.parametrize("tile", ["small", "wide"])
def test_gemm_output_strides(orc, pad, out, tile, monkeypatch):
    """GEMM outputs into a NaN-filled buffer with a row stride of N + pad: rows
    aligned to 16 bytes take the LDS-staged epilogue, the others the direct one;
    nothing is written past column N."""
    monkeypatch.setenv("BITNET_GEMM_TILE", tile)
    M, N, K = 200, 300, 1152
    x, W, ref = _tile_case(orc, M, N, K)
    dt = torch.bfloat16 if out == "bf16" else torch.float32
    pw = tw.pack(W.to(DEV))
    q, a, r = tw.act_quant(x.to(DEV))
    ybuf = torch.full((M, N + pad + 8), float("nan"), device=DEV, dtype=dt)
    y = ybuf.view(-1)[: M * (N + pad)].view(M, N + pad)[:, :N]
    tw.linear(q, a, r, pw, out=y)
    check_y(y, ref["y_bf16"] if out == "bf16" else ref["y"])
    assert torch.isnan(ybuf.view(-1)[: M * (N + pad)].view(M, N + pad)[:, N:].float()).all()


@pytest.mark.parametrize("M", [1, 4, 16, 17, 64])
def test_linear_segments_and_strided_output(orc, M):
    K, segs = 2560, (256, 64, 64)
    N = sum(segs)
    x = wl.draw_activation((M, K), seed=M)
    W = torch.cat([wl.draw_weight((rr, K), seed=10 + i, dist="laplace") * (4.0 ** i)
                   for i, rr in enumerate(segs)]).to(torch.bfloat16)
    ref = orc.linear(bits(x), bits(W), segments=segs)
    pw = tw.pack(W.to(DEV), segs)
    q, a, r = tw.act_quant(x.to(DEV))
    ybuf = torch.full((M, N + 24), float("nan"), device=DEV)
    y = tw.linear(q, a, r, pw, out=ybuf[:, :N])
    check_y(y, ref["y"])
    assert torch.isnan(ybuf[:, N:]).all()            # nothing written past N


def test_batch_invariance(orc):
    """A token's output bits do not depend on M or on the kernel (decode vs GEMM)."""
    K, N = 1152, 300
    x, W = wl.random_case(77, 200, N, K)
    pw = tw.pack(W.to(DEV))
    xd = x.to(DEV)
    y_all = tw.bitlinear(xd, pw)
    for lo, hi in ((0, 1), (5, 13), (100, 116), (150, 167), (0, 200)):
        y_part = tw.bitlinear(xd[lo:hi].contiguous(), pw)
        assert torch.equal(y_part, y_all[lo:hi])


def test_bitlinear_equals_two_calls(orc):
    for M in (1, 9, 40):
        x, W = wl.random_case(M, M, 96, 512)
        pw = tw.pack(W.to(DEV))
        xd = x.to(DEV)
        q, a, r = tw.act_quant(xd)
        y2 = tw.linear(q, a, r, pw, out_dtype=torch.bfloat16)
        y1 = tw.bitlinear(xd, pw, out_dtype=torch.bfloat16)
        assert torch.equal(y1, y2)
        assert np.array_equal(bits(y1), orc.linear(bits(x), bits(W), out="bf16")["y"])


def test_closed_forms_on_device():
    """Permutation weights give acc = q[:, perm]; constant weights give acc = q_rowsum."""
    K = 256
    perm = torch.randperm(K, generator=torch.Generator().manual_seed(1))
    P = torch.zeros((K, K), dtype=torch.bfloat16)
    P[torch.arange(K), perm] = 1.0
    x = wl.draw_activation((20, K), seed=5).to(DEV)
    q, a, r = tw.act_quant(x)
    for M in (1, 20):
        _, acc = tw.linear(q[:M], a[:M], r[:M], tw.pack(P.to(DEV)), acc_debug=True)
        assert torch.equal(acc, q[:M, :K][:, perm.to(DEV)].int())
        _, acc = tw.linear(q[:M], a[:M], r[:M], tw.pack(torch.full((7, K), 0.5, dtype=torch.bfloat16,
                                                                    device=DEV)), acc_debug=True)
        assert torch.equal(acc, r[:M, None].expand(M, 7))


def test_linear_argument_errors_on_device():
    x = torch.zeros((2, 32), dtype=torch.bfloat16, device=DEV)
    q, a, r = tw.act_quant(x)
    pw = tw.pack(torch.ones((4, 32), dtype=torch.bfloat16, device=DEV))
    y = torch.empty((2, 3), device=DEV)
    with pytest.raises(tw.BitnetError) as e:
        _lib.check(_lib.lib().bitnet_linear_forward(None, q.data_ptr(), a.data_ptr(), r.data_ptr(), 2, 32,
                                                    pw.packed.data_ptr(), pw.w_scale.data_ptr(), 4,
                                                    y.data_ptr(), _lib.F32, 3, None))
    assert e.value.status == _lib.ERR_INVALID_ARG


@pytest.mark.parametrize("M,dtype", [(1, torch.bfloat16), (3, torch.bfloat16), (2, torch.float32)])
def test_grouped_matches_oracle_and_single_calls(orc, M, dtype):
    shapes = [(2560, 2560), (640, 2560), (6912, 2560), (2560, 6912), (33, 144), (4304, 1152), (1, 16),
              (1152, 4304), (17, 16384 if M == 1 else 4096)]
    items, refs = [], []
    for i, (N, K) in enumerate(shapes):
        x, W = wl.random_case(500 + i, M, N, K, x_dist="normal_outliers")
        pw = tw.pack(W.to(DEV))
        xd = x.to(DEV).to(dtype)
        y = torch.full((M, N), float("nan"), device=DEV)
        items.append((xd, pw, y))
        xo = bits(x) if dtype == torch.bfloat16 else x.float().numpy()
        refs.append(orc.linear(xo, bits(W)))
    group = tw.GroupedBitLinear(items)
    for rep in range(2):                       # the plan is reusable
        for _, _, y in items:
            y.fill_(float("nan"))
        group()
        torch.cuda.synchronize()
        for (xd, pw, y), ref in zip(items, refs):
            check_y(y, ref["y"])
            assert torch.equal(y, tw.bitlinear(xd, pw))


def test_grouped_large_tokens_use_persistent_kernel(orc):
    """M=16 tokens of K=4096 exceed the streaming kernel's LDS share per workgroup,
    so the plan falls back to the persistent kernel; results are the same."""
    M = 16
    shapes = [(640, 4096), (2560, 4096), (97, 4096), (1000, 2048)]
    items, refs = [], []
    for i, (N, K) in enumerate(shapes):
        x, W = wl.random_case(900 + i, M, N, K)
        pw = tw.pack(W.to(DEV))
        y = torch.full((M, N), float("nan"), device=DEV)
        items.append((x.to(DEV), pw, y))
        refs.append(orc.linear(bits(x), bits(W)))
    group = tw.GroupedBitLinear(items)
    assert group.kernel == "persistent"
    group()
    torch.cuda.synchronize()
    for (_, _, y), ref in zip(items, refs):
        check_y(y, ref["y"])


# Grouped decode items: N values leave ragged last tiles; K=4304 and K=2000
# are not multiples of 128 (padded tails); small N gives one-tile problems.
GROUP_SHAPES = [(2560, 2560), (640, 2560), (6912, 2560), (2560, 6912), (2500, 2560), (1000, 4304),
                (4100, 2000), (64, 2560), (130, 6912)]


def _group_case(orc, M, x_dtype, y_dtype, shapes, seed):
    items, refs = [], []
    for i, (N, K) in enumerate(shapes):
        x, W = wl.random_case(seed + i, M, N, K, x_dist="normal_outliers")
        pw = tw.pack(W.to(DEV))
        items.append((x.to(DEV).to(x_dtype), pw, torch.full((M, N), float("nan"), device=DEV, dtype=y_dtype)))
        xo = bits(x) if x_dtype == torch.bfloat16 else x.float().numpy()
        refs.append(orc.linear(xo, bits(W), out="bf16" if y_dtype == torch.bfloat16 else "f32"))
    return items, refs


@pytest.mark.parametrize("M,x_dtype,y_dtype", [(1, torch.bfloat16, torch.float32), (1, torch.float32, torch.bfloat16),
                                               (2, torch.float32, torch.float32), (3, torch.bfloat16, torch.bfloat16),
                                               (4, torch.float32, torch.bfloat16)])
def test_grouped_kernels_agree_with_oracle(orc, M, x_dtype, y_dtype, monkeypatch):
    """The same group planned for the streaming kernel and for the persistent
    fallback matches the oracle on every launch of the reused plan."""
    items, refs = _group_case(orc, M, x_dtype, y_dtype, GROUP_SHAPES, 1300 + 10 * M)
    for kernel in ("stream", "persistent"):
        if kernel == "stream":
            monkeypatch.delenv("BITNET_GROUP_KERNEL", raising=False)
        else:
            monkeypatch.setenv("BITNET_GROUP_KERNEL", kernel)
        group = tw.GroupedBitLinear(items)
        assert group.kernel == kernel
        for rep in range(3):
            for _, _, y in items:
                y.fill_(float("nan"))
            group()
            torch.cuda.synchronize()
            for (_, _, y), ref in zip(items, refs):
                check_y(y, ref["y"])


@pytest.mark.parametrize("M,y_dtype", [(5, torch.float32), (8, torch.bfloat16), (13, torch.float32),
                                       (16, torch.bfloat16)])
def test_grouped_persistent_many_tokens(orc, M, y_dtype, monkeypatch):
    """The persistent kernel at M = 5 to 16 with bf16 tokens (more tokens than the
    streaming kernel's LDS share takes): every launch of the reused plan matches
    the oracle.  Shapes whose M token rows (K rounded up to 512 bytes) exceed the
    plan's 64 KiB of LDS are left out."""
    shapes = [(N, K) for N, K in GROUP_SHAPES if M * (-(-K // 512) * 512) <= 65536]
    items, refs = _group_case(orc, M, torch.bfloat16, y_dtype, shapes, 1900 + 10 * M)
    monkeypatch.setenv("BITNET_GROUP_KERNEL", "persistent")
    group = tw.GroupedBitLinear(items)
    assert group.kernel == "persistent"
    for rep in range(2):
        for _, _, y in items:
            y.fill_(float("nan"))
        group()
        torch.cuda.synchronize()
        for (_, _, y), ref in zip(items, refs):
            check_y(y, ref["y"])


@pytest.mark.parametrize("M", [1, 2, 4])
def test_grouped_many_problems_per_workgroup(orc, M):
    """A six-layer mix of a decoder's projections (each workgroup's share spans
    several problems, so with M > 1 a batch of quantised token rows crosses
    problem boundaries) next to a two-item group with fewer tiles than
    workgroups, launched back to back."""
    big = [(2560, 2560), (640, 2560), (640, 2560), (2560, 2560), (6912, 2560), (6912, 2560), (2560, 6912)] * 6
    items, refs = _group_case(orc, M, torch.bfloat16, torch.bfloat16, big, 1700 + 7 * M)
    small_items, small_refs = _group_case(orc, M, torch.float32, torch.float32, [(130, 2560), (64, 6912)], 1800 + M)
    g_big, g_small = tw.GroupedBitLinear(items), tw.GroupedBitLinear(small_items)
    assert g_big.kernel == "stream" and g_small.kernel == "stream"
    for rep in range(3):
        for _, _, y in items + small_items:
            y.fill_(float("nan"))
        g_big()
        g_small()
        torch.cuda.synchronize()
        for (_, _, y), ref in zip(items + small_items, refs + small_refs):
            check_y(y, ref["y"])


def test_grouped_lds_limited_shares(orc):
    """Thirty decoder layers at M = 4: the token rows of the problems a share
    spans fill the streaming kernel's LDS, so the planner cuts shares where
    they would overflow.  Every output equals the single-call result, and the
    k/v projections of the first and last layer match the oracle."""
    M, gen = 4, torch.Generator(device="cpu").manual_seed(2400)
    layer = [(2560, 2560), (640, 2560), (640, 2560), (2560, 2560), (6912, 2560), (6912, 2560), (2560, 6912)]
    items, checks = [], []
    for li in range(30):
        for pi, (N, K) in enumerate(layer):
            W = (torch.randn(N, K, generator=gen) * 0.02).to(torch.bfloat16)
            x = torch.randn(M, K, generator=gen).to(torch.bfloat16)
            pw = tw.pack(W.to(DEV))
            items.append((x.to(DEV), pw, torch.full((M, N), float("nan"), device=DEV)))
            if li in (0, 29) and pi in (1, 2):
                checks.append((len(items) - 1, orc.linear(bits(x), bits(W))))
    group = tw.GroupedBitLinear(items)
    assert group.kernel == "stream"
    for rep in range(2):
        for _, _, y in items:
            y.fill_(float("nan"))
        group()
        torch.cuda.synchronize()
        for x, pw, y in items:
            assert torch.equal(y, tw.bitlinear(x, pw))
        for i, ref in checks:
            check_y(items[i][2], ref["y"])


@pytest.mark.parametrize("M", [1, 2])
def test_grouped_few_tall_tiles(orc, M):
    """Two groups with fewer 64-row tiles than CUs (16384-wide rows, so one
    tile is a workgroup's whole share, and a 100 x 2560 + 64 x 4304 group),
    each launched four times with the other in between: every launch of a
    reused plan matches the oracle."""
    items, refs = _group_case(orc, M, torch.bfloat16, torch.float32, [(192, 16384), (50, 16384)], 2100 + M)
    other, other_refs = _group_case(orc, M, torch.float32, torch.bfloat16, [(100, 2560), (64, 4304)], 2200 + M)
    g, g_other = tw.GroupedBitLinear(items), tw.GroupedBitLinear(other)
    assert g.kernel == "stream" and g_other.kernel == "stream"
    for rep in range(4):
        for _, _, y in items + other:
            y.fill_(float("nan"))
        g()
        if rep % 2:
            g_other()
        torch.cuda.synchronize()
        for (_, _, y), ref in zip(items, refs):
            check_y(y, ref["y"])
        if rep % 2:
            for (_, _, y), ref in zip(other, other_refs):
                check_y(y, ref["y"])


def test_grouped_plan_rejects_bad_items():
    x = torch.zeros((1, 64), dtype=torch.bfloat16, device=DEV)
    pw = tw.pack(torch.ones((8, 64), dtype=torch.bfloat16, device=DEV))
    with pytest.raises(ValueError):
        tw.GroupedBitLinear([(x, pw, torch.empty((1, 9), device=DEV))])
    x17 = torch.zeros((17, 64), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(tw.BitnetError) as e:
        tw.GroupedBitLinear([(x17, pw, torch.empty((17, 8), device=DEV))])
    assert e.value.status == _lib.ERR_INVALID_ARG
