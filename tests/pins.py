"""Pins: checks that tie the CPU oracle to things other than itself.

Each ``pin_*`` function takes an ``Oracle`` handle and raises AssertionError if
the oracle disagrees with a hand-worked example from the pages' formulas
(``tests/golden``), a closed form, an invariant, a library routine on a special
case, or a brute force on tiny inputs.  The same functions run against the
committed oracle (all must pass) and against deliberately broken copies of it
(at least one must fail), which shows that the set is sharp enough to catch a
dropped term, a wrong sign or index, or a transposed operand.

Run as a script (``python tests/pins.py <liboracle.so>``) it prints a JSON list
of the pins that failed; the mutation test uses that to isolate each broken
copy in a process of its own.
"""
from __future__ import annotations

import json
import math
import sys
from pathlib import Path

import numpy as np

ROOT = Path(__file__).resolve().parents[1]
GOLDEN = Path(__file__).resolve().parent / "golden"
if str(ROOT) not in sys.path:
    sys.path.insert(0, str(ROOT))

import brute  # noqa: E402  (tests/brute.py: independent fp64 brute force)


def _workloads():
    """The seeded input generators (ternary_weight_bitlinear_amd/workloads.py),
    loaded by path so that the library package itself is not imported."""
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "_pin_workloads", ROOT / "ternary_weight_bitlinear_amd" / "workloads.py")
    if spec.name not in sys.modules:
        mod = importlib.util.module_from_spec(spec)
        sys.modules[spec.name] = mod            # dataclasses look their module up here
        spec.loader.exec_module(mod)
    return sys.modules[spec.name]


# ----------------------------------------------------------------- helpers

def f32_to_bf16_bits(a) -> np.ndarray:
    """Exactly representable fp32 values -> bf16 bit patterns (truncation is exact here)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    bits = a.view(np.uint32)
    assert np.all(bits & 0xFFFF == 0), "fixture value is not exactly representable in bf16"
    return (bits >> 16).astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint32) << 16).view(np.float32)


def read_golden(name: str) -> dict:
    out: dict = {}
    for line in (GOLDEN / name).read_text().splitlines():
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        key, *vals = line.split()
        out.setdefault(key, []).append(vals)
    return out


def rng_bf16(rng: np.random.Generator, shape, scale=1.0, dist="normal") -> np.ndarray:
    if dist == "normal":
        v = rng.standard_normal(shape, dtype=np.float32) * np.float32(scale)
    else:
        v = rng.laplace(0.0, scale / math.sqrt(2.0), size=shape).astype(np.float32)
    # round-to-nearest-even to bf16 done in integer arithmetic (input prep only)
    bits = v.view(np.uint32).astype(np.uint64)
    bits = (bits + 0x7FFF + ((bits >> 16) & 1)) >> 16
    return bits.astype(np.uint16)


# -------------------------------------------------------------------- pins

def pin_bf16_conversions(orc):
    """bf16<->fp32 conversions against the IEEE definition / torch's rounding."""
    import torch
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    widened = np.array([orc.lib.orc_bf16_to_f32(int(b)) for b in allbits[::257]], dtype=np.float32)
    ref = bf16_bits_to_f32(allbits[::257])
    assert np.array_equal(widened.view(np.uint32), ref.view(np.uint32))
    rng = np.random.default_rng(7)
    vals = np.concatenate([
        rng.standard_normal(3000).astype(np.float32) * np.float32(1e3),
        # exact ties: low 16 bits 0x8000, both parities of the kept lsb
        (np.array([0x3F808000, 0x3F818000, 0xBF808000, 0x7F7F8000, 0x00018000, 0x7F7FFFFF],
                  dtype=np.uint32)).view(np.float32),
        np.array([0.0, -0.0, np.inf, -np.inf, 1e-40, -3e-39], dtype=np.float32),
    ])
    mine = orc.bf16_from_f32(vals)
    theirs = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, theirs)
    nan = orc.bf16_from_f32(np.array([np.nan], dtype=np.float32))[0]
    assert (nan & 0x7F80) == 0x7F80 and (nan & 0x7F) != 0


def pin_f16_widening(orc):
    """IEEE binary16 -> fp32 against numpy's float16 (a library routine): every
    one of the 65536 bit patterns, incl. subnormals, zeros of both signs,
    infinities and NaNs; and fp16 activations through the W1.58A16 reference
    equal the same values given as fp32."""
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    mine = np.array([orc.lib.orc_f16_to_f32(int(b)) for b in allbits], dtype=np.float32)
    ref = allbits.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan].view(np.uint32), ref[~nan].view(np.uint32))
    rng = np.random.default_rng(61)
    x16 = (rng.standard_normal((2, 48)) * 3).astype(np.float16)
    t = rng.integers(-1, 2, size=(5, 48)).astype(np.int8)
    ws = rng.random(5).astype(np.float32)
    y16, m16 = orc.linear_a16(x16, t, ws)
    y32, m32 = orc.linear_a16(x16.astype(np.float32), t, ws)
    assert np.array_equal(y16, y32) and np.array_equal(m16, m32)


def pin_weight_ties_golden(orc):
    g = read_golden("weight_ties.txt")
    N, K = int(g["N"][0][0]), int(g["K"][0][0])
    W = f32_to_bf16_bits(np.array(g["W"], dtype=np.float32).reshape(N, K))
    T = np.array(g["T"], dtype=np.int8).reshape(N, K)
    t, w_scale, seg_mean, zeros = orc.weight_quant(W)
    assert seg_mean[0] == np.float32(g["mean"][0][0])
    assert np.all(w_scale == seg_mean[0])
    assert np.array_equal(t, T)
    assert zeros[0] == np.count_nonzero(T == 0)


def pin_act_ties_golden(orc):
    g = read_golden("act_ties.txt")
    K = int(g["K"][0][0])
    x = f32_to_bf16_bits(np.array(g["X"][0], dtype=np.float32).reshape(1, K))
    q, a_scale, rowsum = orc.act_quant(x)
    expect = np.array(g["Q"][0], dtype=np.int8)
    assert q.shape == (1, orc.padded_k(K))
    assert np.array_equal(q[0, :K], expect)
    assert not q[0, K:].any()
    assert a_scale[0] == np.float32(g["a_scale"][0][0])
    assert rowsum[0] == int(g["q_rowsum"][0][0])


def pin_pack_golden(orc):
    g = read_golden("pack_v1.txt")
    K = int(g["K"][0][0])
    t = np.array(g["T"][0], dtype=np.int8).reshape(1, K)
    expect = np.array([int(b, 16) for b in g["BYTES"][0]], dtype=np.uint8)
    packed = orc.pack(t)
    assert packed.shape == (1, expect.size)
    assert np.array_equal(packed[0], expect)
    back, bad = orc.unpack(packed, K)
    assert bad == 0 and np.array_equal(back, t)


def pin_pack_roundtrip_and_padding(orc):
    rng = np.random.default_rng(11)
    for K in (16, 48, 128, 144, 1152, 4304):
        t = rng.integers(-1, 2, size=(5, K), dtype=np.int8)
        packed = orc.pack(t)
        Kp = -(-K // 128) * 128
        assert packed.shape == (5, Kp // 4)
        back, bad = orc.unpack(packed, K)
        assert bad == 0 and np.array_equal(back, t)
        # every 2-bit field at k >= K holds 1, and no field anywhere holds 3
        fields = np.stack([(packed >> s) & 3 for s in (0, 2, 4, 6)], -1)
        assert not np.any(fields == 3)
        # the number of fields equal to u in the whole row = count(t+1 == u) + padding
        for u in (0, 1, 2):
            want = np.count_nonzero(t + 1 == u, axis=1) + (Kp - K) * (u == 1)
            assert np.array_equal(np.count_nonzero(fields == u, axis=(1, 2)), want)


def pin_codes_invariant_and_zero_fraction(orc):
    """Codes lie in {-1,0,1}; zero fraction matches the closed forms."""
    rng = np.random.default_rng(3)
    N, K = 512, 2048
    for dist, p0 in (("normal", math.erf(0.5 * math.sqrt(2 / math.pi) / math.sqrt(2))),
                     ("laplace", 1 - math.exp(-0.5))):
        W = rng_bf16(rng, (N, K), 0.02, dist)
        t, _, _, zeros = orc.weight_quant(W)
        assert set(np.unique(t).tolist()) <= {-1, 0, 1}
        frac = zeros[0] / (N * K)
        sigma = math.sqrt(p0 * (1 - p0) / (N * K))
        assert abs(frac - p0) < 5 * sigma, (dist, frac, p0)
        assert zeros[0] == np.count_nonzero(t == 0)


def pin_max_maps_to_127(orc):
    """Every token's max-|x| element maps to +-127 with its sign; |q| <= 127."""
    rng = np.random.default_rng(5)
    M, K = 256, 512
    mag = np.exp(rng.uniform(-30, 30, size=(M, 1))).astype(np.float32)
    x = rng_bf16_from(rng.standard_normal((M, K)).astype(np.float32) * mag)
    q, a_scale, _ = orc.act_quant(x)
    xv = bf16_bits_to_f32(x)
    idx = np.argmax(np.abs(xv), axis=1)
    top = q[np.arange(M), idx]
    assert np.array_equal(top, np.where(xv[np.arange(M), idx] > 0, 127, -127).astype(np.int8))
    assert np.abs(q.astype(np.int32)).max() <= 127


def rng_bf16_from(v: np.ndarray) -> np.ndarray:
    bits = np.ascontiguousarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    bits = (bits + 0x7FFF + ((bits >> 16) & 1)) >> 16
    return bits.astype(np.uint16)


def pin_permutation_weights(orc):
    """W = a permutation matrix P (non-symmetric): codes = P, acc[m, n] = q[m, pi(n)],
    y = acc * (amax/127) * (1/K) -- a closed form, every step exact for K a power of 2."""
    rng = np.random.default_rng(9)
    K = 64
    perm = rng.permutation(K)
    Wf = np.zeros((K, K), dtype=np.float32)
    Wf[np.arange(K), perm] = 1.0
    W = f32_to_bf16_bits(Wf)
    t, w_scale, seg_mean, _ = orc.weight_quant(W)
    assert seg_mean[0] == np.float32(1.0 / K)
    assert np.array_equal(t, Wf.astype(np.int8))
    x = rng_bf16(rng, (3, K))
    q, a_scale, _ = orc.act_quant(x)
    acc = orc.int_dot(q, t)
    assert np.array_equal(acc, q[:, perm].astype(np.int32))
    y = orc.epilogue(acc, a_scale, w_scale)
    amax = np.abs(bf16_bits_to_f32(x)).max(axis=1)
    want = acc.astype(np.float64) * (amax.astype(np.float32) / np.float32(127)).astype(np.float64)[:, None] / K
    assert np.array_equal(y, want.astype(np.float32))


def pin_constant_weights(orc):
    """W = +c everywhere: codes all +1 and acc = q_rowsum; W = -c gives -q_rowsum."""
    rng = np.random.default_rng(13)
    K, N = 96, 5
    x = rng_bf16(rng, (4, K))
    q, _, rowsum = orc.act_quant(x)
    for sign in (1.0, -1.0):
        W = f32_to_bf16_bits(np.full((N, K), sign * 0.375, dtype=np.float32))
        t, w_scale, _, _ = orc.weight_quant(W)
        assert np.all(t == int(sign)) and np.all(w_scale == np.float32(0.375))
        acc = orc.int_dot(q, t)
        assert np.array_equal(acc, np.repeat((sign * rowsum).astype(np.int32)[:, None], N, 1))
    assert np.array_equal(rowsum, q.astype(np.int64).sum(1).astype(np.int32))


def pin_symmetry_and_pow2_scaling(orc):
    rng = np.random.default_rng(17)
    x = rng_bf16(rng, (8, 160))
    W = rng_bf16(rng, (24, 160), 0.02)
    q, a, r = orc.act_quant(x)
    qn, an, rn = orc.act_quant(x ^ np.uint16(0x8000))          # -x
    assert np.array_equal(qn, -q) and np.array_equal(an, a) and np.array_equal(rn, -r)
    t, ws, _, _ = orc.weight_quant(W)
    tn, wsn, _, _ = orc.weight_quant(W ^ np.uint16(0x8000))      # -W
    assert np.array_equal(tn, -t) and np.array_equal(wsn, ws)
    for j in (-3, 4):                                            # x * 2^j, W * 2^j
        xs = f32_to_bf16_bits(bf16_bits_to_f32(x) * np.float32(2.0 ** j))
        qs, as_, _ = orc.act_quant(xs)
        assert np.array_equal(qs, q) and np.array_equal(as_, a * np.float32(2.0 ** j))
        Ws = f32_to_bf16_bits(bf16_bits_to_f32(W) * np.float32(2.0 ** j))
        ts, wss, _, _ = orc.weight_quant(Ws)
        assert np.array_equal(ts, t) and np.array_equal(wss, ws * np.float32(2.0 ** j))


def pin_zero_token_and_zero_tensor(orc):
    K = 32
    x = np.zeros((2, K), dtype=np.uint16)
    x[1, 5] = f32_to_bf16_bits(np.array([3.0], dtype=np.float32))[0]
    q, a, r = orc.act_quant(x)
    assert not q[0].any() and a[0] == 0 and r[0] == 0
    assert q[1, 5] == 127 and np.count_nonzero(q[1]) == 1 and a[1] == np.float32(3.0) / np.float32(127)
    W = np.zeros((3, K), dtype=np.uint16)
    t, ws, mean, zeros = orc.weight_quant(W)
    assert not t.any() and not ws.any() and mean[0] == 0 and zeros[0] == 3 * K
    y = orc.epilogue(orc.int_dot(q, t), a, ws)
    assert np.array_equal(y, np.zeros((2, 3), dtype=np.float32))  # +0 and -0 both compare equal
    # R5 at the edge of fp32: amax = 2^-122 makes 127/amax overflow, so the token
    # is a zero token; at amax = 2^-121 the scale 127 * 2^121 is still finite and
    # the token quantises normally (-2^-122 * 127 * 2^121 = -63.5, a tie -> -64)
    tiny = np.zeros((2, K), dtype=np.uint16)
    tiny[0, [3, 9]] = f32_to_bf16_bits(np.array([2.0 ** -122, -2.0 ** -123], dtype=np.float32))
    tiny[1, [3, 9]] = f32_to_bf16_bits(np.array([2.0 ** -121, -2.0 ** -122], dtype=np.float32))
    q, a, r = orc.act_quant(tiny)
    assert not q[0].any() and a[0] == 0 and r[0] == 0
    assert q[1, 3] == 127 and q[1, 9] == -64 and np.count_nonzero(q[1]) == 2 and r[1] == 63
    assert a[1] == np.float32(2.0 ** -121) / np.float32(127)
    g = f32_to_bf16_bits(np.ones(K, dtype=np.float32))
    qn, an, rn = orc.rms_act_quant(tiny, g, 0.0)
    assert not qn[0].any() and an[0] == 0 and rn[0] == 0
    assert np.array_equal(qn[1], q[1]) and an[1] > 0


def pin_int_dot_bruteforce(orc):
    """Integer dot equals numpy int64 matmul (a library primitive) on several shapes."""
    rng = np.random.default_rng(19)
    for M, N, K in ((1, 1, 16), (3, 7, 48), (9, 33, 144), (2, 65, 1152)):
        Kp = -(-K // 128) * 128
        q = np.zeros((M, Kp), dtype=np.int8)
        q[:, :K] = rng.integers(-127, 128, size=(M, K))
        t = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
        acc = orc.int_dot(q, t)
        want = q[:, :K].astype(np.int64) @ t.astype(np.int64).T
        assert np.array_equal(acc, want.astype(np.int32))
        mi = rng.integers(0, M, 20)
        ni = rng.integers(0, N, 20)
        assert np.array_equal(orc.int_dot_pairs(q, t, mi, ni), want[mi, ni].astype(np.int32))
    q = np.full((1, 6912), 127, dtype=np.int8)                 # largest K of the workloads:
    t = np.ones((1, 6912), dtype=np.int8)                     # 127 * K fits in int32
    assert orc.int_dot(q, t)[0, 0] == 127 * 6912


def pin_segments(orc):
    """A fused tensor keeps one scale per source tensor, on the right rows."""
    rng = np.random.default_rng(23)
    K = 256
    A = rng_bf16(rng, (40, K), 0.02)
    B = rng_bf16(rng, (24, K), 0.2)
    C = rng_bf16(rng, (8, K), 0.002)
    fused = np.concatenate([A, B, C], 0)
    t, ws, means, zeros = orc.weight_quant(fused, [40, 24, 8])
    for part, rows, sl, sigma in ((A, 40, slice(0, 40), 0.02), (B, 24, slice(40, 64), 0.2),
                                  (C, 8, slice(64, 72), 0.002)):
        tp, wsp, mp, zp = orc.weight_quant(part)
        assert np.array_equal(t[sl], tp) and np.all(ws[sl] == mp[0])
        assert abs(mp[0] / (sigma * math.sqrt(2 / math.pi)) - 1) < 0.1
    assert np.array_equal(means, [ws[0], ws[40], ws[64]])
    t1, ws1, _, _ = orc.weight_quant(fused)                      # one scale for all: differs
    assert not np.array_equal(t1, t)


def pin_float_linear_tiny(orc):
    """y against an independent fp64 brute force of linear(ActQuant(x), WeightQuant(W))."""
    rng = np.random.default_rng(29)
    for M, N, K in ((1, 1, 16), (2, 3, 32), (3, 5, 48), (8, 16, 128), (3, 33, 144)):
        x = rng_bf16(rng, (M, K))
        W = rng_bf16(rng, (N, K), 0.02)
        res = orc.linear(x, W)
        yref, bound, q_b, t_b = brute.linear(bf16_bits_to_f32(x), bf16_bits_to_f32(W))
        assert np.array_equal(res["q"][:, :K], q_b)
        assert np.array_equal(res["t"], t_b)
        err = np.abs(res["y"].astype(np.float64) - yref)
        assert np.all(err <= bound), (M, N, K, float(err.max()))
        bf = orc.epilogue(res["acc"], res["a_scale"], res["w_scale"], "bf16")
        assert np.array_equal(bf, orc.bf16_from_f32(res["y"]))


def pin_act_quant_exact_rational(orc):
    """q against the exact value of the fp32 formula: sa = fl(127/amax) by numpy's
    correctly rounded fp32 division; x*sa is exact in fp64, rounded once to fp32."""
    rng = np.random.default_rng(31)
    x = rng_bf16(rng, (64, 256))
    xv = bf16_bits_to_f32(x)
    q, a, r = orc.act_quant(x)
    amax = np.abs(xv).max(1)
    sa = np.float32(127) / amax
    prod = (xv.astype(np.float64) * sa.astype(np.float64)[:, None]).astype(np.float32)
    want = np.clip(np.rint(prod), -128, 127).astype(np.int8)
    assert np.array_equal(q[:, :256], want)
    assert np.array_equal(a, amax / np.float32(127))
    assert np.array_equal(r, want.astype(np.int64).sum(1).astype(np.int32))


# ------------------------------------------- RMSNorm -> ActQuant, SwiGLU

def _rms_literal(xv: np.ndarray, gv: np.ndarray, eps: float):
    """The composition written out in fp64, straight from the page's pipeline
    (x -> RMSNorm(x, g) -> ActQuant): the normalised vector y, its codes before
    rounding v = y*127/max|y|, and amax(y)/127."""
    x64, g64 = xv.astype(np.float64), gv.astype(np.float64)
    ms = np.array([math.fsum(row) for row in x64 * x64]) / xv.shape[1]
    y = x64 * g64[None, :] / np.sqrt(ms + eps)[:, None]
    amax = np.abs(y).max(1)
    v = y * (127.0 / np.where(amax > 0, amax, 1.0))[:, None]
    return y, v, amax / 127.0


def pin_rms_constant_token(orc):
    """x = c on every k, g = 1: every code is +-127 and a_scale = |c| / sqrt(c^2 + eps) / 127
    (closed form, evaluated with Python's decimal module)."""
    from decimal import Decimal, getcontext
    getcontext().prec = 50
    K, eps = 256, 1e-6
    for c in (0.75, -3.5, 0.001953125, 40.0):
        x = f32_to_bf16_bits(np.full((1, K), c, dtype=np.float32))
        g = f32_to_bf16_bits(np.ones(K, dtype=np.float32))
        q, a, r = orc.rms_act_quant(x, g, eps)
        sign = 1 if c > 0 else -1
        assert np.all(q[0, :K] == 127 * sign) and np.all(q[0, K:] == 0)
        assert r[0] == 127 * K * sign
        dc, de = Decimal(abs(c)), Decimal(np.float32(eps).item())
        want = float(dc / (dc * dc + de).sqrt() / Decimal(127))
        assert abs(float(a[0]) - want) <= 2 * np.spacing(np.float32(want)), (c, float(a[0]), want)


def pin_rms_matches_literal_composition(orc):
    """Codes equal the fp64 composition RMSNorm then ActQuant wherever the value
    before rounding is not within 2e-5 of a .5 tie (the fp32 product decides those),
    and a_scale equals amax(y)/127 to 2 fp32 ulps."""
    rng = np.random.default_rng(41)
    M, K, eps = 24, 384, 1e-6
    x = rng_bf16(rng, (M, K))
    x[3] = rng_bf16(rng, (1, K), scale=1e-4)          # eps matters for this token
    x[5, 17] = f32_to_bf16_bits(np.array([60.0], dtype=np.float32))[0]   # an outlier
    g = rng_bf16(rng, (K,), scale=0.2)
    gv = bf16_bits_to_f32(g) + np.float32(1.0)
    g = f32_to_bf16_bits(bf16_bits_to_f32(rng_bf16_from(gv)))
    xv, gv = bf16_bits_to_f32(x), bf16_bits_to_f32(g)
    q, a, rs = orc.rms_act_quant(x, g, eps)
    _, v, a_lit = _rms_literal(xv, gv, np.float64(np.float32(eps)))
    clear = np.abs(np.abs(v - np.trunc(v)) - 0.5) > 2e-5
    want = np.clip(np.rint(v), -128, 127)
    assert clear.mean() > 0.99
    assert np.array_equal(q[:, :K][clear], want[clear].astype(np.int8))
    assert np.all(np.abs(a.astype(np.float64) - a_lit) <= 2 * np.spacing(a))
    assert np.array_equal(rs, q.astype(np.int64).sum(1).astype(np.int32))


def pin_rms_eps_and_zero_weight(orc):
    """A token far below sqrt(eps) is scaled by about 1/sqrt(eps); a zero norm
    weight gives zero codes and a zero scale; eps = 0 with power-of-two scaling
    of x leaves codes and a_scale unchanged."""
    rng = np.random.default_rng(43)
    K = 128
    x = rng_bf16(rng, (1, K), scale=1e-6)
    g = f32_to_bf16_bits(np.ones(K, dtype=np.float32))
    q, a, _ = orc.rms_act_quant(x, g, 1e-6)
    xv = bf16_bits_to_f32(x).astype(np.float64)
    ms = math.fsum(xv[0] ** 2) / K
    want = np.abs(xv).max() / math.sqrt(ms + float(np.float32(1e-6))) / 127
    assert abs(float(a[0]) - want) <= 2 * np.spacing(np.float32(want))
    q0, a0, r0 = orc.rms_act_quant(rng_bf16(rng, (2, K)), np.zeros(K, dtype=np.float32), 1e-6)
    assert not q0.any() and not a0.any() and not r0.any()
    x = rng_bf16(rng, (3, K))
    base = orc.rms_act_quant(x, g, 0.0)
    for j in (-3, 5):
        xs = f32_to_bf16_bits(bf16_bits_to_f32(x) * np.float32(2.0 ** j))
        got = orc.rms_act_quant(xs, g, 0.0)
        assert np.array_equal(got[0], base[0]) and np.array_equal(got[1], base[1])


def pin_swiglu_decimal(orc):
    """silu(a)*u against Python's decimal module (50 digits): the oracle evaluates
    the definition in fp64 and rounds once (R14), so every result is the correctly
    rounded fp32 value up to the fp64 error (half an fp32 ulp plus 2^-40 relative);
    exact for silu(0) = 0, u = 0 and silu(60) = 60, and the tiny value of silu(-100)
    (about -3.7e-42, an fp32 subnormal) comes out right too."""
    from decimal import Decimal, getcontext
    getcontext().prec = 50
    rng = np.random.default_rng(47)
    a = rng_bf16(rng, (4, 48), scale=3.0)
    u = rng_bf16(rng, (4, 48))
    a[0, :5] = f32_to_bf16_bits(np.array([0.0, -0.0, 60.0, -60.0, -100.0], dtype=np.float32))
    u[0, 4] = f32_to_bf16_bits(np.array([1.0], dtype=np.float32))[0]
    u[1, :3] = 0
    h = orc.swiglu(a, u)
    av, uv = bf16_bits_to_f32(a), bf16_bits_to_f32(u)
    for i in range(av.shape[0]):
        for k in range(av.shape[1]):
            da, du = Decimal(float(av[i, k])), Decimal(float(uv[i, k]))
            exact = da / (1 + (-da).exp()) * du
            if exact == 0:
                assert h[i, k] == 0, (i, k)
                continue
            half_ulp = Decimal(float(np.spacing(np.float32(abs(float(exact)))))) / 2
            slack = abs(exact) * Decimal(2) ** -40
            assert abs(Decimal(float(h[i, k])) - exact) <= half_ulp + slack, (i, k, float(h[i, k]), float(exact))
    assert h[0, 0] == 0 and h[0, 1] == 0 and np.all(h[1, :3] == 0)
    assert h[0, 2] == np.float32(60.0) * uv[0, 2]
    assert h[0, 4] < 0 and abs(float(h[0, 4]) + 3.72e-42) < 2e-44


def _exact_abs_ints(W: np.ndarray):
    """|W| of bf16 bit patterns as exact integers: a bf16 value is an 8-bit
    integer significand times a power of two, so |W| = ints * 2**scale_exp with
    every significand shifted to the smallest exponent present (int64, asserted
    to leave room for sums of up to 2^14 values)."""
    bits = W.astype(np.int64) & 0x7FFF
    e = bits >> 7
    mant = np.where(e > 0, (bits & 0x7F) | 0x80, bits & 0x7F)
    e_eff = np.where(e > 0, e, 1)
    nz = mant != 0
    emin = int(e_eff[nz].min()) if nz.any() else 1
    assert int(e_eff.max()) - emin <= 40, "exponent spread too wide for exact int64 sums"
    return mant << (e_eff - emin), emin - 127 - 7


def pin_segment_mean_exact(orc):
    """R2 on the c5 prefill tensors (seeded generators, full size): every segment
    mean equals fp32(S / (rows * K)) where S is the exact sum of |W| rounded once
    to fp64 (integer arithmetic, Python's correctly rounded int -> float), and the
    oracle's fp64 row sums are the exact row sums -- the fused 13824 x 2560
    gate|up (two 6912-row segments), the 6912 x 2560 gate segment on its own and
    the 2560 x 6912 down projection.  For bf16 weights of this magnitude the
    fixed-order fp64 sum makes no rounding at all, so this is the correctly
    rounded mean; an fp32 row sum or segment total moves it by several ulps."""
    import torch
    wl = _workloads()
    w = wl.WORKLOADS["c5"]

    def bits_of(t):
        return t.contiguous().view(torch.int16).numpy().view(np.uint16)

    gu, dn = bits_of(wl.weight_for(w, 0)), bits_of(wl.weight_for(w, 1))
    exact = {}
    for key, W in (("gate", gu[:6912]), ("up", gu[6912:]), ("down", dn)):
        W = np.ascontiguousarray(W)
        ints, sexp = _exact_abs_ints(W)
        rows = ints.sum(axis=1)                              # < 2^62: exact in int64
        total = sum(int(r) for r in rows)                    # Python int: exact
        exact[key] = np.float32(math.ldexp(float(total), sexp) / W.size)
        for n in (0, 1, W.shape[0] // 2, W.shape[0] - 1):
            got = orc.lib.orc_row_abs_sum(W.ctypes.data, 1, n, W.shape[1], W.shape[1])
            assert got == math.ldexp(float(int(rows[n])), sexp), (key, n)
    _, w_scale, seg_mean, _ = orc.weight_quant(gu, [6912, 6912])
    assert seg_mean[0] == exact["gate"] and seg_mean[1] == exact["up"], (seg_mean, exact)
    assert np.all(w_scale[:6912] == exact["gate"]) and np.all(w_scale[6912:] == exact["up"])
    _, _, seg_mean, _ = orc.weight_quant(np.ascontiguousarray(gu[:6912]))
    assert seg_mean[0] == exact["gate"]
    _, w_scale, seg_mean, _ = orc.weight_quant(dn)
    assert seg_mean[0] == exact["down"] and np.all(w_scale == exact["down"])


def _exact_block_abs_sums(W: np.ndarray, K: int) -> np.ndarray:
    """sum of |W| over each 256-weight block of each row, exactly (integer sums
    of _exact_abs_ints; each below 2^53, so exact in fp64)."""
    ints, sexp = _exact_abs_ints(W)
    nb = -(-K // 256)
    out = np.empty((W.shape[0], nb), dtype=np.float64)
    for b in range(nb):
        s_ = ints[:, 256 * b:min(256 * b + 256, K)].sum(axis=1)
        assert s_.max() < 2 ** 53
        out[:, b] = np.ldexp(s_.astype(np.float64), sexp)
    return out


def pin_block_scales_exact(orc):
    """R18 on a full-size 2560 x 6912 tensor (27 blocks, all full) and a
    300 x 1152 one (last block partial, 128 weights): every block scale equals
    fp32(exact block sum of |W| / block count), the block sums being computed
    exactly in integer arithmetic.  An fp32 block sum misses by ulps."""
    rng = np.random.default_rng(83)
    for N, K in ((2560, 6912), (300, 1152)):
        W = rng_bf16(rng, (N, K), 0.02)
        _, bs = orc.weight_quant_blocked(W)
        sums = _exact_block_abs_sums(W, K)
        counts = np.array([min(256, K - 256 * b) for b in range(sums.shape[1])], dtype=np.float64)
        want = (sums / counts[None, :]).astype(np.float32).T
        assert np.array_equal(bs, want), (N, K, int(np.count_nonzero(bs != want)))


def pin_blocked_order_fp32(orc):
    """R19 fixes how the block terms are combined: fp32, total = total +
    fp32(acc_b) * scale_b for b ascending, then one product with a_scale.  The
    exact block sums come from numpy's int64 matrix product (a library routine),
    the fp32 evaluation from numpy's IEEE single-precision operations, one
    rounding per operation; the oracle's y must agree bit for bit at K = 6912
    (27 blocks) and K = 1152 (partial last block).  Reordering the blocks or
    accumulating in fp64 changes last bits."""
    rng = np.random.default_rng(89)
    for M, N, K in ((6, 200, 6912), (4, 96, 1152)):
        W = rng_bf16(rng, (N, K), 0.02)
        x = rng_bf16(rng, (M, K))
        t, bs = orc.weight_quant_blocked(W)
        q, a_scale, _ = orc.act_quant(x)
        y, _ = orc.linear_blocked_q(q, a_scale, t, bs)
        nb = bs.shape[0]
        total = np.zeros((M, N), dtype=np.float32)
        for b in range(nb):
            sl = slice(256 * b, min(256 * b + 256, K))
            acc_b = q[:, sl].astype(np.int64) @ t[:, sl].astype(np.int64).T
            term = acc_b.astype(np.float32) * bs[b][None, :]
            total = (total + term).astype(np.float32)
        want = (total * a_scale[:, None]).astype(np.float32)
        assert np.array_equal(y.view(np.uint32), want.view(np.uint32)), (M, N, K)


# ----------------------------------------------------------------- W1.58A16

def pin_a16_closed_forms_and_matmul(orc):
    """W = permutation P gives y = x[:, pi] * w_scale exactly; constant codes give
    y = (sum_k x) * w_scale; random codes agree with numpy's fp64 matmul to 1e-12
    of sum |x*t| (a library routine on a special case); mag is that sum."""
    rng = np.random.default_rng(59)
    K = 64
    x = rng_bf16(rng, (3, K))
    xv = bf16_bits_to_f32(x).astype(np.float64)
    perm = rng.permutation(K)
    t = np.zeros((K, K), dtype=np.int8)
    t[np.arange(K), perm] = 1
    ws = np.full(K, 0.375, dtype=np.float32)
    y, mag = orc.linear_a16(x, t, ws)
    assert np.array_equal(y, xv[:, perm] * 0.375)
    tc = -np.ones((5, K), dtype=np.int8)
    y, _ = orc.linear_a16(x, tc, np.ones(5, dtype=np.float32))
    assert np.allclose(y, -xv.sum(1)[:, None], rtol=0, atol=1e-12)
    t = rng.integers(-1, 2, size=(40, K)).astype(np.int8)
    ws = rng.random(40).astype(np.float32)
    y, mag = orc.linear_a16(x, t, ws)
    want = (xv @ t.T.astype(np.float64)) * ws.astype(np.float64)
    absum = np.abs(xv) @ np.abs(t.T.astype(np.float64))
    assert np.all(np.abs(y - want) <= 1e-12 * absum * ws + 1e-300)
    assert np.allclose(mag, absum, rtol=1e-15, atol=0)


# --------------------------------------------------------------------- I2_S

def pin_i2s_golden(orc):
    """One block worked by hand from the page's byte formula, both readings of
    which values share a byte (tests/golden/i2s_block.txt)."""
    g = read_golden("i2s_block.txt")
    t = np.array([int(v) for v in g["T"][0]], dtype=np.int8).reshape(1, 128)
    scale = float(g["SCALE"][0][0])
    for order, key in (("strided", "STRIDED"), ("consecutive", "CONSECUTIVE")):
        want = np.array([int(b, 16) for b in g[key][0]], dtype=np.uint8)
        got = orc.i2s_pack(t, scale, order)
        assert np.array_equal(got, want), order
        t2, s2, bad = orc.i2s_unpack(want, 1, 128, order)
        assert np.array_equal(t2, t) and s2 == np.float32(scale) and bad == 0


def pin_i2s_roundtrip_and_blocks(orc):
    """unpack(pack(t)) = t with blocks that cross rows (K = 48); each 32-byte block
    holds the same multiset of codes under both readings (they only permute
    values inside a block); codes of other blocks do not move; fields never hold 3."""
    rng = np.random.default_rng(53)
    N, K = 16, 48
    t = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
    for order in ("strided", "consecutive"):
        buf = orc.i2s_pack(t, 0.25, order)
        t2, s2, bad = orc.i2s_unpack(buf, N, K, order)
        assert np.array_equal(t2, t) and s2 == np.float32(0.25) and bad == 0
        fields = np.stack([(buf[:-4] >> sh) & 3 for sh in (6, 4, 2, 0)], 1)
        assert fields.max() <= 2
    a, b = orc.i2s_pack(t, 1.0, "strided"), orc.i2s_pack(t, 1.0, "consecutive")
    flat = t.reshape(-1)
    for blk in range(flat.size // 128):
        def counts(buf):
            f = np.stack([(buf[32 * blk:32 * blk + 32] >> sh) & 3 for sh in (6, 4, 2, 0)], 1).reshape(-1)
            return np.bincount(f, minlength=3)
        want = np.bincount(flat[128 * blk:128 * blk + 128] + 1, minlength=3)
        assert np.array_equal(counts(a), want) and np.array_equal(counts(b), want)
    t3 = t.copy()
    t3.reshape(-1)[200] = -t3.reshape(-1)[200] if t3.reshape(-1)[200] else 1
    d = np.nonzero(orc.i2s_pack(t3, 1.0, "strided") != a)[0]
    assert d.size == 1 and d[0] // 32 == 200 // 128


# ------------------------------------------- per-block weight scales (R15, R16)

def _blocked_fp32_bound(acc_blocks, bs, a_scale):
    """Exact value a_scale * sum_b acc_b * bs_b (fp64 of exact products) and a
    bound on the sequential fp32 evaluation: every product and partial sum
    rounds once (2**-24 relative each), then one product with a_scale."""
    M, nb, N = acc_blocks.shape
    terms = acc_blocks.astype(np.float64) * bs.astype(np.float64)[None, :, :]
    exact = terms.sum(axis=1) * a_scale.astype(np.float64)[:, None]
    mag = np.abs(terms).sum(axis=1) * a_scale.astype(np.float64)[:, None]
    return exact, (nb + 2) * 2.0 ** -24 * mag + 1e-30


def pin_blocked_closed_form(orc):
    """Blocks of constant magnitude c[n][b] with a sign pattern and 10% zeros:
    each block's absmean is c * nonzeros / count (the last block of K = 1152
    holds 128 weights), every nonzero weight maps to its sign, and y equals
    a_scale * sum_b c-scaled integer block sums within the fp32 bound."""
    rng = np.random.default_rng(71)
    N, K = 6, 1152
    nb = orc.block_count(K)
    assert nb == 5
    sigma = rng.choice(np.array([-1, 1], dtype=np.int8), size=(N, K))
    sigma[rng.random((N, K)) < 0.1] = 0
    c = (2.0 ** rng.integers(-9, -3, size=(N, nb))) * rng.choice([1.0, 1.5, 1.25], size=(N, nb))
    W32 = np.zeros((N, K), dtype=np.float32)
    for b in range(nb):
        W32[:, 256 * b:256 * b + 256] = c[:, b:b + 1] * sigma[:, 256 * b:256 * b + 256]
    W = f32_to_bf16_bits(W32)
    t, bs = orc.weight_quant_blocked(W)
    assert np.array_equal(t, sigma)
    for n in range(N):
        for b in range(nb):
            blk = sigma[n, 256 * b:256 * b + 256]
            assert bs[b, n] == np.float32(c[n, b] * np.count_nonzero(blk) / blk.size)
    x = rng_bf16(rng, (3, K))
    q, a_scale, _ = orc.act_quant(x)
    y, accb = orc.linear_blocked_q(q, a_scale, t, bs)
    want = np.stack([(q[:, 256 * b:min(256 * b + 256, K)].astype(np.int64)
                      @ sigma[:, 256 * b:min(256 * b + 256, K)].astype(np.int64).T) for b in range(nb)], axis=1)
    assert np.array_equal(accb, want)
    exact, bound = _blocked_fp32_bound(want, bs, a_scale)
    assert np.all(np.abs(y.astype(np.float64) - exact) <= bound)


def pin_blocked_reduces_to_tensor(orc):
    """When every block has the tensor's absmean (W = mu * sign), the block codes
    and scales are the per-tensor ones and the block sums add up to the
    per-tensor integer dot exactly."""
    rng = np.random.default_rng(73)
    N, K = 5, 2560
    sign = rng.choice(np.array([-1, 1], dtype=np.int8), size=(N, K))
    W = f32_to_bf16_bits((np.float32(0.046875) * sign).astype(np.float32))
    t_b, bs = orc.weight_quant_blocked(W)
    t, w_scale, _, _ = orc.weight_quant(W)
    assert np.array_equal(t_b, t) and np.all(bs == w_scale[None, :])
    x = rng_bf16(rng, (4, K))
    q, a_scale, _ = orc.act_quant(x)
    y_b, accb = orc.linear_blocked_q(q, a_scale, t_b, bs)
    acc = orc.int_dot(q, t)
    assert np.array_equal(accb.astype(np.int64).sum(axis=1), acc.astype(np.int64))
    y = orc.epilogue(acc, a_scale, w_scale)
    assert np.allclose(y_b, y, rtol=4e-6, atol=0)


def pin_blocked_random_codes_and_float(orc):
    """Random weights with a different spread in every row: codes are the sign
    where |W| >= 1.5 * block mean and 0 where |W| <= 0.5 * block mean (away from
    the two rounding boundaries); y is within the fp32 bound of the exact
    a_scale * sum_k q * t * block_scale (K = 400: blocks of 256 and 144)."""
    rng = np.random.default_rng(79)
    N, K = 7, 400
    W32 = (rng.standard_normal((N, K)) * (0.01 * (1 + np.arange(N)))[:, None]).astype(np.float32)
    W = rng_bf16_from(W32)
    Wf = bf16_bits_to_f32(W).astype(np.float64)
    t, bs = orc.weight_quant_blocked(W)
    assert set(np.unique(t)) <= {-1, 0, 1}
    for b in range(orc.block_count(K)):
        sl = slice(256 * b, min(256 * b + 256, K))
        mean = np.abs(Wf[:, sl]).mean(axis=1)
        assert np.allclose(bs[b], mean, rtol=2 ** -23)
        ratio = np.abs(Wf[:, sl]) / mean[:, None]
        tb = t[:, sl]
        big, small = ratio >= 1.5 * (1 + 1e-6), ratio <= 0.5 * (1 - 1e-6)
        assert np.array_equal(tb[big], np.sign(Wf[:, sl])[big].astype(np.int8))
        assert np.all(tb[small] == 0)
    x = rng_bf16(rng, (3, K))
    q, a_scale, _ = orc.act_quant(x)
    y, accb = orc.linear_blocked_q(q, a_scale, t, bs)
    exact, bound = _blocked_fp32_bound(accb, bs, a_scale)
    qt = np.stack([q[:, 256 * b:min(256 * b + 256, K)].astype(np.int64)
                   @ t[:, 256 * b:min(256 * b + 256, K)].astype(np.int64).T for b in range(2)], axis=1)
    assert np.array_equal(accb, qt)
    assert np.all(np.abs(y.astype(np.float64) - exact) <= bound)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]


def failing_pins(orc) -> list:
    bad = []
    for pin in ALL_PINS:
        try:
            pin(orc)
        except Exception:  # an assertion, or a mutant that breaks a precondition
            bad.append(pin.__name__)
    return bad


if __name__ == "__main__":
    sys.path.insert(0, str(ROOT))
    from oracle.oracle import Oracle

    print(json.dumps(failing_pins(Oracle(sys.argv[1]))))
