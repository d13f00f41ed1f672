"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, rejects bad arguments before launching anything, and its host
packer (BITNET_MEM_HOST) produces the oracle's bytes, scales and counts."""
import ctypes
import re
from pathlib import Path

import numpy as np
import pytest
import torch

import ternary_weight_bitlinear_amd as tw
from ternary_weight_bitlinear_amd import _lib
from ternary_weight_bitlinear_amd import workloads as wl

HEADER = Path(__file__).resolve().parents[1] / "include" / "bitnet.h"


def declared_functions():
    text = re.sub(r"/\*.*?\*/", "", HEADER.read_text(), flags=re.S)
    return sorted(set(re.findall(r"\b(bitnet_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_three_main_calls():
    names = declared_functions()
    for fn in ("bitnet_pack_weights", "bitnet_act_quant", "bitnet_linear_forward"):
        assert fn in names


def test_library_exports_every_declared_symbol():
    handle = ctypes.CDLL(tw.library_path())
    for name in declared_functions():
        assert hasattr(handle, name), name
    assert set(declared_functions()) == set(_lib.SIGNATURES)


def test_sizes_and_strings():
    L = _lib.lib()
    assert L.bitnet_abi_version() == 1
    assert [L.bitnet_padded_k(k) for k in (16, 128, 144, 1152, 4304, 6912)] == [128, 128, 256, 1152, 4352, 6912]
    assert [L.bitnet_padded_k(k) for k in (0, -16, 8, 100, (1 << 20) + 16)] == [-1] * 5
    assert L.bitnet_packed_bytes(3, 4304) == 3 * 4352 // 4
    assert L.bitnet_packed_bytes(0, 16) == -1
    for s in range(5):
        assert L.bitnet_status_string(s)


def test_group_table_and_plan_handle():
    """The table holds one descriptor per item plus a fixed block of share
    bounds; a handle that bitnet_group_plan did not fill names no kernel."""
    L = _lib.lib()
    assert L.bitnet_group_table_bytes(0) == -1
    one, two = L.bitnet_group_table_bytes(1), L.bitnet_group_table_bytes(2)
    per_item = two - one
    assert per_item > 0 and per_item % 8 == 0 and one > per_item
    assert L.bitnet_group_table_bytes(210) == one + 209 * per_item
    assert L.bitnet_group_plan_kernel(ctypes.byref(_lib.GroupPlan())) == b""
    assert L.bitnet_group_plan_kernel(None) == b""


def _status_and_error(fn, *args):
    st = fn(*args)
    return st, _lib.lib().bitnet_last_error().decode()


def test_blocked_sizes_and_limits():
    L = _lib.lib()
    assert [L.bitnet_block_count(k) for k in (16, 256, 272, 1152, 6912, 8192)] == [1, 1, 2, 5, 27, 32]
    assert L.bitnet_block_count(0) == -1 and L.bitnet_block_count(24) == -1
    buf = (ctypes.c_uint8 * 256)()
    p16 = (ctypes.addressof(buf) + 15) // 16 * 16
    assert L.bitnet_linear_blocked_forward(None, p16, p16, 1, 8208, p16, p16, 4, p16, _lib.F32, 4) == \
        _lib.ERR_UNSUPPORTED
    assert b"8192" in L.bitnet_last_error()
    assert L.bitnet_pack_weights_blocked(None, p16, _lib.BF16, 4, 8208, 8208, p16, p16) == _lib.ERR_UNSUPPORTED


def test_argument_errors_launch_nothing():
    """Every call here fails validation on the host, so no HIP call is made."""
    L = _lib.lib()
    buf = (ctypes.c_uint8 * 4096)()
    p = ctypes.addressof(buf)
    p16 = (p + 15) // 16 * 16
    cases = [
        (L.bitnet_act_quant, (None, p16, _lib.BF16, 1, 15, 16, p16, p16, p16), "K=15"),
        (L.bitnet_pack_weights_blocked, (None, p16, _lib.BF16, 4, 24, 24, p16, p16), "K=24"),
        (L.bitnet_pack_weights_blocked, (None, p16, _lib.BF16, 4, 16, 8, p16, p16), "ldw"),
        (L.bitnet_pack_weights_blocked, (None, p16, _lib.BF16, 4, 16, 16, p16 + 4, p16), "aligned"),
        (L.bitnet_pack_weights_blocked, (None, p16, _lib.BF16, 4, 16, 16, p16, None), "NULL"),
        (L.bitnet_pack_weights_blocked, (None, p16, 5, 4, 16, 16, p16, p16), "dtype"),
        (L.bitnet_linear_blocked_forward, (None, p16, p16, 1, 16, p16, p16, 4, p16, _lib.F32, 3), "ldy"),
        (L.bitnet_linear_blocked_forward, (None, p16 + 8, p16, 1, 16, p16, p16, 4, p16, _lib.F32, 4), "aligned"),
        (L.bitnet_linear_blocked_forward, (None, p16, p16, 0, 16, p16, p16, 4, p16, _lib.F32, 4), "M=0"),
        (L.bitnet_linear_blocked_forward, (None, p16, None, 1, 16, p16, p16, 4, p16, _lib.F32, 4), "NULL"),
        (L.bitnet_act_quant, (None, p16, _lib.BF16, 0, 16, 16, p16, p16, p16), "M=0"),
        (L.bitnet_act_quant, (None, p16, _lib.BF16, 1, 16, 8, p16, p16, p16), "ldx"),
        (L.bitnet_act_quant, (None, None, _lib.BF16, 1, 16, 16, p16, p16, p16), "NULL"),
        (L.bitnet_act_quant, (None, p16, 7, 1, 16, 16, p16, p16, p16), "dtype"),
        (L.bitnet_act_quant, (None, p16, _lib.BF16, 1, 16, 16, p16 + 4, p16, p16), "aligned"),
        (L.bitnet_linear_forward, (None, p16, p16, p16, 1, 16, p16, p16, 4, p16, _lib.F32, 3, None), "ldy"),
        (L.bitnet_linear_forward, (None, p16, p16, p16, 1, 16, p16 + 8, p16, 4, p16, _lib.F32, 4, None), "aligned"),
        (L.bitnet_linear_forward, (None, p16, p16, p16, 1, 16, p16, p16, 0, p16, _lib.F32, 4, None), "N=0"),
        (L.bitnet_linear_forward, (None, p16, p16, None, 1, 16, p16, p16, 4, p16, _lib.F32, 4, None), "NULL"),
        (L.bitnet_linear_forward, (None, p16, p16, p16, 1, 16, p16, p16, 4, p16, 5, 4, None), "dtype"),
        (L.bitnet_bitlinear_forward, (None, p16, _lib.BF16, 2, 32, 32, p16, p16, 4, p16, _lib.F32, 2,
                                      p16, p16, p16), "ldy"),
        (L.bitnet_rmsnorm_act_quant, (None, p16, None, _lib.BF16, 1, 16, 16, None, _lib.BF16, 1e-6,
                                      p16, p16, p16), "norm_w is NULL"),
        (L.bitnet_rmsnorm_act_quant, (None, p16, None, _lib.BF16, 1, 16, 16, p16, 3, 1e-6, p16, p16, p16),
         "norm_w dtype"),
        (L.bitnet_rmsnorm_act_quant, (None, p16, None, _lib.BF16, 1, 16, 16, p16, _lib.BF16, -1.0,
                                      p16, p16, p16), "eps"),
        (L.bitnet_rmsnorm_act_quant, (None, p16, None, _lib.BF16, 1, 16, 16, p16, _lib.BF16, float("nan"),
                                      p16, p16, p16), "eps"),
        (L.bitnet_rmsnorm_act_quant, (None, p16, p16 + 1, _lib.BF16, 1, 16, 16, p16, _lib.BF16, 1e-6,
                                      p16, p16, p16), "misaligned up"),
        (L.bitnet_rmsnorm_act_quant, (None, p16, None, _lib.BF16, 1, 20, 20, p16, _lib.BF16, 1e-6,
                                      p16, p16, p16), "K=20"),
        (L.bitnet_pack_weights, (_lib.MEM_HOST, None, p16, _lib.BF16, 4, 16, 16,
                                 (ctypes.c_int64 * 2)(2, 1), 2, p16, p16, None, None), "segment"),
        (L.bitnet_pack_weights, (_lib.MEM_HOST, None, p16, _lib.BF16, 4, 16, 16,
                                 (ctypes.c_int64 * 2)(4, 0), 2, p16, p16, None, None), "segment 1"),
        (L.bitnet_pack_weights, (9, None, p16, _lib.BF16, 4, 16, 16, None, 0, p16, p16, None, None), "memory"),
        (L.bitnet_pack_weights, (_lib.MEM_DEVICE, None, p16, _lib.BF16, 4, 24, 24, None, 0, p16, p16, None,
                                 None), "K=24"),
        (L.bitnet_pack_weights_static, (None, p16, _lib.BF16, 4, 24, 24, None, 0, p16, p16, None, None), "K=24"),
        (L.bitnet_pack_weights_static, (None, p16, _lib.BF16, 4, 16, 8, None, 0, p16, p16, None, None), "ldw"),
        (L.bitnet_pack_weights_static, (None, p16, _lib.BF16, 4, 16, 16, None, 0, p16 + 4, p16, None, None),
         "aligned"),
        (L.bitnet_pack_weights_static, (None, p16, _lib.BF16, 4, 16, 16, (ctypes.c_int64 * 2)(2, 1), 2, p16, p16,
                                        None, None), "segment"),
    ]
    for fn, args, needle in cases:
        st, msg = _status_and_error(fn, *args)
        assert st == _lib.ERR_INVALID_ARG, (fn.__name__, needle, st, msg)
        assert needle in msg, (needle, msg)


def test_static_pack_limits():
    """The allocation-free pack refuses, before any launch, what its fixed
    temporaries cannot hold."""
    L = _lib.lib()
    buf = (ctypes.c_uint8 * 4096)()
    p16 = (ctypes.addressof(buf) + 15) // 16 * 16
    big = _lib.lib().bitnet_pack_weights_static
    st, msg = _status_and_error(big, None, p16, _lib.BF16, 131073, 16, 16, None, 0, p16, p16, None, None)
    assert st == _lib.ERR_UNSUPPORTED and "131072" in msg, msg
    segs = (ctypes.c_int64 * 65)(*([1] * 65))
    st, msg = _status_and_error(L.bitnet_pack_weights_static, None, p16, _lib.BF16, 65, 16, 16, segs, 65, p16, p16,
                                None, None)
    assert st == _lib.ERR_UNSUPPORTED and "segments" in msg, msg


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("N,K,segments,dtype,ldw_extra", [
    (1, 16, None, torch.bfloat16, 0),
    (33, 144, None, torch.bfloat16, 16),
    (64, 1152, (32, 16, 16), torch.bfloat16, 0),
    (17, 4304, None, torch.bfloat16, 0),
    (40, 256, (8, 32), torch.float32, 32),
])
def test_host_packer_matches_oracle(orc, N, K, segments, dtype, ldw_extra):
    base = wl.draw_weight((N, K + ldw_extra), seed=N * 1000 + K, dist="normal")
    if segments:  # very different scales per segment
        scales = torch.cat([torch.full((r, 1), 10.0 ** i) for i, r in enumerate(segments)])
        base = (base.float() * scales).to(torch.bfloat16)
    W = base.to(dtype)[:, :K]          # a strided view when ldw_extra > 0
    pw = tw.pack(W, segments)
    Wn = _bits(W.contiguous()) if dtype == torch.bfloat16 else W.contiguous().numpy()
    t, w_scale, seg_mean, zeros = orc.weight_quant(Wn, segments)
    assert np.array_equal(pw.packed.numpy(), orc.pack(t))
    assert np.array_equal(pw.w_scale.numpy().view(np.uint32), w_scale.view(np.uint32))
    assert np.array_equal(pw.seg_mean.numpy().view(np.uint32), seg_mean.view(np.uint32))
    assert np.array_equal(pw.zero_count.numpy(), zeros)


def test_host_packer_rejects_non_finite():
    W = wl.draw_weight((4, 32), seed=5)
    W[2, 7] = float("inf")
    with pytest.raises(tw.BitnetError) as e:
        tw.pack(W)
    assert e.value.status == _lib.ERR_NONFINITE
    W[2, 7] = float("nan")
    with pytest.raises(tw.BitnetError):
        tw.pack(W)


def test_host_packer_degenerate_tensors(orc):
    W = torch.zeros((3, 48), dtype=torch.bfloat16)
    pw = tw.pack(W)
    assert torch.all(pw.packed == 0x55) and torch.all(pw.w_scale == 0) and pw.zero_count[0] == 3 * 48
    W = torch.full((2, 16), -0.25, dtype=torch.bfloat16)
    pw = tw.pack(W)
    t, _ = orc.unpack(pw.packed.numpy(), 16)
    assert np.all(t == -1)


# ------------------------------------------------------------------ I2_S (host memory)

@pytest.mark.parametrize("N,K", [(1, 128), (24, 48), (40, 2560), (9, 4352)])
@pytest.mark.parametrize("order", ["strided", "consecutive"])
def test_host_i2s_matches_oracle(orc, N, K, order):
    """Export of a host-packed weight equals the oracle's I2_S bytes of the same
    codes and scale; import of those bytes gives back the layout-v1 bytes."""
    W = wl.draw_weight((N, K), seed=N * 3 + K, dist="laplace")
    pw = tw.pack(W)
    t, ws, _, _ = orc.weight_quant(_bits(W))
    buf = tw.i2s_export(pw, order)
    assert np.array_equal(buf.numpy(), orc.i2s_pack(t, np.float32(1) / ws[0], order))
    back = tw.i2s_import(buf, N, K, order)
    assert torch.equal(back.packed, pw.packed)
    assert torch.equal(back.w_scale, torch.full((N,), np.float32(1) / (np.float32(1) / ws[0])))


def test_host_i2s_golden_block():
    """The hand-worked block of tests/golden/i2s_block.txt through the library."""
    import pins
    g = pins.read_golden("i2s_block.txt")
    t = np.array([int(v) for v in g["T"][0]], dtype=np.int8)
    for order, key in (("strided", "STRIDED"), ("consecutive", "CONSECUTIVE")):
        raw = torch.tensor([int(b, 16) for b in g[key][0]], dtype=torch.uint8)
        pw = tw.i2s_import(raw, 1, 128, order)
        assert pw.w_scale.item() == 2.0                     # 1 / 0.5
        fields = torch.stack([(pw.packed[0] >> sh) & 3 for sh in (0, 2, 4, 6)], -1)   # [32 bytes, p]
        k = torch.arange(128)
        got = fields[4 * (k // 16) + k % 4, (k % 16) // 4].to(torch.int8) - 1
        assert np.array_equal(got.numpy(), t)
        assert torch.equal(tw.i2s_export(pw, order), raw)


def test_host_i2s_errors():
    L = _lib.lib()
    assert L.bitnet_i2s_bytes(3, 16) == -1 and L.bitnet_i2s_bytes(8, 16) == 36 and L.bitnet_i2s_bytes(1, 24) == -1
    W = wl.draw_weight((4, 64), seed=1)
    pw = tw.pack(W)
    buf = tw.i2s_export(pw)
    bad = buf.clone()
    bad[5] = 0xFF                                           # fields holding 3
    with pytest.raises(tw.BitnetError, match="holds 3"):
        tw.i2s_import(bad, 4, 64)
    neg = buf.clone()
    neg[-4:] = torch.tensor(np.array([-1.0], dtype=np.float32).view(np.uint8))
    with pytest.raises(tw.BitnetError, match="not positive"):
        tw.i2s_import(neg, 4, 64)
    two = tw.pack(W, (2, 2))                                # two source tensors: two scales
    if two.w_scale[0] != two.w_scale[2]:
        with pytest.raises(tw.BitnetError, match="differs between rows"):
            tw.i2s_export(two)
    st = L.bitnet_i2s_import(_lib.MEM_HOST, None, buf.data_ptr(), 4, 64, 7, pw.packed.data_ptr(),
                             pw.w_scale.data_ptr())
    assert st == _lib.ERR_INVALID_ARG and b"order" in L.bitnet_last_error()


# -------------------------------------------------------------- packed-weight files

def test_packed_file_roundtrip_and_damage(tmp_path):
    W = wl.draw_weight((70, 304), seed=9, dist="laplace")
    pw = tw.pack(W, (30, 40))
    f = tmp_path / "w.btnl"
    tw.save_packed(f, pw, (30, 40))
    raw = f.read_bytes()
    assert raw[:8] == b"BTNLV1\0\0" and len(raw) == 64 + 70 * tw.padded_k(304) // 4 + 70 * 4 + 2 * 8 + 2 * 4
    back, segs = tw.load_packed(f)
    assert segs == [30, 40] and (back.N, back.K) == (70, 304)
    assert torch.equal(back.packed, pw.packed) and torch.equal(back.w_scale, pw.w_scale)
    assert torch.equal(back.seg_mean, pw.seg_mean)
    damaged = bytearray(raw)
    damaged[64 + 100] ^= 0x04                          # one code field changed
    (tmp_path / "d.btnl").write_bytes(bytes(damaged))
    with pytest.raises(tw.BitnetError, match="checksum"):
        tw.load_packed(tmp_path / "d.btnl")
    newer = bytearray(raw)
    newer[8] = 2                                       # version 2
    (tmp_path / "v.btnl").write_bytes(bytes(newer))
    with pytest.raises(tw.BitnetError) as e:
        tw.load_packed(tmp_path / "v.btnl")
    assert e.value.status == _lib.ERR_UNSUPPORTED
    (tmp_path / "t.btnl").write_bytes(raw[:-10])
    with pytest.raises(tw.BitnetError, match="truncated"):
        tw.load_packed(tmp_path / "t.btnl")
    (tmp_path / "m.btnl").write_bytes(b"NOTAFILE" + raw[8:])
    with pytest.raises(tw.BitnetError, match="not a packed-weight file"):
        tw.load_packed(tmp_path / "m.btnl")
    with pytest.raises(ValueError):
        tw.save_packed(f, pw)                          # two segments need two row counts


def _load_raw(path, limit_bytes=1 << 26):
    """bitnet_load_packed through the C ABI with buffers sized exactly from the
    header query (so an over-read or over-write shows under AddressSanitizer)."""
    L = _lib.lib()
    N, K, ns = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int32()
    st = L.bitnet_load_packed(str(path).encode(), ctypes.byref(N), ctypes.byref(K), ctypes.byref(ns),
                              None, None, None, None)
    if st != _lib.OK:
        return st
    N, K, ns = N.value, K.value, ns.value
    kp = L.bitnet_padded_k(K)
    assert N > 0 and kp > 0 and 0 < ns <= N
    if N * kp // 4 + N * 4 > limit_bytes:
        return "too large to load"
    packed = np.empty(N * kp // 4, dtype=np.uint8)
    w_scale = np.empty(N, dtype=np.float32)
    segs = np.empty(ns, dtype=np.int64)
    means = np.empty(ns, dtype=np.float32)
    d = ctypes.c_int64()
    return L.bitnet_load_packed(str(path).encode(), ctypes.byref(d), ctypes.byref(ctypes.c_int64()),
                                ctypes.byref(ctypes.c_int32()), packed.ctypes.data, w_scale.ctypes.data,
                                segs.ctypes.data, means.ctypes.data)


def test_packed_file_fuzz(tmp_path):
    """Damaged files: every header byte flipped, extreme header fields,
    truncations at many lengths and random payload damage.  The loader must
    return a status (OK only for an undamaged file) and never read or write out
    of bounds."""
    import struct
    W = wl.draw_weight((24, 160), seed=21)
    pw = tw.pack(W, (8, 16))
    f = tmp_path / "w.btnl"
    tw.save_packed(f, pw, (8, 16))
    raw = f.read_bytes()
    assert _load_raw(f) == _lib.OK
    rng = np.random.default_rng(5)
    cases = []
    for pos in range(64):                                   # every header byte, two flips each
        for bit in rng.choice(8, size=2, replace=False):
            b = bytearray(raw)
            b[pos] ^= 1 << int(bit)
            cases.append(bytes(b))
    for off, fmt, val in ((16, "<q", 1 << 40), (16, "<q", -5), (24, "<q", 1 << 30), (24, "<q", 17),
                          (32, "<q", 1 << 20), (40, "<i", 1 << 30), (40, "<i", -1), (40, "<i", 0),
                          (24, "<q", 0), (16, "<q", 0)):
        b = bytearray(raw)
        struct.pack_into(fmt, b, off, val)
        cases.append(bytes(b))
    for n in sorted(set(rng.integers(0, len(raw), size=40).tolist()) | {0, 1, 63, 64, len(raw) - 1}):
        cases.append(raw[:n])
    for _ in range(20):
        b = bytearray(raw)
        for p in rng.integers(64, len(raw), size=3):
            b[int(p)] = int(rng.integers(0, 256))
        cases.append(bytes(b))
    for _ in range(10):
        cases.append(rng.integers(0, 256, size=int(rng.integers(1, 400)), dtype=np.uint8).tobytes())
    for i, data in enumerate(cases):
        g = tmp_path / f"c{i}.btnl"
        g.write_bytes(data)
        st = _load_raw(g)
        assert st in (_lib.OK, _lib.ERR_INVALID_ARG, _lib.ERR_UNSUPPORTED, "too large to load"), (i, st)
        if data != raw:
            assert st != _lib.OK, f"case {i}: a damaged file loaded"


def test_host_i2s_import_fuzz():
    """Random I2_S buffers into the host importer: every field value 3 is an
    error, other bytes import, nothing out of bounds."""
    L = _lib.lib()
    rng = np.random.default_rng(6)
    for N, K in ((4, 32), (2, 64), (3, 128)):
        nbytes = L.bitnet_i2s_bytes(N, K)
        kp = L.bitnet_padded_k(K)
        for _ in range(30):
            buf = rng.integers(0, 256, size=nbytes, dtype=np.uint8)
            buf[-4:] = np.frombuffer(np.float32(rng.uniform(-2, 8)).tobytes(), dtype=np.uint8)
            packed = np.empty(N * kp // 4, dtype=np.uint8)
            ws = np.empty(N, dtype=np.float32)
            st = L.bitnet_i2s_import(_lib.MEM_HOST, None, buf.ctypes.data, N, K, int(rng.integers(0, 2)),
                                     packed.ctypes.data, ws.ctypes.data)
            fields = np.stack([(buf[:-4] >> s) & 3 for s in (0, 2, 4, 6)])
            scale = np.frombuffer(buf[-4:].tobytes(), dtype=np.float32)[0]
            ok = not (fields == 3).any() and scale > 0
            assert (st == _lib.OK) == ok, (st, ok)
