"""W1.58A8 BitLinear on MI355X (gfx950): Python binding of libbitnet_hip.so.

    y = linear(ActQuant(x), WeightQuant(W))

("BitVLA -- 1.58-bit Vision-Language-Action on Core AI", s1 and s2;
"BitNet-Embeddings-0.6B/270M: I2_S Conversion and Inference Optimization
Guide", s2 and s3.3.)  Every function here only marshals arguments: torch
supplies device memory and the current HIP stream, the C ABI in
``include/bitnet.h`` does all of the work in HIP kernels.  Non-OK statuses
raise ``BitnetError``.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import torch

from . import _lib
from ._lib import BitnetError

__all__ = ["BitnetError", "PackedWeight", "padded_k", "packed_bytes", "pack", "act_quant",
           "linear", "bitlinear", "GroupedBitLinear", "library_path"]

_DT = {torch.float32: _lib.F32, torch.bfloat16: _lib.BF16}
_DT_A16 = {torch.bfloat16: _lib.BF16, torch.float16: _lib.F16}     # W1.58A16 activations


def library_path() -> str:
    return str(_lib.LIBRARY)


def _stream(t: torch.Tensor):
    return torch.cuda.current_stream(t.device).cuda_stream


def _dtype(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise TypeError(f"expected float32 or bfloat16, got {t.dtype}")
    return _DT[t.dtype]


def _rows(t: torch.Tensor, name: str) -> int:
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be a 2-D tensor with unit column stride")
    return t.stride(0)


def _vector(t, n: int, dtype, name: str) -> None:
    if not isinstance(t, torch.Tensor) or t.dtype != dtype or t.dim() != 1 or t.numel() != n or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape [{n}]")


def _quantised(q, a_scale, q_rowsum, K: int) -> int:
    """Check ActQuant outputs for a weight of K columns; returns M."""
    Kp = padded_k(K)
    if (not isinstance(q, torch.Tensor) or q.dtype != torch.int8 or q.dim() != 2 or q.shape[1] != Kp
            or not q.is_contiguous()):
        raise ValueError(f"q must be a contiguous int8 tensor of shape [M, {Kp}] (Kp of the weight's K={K})")
    M = q.shape[0]
    if M < 1:
        raise ValueError("q must hold at least one token")
    _vector(a_scale, M, torch.float32, "a_scale")
    if q_rowsum is not None:
        _vector(q_rowsum, M, torch.int32, "q_rowsum")
    return M


def _weight(w) -> None:
    Kp = padded_k(w.K)
    if Kp < 0 or w.N < 1:
        raise ValueError(f"packed weight has a bad shape N={w.N}, K={w.K}")
    if (w.packed.dtype != torch.uint8 or tuple(w.packed.shape) != (w.N, Kp // 4)
            or not w.packed.is_contiguous()):
        raise ValueError(f"packed must be a contiguous uint8 tensor of shape [{w.N}, {Kp // 4}]")
    scale = getattr(w, "w_scale", None)
    if scale is not None:
        _vector(scale, w.N, torch.float32, "w_scale")
    else:
        nb = -(-w.K // 256)
        if (w.block_scale.dtype != torch.float32 or tuple(w.block_scale.shape) != (nb, w.N)
                or not w.block_scale.is_contiguous()):
            raise ValueError(f"block_scale must be a contiguous float32 tensor of shape [{nb}, {w.N}]")


def _output(y, M: int, N: int) -> int:
    """Check an output tensor [M, N] (fp32 or bf16, unit column stride); returns its row stride."""
    if not isinstance(y, torch.Tensor) or y.dim() != 2 or tuple(y.shape) != (M, N):
        raise ValueError(f"out must be a tensor of shape [{M}, {N}]")
    if y.dtype not in _DT:
        raise TypeError(f"out must be float32 or bfloat16, not {y.dtype}")
    return _rows(y, "out")


def _on_device(device, **tensors) -> None:
    """Every tensor must be a CUDA tensor on ``device``."""
    for name, t in tensors.items():
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a CUDA tensor")
        if t.device != device:
            raise ValueError(f"{name} is on {t.device}, expected {device}")


def padded_k(K: int) -> int:
    """Kp = K rounded up to a multiple of 128 (-1 if K is not a positive multiple of 16)."""
    return int(_lib.lib().bitnet_padded_k(K))


def packed_bytes(N: int, K: int) -> int:
    return int(_lib.lib().bitnet_packed_bytes(N, K))


@dataclass
class PackedWeight:
    packed: torch.Tensor      # uint8 [N, Kp/4], layout v1
    w_scale: torch.Tensor     # float32 [N]
    N: int
    K: int
    seg_mean: torch.Tensor    # float32 [segments] (host)
    zero_count: torch.Tensor  # int64 [segments] (host)


def pack(W: torch.Tensor, segments=None) -> PackedWeight:
    """WeightQuant + pack of W [N, K] (bf16 or fp32).  A CUDA tensor is packed by the
    device kernels, a CPU tensor by the library's host packer (chosen by where W lives)."""
    ldw = _rows(W, "W")
    N, K = W.shape
    Kp = padded_k(K)
    if Kp < 0:
        raise ValueError(f"K={K} must be a positive multiple of 16")
    segs = list(segments) if segments else [N]
    seg_arr = (torch.tensor(segs, dtype=torch.int64))
    packed = torch.empty((N, Kp // 4), dtype=torch.uint8, device=W.device)
    w_scale = torch.empty(N, dtype=torch.float32, device=W.device)
    seg_mean = torch.empty(len(segs), dtype=torch.float32)
    zeros = torch.empty(len(segs), dtype=torch.int64)
    on_gpu = W.is_cuda
    with torch.cuda.device(W.device) if on_gpu else _nullctx():
        st = _lib.lib().bitnet_pack_weights(
            _lib.MEM_DEVICE if on_gpu else _lib.MEM_HOST, _stream(W) if on_gpu else None,
            W.data_ptr(), _dtype(W), N, K, ldw, seg_arr.data_ptr(), len(segs),
            packed.data_ptr(), w_scale.data_ptr(), seg_mean.data_ptr(), zeros.data_ptr())
    _lib.check(st)
    return PackedWeight(packed, w_scale, N, K, seg_mean, zeros)


_I2S_ORDERS = {"strided": 0, "consecutive": 1}


def i2s_import(buf: torch.Tensor, N: int, K: int, order: str = "strided") -> PackedWeight:
    """An I2_S buffer (uint8, bitnet_i2s_bytes(N, K) bytes, CPU or CUDA) of one [N, K]
    tensor as a layout-v1 PackedWeight on the same device.  seg_mean holds 1/s; the
    zero count is not known for imported weights (-1)."""
    nbytes = int(_lib.lib().bitnet_i2s_bytes(N, K))
    if nbytes < 0:
        raise ValueError("need K % 16 == 0 and N*K % 128 == 0")
    if buf.dtype != torch.uint8 or buf.numel() < nbytes or not buf.is_contiguous():
        raise ValueError(f"buf must be a contiguous uint8 tensor of at least {nbytes} bytes")
    Kp = padded_k(K)
    packed = torch.empty((N, Kp // 4), dtype=torch.uint8, device=buf.device)
    w_scale = torch.empty(N, dtype=torch.float32, device=buf.device)
    on_gpu = buf.is_cuda
    with torch.cuda.device(buf.device) if on_gpu else _nullctx():
        _lib.check(_lib.lib().bitnet_i2s_import(
            _lib.MEM_DEVICE if on_gpu else _lib.MEM_HOST, _stream(buf) if on_gpu else None, buf.data_ptr(),
            N, K, _I2S_ORDERS[order], packed.data_ptr(), w_scale.data_ptr()))
    return PackedWeight(packed, w_scale, N, K, w_scale[:1].cpu().clone(), torch.tensor([-1], dtype=torch.int64))


def i2s_export(w: PackedWeight, order: str = "strided") -> torch.Tensor:
    """The I2_S buffer (uint8, on w's device) of a single-tensor PackedWeight."""
    nbytes = int(_lib.lib().bitnet_i2s_bytes(w.N, w.K))
    if nbytes < 0:
        raise ValueError("need K % 16 == 0 and N*K % 128 == 0")
    out = torch.empty(nbytes, dtype=torch.uint8, device=w.packed.device)
    on_gpu = w.packed.is_cuda
    with torch.cuda.device(w.packed.device) if on_gpu else _nullctx():
        _lib.check(_lib.lib().bitnet_i2s_export(
            _lib.MEM_DEVICE if on_gpu else _lib.MEM_HOST, _stream(w.packed) if on_gpu else None,
            w.packed.data_ptr(), w.w_scale.data_ptr(), w.N, w.K, _I2S_ORDERS[order], out.data_ptr()))
    return out


def save_packed(path, w: PackedWeight, segments=None):
    """Write w (with the row counts of its source tensors, default one) to a
    versioned packed-weight file."""
    segs = torch.tensor(list(segments) if segments else [w.N], dtype=torch.int64)
    if segs.numel() != w.seg_mean.numel():
        raise ValueError("one row count per segment of w")
    packed, w_scale = w.packed.cpu().contiguous(), w.w_scale.cpu().contiguous()
    seg_mean = w.seg_mean.to(torch.float32).contiguous()
    _lib.check(_lib.lib().bitnet_save_packed(str(path).encode(), packed.data_ptr(), w_scale.data_ptr(), w.N, w.K,
                                             segs.data_ptr(), seg_mean.data_ptr(), segs.numel()))


def load_packed(path, device="cpu"):
    """(PackedWeight, segment row counts) from a packed-weight file; tensors on ``device``."""
    L = _lib.lib()
    N, K, ns = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int32()
    _lib.check(L.bitnet_load_packed(str(path).encode(), ctypes.byref(N), ctypes.byref(K), ctypes.byref(ns),
                                    None, None, None, None))
    N, K, ns = N.value, K.value, ns.value
    packed = torch.empty((N, padded_k(K) // 4), dtype=torch.uint8)
    w_scale = torch.empty(N, dtype=torch.float32)
    segs = torch.empty(ns, dtype=torch.int64)
    seg_mean = torch.empty(ns, dtype=torch.float32)
    _lib.check(L.bitnet_load_packed(str(path).encode(), ctypes.byref(ctypes.c_int64()), ctypes.byref(ctypes.c_int64()),
                                    ctypes.byref(ctypes.c_int32()), packed.data_ptr(), w_scale.data_ptr(),
                                    segs.data_ptr(), seg_mean.data_ptr()))
    w = PackedWeight(packed.to(device), w_scale.to(device), N, K, seg_mean, torch.full((ns,), -1, dtype=torch.int64))
    return w, segs.tolist()


class _nullctx:
    def __enter__(self):
        return None

    def __exit__(self, *a):
        return False


def act_quant(x: torch.Tensor):
    """Per-token ActQuant of x [M, K] (CUDA, bf16 or fp32) -> (q [M, Kp] int8, a_scale [M], q_rowsum [M])."""
    ldx = _rows(x, "x")
    M, K = x.shape
    Kp = padded_k(K)
    if Kp < 0:
        raise ValueError(f"K={K} must be a positive multiple of 16")
    _on_device(x.device, x=x)
    q = torch.empty((M, Kp), dtype=torch.int8, device=x.device)
    a_scale = torch.empty(M, dtype=torch.float32, device=x.device)
    rowsum = torch.empty(M, dtype=torch.int32, device=x.device)
    with torch.cuda.device(x.device):
        _lib.check(_lib.lib().bitnet_act_quant(_stream(x), x.data_ptr(), _dtype(x), M, K, ldx,
                                               q.data_ptr(), a_scale.data_ptr(), rowsum.data_ptr()))
    return q, a_scale, rowsum


def rmsnorm_act_quant(x: torch.Tensor, norm_w: torch.Tensor, eps: float = 1e-6, up: torch.Tensor | None = None):
    """ActQuant(RMSNorm(h, norm_w)) with h = x, or h = silu(x) * up when ``up`` is given
    (same shape, dtype and row stride as x) -> (q [M, Kp] int8, a_scale [M], q_rowsum [M])."""
    ldx = _rows(x, "x")
    M, K = x.shape
    Kp = padded_k(K)
    if Kp < 0:
        raise ValueError(f"K={K} must be a positive multiple of 16")
    if norm_w.shape != (K,) or not norm_w.is_contiguous():
        raise ValueError("norm_w must be a contiguous [K] tensor")
    if up is not None and (up.shape != x.shape or up.dtype != x.dtype or _rows(up, "up") != ldx):
        raise ValueError("up must match x in shape, dtype and row stride")
    _on_device(x.device, x=x, norm_w=norm_w, up=up)
    q = torch.empty((M, Kp), dtype=torch.int8, device=x.device)
    a_scale = torch.empty(M, dtype=torch.float32, device=x.device)
    rowsum = torch.empty(M, dtype=torch.int32, device=x.device)
    with torch.cuda.device(x.device):
        _lib.check(_lib.lib().bitnet_rmsnorm_act_quant(
            _stream(x), x.data_ptr(), up.data_ptr() if up is not None else None, _dtype(x), M, K, ldx,
            norm_w.data_ptr(), _dtype(norm_w), float(eps), q.data_ptr(), a_scale.data_ptr(), rowsum.data_ptr()))
    return q, a_scale, rowsum


def linear(q: torch.Tensor, a_scale: torch.Tensor, q_rowsum: torch.Tensor, w: PackedWeight,
           out_dtype=torch.float32, out: torch.Tensor | None = None, acc_debug: bool = False):
    """y [M, N] = (acc) * (a_scale[m] * w_scale[n]) with acc the exact int32 sum of q*t.
    Returns y, or (y, acc) when acc_debug is set."""
    M = _quantised(q, a_scale, q_rowsum, w.K)
    _weight(w)
    y = out if out is not None else torch.empty((M, w.N), dtype=out_dtype, device=q.device)
    ldy = _output(y, M, w.N)
    _on_device(q.device, q=q, a_scale=a_scale, q_rowsum=q_rowsum, packed=w.packed, w_scale=w.w_scale, out=y)
    acc = torch.empty((M, w.N), dtype=torch.int32, device=q.device) if acc_debug else None
    with torch.cuda.device(q.device):
        _lib.check(_lib.lib().bitnet_linear_forward(
            _stream(q), q.data_ptr(), a_scale.data_ptr(), q_rowsum.data_ptr(), M, w.K,
            w.packed.data_ptr(), w.w_scale.data_ptr(), w.N, y.data_ptr(), _dtype(y), ldy,
            acc.data_ptr() if acc is not None else None))
    return (y, acc) if acc_debug else y


@dataclass
class BlockPackedWeight:
    packed: torch.Tensor       # uint8 [N, Kp/4], layout v1
    block_scale: torch.Tensor  # float32 [ceil(K/256), N], block-major
    N: int
    K: int


def pack_blocked(W: torch.Tensor) -> BlockPackedWeight:
    """WeightQuant with one absmean scale per 256 weights of a row (device W)."""
    ldw = _rows(W, "W")
    N, K = W.shape
    nb = int(_lib.lib().bitnet_block_count(K))
    if nb < 0:
        raise ValueError(f"K={K} must be a positive multiple of 16")
    packed = torch.empty((N, padded_k(K) // 4), dtype=torch.uint8, device=W.device)
    block_scale = torch.empty((nb, N), dtype=torch.float32, device=W.device)
    with torch.cuda.device(W.device):
        _lib.check(_lib.lib().bitnet_pack_weights_blocked(_stream(W), W.data_ptr(), _dtype(W), N, K, ldw,
                                                          packed.data_ptr(), block_scale.data_ptr()))
    return BlockPackedWeight(packed, block_scale, N, K)


def linear_blocked(q: torch.Tensor, a_scale: torch.Tensor, w: BlockPackedWeight, out_dtype=torch.float32,
                   out: torch.Tensor | None = None) -> torch.Tensor:
    """y [M, N] = a_scale[m] * sum_b acc_b * block_scale[b][n] (fp32, blocks in order)."""
    M = _quantised(q, a_scale, None, w.K)
    _weight(w)
    y = out if out is not None else torch.empty((M, w.N), dtype=out_dtype, device=q.device)
    ldy = _output(y, M, w.N)
    _on_device(q.device, q=q, a_scale=a_scale, packed=w.packed, block_scale=w.block_scale, out=y)
    with torch.cuda.device(q.device):
        _lib.check(_lib.lib().bitnet_linear_blocked_forward(
            _stream(q), q.data_ptr(), a_scale.data_ptr(), M, w.K, w.packed.data_ptr(), w.block_scale.data_ptr(),
            w.N, y.data_ptr(), _dtype(y), ldy))
    return y


def bitlinear(x: torch.Tensor, w: PackedWeight, out_dtype=torch.float32, out: torch.Tensor | None = None,
              workspace=None):
    """y = linear(ActQuant(x), WeightQuant(W)) from activations x [M, K].
    ``workspace`` may pass preallocated (q, a_scale, q_rowsum) buffers."""
    ldx = _rows(x, "x")
    M, K = x.shape
    if K != w.K:
        raise ValueError("x and the packed weight disagree on K")
    _weight(w)
    if workspace is None:
        workspace = (torch.empty((M, padded_k(K)), dtype=torch.int8, device=x.device),
                     torch.empty(M, dtype=torch.float32, device=x.device),
                     torch.empty(M, dtype=torch.int32, device=x.device))
    q, a_scale, rowsum = workspace
    if _quantised(q, a_scale, rowsum, K) != M:
        raise ValueError("workspace must hold M tokens")
    y = out if out is not None else torch.empty((M, w.N), dtype=out_dtype, device=x.device)
    ldy = _output(y, M, w.N)
    _on_device(x.device, x=x, q=q, a_scale=a_scale, q_rowsum=rowsum, packed=w.packed, w_scale=w.w_scale, out=y)
    with torch.cuda.device(x.device):
        _lib.check(_lib.lib().bitnet_bitlinear_forward(
            _stream(x), x.data_ptr(), _dtype(x), M, K, ldx, w.packed.data_ptr(), w.w_scale.data_ptr(),
            w.N, y.data_ptr(), _dtype(y), ldy, q.data_ptr(), a_scale.data_ptr(), rowsum.data_ptr()))
    return y


def linear_a16(x: torch.Tensor, w: PackedWeight, out_dtype=torch.float32, out: torch.Tensor | None = None):
    """W1.58A16: y = w_scale * (x . t) with bf16 or fp16 activations x [M, K] kept unquantised."""
    ldx = _rows(x, "x")
    M, K = x.shape
    if K != w.K:
        raise ValueError("x and the packed weight disagree on K")
    _weight(w)
    y = out if out is not None else torch.empty((M, w.N), dtype=out_dtype, device=x.device)
    ldy = _output(y, M, w.N)
    _on_device(x.device, x=x, packed=w.packed, w_scale=w.w_scale, out=y)
    with torch.cuda.device(x.device):
        _lib.check(_lib.lib().bitnet_linear_a16(_stream(x), x.data_ptr(), _DT_A16.get(x.dtype, _lib.F32), M, K, ldx,
                                                w.packed.data_ptr(),
                                                w.w_scale.data_ptr(), w.N, y.data_ptr(), _dtype(y), ldy))
    return y


def rmsnorm_bitlinear(x: torch.Tensor, norm_w: torch.Tensor, w: PackedWeight, eps: float = 1e-6,
                      up: torch.Tensor | None = None, out_dtype=torch.float32, out: torch.Tensor | None = None,
                      workspace=None):
    """y = linear(ActQuant(RMSNorm(h, norm_w)), WeightQuant(W)) with h = x, or h = silu(x) * up."""
    ldx = _rows(x, "x")
    M, K = x.shape
    if K != w.K:
        raise ValueError("x and the packed weight disagree on K")
    if norm_w.shape != (K,) or not norm_w.is_contiguous():
        raise ValueError("norm_w must be a contiguous [K] tensor")
    if up is not None and (up.shape != x.shape or up.dtype != x.dtype or _rows(up, "up") != ldx):
        raise ValueError("up must match x in shape, dtype and row stride")
    _weight(w)
    if workspace is None:
        workspace = (torch.empty((M, padded_k(K)), dtype=torch.int8, device=x.device),
                     torch.empty(M, dtype=torch.float32, device=x.device),
                     torch.empty(M, dtype=torch.int32, device=x.device))
    q, a_scale, rowsum = workspace
    if _quantised(q, a_scale, rowsum, K) != M:
        raise ValueError("workspace must hold M tokens")
    y = out if out is not None else torch.empty((M, w.N), dtype=out_dtype, device=x.device)
    ldy = _output(y, M, w.N)
    _on_device(x.device, x=x, up=up, norm_w=norm_w, q=q, a_scale=a_scale, q_rowsum=rowsum, packed=w.packed,
               w_scale=w.w_scale, out=y)
    with torch.cuda.device(x.device):
        _lib.check(_lib.lib().bitnet_rmsnorm_bitlinear_forward(
            _stream(x), x.data_ptr(), up.data_ptr() if up is not None else None, _dtype(x), M, K, ldx,
            norm_w.data_ptr(), _dtype(norm_w), float(eps), w.packed.data_ptr(), w.w_scale.data_ptr(),
            w.N, y.data_ptr(), _dtype(y), ldy, q.data_ptr(), a_scale.data_ptr(), rowsum.data_ptr()))
    return y


class GroupedBitLinear:
    """Many independent decode-size BitLinears (shared M <= 16) run as one launch.

    ``items`` is a list of (x [M, K], PackedWeight, y [M, N]) device tensors; the
    plan keeps pointers to them, so they must stay alive and in place.  Calling
    the object writes y_i = linear(ActQuant(x_i), WeightQuant(W_i)) for all i.
    With BlockPackedWeight items (per-256-block scales) every y_i is
    linear_blocked's result for that item."""

    def __init__(self, items, norms=None, a16=False):
        """``norms``: None, or one entry per item, each None or (norm_w [K], up or None, eps):
        the item's input is then RMSNorm(x or silu(x) * up, norm_w) before ActQuant.
        ``a16``: the W1.58A16 variant, y_i = w_scale_i * (x_i . t_i) with bf16 x_i kept
        unquantised (as linear_a16 per item); no norms."""
        if not items:
            raise ValueError("need at least one item")
        if norms is not None and len(norms) != len(items):
            raise ValueError("norms needs one entry per item")
        if a16 and norms is not None:
            raise ValueError("the W1.58A16 group takes no input norms")
        if a16 and any(x.dtype not in _DT_A16 or x.dtype != items[0][0].dtype for x, _, _ in items):
            raise ValueError("the W1.58A16 group takes bf16 or fp16 activations, one dtype for all items")
        blocked = isinstance(items[0][1], BlockPackedWeight)
        if any(isinstance(w, BlockPackedWeight) != blocked for _, w, _ in items):
            raise ValueError("a group takes either per-tensor or per-256-block scaled weights, not both")
        if blocked and (a16 or norms is not None):
            raise ValueError("the block-scaled group takes neither input norms nor 16-bit activations")
        x0 = items[0][0]
        M = x0.shape[0]
        self._keep = list(items)
        arr = (_lib.GroupItem * len(items))()
        for i, (x, w, y) in enumerate(items):
            if x.shape != (M, w.K) or y.shape != (M, w.N):
                raise ValueError(f"item {i}: shapes do not match")
            if x.dtype != x0.dtype or y.dtype != items[0][2].dtype:
                raise ValueError(f"item {i}: every x must share one dtype, and every y another")
            _weight(w)
            _output(y, M, w.N)
            scale = w.block_scale if blocked else w.w_scale
            _on_device(x0.device, x=x, packed=w.packed, w_scale=scale, out=y)
            arr[i] = _lib.GroupItem(x.data_ptr(), _rows(x, "x"), w.packed.data_ptr(), scale.data_ptr(),
                                    y.data_ptr(), _rows(y, "y"), w.N, w.K)
        nrm = None
        if norms is not None:
            nrm = (_lib.GroupNorm * len(items))()
            for i, entry in enumerate(norms):
                if entry is None:
                    continue
                g, up, eps = entry
                x = items[i][0]
                if g.shape != (x.shape[1],) or not g.is_contiguous():
                    raise ValueError(f"item {i}: norm_w must be a contiguous [K] tensor")
                if up is not None and (up.shape != x.shape or up.dtype != x.dtype or _rows(up, "up") != _rows(x, "x")):
                    raise ValueError(f"item {i}: up must match x in shape, dtype and row stride")
                _on_device(x0.device, norm_w=g, up=up)
                nrm[i] = _lib.GroupNorm(up.data_ptr() if up is not None else None, g.data_ptr(), _dtype(g),
                                        float(eps))
                self._keep.append((g, up))
        nbytes = int(_lib.lib().bitnet_group_table_bytes(len(items)))
        self.table = torch.empty(nbytes, dtype=torch.uint8, device=x0.device)
        self.plan = _lib.GroupPlan()
        self.device = x0.device
        with torch.cuda.device(x0.device):
            if blocked:
                _lib.check(_lib.lib().bitnet_group_plan_blocked(
                    _stream(x0), ctypes.cast(arr, ctypes.c_void_p), len(items), M, _dtype(x0),
                    _dtype(items[0][2]), self.table.data_ptr(), nbytes, ctypes.byref(self.plan)))
            elif a16:
                plan_fn = (_lib.lib().bitnet_group_plan_a16_fp16 if x0.dtype == torch.float16
                           else _lib.lib().bitnet_group_plan_a16)
                _lib.check(plan_fn(
                    _stream(x0), ctypes.cast(arr, ctypes.c_void_p), len(items), M, _dtype(items[0][2]),
                    self.table.data_ptr(), nbytes, ctypes.byref(self.plan)))
            elif nrm is None:
                _lib.check(_lib.lib().bitnet_group_plan(
                    _stream(x0), ctypes.cast(arr, ctypes.c_void_p), len(items), M, _dtype(x0),
                    _dtype(items[0][2]), self.table.data_ptr(), nbytes, ctypes.byref(self.plan)))
            else:
                _lib.check(_lib.lib().bitnet_group_plan_rmsnorm(
                    _stream(x0), ctypes.cast(arr, ctypes.c_void_p), ctypes.cast(nrm, ctypes.c_void_p), len(items),
                    M, _dtype(x0), _dtype(items[0][2]), self.table.data_ptr(), nbytes, ctypes.byref(self.plan)))
        self.bytes = sum(w.N * w.K // 4 for _, w, _ in items)
        # which kernel the plan launches: "stream", "persistent", "stream-a16" or "stream-blocked"
        self.kernel = _lib.lib().bitnet_group_plan_kernel(ctypes.byref(self.plan)).decode()

    def __call__(self):
        with torch.cuda.device(self.device):
            _lib.check(_lib.lib().bitnet_bitlinear_grouped(torch.cuda.current_stream(self.device).cuda_stream,
                                                           ctypes.byref(self.plan)))
