"""numpy-facing wrapper of the plain C oracle (``bitnet_oracle.c``).

TEST INFRASTRUCTURE ONLY.  Imported by ``tests/``, by the smoke check and by
the CPU-baseline leg of ``bench.py``; the library package never imports it.
It shares no code with the HIP path (no common headers, helpers, tables or
generators); the only thing both sides see is the seeded input bytes.

Each wrapper says which step of the method it runs; the C file cites the page
passage for every step.  Arrays are numpy: bf16 data travels as ``uint16`` bit
patterns, so nothing here depends on torch.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

HERE = Path(__file__).resolve().parent
SOURCE = HERE / "bitnet_oracle.c"
LIBRARY = HERE / "liboracle.so"

F32, BF16, F16 = 0, 1, 2
CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
          "-shared", "-fopenmp", "-Wall", "-Wextra"]


def build(source: Path = SOURCE, out: Path = LIBRARY) -> Path:
    """Compile the oracle with gcc (plain C11, no fast-math, no contraction)."""
    tmp = Path(str(out) + f".tmp{os.getpid()}")
    subprocess.run(["gcc", *CFLAGS, str(source), "-o", str(tmp), "-lm"], check=True)
    os.replace(tmp, out)
    return out


SANITIZED = HERE / "liboracle_san.so"


def build_sanitized(out: Path = SANITIZED) -> Path:
    """The oracle built with AddressSanitizer and UndefinedBehaviorSanitizer by
    the ROCm clang, to run under that compiler's ASan runtime (CPU tests only)."""
    clang = "/opt/rocm/llvm/bin/clang"
    flags = [f for f in CFLAGS if f not in ("-O2", "-fopenmp")] + [
        "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
    tmp = Path(str(out) + f".tmp{os.getpid()}")
    subprocess.run([clang, *flags, str(SOURCE), "-o", str(tmp), "-lm"], check=True)
    os.replace(tmp, out)
    return out


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.float16:
        return F16                      # passed as its bit patterns; widened by orc_f16_to_f32
    raise TypeError(f"oracle inputs are bf16 bit patterns (uint16), float16 or float32, not {a.dtype}")


class Oracle:
    """Handle on one compiled oracle shared object."""

    def __init__(self, path: Path | str | None = None):
        if path is None and os.environ.get("BITNET_ORACLE_LIBRARY"):
            path = os.environ["BITNET_ORACLE_LIBRARY"]     # e.g. the sanitized build
        path = Path(path) if path is not None else LIBRARY
        if path == LIBRARY and (not path.exists() or path.stat().st_mtime < SOURCE.stat().st_mtime):
            build(out=path)
        self.path = path
        lib = ctypes.CDLL(str(path))
        i64, i32, vp, f32 = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_float
        lib.orc_bf16_to_f32.argtypes, lib.orc_bf16_to_f32.restype = [ctypes.c_uint16], f32
        lib.orc_f16_to_f32.argtypes, lib.orc_f16_to_f32.restype = [ctypes.c_uint16], f32
        lib.orc_f32_to_bf16.argtypes, lib.orc_f32_to_bf16.restype = [f32], ctypes.c_uint16
        lib.orc_f32_to_bf16_array.argtypes, lib.orc_f32_to_bf16_array.restype = [vp, i64, vp], None
        lib.orc_padded_k.argtypes, lib.orc_padded_k.restype = [i64], i64
        lib.orc_row_abs_sum.argtypes, lib.orc_row_abs_sum.restype = [vp, ctypes.c_int, i64, i64, i64], ctypes.c_double
        lib.orc_segment_mean.argtypes = [vp, ctypes.c_int, i64, i64, i64, i64]
        lib.orc_segment_mean.restype = f32
        lib.orc_ternary.argtypes, lib.orc_ternary.restype = [f32, f32], ctypes.c_int8
        lib.orc_weight_quant.argtypes = [vp, ctypes.c_int, i64, i64, i64, vp, i32, vp, vp, vp, vp]
        lib.orc_weight_quant.restype = ctypes.c_int
        lib.orc_pack.argtypes, lib.orc_pack.restype = [vp, i64, i64, vp], ctypes.c_int
        lib.orc_unpack.argtypes, lib.orc_unpack.restype = [vp, i64, i64, vp], i64
        lib.orc_i2s_pack.argtypes, lib.orc_i2s_pack.restype = [vp, i64, i64, f32, ctypes.c_int, vp], ctypes.c_int
        lib.orc_i2s_unpack.argtypes = [vp, i64, i64, ctypes.c_int, vp, vp]
        lib.orc_i2s_unpack.restype = i64
        lib.orc_act_quant.argtypes = [vp, ctypes.c_int, i64, i64, i64, vp, vp, vp]
        lib.orc_act_quant.restype = ctypes.c_int
        lib.orc_rms_act_quant.argtypes = [vp, ctypes.c_int, vp, ctypes.c_int, i64, i64, i64, f32, vp, vp, vp]
        lib.orc_rms_act_quant.restype = ctypes.c_int
        lib.orc_swiglu.argtypes = [vp, vp, ctypes.c_int, i64, i64, i64, vp]
        lib.orc_swiglu.restype = None
        lib.orc_linear_a16.argtypes = [vp, ctypes.c_int, i64, i64, i64, vp, i64, vp, vp, vp]
        lib.orc_linear_a16.restype = None
        lib.orc_int_dot.argtypes = [vp, i64, i64, vp, i64, vp, ctypes.c_int]
        lib.orc_int_dot.restype = ctypes.c_int
        lib.orc_int_dot_pairs.argtypes = [vp, i64, vp, i64, vp, vp, vp]
        lib.orc_int_dot_pairs.restype = ctypes.c_int
        lib.orc_dequant_one.argtypes, lib.orc_dequant_one.restype = [i32, f32, f32], f32
        lib.orc_epilogue.argtypes = [vp, i64, i64, vp, vp, ctypes.c_int, vp, i64]
        lib.orc_epilogue.restype = None
        lib.orc_max_threads.argtypes, lib.orc_max_threads.restype = [], ctypes.c_int
        lib.orc_block_count.argtypes, lib.orc_block_count.restype = [i64], i64
        lib.orc_weight_quant_blocked.argtypes = [vp, ctypes.c_int, i64, i64, i64, vp, vp]
        lib.orc_weight_quant_blocked.restype = ctypes.c_int
        lib.orc_linear_blocked.argtypes = [vp, vp, i64, i64, vp, vp, i64, vp, vp]
        lib.orc_linear_blocked.restype = ctypes.c_int
        self.lib = lib

    # ----------------------------------------------------------- scalars
    def padded_k(self, K: int) -> int:
        return int(self.lib.orc_padded_k(K))

    def bf16_from_f32(self, v: np.ndarray) -> np.ndarray:
        """fp32 -> bf16 bit patterns, round to nearest even (the C element loop)."""
        v = np.ascontiguousarray(v, dtype=np.float32)
        out = np.empty(v.shape, dtype=np.uint16)
        self.lib.orc_f32_to_bf16_array(_ptr(v), v.size, _ptr(out))
        return out

    def ternary(self, w: float, s: float) -> int:
        return int(self.lib.orc_ternary(w, s))

    # ------------------------------------------------------ WeightQuant
    def segment_mean(self, W: np.ndarray, row0: int, rows: int) -> np.float32:
        W = np.ascontiguousarray(W)
        return np.float32(self.lib.orc_segment_mean(_ptr(W), _dtype_code(W), row0, rows,
                                                    W.shape[1], W.shape[1]))

    def weight_quant(self, W: np.ndarray, segments=None):
        """Codes t [N,K] int8, w_scale [N], seg_mean [S], zero_count [S]."""
        W = np.ascontiguousarray(W)
        N, K = W.shape
        segs = np.asarray(segments if segments else [N], dtype=np.int64)
        t = np.empty((N, K), dtype=np.int8)
        w_scale = np.empty(N, dtype=np.float32)
        seg_mean = np.empty(len(segs), dtype=np.float32)
        zeros = np.empty(len(segs), dtype=np.int64)
        rc = self.lib.orc_weight_quant(_ptr(W), _dtype_code(W), N, K, K, _ptr(segs), len(segs),
                                       _ptr(t), _ptr(w_scale), _ptr(seg_mean), _ptr(zeros))
        if rc == -1:
            raise ValueError("segment rows do not add up to N")
        if rc == -2:
            raise ValueError("non-finite weight")
        return t, w_scale, seg_mean, zeros

    def pack(self, t: np.ndarray) -> np.ndarray:
        """Layout-v1 bytes [N, Kp/4] of codes t [N, K]."""
        t = np.ascontiguousarray(t, dtype=np.int8)
        N, K = t.shape
        Kp = self.padded_k(K)
        if Kp < 0:
            raise ValueError("K must be a positive multiple of 16")
        out = np.empty((N, Kp // 4), dtype=np.uint8)
        self.lib.orc_pack(_ptr(t), N, K, _ptr(out))
        return out

    def unpack(self, packed: np.ndarray, K: int):
        """Codes t [N, K] of layout-v1 bytes, and the count of invalid fields (value 3)."""
        packed = np.ascontiguousarray(packed, dtype=np.uint8)
        N = packed.shape[0]
        t = np.empty((N, K), dtype=np.int8)
        bad = self.lib.orc_unpack(_ptr(packed), N, K, _ptr(t))
        if bad < 0:
            raise ValueError("K must be a positive multiple of 16")
        return t, int(bad)

    # ------------------------------------------------------------- I2_S
    def i2s_pack(self, t: np.ndarray, s: float, order: str = "strided") -> np.ndarray:
        """I2_S bytes of codes t [N, K] (N*K % 128 == 0) and scale s = 1/mean|W|."""
        t = np.ascontiguousarray(t, dtype=np.int8)
        N, K = t.shape
        out = np.empty(N * K // 4 + 4, dtype=np.uint8)
        if self.lib.orc_i2s_pack(_ptr(t), N, K, float(s), int(order == "consecutive"), _ptr(out)) != 0:
            raise ValueError("N*K must be a positive multiple of 128")
        return out

    def i2s_unpack(self, buf: np.ndarray, N: int, K: int, order: str = "strided"):
        """Codes t [N, K], the scale s, and the count of invalid fields (value 3)."""
        buf = np.ascontiguousarray(buf, dtype=np.uint8)
        if buf.size < N * K // 4 + 4:
            raise ValueError("buffer too small")
        t = np.empty((N, K), dtype=np.int8)
        s = np.empty(1, dtype=np.float32)
        bad = self.lib.orc_i2s_unpack(_ptr(buf), N, K, int(order == "consecutive"), _ptr(t), _ptr(s))
        if bad < 0:
            raise ValueError("N*K must be a positive multiple of 128")
        return t, np.float32(s[0]), int(bad)

    # --------------------------------------------------------- ActQuant
    def act_quant(self, x: np.ndarray):
        """q [M, Kp] int8 (tail 0), a_scale [M] f32, q_rowsum [M] i32."""
        x = np.ascontiguousarray(x)
        M, K = x.shape
        Kp = self.padded_k(K)
        if Kp < 0:
            raise ValueError("K must be a positive multiple of 16")
        q = np.empty((M, Kp), dtype=np.int8)
        a_scale = np.empty(M, dtype=np.float32)
        rowsum = np.empty(M, dtype=np.int32)
        self.lib.orc_act_quant(_ptr(x), _dtype_code(x), M, K, K, _ptr(q), _ptr(a_scale), _ptr(rowsum))
        return q, a_scale, rowsum

    def rms_act_quant(self, x: np.ndarray, g: np.ndarray, eps: float = 1e-6):
        """ActQuant(RMSNorm(x, g)): q [M, Kp] int8, a_scale [M] f32, q_rowsum [M] i32."""
        x = np.ascontiguousarray(x)
        g = np.ascontiguousarray(g)
        M, K = x.shape
        if g.shape != (K,):
            raise ValueError("g must have K entries")
        Kp = self.padded_k(K)
        if Kp < 0:
            raise ValueError("K must be a positive multiple of 16")
        q = np.empty((M, Kp), dtype=np.int8)
        a_scale = np.empty(M, dtype=np.float32)
        rowsum = np.empty(M, dtype=np.int32)
        self.lib.orc_rms_act_quant(_ptr(x), _dtype_code(x), _ptr(g), _dtype_code(g), M, K, K, float(eps),
                                   _ptr(q), _ptr(a_scale), _ptr(rowsum))
        return q, a_scale, rowsum

    def swiglu(self, gate: np.ndarray, up: np.ndarray) -> np.ndarray:
        """silu(gate) * up, fp32 [M, K]: the definition in fp64, rounded once
        (reading R14 of the C file); gate and up of one dtype and shape."""
        gate = np.ascontiguousarray(gate)
        up = np.ascontiguousarray(up)
        if gate.shape != up.shape or gate.dtype != up.dtype:
            raise ValueError("gate and up must match")
        M, K = gate.shape
        h = np.empty((M, K), dtype=np.float32)
        self.lib.orc_swiglu(_ptr(gate), _ptr(up), _dtype_code(gate), M, K, K, _ptr(h))
        return h

    def swiglu_rms_act_quant(self, gate: np.ndarray, up: np.ndarray, g: np.ndarray, eps: float = 1e-6):
        """ActQuant(RMSNorm(silu(gate) * up, g)) for the down projection."""
        return self.rms_act_quant(self.swiglu(gate, up), g, eps)

    # --------------------------------------------------------- W1.58A16
    def linear_a16(self, x: np.ndarray, t: np.ndarray, w_scale: np.ndarray):
        """fp64 y [M, N] = w_scale * (x @ t.T) with bf16/fp32 x, and sum |x*t| per output."""
        x = np.ascontiguousarray(x)
        t = np.ascontiguousarray(t, dtype=np.int8)
        w_scale = np.ascontiguousarray(w_scale, dtype=np.float32)
        M, K = x.shape
        N = t.shape[0]
        y = np.empty((M, N), dtype=np.float64)
        mag = np.empty((M, N), dtype=np.float64)
        self.lib.orc_linear_a16(_ptr(x), _dtype_code(x), M, K, K, _ptr(t), N, _ptr(w_scale), _ptr(y), _ptr(mag))
        return y, mag

    # ------------------------------------------------------ integer dot
    def int_dot(self, q: np.ndarray, t: np.ndarray, nthreads: int = 1) -> np.ndarray:
        q = np.ascontiguousarray(q, dtype=np.int8)
        t = np.ascontiguousarray(t, dtype=np.int8)
        M, N, K = q.shape[0], t.shape[0], t.shape[1]
        if q.shape[1] != self.padded_k(K):
            raise ValueError("q must be [M, Kp]")
        acc = np.empty((M, N), dtype=np.int32)
        if self.lib.orc_int_dot(_ptr(q), M, K, _ptr(t), N, _ptr(acc), nthreads) != 0:
            raise OverflowError("int32 accumulator overflow")
        return acc

    def int_dot_pairs(self, q: np.ndarray, t: np.ndarray, m_idx, n_idx) -> np.ndarray:
        q = np.ascontiguousarray(q, dtype=np.int8)
        t = np.ascontiguousarray(t, dtype=np.int8)
        m_idx = np.ascontiguousarray(m_idx, dtype=np.int64)
        n_idx = np.ascontiguousarray(n_idx, dtype=np.int64)
        K = t.shape[1]
        acc = np.empty(m_idx.size, dtype=np.int32)
        self.lib.orc_int_dot_pairs(_ptr(q), K, _ptr(t), m_idx.size, _ptr(m_idx), _ptr(n_idx), _ptr(acc))
        return acc

    # --------------------------------------------------------- epilogue
    def epilogue(self, acc: np.ndarray, a_scale: np.ndarray, w_scale: np.ndarray,
                 out: str = "f32") -> np.ndarray:
        acc = np.ascontiguousarray(acc, dtype=np.int32)
        a_scale = np.ascontiguousarray(a_scale, dtype=np.float32)
        w_scale = np.ascontiguousarray(w_scale, dtype=np.float32)
        M, N = acc.shape
        y = np.empty((M, N), dtype=np.float32 if out == "f32" else np.uint16)
        self.lib.orc_epilogue(_ptr(acc), M, N, _ptr(a_scale), _ptr(w_scale),
                              F32 if out == "f32" else BF16, _ptr(y), N)
        return y

    def dequant_one(self, acc: int, a_scale: float, w_scale: float) -> np.float32:
        return np.float32(self.lib.orc_dequant_one(int(acc), float(a_scale), float(w_scale)))

    # ----------------------------------------------------- whole method
    def linear(self, x: np.ndarray, W: np.ndarray, segments=None, out: str = "f32",
               nthreads: int = 1) -> dict:
        """y = linear(ActQuant(x), WeightQuant(W)) and every intermediate."""
        t, w_scale, seg_mean, zeros = self.weight_quant(W, segments)
        packed = self.pack(t)
        q, a_scale, rowsum = self.act_quant(x)
        acc = self.int_dot(q, t, nthreads)
        y = self.epilogue(acc, a_scale, w_scale, out)
        return dict(t=t, packed=packed, w_scale=w_scale, seg_mean=seg_mean, zero_count=zeros,
                    q=q, a_scale=a_scale, q_rowsum=rowsum, acc=acc, y=y)

    # ------------------------------------------- per-block weight scales
    def block_count(self, K: int) -> int:
        return int(self.lib.orc_block_count(K))

    def weight_quant_blocked(self, W: np.ndarray):
        """Codes t [N, K] and block_scale [nb, N]: one absmean scale per 256
        weights of a row (reading R18 of the C file)."""
        W = np.ascontiguousarray(W)
        N, K = W.shape
        nb = self.block_count(K)
        if nb < 0:
            raise ValueError("K must be a positive multiple of 16")
        t = np.empty((N, K), dtype=np.int8)
        bs = np.empty((nb, N), dtype=np.float32)
        rc = self.lib.orc_weight_quant_blocked(_ptr(W), _dtype_code(W), N, K, K, _ptr(t), _ptr(bs))
        if rc == -2:
            raise FloatingPointError("non-finite weight")
        return t, bs

    def linear_blocked_q(self, q: np.ndarray, a_scale: np.ndarray, t: np.ndarray, block_scale: np.ndarray):
        """fp32 y [M, N] and exact block sums [M, nb, N] from quantised
        operands (reading R19 of the C file)."""
        q = np.ascontiguousarray(q, dtype=np.int8)
        a_scale = np.ascontiguousarray(a_scale, dtype=np.float32)
        t = np.ascontiguousarray(t, dtype=np.int8)
        block_scale = np.ascontiguousarray(block_scale, dtype=np.float32)
        M, (N, K) = q.shape[0], t.shape
        if q.shape[1] != self.padded_k(K) or block_scale.shape != (self.block_count(K), N):
            raise ValueError("q must be [M, Kp] and block_scale [nb, N]")
        y = np.empty((M, N), dtype=np.float32)
        accb = np.empty((M, block_scale.shape[0], N), dtype=np.int32)
        self.lib.orc_linear_blocked(_ptr(q), _ptr(a_scale), M, K, _ptr(t), _ptr(block_scale), N, _ptr(y),
                                    _ptr(accb))
        return y, accb

    def linear_blocked(self, x: np.ndarray, W: np.ndarray, out: str = "f32") -> dict:
        """y = linear(ActQuant(x), blocked WeightQuant(W)) and its intermediates."""
        t, bs = self.weight_quant_blocked(W)
        packed = self.pack(t)
        q, a_scale, rowsum = self.act_quant(x)
        y, accb = self.linear_blocked_q(q, a_scale, t, bs)
        if out == "bf16":
            y = self.bf16_from_f32(y)
        return dict(t=t, packed=packed, block_scale=bs, q=q, a_scale=a_scale, q_rowsum=rowsum,
                    acc_blocks=accb, y=y)

    def max_threads(self) -> int:
        return int(self.lib.orc_max_threads())


_default: Oracle | None = None


def get() -> Oracle:
    """The oracle built from the committed source (built on first use)."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default
