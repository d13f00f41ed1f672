"""Plant one plausible mistake at a time in a copy of the oracle (on the CPU)
and check that the pins catch every one of them.

Each mutant is compiled from the committed C source with one textual change and
its pins run in a process of their own, so a mutant that misbehaves cannot take
the test runner down.  Every mutation keeps all memory accesses in bounds.
"""
import json
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor
from pathlib import Path

from oracle import oracle as orc_mod

HERE = Path(__file__).resolve().parent

MUTANTS = [
    ("block mean divides by 256 in a partial block",
     "float mean = (float)(sum / (double)(k1 - k0));", "float mean = (float)(sum / 256.0);"),
    ("block scales stored row-major", "block_scale[b * N + n] = mean;", "block_scale[n * nb + b] = mean;"),
    ("blocked sum drops the last block",
     "for (int64_t b = 0; b < nb; ++b) {\n                int64_t k0",
     "for (int64_t b = 0; b < nb - 1; ++b) {\n                int64_t k0"),
    ("blocked output omits a_scale", "y[m * N + n] = total * a_scale[m];", "y[m * N + n] = total;"),
    ("block codes use the tensor's first block scale",
     "float s = 1.0f / mean;\n            block_scale[b * N + n] = mean;",
     "float s = 1.0f / (float)(fabs((double)load_elem(W, dtype, n * ldw + 0)) + 1e-30);\n"
     "            block_scale[b * N + n] = mean;"),
    ("weight rounding half away from zero",
     "float r = round_half_even(p);", "float r = roundf(p);"),
    ("activation rounding half away from zero",
     "float r = round_half_even(load_elem(x, dtype, m * ldx + k) * sa);",
     "float r = roundf(load_elem(x, dtype, m * ldx + k) * sa);"),
    ("activation factor applied as (x*127)/amax",
     "float r = round_half_even(load_elem(x, dtype, m * ldx + k) * sa);",
     "float r = round_half_even(load_elem(x, dtype, m * ldx + k) * 127.0f / amax);"),
    ("stored code sign flipped",
     "(unsigned)(t[n * K + k] + 1)", "(unsigned)(1 - t[n * K + k])"),
    ("padding code 0 instead of 1",
     "(unsigned)(t[n * K + k] + 1) : 1u;", "(unsigned)(t[n * K + k] + 1) : 0u;"),
    ("byte and bit roles of the layout transposed",
     "static int64_t v1_byte(int64_t k) { return 4 * (k / 16) + (k % 4); }\n"
     "static int v1_shift(int64_t k) { return (int)(2 * ((k % 16) / 4)); }",
     "static int64_t v1_byte(int64_t k) { return 4 * (k / 16) + (k % 16) / 4; }\n"
     "static int v1_shift(int64_t k) { return (int)(2 * (k % 4)); }"),
    ("mean divides by K instead of rows*K",
     "return (float)(total / (double)(rows * K));", "return (float)(total / (double)(K));"),
    ("segments ignored (one scale for the fused tensor)",
     "float mean = orc_segment_mean(W, dtype, row0, seg_rows[i], K, ldw);",
     "float mean = orc_segment_mean(W, dtype, 0, N, K, ldw);"),
    ("absolute value dropped in amax",
     "float a = fabsf(load_elem(x, dtype, m * ldx + k));",
     "float a = load_elem(x, dtype, m * ldx + k);"),
    ("absolute value dropped in mean|W|",
     "s += fabs((double)load_elem(W, dtype, n * ldw + k));",
     "s += (double)load_elem(W, dtype, n * ldw + k);"),
    ("q_rowsum drops the last element",
     "sum += (int8_t)r;", "sum += (k + 1 < K) ? (int8_t)r : 0;"),
    ("integer dot reads the codes transposed",
     "s += (int64_t)q[m * Kp + k] * (int64_t)t[n * K + k];",
     "s += (int64_t)q[m * Kp + k] * (int64_t)t[k * N + n];"),
    ("integer dot drops the last k",
     "for (int64_t k = 0; k < K; ++k)\n                s += (int64_t)q[m * Kp + k]",
     "for (int64_t k = 0; k < K - 1; ++k)\n                s += (int64_t)q[m * Kp + k]"),
    ("epilogue drops w_scale", "float f = a_scale * w_scale;", "float f = a_scale;"),
    ("epilogue uses a_scale twice", "float f = a_scale * w_scale;", "float f = a_scale * a_scale;"),
    ("a_scale stored as 127/amax", "a_scale[m] = amax / 127.0f;", "a_scale[m] = 127.0f / amax;"),
    ("bf16 output truncates", "if (rest > 0x8000u)", "if (rest > 0xFFFFu)"),
    ("bf16 ties away from zero",
     "else if (rest == 0x8000u && (upper & 1u))", "else if (rest == 0x8000u)"),
    ("q tail left non-zero",
     "for (int64_t k = K; k < Kp; ++k)\n                q[m * Kp + k] = 0;",
     "for (int64_t k = K; k < Kp; ++k)\n                q[m * Kp + k] = 1;"),
    ("weight clamp at +-2",
     "if (r > 1.0f)\n        r = 1.0f;\n    if (r < -1.0f)\n        r = -1.0f;",
     "if (r > 2.0f)\n        r = 2.0f;\n    if (r < -2.0f)\n        r = -2.0f;"),
    ("zero count counts non-zeros", "zeros += (c == 0);", "zeros += (c != 0);"),
    ("unpack offset wrong", "t[n * K + k] = (int8_t)((int)u - 1);", "t[n * K + k] = (int8_t)((int)u - 2);"),
    ("RMSNorm drops eps",
     "double r = 1.0 / sqrt(squares / (double)K + (double)eps);",
     "double r = 1.0 / sqrt(squares / (double)K);"),
    ("RMSNorm sums instead of averaging",
     "double r = 1.0 / sqrt(squares / (double)K + (double)eps);",
     "double r = 1.0 / sqrt(squares + (double)eps);"),
    ("RMSNorm without the square root",
     "double r = 1.0 / sqrt(squares / (double)K + (double)eps);",
     "double r = 1.0 / (squares / (double)K + (double)eps);"),
    ("RMSNorm codes ignore the norm weight",
     "float z = load_elem(x, x_dtype, m * ldx + k) * load_elem(g, g_dtype, k);\n                float c",
     "float z = load_elem(x, x_dtype, m * ldx + k);\n                float c"),
    ("RMSNorm scale leaves out r",
     "a_scale[m] = (float)((double)amax * r / 127.0);", "a_scale[m] = (float)((double)amax / 127.0);"),
    ("RMSNorm squares the weighted value",
     "squares += (double)xv * (double)xv;", "squares += (double)z * (double)z;"),
    ("silu sign flipped", "(float)(a / (1.0 + exp(-a)) * u)", "(float)(a / (1.0 + exp(a)) * u)"),
    ("gated product drops up", "(float)(a / (1.0 + exp(-a)) * u)", "(float)(a / (1.0 + exp(-a)))"),
    ("silu divides by 1 - exp", "(float)(a / (1.0 + exp(-a)) * u)", "(float)(a / (2.0 - exp(-a)) * u)"),
    ("silu evaluated in fp32", "h[m * K + k] = (float)(a / (1.0 + exp(-a)) * u);",
     "h[m * K + k] = (float)a / (1.0f + expf(-(float)a)) * (float)u;"),
    ("row sum of |W| in fp32",
     "double s = 0.0;\n    for (int64_t k = 0; k < K; ++k)\n        s += fabs((double)load_elem(W, dtype, n * ldw + k));",
     "float s = 0.0f;\n    for (int64_t k = 0; k < K; ++k)\n        s += fabsf(load_elem(W, dtype, n * ldw + k));"),
    ("segment total in fp32", "double total = 0.0;\n    for (int64_t n = row0;", "float total = 0.0f;\n    for (int64_t n = row0;"),
    ("block sum of |W| in fp32", "double sum = 0.0;\n            for (int64_t k = k0;",
     "float sum = 0.0f;\n            for (int64_t k = k0;"),
    ("block terms added in reverse order",
     "for (int64_t b = 0; b < nb; ++b) {\n                int64_t k0",
     "for (int64_t b = nb - 1; b >= 0; --b) {\n                int64_t k0"),
    ("block terms accumulated in fp64", "float total = 0.0f;\n            for (int64_t b = 0;",
     "double total = 0.0;\n            for (int64_t b = 0;"),
    ("fp16 exponent bias off by one", "v = ldexpf((float)(1024 + f), e - 25);",
     "v = ldexpf((float)(1024 + f), e - 24);"),
    ("fp16 subnormals flushed to zero", "v = ldexpf((float)f, -24);", "v = 0.0f * (float)f;"),
    ("A16 product transposed",
     "double p = (double)load_elem(x, dtype, m * ldx + k) * (double)t[n * K + k];",
     "double p = (double)load_elem(x, dtype, m * ldx + k) * (double)t[(k % N) * K + (n % K)];"),
    ("A16 scale left out", "y[m * N + n] = s * (double)w_scale[n];", "y[m * N + n] = s;"),
    ("A16 drops the last k", "for (int64_t k = 0; k < K; ++k) {\n                double p",
     "for (int64_t k = 0; k < K - 1; ++k) {\n                double p"),
    ("I2_S strided fields in reversed bit order", "6 - 2 * (int)(v / 32)", "2 * (int)(v / 32)"),
    ("I2_S consecutive fields in reversed bit order", "6 - 2 * (int)(v % 4)", "2 * (int)(v % 4)"),
    ("I2_S stride of 16", "return consecutive ? v / 4 : v % 32;", "return consecutive ? v / 4 : v % 16;"),
    ("I2_S scale not stored", "memcpy(out + total / 4, &s, sizeof s);", "(void)s;"),
    ("I2_S codes offset by 2", "unsigned c = (unsigned)(t[i] + 1);", "unsigned c = (unsigned)(t[i] + 2) & 3u;"),
    ("ActQuant of a token whose 127/amax overflows fp32 (R5 only for amax == 0)",
     "if (!(sa <= FLT_MAX)) {                    /* R5 */\n            for (int64_t k = 0; k < Kp; ++k)",
     "if (amax == 0.0f) {\n            for (int64_t k = 0; k < Kp; ++k)"),
    ("RMSNorm -> ActQuant of a token whose 127/amax overflows fp32",
     "if (!(sa <= FLT_MAX)) {                    /* R5 */\n            a_scale[m] = 0.0f;",
     "if (amax == 0.0f) {\n            a_scale[m] = 0.0f;"),
]


def _run_mutant(args):
    idx, (name, old, new), src, tmp = args
    assert src.count(old) == 1, f"mutation '{name}' does not match the source exactly once"
    c_file = tmp / f"mutant{idx}.c"
    c_file.write_text(src.replace(old, new))
    so = tmp / f"mutant{idx}.so"
    orc_mod.build(source=c_file, out=so)
    out = subprocess.run([sys.executable, str(HERE / "pins.py"), str(so)],
                         capture_output=True, text=True, timeout=300)
    caught = json.loads(out.stdout.strip().splitlines()[-1]) if out.returncode == 0 else ["<crashed>"]
    return name, caught


def test_every_planted_mistake_is_caught(tmp_path):
    src = orc_mod.SOURCE.read_text()
    jobs = [(i, m, src, tmp_path) for i, m in enumerate(MUTANTS)]
    with ThreadPoolExecutor(max_workers=6) as pool:
        results = list(pool.map(_run_mutant, jobs))
    missed = [name for name, caught in results if not caught]
    assert not missed, f"pins missed: {missed}"
