#!/usr/bin/env python3
"""Throughput of the W1.58A8 BitLinear on one MI355X; prints one JSON line.

Headline (``value``): decode GEMV packed-weight GB/s at M = 1 on the
BitNet-b1.58-2B-shaped 30-layer stream (210 projections, 521 MB of packed
ternary weights, one token per projection).  A step is one pass over all 210
projections: per-token ActQuant, the ternary product and the dequant epilogue,
run as one grouped launch.

``gemm``: prefill int8 TOPS at M = 4096 on the BitNet-b1.58-2B-shaped prefill
(fused gate|up 2560->13824, down 6912->2560, q|k|v 2560->3840).  A step is,
for each projection, ActQuant followed by the int8-MFMA GEMM.

Each part carries a ``roofline`` object for its dominant kernel (algorithmic
bytes or int ops per launch over the launch's average duration, timed with HIP
events on the stream the kernel runs on) and a ``cpu_baseline`` object: the
plain CPU oracle, untuned, timed on a bounded sample of the same workload on
this host's cores.  Inputs are seeded synthetic tensors of the workloads'
shapes; weights are packed before timing (packing is offline).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

METRIC = "BitLinear GEMV packed-weight GB/s (M=1) and GEMM int8 TOPS (M=4096), % of peak"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
INT8_PEAK_TOPS = 5000.0         # MI355X dense int8 MFMA, published (5.0 POPS)
PROFILES = ROOT / "profiles"


def kernel_source_hash(*names: str) -> str:
    h = hashlib.sha256()
    for n in names:
        h.update((ROOT / "ternary_weight_bitlinear_amd" / "csrc" / n).read_bytes())
    return h.hexdigest()[:16]


def traffic_from_profile(name: str, src_hash: str, key: str = "hbm_bytes_per_launch"):
    """HBM bytes per launch from a committed counter summary (profiles/<name>_traffic.md,
    lines "- key: value"; `key` names the figure when the summary covers several
    shapes), or None when it was taken on a different kernel source."""
    f = PROFILES / f"{name}_traffic.md"
    if not f.exists():
        return None
    fields = {}
    for ln in f.read_text().splitlines():
        if ln.startswith("- ") and ": " in ln:
            k, v = ln[2:].split(": ", 1)
            fields[k.strip()] = v.strip().strip("`")
    if fields.get("kernel_source_hash") != src_hash:
        return None
    try:
        return float(fields[key])
    except (KeyError, ValueError):
        return None


def progress(msg: str) -> None:
    """A line on stderr per finished leg (the JSON result goes to stdout)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ------------------------------------------------------------------- decode

def setup_decode(tw, wl, torch, layers: int):
    w = wl.WORKLOADS["c2"]
    items, nbytes = [], 0
    for layer in range(layers):
        for i, p in enumerate(w.projections):
            W = wl.weight_for(w, i, layer=layer, device="cuda")
            pw = tw.pack(W)
            del W
            x = wl.activation_for(w, i, layer=layer, device="cuda")
            y = torch.empty((1, p.N), dtype=torch.float32, device="cuda")
            items.append((x, pw, y))
            nbytes += p.N * p.K // 4
    return items, nbytes


# Measured on MI355X: after the GPU has been idle (setup, another leg), its
# throughput climbs for tens of milliseconds of continuous work (the c2 decode
# from 5.09 to a steady 5.36-5.38 TB/s over ~10 ms of launches, the c5 prefill
# step from 1.56 to 1.82 int8 POPS over ~40 ms), so every timed region follows
# a warm-up: the headline legs exactly `warmup` steps (default 300, 30 ms of
# decode launches), the others at least MIN_WARM_MS of work.
MIN_WARM_MS = 30.0


def time_region(torch, fn, steps: int, warmup: int, min_warm_ms: float = MIN_WARM_MS):
    t0 = time.perf_counter()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    while (time.perf_counter() - t0) * 1e3 < min_warm_ms:
        for _ in range(8):
            fn()
        torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        fn()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps      # ms per step


def time_each(torch, fn, n: int, warmup: int = 2):
    """Device time of each of n calls of fn (HIP events around every call on the
    current stream): a list of ms, for per-dispatch median and min."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for a, b in ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]


def time_calls_graph(torch, fn, steps: int, reps: int = 10):
    """Device time of one call of fn: a HIP graph of `reps` back-to-back calls,
    replayed (host launch overhead excluded, as in the other single-call legs)."""
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            fn()
    return time_region(torch, g.replay, steps, 2) / reps


def dispatch_stats(times_ms):
    xs = sorted(times_ms)
    return dict(n=len(xs), median_us=xs[len(xs) // 2] * 1e3, min_us=xs[0] * 1e3, max_us=xs[-1] * 1e3)


def cpu_model() -> str:
    try:
        for ln in Path("/proc/cpuinfo").read_text().splitlines():
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def applicable_roofline(M: int, N: int, K: int, out_bytes: int, seconds: float) -> dict:
    """The shape's bound: the larger of its MFMA time (2MNK at the int8 peak) and
    its HBM time (M*Kp + N*K/4 + M*N*out_bytes at the HBM peak)."""
    Kp = (K + 127) // 128 * 128
    ops = 2 * M * N * K
    nbytes = M * Kp + N * K // 4 + M * N * out_bytes
    t_mfma = ops / (INT8_PEAK_TOPS * 1e12)
    t_hbm = nbytes / (HBM_PEAK_GBPS * 1e9)
    return dict(bound="mfma" if t_mfma >= t_hbm else "hbm", frac_of_mfma_peak=t_mfma / seconds,
                frac_of_applicable=max(t_mfma, t_hbm) / seconds, algorithmic_bytes=nbytes)


def zero_fraction(pws) -> float:
    """Zero codes over all weights of the packed tensors (the packer's counts)."""
    zeros = sum(int(pw.zero_count.sum()) for pw in pws)
    total = sum(pw.N * pw.K for pw in pws)
    return zeros / total


def bench_decode(tw, wl, torch, steps, warmup, per_call: bool):
    items, nbytes = setup_decode(tw, wl, torch, 30)
    group = tw.GroupedBitLinear(items)
    ms = time_region(torch, group, steps, warmup, min_warm_ms=0.0)     # one launch per step; exactly W warm-up
    gbps = nbytes / (ms * 1e-3) / 1e9
    per = dispatch_stats(time_each(torch, group, max(steps, 20)))
    src = kernel_source_hash("gemv.hip", "gemv.h", "device_common.h", "codes_bf16.h")
    out = dict(value=gbps, ms_per_step=ms, bytes=nbytes, launches_per_step=1, per_dispatch=per,
               zero_code_fraction=zero_fraction([pw for _, pw, _ in items]),
               roofline=dict(bound="hbm", achieved=gbps, peak=HBM_PEAK_GBPS, unit="GB/s",
                             frac=gbps / HBM_PEAK_GBPS,
                             traffic=traffic_from_profile("decode_gemv_bitnet2b_30_layers_m1", src)))
    if per_call:
        # the same 210 projections as 210 single-problem calls (one fused launch each),
        # replayed from a HIP graph: what a decoder that cannot group its calls pays
        ws = [(torch.empty((1, tw.padded_k(pw.K)), dtype=torch.int8, device="cuda"),
               torch.empty(1, dtype=torch.float32, device="cuda"),
               torch.empty(1, dtype=torch.int32, device="cuda")) for _, pw, _ in items]

        def calls():
            for (x, pw, y), w_ in zip(items, ws):
                tw.bitlinear(x, pw, out=y, workspace=w_)
        calls()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            calls()
        ms_pc = time_region(torch, g.replay, max(steps // 2, 3), 2)
        out["per_call"] = dict(value=nbytes / (ms_pc * 1e-3) / 1e9, unit="GB/s", ms_per_step=ms_pc,
                               launches_per_step=len(items), note="one fused launch per projection, HIP graph")
    del group, items
    torch.cuda.empty_cache()
    return out


def bench_norm(tw, wl, torch, steps, warmup):
    """The projections' input norm ("BitNet-Embeddings" guide, s3.1): the c2 grouped
    decode with an RMSNorm before every projection (the down projection's input being
    silu(gate) * up), and the standalone RMSNorm -> ActQuant kernel at the prefill
    token count."""
    items, nbytes = setup_decode(tw, wl, torch, 30)
    norms = []
    for x, pw, _ in items:
        K = pw.K
        g = (1.0 + 0.2 * torch.randn(K, device="cuda")).to(torch.bfloat16)
        up = torch.randn_like(x) if K == 6912 else None
        norms.append((g, up, 1e-6))
    group = tw.GroupedBitLinear(items, norms)
    ms = time_region(torch, group, steps, warmup)
    out = dict(decode=dict(value=nbytes / (ms * 1e-3) / 1e9, unit="GB/s", ms_per_step=ms, kernel=group.kernel,
                           note="c2 grouped decode with a per-projection RMSNorm (down: silu(gate)*up) "
                                "fused into the token prologue; GB/s of packed weights"))
    del group, items, norms
    torch.cuda.empty_cache()
    # standalone RMSNorm -> ActQuant at M = 4096 (prefill): HBM-bound, bytes = inputs + g + q + scales
    res = {}
    for name, K, gated in (("qkv_gate_up_input", 2560, False), ("down_input", 6912, True)):
        M = 4096
        x = torch.randn((M, K), device="cuda").to(torch.bfloat16)
        up = torch.randn_like(x) if gated else None
        g = (1.0 + 0.2 * torch.randn(K, device="cuda")).to(torch.bfloat16)
        q = torch.empty((M, tw.padded_k(K)), dtype=torch.int8, device="cuda")
        a = torch.empty(M, dtype=torch.float32, device="cuda")
        r = torch.empty(M, dtype=torch.int32, device="cuda")
        stream = torch.cuda.current_stream().cuda_stream
        L = tw._lib.lib()

        def run():
            tw._lib.check(L.bitnet_rmsnorm_act_quant(stream, x.data_ptr(), up.data_ptr() if gated else None,
                                                     tw._lib.BF16, M, K, K, g.data_ptr(), tw._lib.BF16, 1e-6,
                                                     q.data_ptr(), a.data_ptr(), r.data_ptr()))
        ms_k = time_region(torch, run, steps * 5, warmup)
        nb = (2 if gated else 1) * 2 * M * K + 2 * K + M * tw.padded_k(K) + 8 * M
        gbps = nb / (ms_k * 1e-3) / 1e9
        src = kernel_source_hash("act_quant.hip", "device_common.h")
        res[name] = dict(M=M, K=K, gated=gated, us_per_launch=ms_k * 1e3, value=gbps, unit="GB/s",
                         roofline=dict(bound="hbm", achieved=gbps, peak=HBM_PEAK_GBPS, unit="GB/s",
                                       frac=gbps / HBM_PEAK_GBPS, algorithmic_bytes=nb,
                                       traffic=traffic_from_profile("rmsnorm_act_quant_m4096", src,
                                                                    f"hbm_bytes_per_launch_{name}")))
        del x, up, g, q, a, r
    out["rmsnorm_act_quant"] = res
    torch.cuda.empty_cache()
    return out


def bench_a16(tw, wl, torch, steps, warmup):
    """The W1.58A16 variant (BitVLA s5: bf16 activations, ternary weights) at M = 1:
    the c2 30-layer stream as one grouped streaming launch and as a HIP graph of
    210 launches, and one large projection (gate|up 13824 x 2560) alone; GB/s of
    packed weights."""
    items, nbytes = setup_decode(tw, wl, torch, 30)

    def calls():
        for x, pw, y in items:
            tw.linear_a16(x, pw, out=y)
    calls()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    ms = time_region(torch, g.replay, steps, 2)     # a graph of many calls: 2 replays + the minimum warm-up time
    out = dict(stream=dict(value=nbytes / (ms * 1e-3) / 1e9, unit="GB/s", ms_per_step=ms, launches_per_step=210))
    group = tw.GroupedBitLinear(items, a16=True)
    msg = time_region(torch, group, steps, warmup)
    gbps_g = nbytes / (msg * 1e-3) / 1e9
    src = kernel_source_hash("gemv.hip", "gemv.h", "device_common.h", "codes_bf16.h")
    out["grouped"] = dict(value=gbps_g, unit="GB/s", ms_per_step=msg, kernel=group.kernel, launches_per_step=1,
                          roofline=dict(bound="hbm", achieved=gbps_g, peak=HBM_PEAK_GBPS, unit="GB/s",
                                        frac=gbps_g / HBM_PEAK_GBPS,
                                        traffic=traffic_from_profile("decode_a16_bitnet2b_30_layers_m1", src)))
    # the same group with fp16 activations (fp16 matrix cores)
    items16 = [(x.to(torch.float16), pw, y) for x, pw, y in items]
    group16 = tw.GroupedBitLinear(items16, a16=True)
    ms16 = time_region(torch, group16, steps, warmup)
    out["grouped_fp16"] = dict(value=nbytes / (ms16 * 1e-3) / 1e9, unit="GB/s", ms_per_step=ms16,
                               kernel=group16.kernel, launches_per_step=1, activations="float16")
    del g, group, group16, items, items16
    torch.cuda.empty_cache()
    W = wl.draw_weight((13824, 2560), seed=3, device="cuda")
    pw = tw.pack(W)
    x = wl.draw_activation((1, 2560), seed=4, device="cuda")
    y = torch.empty((1, 13824), device="cuda")
    ms1 = time_calls_graph(torch, lambda: tw.linear_a16(x, pw, out=y), steps)
    nb = 13824 * 2560 // 4
    gbps = nb / (ms1 * 1e-3) / 1e9
    src1 = kernel_source_hash("gemv_a16.hip", "gemv.h", "device_common.h", "codes_bf16.h")
    out["gate_up_13824x2560"] = dict(value=gbps, unit="GB/s", us_per_launch=ms1 * 1e3,
                                     roofline=dict(bound="hbm", achieved=gbps, peak=HBM_PEAK_GBPS, unit="GB/s",
                                                   frac=gbps / HBM_PEAK_GBPS,
                                                   traffic=traffic_from_profile("decode_a16_single_13824x2560",
                                                                                src1)))
    return out


def cpu_baseline_decode(wl, torch, budget_s: float, max_layers: int = 3):
    """The oracle's ActQuant + int dot + epilogue over the first layers' projections
    (weights quantised once, untimed), cycled until budget_s of timed work, on all
    the host's threads and again on one."""
    res = _cpu_decode(wl, torch, budget_s / 2, max_layers, None)
    one = _cpu_decode(wl, torch, budget_s / 2, max_layers, 1)
    res["one_thread"] = dict(value=one["value"], unit=one["unit"], cores=1, sample=one["sample"])
    res["cpu_model"] = cpu_model()
    return res


def _cpu_decode(wl, torch, budget_s: float, max_layers: int, nthreads):
    from oracle.oracle import Oracle
    orc = Oracle()
    w = wl.WORKLOADS["c2"]
    threads = nthreads or orc.max_threads()
    prepared = []
    for layer in range(max_layers):
        for i, p in enumerate(w.projections):
            W = wl.weight_for(w, i, layer=layer, device="cuda").cpu()
            x = wl.activation_for(w, i, layer=layer, device="cuda").cpu()
            t, ws, _, _ = orc.weight_quant(W.view(torch.int16).numpy().view("uint16"))
            prepared.append((x.view(torch.int16).numpy().view("uint16"), t, ws, p.N * p.K // 4))
    done_bytes, spent, passes = 0, 0.0, 0
    while spent < budget_s:
        for xb, t, ws, nb in prepared:
            t0 = time.perf_counter()
            q, a, _ = orc.act_quant(xb)
            acc = orc.int_dot(q, t, nthreads=threads)
            orc.epilogue(acc, a, ws)
            spent += time.perf_counter() - t0
            done_bytes += nb
        passes += 1
    return dict(value=done_bytes / spent / 1e9, unit="GB/s", cores=threads, kind="oracle",
                sample=f"the first {max_layers} of 30 decode layers ({len(prepared)} projections, "
                       f"{sum(nb for *_, nb in prepared) / 1e6:.1f} MB packed) {passes} times over, "
                       f"ActQuant + int dot + epilogue, {spent:.1f} s")


# ------------------------------------------------------------------- prefill

def bench_prefill(tw, wl, torch, steps, warmup, out_dtype):
    w = wl.WORKLOADS["c5"]
    projs = []
    for i, p in enumerate(w.projections):
        pw = tw.pack(wl.weight_for(w, i, device="cuda"), p.segments or None)
        x = wl.activation_for(w, i, device="cuda")
        q = torch.empty((w.M, tw.padded_k(p.K)), dtype=torch.int8, device="cuda")
        a = torch.empty(w.M, dtype=torch.float32, device="cuda")
        r = torch.empty(w.M, dtype=torch.int32, device="cuda")
        y = torch.empty((w.M, p.N), dtype=out_dtype, device="cuda")
        projs.append((p, pw, x, q, a, r, y))
    ops = sum(2 * w.M * p.N * p.K for p, *_ in projs)

    def quant(p, x, q, a, r):
        tw._lib.check(tw._lib.lib().bitnet_act_quant(torch.cuda.current_stream().cuda_stream, x.data_ptr(),
                                                     tw._dtype(x), w.M, p.K, p.K, q.data_ptr(), a.data_ptr(),
                                                     r.data_ptr()))

    def step():
        for p, pw, x, q, a, r, y in projs:
            quant(p, x, q, a, r)
            tw.linear(q, a, r, pw, out=y)

    def gemms():
        for p, pw, x, q, a, r, y in projs:
            tw.linear(q, a, r, pw, out=y)

    # Both timed regions replay HIP graphs, so host-side submission never leaves
    # the GPU idle between launches: a step is ActQuant + GEMM per projection;
    # the GEMM-only graph gives the average duration of one GEMM launch.
    step()
    torch.cuda.synchronize()
    g_step, g_gemm = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_step):
        step()
    reps = 4
    with torch.cuda.graph(g_gemm):
        for _ in range(reps):
            gemms()
    ms = time_region(torch, g_step.replay, steps, warmup, min_warm_ms=0.0)   # exactly W warm-up steps
    gemm_ms = time_region(torch, g_gemm.replay, max(steps // 2, 3), 2) / (reps * len(projs))
    per_shape = {}
    for p, pw, x, q, a, r, y in projs:
        t_each = time_each(torch, lambda: tw.linear(q, a, r, pw, out=y), max(steps, 20))
        st = dispatch_stats(t_each)
        st["tops_at_median"] = 2 * w.M * p.N * p.K / (st["median_us"] * 1e-6) / 1e12
        per_shape[f"{p.name} {w.M}x{p.N}x{p.K}"] = st
    ops_per_launch = ops / len(projs)
    achieved = ops_per_launch / (gemm_ms * 1e-3) / 1e12
    tops = ops / (ms * 1e-3) / 1e12
    src = kernel_source_hash("gemm.hip", "device_common.h")
    return dict(metric="GEMM int8 TOPS (M=4096)", value=tops, unit="TOPS", ms_per_step=ms,
                config=dict(workload=w.name, M=w.M, projections=[f"{p.name} {p.K}->{p.N}" for p, *_ in projs],
                            out_dtype=str(out_dtype).replace("torch.", ""),
                            step="ActQuant + GEMM per projection"),
                roofline=dict(bound="mfma", achieved=achieved, peak=INT8_PEAK_TOPS, unit="TOPS",
                              frac=achieved / INT8_PEAK_TOPS,
                              traffic=traffic_from_profile("prefill_gemm_bitnet2b_m4096", src)),
                gemm_ms_per_launch=gemm_ms, launches_per_step=2 * len(projs), per_dispatch=per_shape,
                zero_code_fraction=zero_fraction([pw for _, pw, *_ in projs]),
                timing="HIP graph replays: whole steps, and GEMM launches alone; per_dispatch: HIP events "
                       "around single launches")


def bench_configs(tw, wl, torch, steps, warmup):
    """The other configurations, each timed on its own: the c1 2560 x 2560
    decode cold (a ring of 320 distinct packed copies, 524 MB, more than twice
    the MALL, as single calls replayed from a HIP graph and as one grouped
    launch) and warm as one call repeated on cached weights, the c2 stream at
    M = 2, 4, 8 (grouped), the c3 (SigLIP, M = 2048), c4 (embedder, M = 8192)
    and c5 prefill GEMMs per shape with bf16 and fp32 output (each against the
    MFMA peak and its applicable roofline), with each workload's zero-code
    fraction, c4 again with its shared-input projections fused (q|k|v and
    gate|up as segmented weights), and ActQuant alone at the c5 inputs."""
    steps = max(3, min(steps, 10))
    out = {}
    # c1 ring
    w1 = wl.WORKLOADS["c1"]
    p1 = w1.projections[0]
    ring = []
    for i in range(320):
        pw = tw.pack(wl.weight_for(w1, 0, layer=i, device="cuda"))
        x = wl.activation_for(w1, 0, layer=i, device="cuda")
        ring.append((x, pw, torch.empty((1, p1.N), device="cuda")))
    nb = len(ring) * p1.N * p1.K // 4
    ws = (torch.empty((1, tw.padded_k(p1.K)), dtype=torch.int8, device="cuda"), torch.empty(1, device="cuda"),
          torch.empty(1, dtype=torch.int32, device="cuda"))

    def calls():
        for x, pw, y in ring:
            tw.bitlinear(x, pw, out=y, workspace=ws)
    calls()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    ms = time_region(torch, g.replay, steps, 2)     # a graph of many calls: 2 replays + the minimum warm-up time
    out["c1_ring_single_calls"] = dict(value=nb / (ms * 1e-3) / 1e9, unit="GB/s", us_per_call=ms * 1e3 / len(ring),
                                       calls=len(ring), bytes=nb)
    group = tw.GroupedBitLinear(ring)
    msg = time_region(torch, group, steps, warmup)
    out["c1_ring_grouped"] = dict(value=nb / (msg * 1e-3) / 1e9, unit="GB/s", ms_per_launch=msg, kernel=group.kernel)
    x0, pw0, y0 = ring[0]
    warm = dispatch_stats(time_each(torch, lambda: tw.bitlinear(x0, pw0, out=y0, workspace=ws), 200, warmup=20))
    out["c1_warm_single_call"] = dict(warm, note="one 2560 x 2560 BitLinear called repeatedly on the same "
                                            "weights (in cache): per-call device time, HIP events",
                                      zero_code_fraction=zero_fraction([pw0]))
    del g, group, ring
    torch.cuda.empty_cache()
    # c2 at M = 2, 4, 8
    items, nbytes = setup_decode(tw, wl, torch, 30)
    res = {}
    for M in (2, 4, 8):
        its = [(wl.draw_activation((M, pw.K), seed=7000 + 10 * M + i, device="cuda"), pw,
                torch.empty((M, pw.N), device="cuda")) for i, (_, pw, _) in enumerate(items)]
        gm = tw.GroupedBitLinear(its)
        msm = time_region(torch, gm, steps, warmup)
        res[f"M{M}"] = dict(value=nbytes / (msm * 1e-3) / 1e9, unit="GB/s", ms_per_step=msm, kernel=gm.kernel)
        del gm, its
    out["c2_grouped_multi_token"] = res
    del items
    torch.cuda.empty_cache()
    # prefill GEMMs per shape

    def time_projections(M, projs, out_dtypes):
        """int8 TOPS of each projection (name, N, K, packed weight, activation) with each
        output dtype, % of the MFMA peak and % of the shape's applicable min(MFMA, HBM)
        roofline, and the aggregate over the projections."""
        res = dict(zero_code_fraction=zero_fraction([pw for _, _, _, pw, _ in projs]))
        quant = [tw.act_quant(x) for *_, x in projs]
        for out_dtype in out_dtypes:
            rows, tot_ops, tot_ms, tot_bound = [], 0, 0.0, 0.0
            for (pname, N, K, pw, _), (q, a, r) in zip(projs, quant):
                y = torch.empty((M, N), dtype=out_dtype, device="cuda")
                gg = torch.cuda.CUDAGraph()
                tw.linear(q, a, r, pw, out=y)
                torch.cuda.synchronize()
                with torch.cuda.graph(gg):
                    for _ in range(4):
                        tw.linear(q, a, r, pw, out=y)
                ms_l = time_region(torch, gg.replay, steps, 2) / 4
                ops = 2 * M * N * K
                tops = ops / (ms_l * 1e-3) / 1e12
                roof = applicable_roofline(M, N, K, y.element_size(), ms_l * 1e-3)
                rows.append(dict(shape=f"{pname} {M}x{N}x{K}", us=ms_l * 1e3, tops=tops, **roof))
                tot_ops += ops
                tot_ms += ms_l
                tot_bound += roof["frac_of_applicable"] * ms_l
                del y, gg
            agg = tot_ops / (tot_ms * 1e-3) / 1e12
            res[str(out_dtype).replace("torch.", "")] = dict(
                tops=agg, frac_of_mfma_peak=agg / INT8_PEAK_TOPS, frac_of_applicable=tot_bound / tot_ms, shapes=rows)
        del quant
        return res

    def gemm_shapes(name, out_dtypes):
        """Every projection of a prefill workload, one launch each."""
        w = wl.WORKLOADS[name]
        projs = [(p.name, p.N, p.K, tw.pack(wl.weight_for(w, i, device="cuda"), p.segments or None),
                  wl.activation_for(w, i, device="cuda")) for i, p in enumerate(w.projections)]
        res = dict(workload=w.name, **time_projections(w.M, projs, out_dtypes))
        del projs
        torch.cuda.empty_cache()
        return res

    def gemm_c4_shared_inputs(out_dtypes):
        """c4 with the projections that read the same input packed as one segmented
        weight, as c5 packs its gate|up and q|k|v: q|k|v (N = 4096, segments
        2048/1024/1024) and gate|up (N = 6144, 3072/3072), each segment with its own
        scale, so every code and output equals that of the separate projection; o and
        down as before.  Four launches instead of seven for the same int ops."""
        w = wl.WORKLOADS["c4"]
        idx = {p.name: i for i, p in enumerate(w.projections)}
        projs = []
        for label, members in (("q|k|v", ("q_proj", "k_proj", "v_proj")), ("o", ("o_proj",)),
                               ("gate|up", ("gate_proj", "up_proj")), ("down", ("down_proj",))):
            ps = [w.projections[idx[m]] for m in members]
            W = torch.cat([wl.weight_for(w, idx[m], device="cuda") for m in members], 0)
            pw = tw.pack(W, [p.N for p in ps] if len(ps) > 1 else None)
            projs.append((label, W.shape[0], ps[0].K, pw, wl.activation_for(w, idx[members[0]], device="cuda")))
            del W
        res = dict(workload=w.name + "-shared-input-projections-fused", **time_projections(w.M, projs, out_dtypes))
        del projs
        torch.cuda.empty_cache()
        return res
    out["gemm_c3"] = gemm_shapes("c3", (torch.bfloat16, torch.float32))
    out["gemm_c4"] = gemm_shapes("c4", (torch.bfloat16, torch.float32))
    out["gemm_c4_shared_inputs_fused"] = gemm_c4_shared_inputs((torch.bfloat16, torch.float32))
    out["gemm_c5"] = gemm_shapes("c5", (torch.bfloat16, torch.float32))
    # ActQuant alone (HBM-bound: 2 B in + 1 B out per element, 8 B per token)
    aq = {}
    for K in (2560, 6912):
        M = 4096
        x = wl.draw_activation((M, K), seed=9000 + K, device="cuda")
        q = torch.empty((M, tw.padded_k(K)), dtype=torch.int8, device="cuda")
        a = torch.empty(M, dtype=torch.float32, device="cuda")
        r = torch.empty(M, dtype=torch.int32, device="cuda")
        L = tw._lib.lib()
        stream = torch.cuda.current_stream().cuda_stream

        def run():
            tw._lib.check(L.bitnet_act_quant(stream, x.data_ptr(), tw._lib.BF16, M, K, K, q.data_ptr(), a.data_ptr(),
                                             r.data_ptr()))
        ms_a = time_region(torch, run, steps * 5, warmup)
        nb_a = 2 * M * K + M * tw.padded_k(K) + 8 * M
        gbps = nb_a / (ms_a * 1e-3) / 1e9
        src = kernel_source_hash("act_quant.hip", "device_common.h")
        aq[f"M{M}_K{K}"] = dict(us=ms_a * 1e3, value=gbps, unit="GB/s", frac_of_hbm_peak=gbps / HBM_PEAK_GBPS,
                                roofline=dict(bound="hbm", achieved=gbps, peak=HBM_PEAK_GBPS, unit="GB/s",
                                              frac=gbps / HBM_PEAK_GBPS, algorithmic_bytes=nb_a,
                                              traffic=traffic_from_profile("act_quant_m4096", src,
                                                                           f"hbm_bytes_per_launch_k{K}")))
        del x, q, a, r
    out["act_quant"] = aq
    # per-256-block weight scales: the c5 GEMMs with block-scaled weights (bf16 out),
    # and one 2560 x 2560 projection at M = 1
    w5 = wl.WORKLOADS["c5"]
    rows, tot_ops, tot_ms = [], 0, 0.0
    for i, p in enumerate(w5.projections):
        pb = tw.pack_blocked(wl.weight_for(w5, i, device="cuda"))
        q, a, _ = tw.act_quant(wl.activation_for(w5, i, device="cuda"))
        y = torch.empty((w5.M, p.N), dtype=torch.bfloat16, device="cuda")
        gg = torch.cuda.CUDAGraph()
        tw.linear_blocked(q, a, pb, out=y)
        torch.cuda.synchronize()
        with torch.cuda.graph(gg):
            for _ in range(4):
                tw.linear_blocked(q, a, pb, out=y)
        ms_l = time_region(torch, gg.replay, steps, 2) / 4
        ops = 2 * w5.M * p.N * p.K
        rows.append(dict(shape=f"{p.name} {w5.M}x{p.N}x{p.K}", us=ms_l * 1e3, tops=ops / (ms_l * 1e-3) / 1e12))
        tot_ops += ops
        tot_ms += ms_l
        del pb, q, a, y, gg
    agg = tot_ops / (tot_ms * 1e-3) / 1e12
    pb = tw.pack_blocked(wl.draw_weight((2560, 2560), seed=9100, device="cuda"))
    q, a, _ = tw.act_quant(wl.draw_activation((1, 2560), seed=9101, device="cuda"))
    y = torch.empty((1, 2560), dtype=torch.float32, device="cuda")
    ms_1 = time_calls_graph(torch, lambda: tw.linear_blocked(q, a, pb, out=y), steps)
    out["block_scaled"] = dict(gemm_c5=dict(tops=agg, frac_of_peak=agg / INT8_PEAK_TOPS, shapes=rows),
                               m1_2560x2560=dict(us=ms_1 * 1e3, value=2560 * 2560 / 4 / (ms_1 * 1e-3) / 1e9,
                                                 unit="GB/s", note="warm, single call on the streaming kernel, device time (HIP graph of 10 calls)"))
    del pb, q, a, y
    torch.cuda.empty_cache()
    # the c2 decode stream with block-scaled weights, one grouped launch (ActQuant fused)
    w2 = wl.WORKLOADS["c2"]
    items, nb_codes, nb_scales = [], 0, 0
    for layer in range(w2.layers):
        for i, p in enumerate(w2.projections):
            items.append((wl.activation_for(w2, i, layer=layer, device="cuda"),
                          tw.pack_blocked(wl.weight_for(w2, i, layer=layer, device="cuda")),
                          torch.empty((1, p.N), device="cuda")))
            nb_codes += p.N * p.K // 4
            nb_scales += (p.K + 255) // 256 * p.N * 4
    group = tw.GroupedBitLinear(items)
    ms_g = time_region(torch, group, steps, warmup)
    gbps = nb_codes / (ms_g * 1e-3) / 1e9
    srcb = kernel_source_hash("gemv.hip", "gemv.h", "device_common.h", "codes_bf16.h")
    out["block_scaled"]["c2_grouped_m1"] = dict(
        value=gbps, unit="GB/s", ms_per_step=ms_g, kernel=group.kernel, packed_bytes=nb_codes, scale_bytes=nb_scales,
        roofline=dict(bound="hbm", achieved=gbps, peak=HBM_PEAK_GBPS, unit="GB/s", frac=gbps / HBM_PEAK_GBPS,
                      traffic=traffic_from_profile("decode_blocked_bitnet2b_30_layers_m1", srcb)),
        with_scales_gbps=(nb_codes + nb_scales) / (ms_g * 1e-3) / 1e9, frac_of_hbm_peak=gbps / HBM_PEAK_GBPS,
        per_dispatch=dispatch_stats(time_each(torch, group, 20)),
        note="packed-code GB/s (N*K/4 per projection); with_scales counts the fp32 block scales too")
    del group, items
    torch.cuda.empty_cache()
    return out


def cpu_baseline_prefill(wl, torch, budget_s: float):
    """The oracle's ActQuant + int dot + epilogue on slices of 64 tokens of the
    prefill activations through all three projections, until budget_s of timed
    work or all 4096 tokens (weights quantised once, untimed), on all the host's
    threads and again on one."""
    res = _cpu_prefill(wl, torch, budget_s / 2, None)
    one = _cpu_prefill(wl, torch, budget_s / 2, 1)
    res["one_thread"] = dict(value=one["value"], unit=one["unit"], cores=1, sample=one["sample"])
    res["cpu_model"] = cpu_model()
    return res


def _cpu_prefill(wl, torch, budget_s: float, nthreads):
    from oracle.oracle import Oracle
    orc = Oracle()
    w = wl.WORKLOADS["c5"]
    threads = nthreads or orc.max_threads()
    prepared = []
    for i, p in enumerate(w.projections):
        W = wl.weight_for(w, i, device="cuda").cpu()
        t, ws, _, _ = orc.weight_quant(W.view(torch.int16).numpy().view("uint16"), p.segments or None)
        x = wl.activation_for(w, i, device="cuda").cpu().view(torch.int16).numpy().view("uint16")
        prepared.append((p, t, ws, x))
    ops, spent, tokens, rows = 0, 0.0, 0, 64
    while spent < budget_s and tokens < w.M:
        for p, t, ws, x in prepared:
            t0 = time.perf_counter()
            q, a, _ = orc.act_quant(x[tokens:tokens + rows])
            acc = orc.int_dot(q, t, nthreads=threads)
            orc.epilogue(acc, a, ws)
            spent += time.perf_counter() - t0
            ops += 2 * rows * p.N * p.K
        tokens += rows
    return dict(value=ops / spent / 1e12, unit="TOPS", cores=threads, kind="oracle",
                sample=f"{tokens} of 4096 tokens through all 3 prefill projections "
                       f"({ops / 1e9:.1f} G int ops), ActQuant + int dot + epilogue, {spent:.1f} s")


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=300,
                    help="untimed steps before each headline timed region (the GPU's throughput climbs "
                         "for tens of ms after idle; 300 decode launches are ~30 ms)")
    ap.add_argument("--cpu-seconds", type=float, default=16.0,
                    help="budget per CPU-baseline leg (half on all host threads, half on one)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-per-call", action="store_true")
    ap.add_argument("--no-norm", action="store_true", help="skip the input-norm measurements")
    ap.add_argument("--no-a16", action="store_true", help="skip the W1.58A16 measurements")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other configurations (c1 ring, c2 at M>1, c3/c4 GEMMs, ActQuant alone)")
    ap.add_argument("--only", choices=["decode", "prefill"], default=None)
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="first fill and copy a buffer of this many MiB three times: plain kernels of "
                         "known HBM traffic, for scaling FETCH_SIZE/WRITE_SIZE counters in a profiled run")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this BitLinear path runs on a single MI355X "
              "(multi-GPU sharding is a design note, not built). Run with --gpus 1.", file=sys.stderr)
        return 2

    import torch
    import ternary_weight_bitlinear_amd as tw
    from ternary_weight_bitlinear_amd import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    tw._lib.lib()   # fail loudly now if the HIP library is not built

    if args.calib_copy_mib > 0:
        src = torch.empty(args.calib_copy_mib << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            src.fill_(1)          # writes n bytes
            dst.copy_(src)        # reads n bytes, writes n bytes
        torch.cuda.synchronize()
        del src, dst
        torch.cuda.empty_cache()

    line = dict(metric=METRIC, value=None, unit="GB/s", n_gpus=1, steps=args.steps, warmup=args.warmup,
                ms_per_step=None, higher_is_better=True, scaling="weak", vs_baseline=None, dtype="int8",
                data="synthetic",
                config=dict(workload=wl.WORKLOADS["c2"].name, M=1, layers=30, projections=210,
                            launch="grouped: all 210 projections in one launch, ActQuant fused",
                            weights="bf16 latent N(0, 0.02), per-tensor absmean ternary",
                            activations="bf16 N(0, 1), one token per projection", out_dtype="float32"))
    if args.only in (None, "decode"):
        d = bench_decode(tw, wl, torch, args.steps, args.warmup, not args.no_per_call)
        progress("decode done")
        line.update(value=d["value"], ms_per_step=d["ms_per_step"], roofline=d["roofline"])
        line["config"]["packed_bytes"] = d["bytes"]
        if "per_call" in d:
            line["per_call"] = d["per_call"]
        if not args.no_cpu_baseline:
            line["cpu_baseline"] = cpu_baseline_decode(wl, torch, args.cpu_seconds)
            progress("decode cpu baseline done")
        if not args.no_norm:
            line["input_norm"] = bench_norm(tw, wl, torch, args.steps, args.warmup)
            progress("input norm done")
        if not args.no_a16:
            line["w158a16"] = bench_a16(tw, wl, torch, args.steps, args.warmup)
            progress("w158a16 done")
    if args.only in (None, "prefill"):
        g = bench_prefill(tw, wl, torch, args.steps, args.warmup, torch.bfloat16)
        progress("prefill done")
        if not args.no_cpu_baseline:
            g["cpu_baseline"] = cpu_baseline_prefill(wl, torch, args.cpu_seconds)
            progress("prefill cpu baseline done")
        line["gemm"] = g
        if args.only == "prefill":
            line.update(value=g["value"], unit="TOPS", ms_per_step=g["ms_per_step"], roofline=g["roofline"],
                        config=g["config"])
            line["config"]["workload"] = wl.WORKLOADS["c5"].name
    if args.only is None and not args.no_configs:
        line["configs"] = bench_configs(tw, wl, torch, args.steps, args.warmup)
        progress("configs done")
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
