"""Benchmark of the block-FP4 hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--skip-secondary] [--no-cpu-baseline]

Flagship step: one W4A16 decode product (8 bf16 activation rows x a 14336 x 4096 weight
matrix in two-level block FP4, bf16 output). Its throughput in GB/s of algorithmic
traffic is ``value``. Weights are pre-quantized on the device and kept resident in HBM;
the timed region rotates through 16 copies (over 512 MB) so the 256 MB Infinity Cache
cannot hold the stream, and launches are replayed from a HIP graph.

Also reported (same JSON line, "secondary"): the W4A4 prefill product (2048 x 4096 x
4096, activations quantized on the device every step) in TFLOP/s, the 8-layer W4A4/W4A8
policy stack, the 128-expert top-8 mixture-of-experts layer, quantization, the layout
repack, decode attention over the FP4 KV cache, the MX-native FP4 product, and the policy
stack under the W8A8 ("sensitive-w8") and static-activation-scale modes, each with its
roofline fraction; the oracle's CPU time on a bounded sample ("cpu_baseline").

Every leg's operands are rotated over more memory than the 256 MB Infinity Cache holds
(20 operand sets for the prefill-size products, 3 copies of the 8-layer stacks, the
mixture-of-experts weights alone are 344 MB), and every leg reports the per-launch
p10 / p50 / p90 over graph replays beside its average. The line also records the device's
clocks and power before and after, and the two ceilings measured on the same device in
the same run (the HBM read floor at the decode weights' size, and the sustained FP16 MFMA
rate with register operands), so that each roofline fraction is given against the spec
peak and against the measured ceiling.

Rank 0 prints one JSON line. Only one GPU is used; --gpus above 1 exits with a message.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "block-FP4 W4A4 GEMM TFLOPS + decode GEMV GB/s, as fraction of roofline"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0   # dense MFMA bf16/fp16
FP4_PEAK_TFLOPS = 10100.0   # dense MFMA fp4 (not reachable with 16-element E4M3 scales)
ROTATE = 16
ROTATE_GEMM = 20  # operand sets of the prefill-size products (20 x 25.7 MB > 256 MB)
STACK_COPIES = 3  # copies of the 8-layer stacks (3 x 153 MB)


def algorithmic_bytes_gemv(m, n, k):
    """Bytes the decode product must move: codes + micro + macro + A + C (bf16)."""
    return n * k // 2 + n * k // 16 + n * (k // 256) * 2 + m * k * 2 + m * n * 2


def algorithmic_bytes_gemm(m, n, k):
    """Prefill product with dynamic activation quantization: read A (bf16) once, read
    packed W once, write C (bf16)."""
    return m * k * 2 + n * k // 2 + n * k // 16 + n * (k // 256) * 2 + m * n * 2


def source_hash(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


KERNEL_SOURCES = {
    "gemv": ["block_scaled_fp4_e2m1_amd/csrc/gemv.hip", "block_scaled_fp4_e2m1_amd/csrc/fp4_device.h"],
    "gemm": ["block_scaled_fp4_e2m1_amd/csrc/gemm.hip", "block_scaled_fp4_e2m1_amd/csrc/fp4_device.h"],
    "attention": ["block_scaled_fp4_e2m1_amd/csrc/attention.hip", "block_scaled_fp4_e2m1_amd/csrc/fp4_device.h"],
    "quant": ["block_scaled_fp4_e2m1_amd/csrc/quant.hip", "block_scaled_fp4_e2m1_amd/csrc/fp4_device.h"],
    "repack": ["block_scaled_fp4_e2m1_amd/csrc/repack.hip", "block_scaled_fp4_e2m1_amd/csrc/fp4_device.h"],
    "probes": ["block_scaled_fp4_e2m1_amd/csrc/probes.hip"],
    "gemm_r8": ["block_scaled_fp4_e2m1_amd/csrc/gemm_r8.hip", "block_scaled_fp4_e2m1_amd/csrc/gemm_ops.h",
                "block_scaled_fp4_e2m1_amd/csrc/fp4_device.h"],
}


def load_traffic(name: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None when
    there is none or the kernel source changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"{name}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("source_hash") != source_hash(KERNEL_SOURCES[rec["kernel_group"]]):
        return None
    return rec.get("bytes_per_launch")


class Timer:
    """HIP-event timing on the stream the work is enqueued on."""

    def __init__(self, torch):
        self.torch = torch

    def region(self, fn, reps):
        t = self.torch
        s = t.cuda.current_stream()
        t.cuda.synchronize()
        e0, e1 = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        e0.record(s)
        for _ in range(reps):
            fn()
        e1.record(s)
        t.cuda.synchronize()
        return e0.elapsed_time(e1) / 1e3  # seconds


def capture(torch, fns):
    """A HIP graph replaying the given launches in order."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for f in fns:
            f()
    return g


def run_steps(torch, timer, graph, fns, steps):
    """Exactly ``steps`` launches: whole graph replays plus an eager remainder."""
    full, rest = divmod(steps, len(fns))

    def body():
        for _ in range(full):
            graph.replay()
        for f in fns[:rest]:
            f()
    return timer.region(body, 1)


def replay_samples(torch, graph, launches, reps):
    """Per-launch seconds of each graph replay (each replay's time over its `launches`
    launches), on the stream the replays run on: at least `reps` replays, at least 16, and
    at least 200 launches in all."""
    reps = max(reps, 16, -(-200 // max(1, launches)))
    s = torch.cuda.current_stream()
    evs = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        graph.replay()
        e1.record(s)
        evs.append((e0, e1))
    torch.cuda.synchronize()
    return np.array([a.elapsed_time(b) / 1e3 / launches for a, b in evs])


def pct_us(samples):
    """p10 / p50 / p90 of per-launch seconds, in microseconds."""
    return [round(float(np.percentile(samples, q)) * 1e6, 3) for q in (10, 50, 90)]


def count_histogram(counts, width):
    """Experts per bin of `width` routed rows: the first bin starts at the smallest count
    rounded down to a multiple of `width`."""
    lo = int(counts.min()) // width * width
    nb = (int(counts.max()) - lo) // width + 1
    hist = np.bincount((counts - lo) // width, minlength=nb)
    return dict(bin_rows=width, first_bin_start=lo, experts=[int(v) for v in hist])


def clone_q(fp4, q):
    """A device copy of a quantized tensor (its own memory: rotation defeats the caches)."""
    return fp4.QTensor(q.codes.clone(), q.micro.clone(), q.macro.clone(), q.rows, q.k, q.elem, q.layout)


def bench_decode(torch, fp4, workloads, steps, warmup):
    m, k, n = 8, 4096, 14336
    a, w, _ = workloads.decode()
    wq0 = fp4.quantize_fp4(torch.from_numpy(w).cuda(), layout=fp4.LAYOUT_TILED)
    del w
    copies = [wq0] + [fp4.QTensor(wq0.codes.clone(), wq0.micro.clone(), wq0.macro.clone(), n, k,
                                  0, fp4.LAYOUT_TILED) for _ in range(ROTATE - 1)]
    ad = torch.from_numpy(a).cuda().to(torch.bfloat16)
    outs = [torch.empty(m, n, dtype=torch.bfloat16, device="cuda") for _ in range(ROTATE)]
    fns = [(lambda q=q, o=o: fp4.gemm_w4aX(fp4.A16, ad, q, out=o)) for q, o in zip(copies, outs)]
    for i in range(warmup):
        fns[i % ROTATE]()
    torch.cuda.synchronize()
    g = capture(torch, fns)
    g.replay()
    torch.cuda.synchronize()
    timer = Timer(torch)
    secs = run_steps(torch, timer, g, fns, steps)
    per = secs / steps
    nbytes = algorithmic_bytes_gemv(m, n, k)
    # spread: per-launch average of each graph replay (16 launches), separate pass
    reps = []
    s_ = torch.cuda.current_stream()
    for _ in range(max(8, steps // ROTATE)):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s_)
        g.replay()
        e1.record(s_)
        reps.append((e0, e1))
    torch.cuda.synchronize()
    per_rep = np.array([a.elapsed_time(b) * 1e3 / ROTATE for a, b in reps])
    same = all(torch.equal(outs[0], o) for o in outs[1:])
    return dict(m=m, n=n, k=k, seconds=secs, per_launch_s=per, bytes=nbytes,
                gbs=nbytes / per / 1e9, flops=2 * m * n * k, outputs_identical=bool(same),
                launch_us_p10_p50_p90=[round(float(np.percentile(per_rep, q)), 3) for q in (10, 50, 90)])


def bench_prefill(torch, fp4, workloads, steps):
    """The W4A4 prefill product per step: activation pass + product, over 20 rotated
    (A, W, C) sets (514 MB of operands), from HIP graph replays."""
    m, k, n = 2048, 4096, 4096
    a, w, _ = workloads.prefill()
    wq0 = fp4.quantize_fp4(torch.from_numpy(w).cuda(), layout=fp4.LAYOUT_TILED)
    a0 = torch.from_numpy(a).cuda().to(torch.bfloat16)
    del a, w
    sets = [(a0, wq0)] + [(a0.clone(), clone_q(fp4, wq0)) for _ in range(ROTATE_GEMM - 1)]
    outs = [torch.empty(m, n, dtype=torch.bfloat16, device="cuda") for _ in sets]
    ws = torch.empty(fp4.fp4_workspace_bytes(fp4.A4, m, n, k), dtype=torch.uint8, device="cuda")
    fns = [(lambda x=x, q=q, o=o: fp4.gemm_w4aX(fp4.A4, x, q, out=o, workspace=ws)) for (x, q), o in zip(sets, outs)]
    for f in fns:
        f()
    g = capture(torch, fns)
    g.replay()
    timer = Timer(torch)
    steps = max(steps, len(fns))
    secs = run_steps(torch, timer, g, fns, steps)
    per = secs / steps
    spread = replay_samples(torch, g, len(fns), 8)
    same = all(torch.equal(outs[0], o) for o in outs[1:])
    flops = 2 * m * n * k
    tfl = flops / per / 1e12
    return dict(m=m, n=n, k=k, per_step_s=per, tflops=tfl, operand_sets_rotated=len(fns),
                step_us_p10_p50_p90=pct_us(spread), outputs_identical=bool(same),
                kernel=fp4.fp4_product_kernel(fp4.A4, torch.bfloat16, m, n, k),
                frac_bf16_peak=tfl / BF16_PEAK_TFLOPS, frac_fp4_peak=tfl / FP4_PEAK_TFLOPS,
                bytes=algorithmic_bytes_gemm(m, n, k))


def bench_mx(torch, fp4, workloads, steps):
    """The prefill product (2048 x 4096 x 4096) in the MX-native FP4 format on the
    block-scaled FP4 matrix instruction: per step the activations are quantized (E2M1,
    E8M0 per 32) and multiplied; the weights are quantized once. Also reports the accuracy
    of both formats against the unquantized float32 product of the same inputs (relative
    Frobenius error), the two-level W4A4 path of the pages beside the MX one."""
    m, k, n = 2048, 4096, 4096
    a, w, _ = workloads.prefill()
    wd = torch.from_numpy(w).cuda()
    ad = torch.from_numpy(a).cuda().to(torch.bfloat16)
    wq = fp4.quantize_mxfp4(wd)
    aq = fp4.quantize_mxfp4(ad)
    # 20 rotated operand sets (activations, their MX codes, weights, output)
    sets = []
    for i in range(ROTATE_GEMM):
        x = ad if i == 0 else ad.clone()
        wqi = wq if i == 0 else fp4.MxTensor(wq.codes.clone(), wq.scales.clone(), wq.rows, wq.k)
        sets.append((x, fp4.quantize_mxfp4(x), wqi, torch.empty(m, n, dtype=torch.bfloat16, device="cuda")))
    steps_fns = [(lambda x=x, q=q, wv=wv, o=o: (fp4.quantize_mxfp4(x, out=q), fp4.gemm_mxfp4(q, wv, out=o)))
                 for x, q, wv, o in sets]
    gemm_fns = [(lambda q=q, wv=wv, o=o: fp4.gemm_mxfp4(q, wv, out=o)) for x, q, wv, o in sets]
    timer = Timer(torch)
    res, spread = {}, {}
    for name, fns in (("step", steps_fns), ("gemm", gemm_fns)):
        for f in fns:
            f()
        g = capture(torch, fns)
        g.replay()
        n_steps = max(steps, len(fns))
        res[name] = run_steps(torch, timer, g, fns, n_steps) / n_steps
        spread[name] = pct_us(replay_samples(torch, g, len(fns), 8))
    flops = 2 * m * n * k
    # accuracy against the float32 product of the unquantized (bf16) activations and weights
    ref = ad.float() @ wd.t()
    mx = fp4.gemm_mxfp4(aq, wq, out_dtype=torch.float32)
    wq2 = fp4.quantize_fp4(wd, layout=fp4.LAYOUT_TILED)
    two = fp4.gemm_w4aX(fp4.A4, ad, wq2, out_dtype=torch.float32)
    nref = torch.linalg.norm(ref).item()
    err_mx = torch.linalg.norm(mx - ref).item() / nref
    err_two = torch.linalg.norm(two - ref).item() / nref
    torch.cuda.synchronize()
    tfl = flops / res["step"] / 1e12
    tfl_g = flops / res["gemm"] / 1e12
    return dict(m=m, n=n, k=k, per_step_s=res["step"], gemm_s=res["gemm"], tflops=tfl, gemm_tflops=tfl_g,
                operand_sets_rotated=len(sets), step_us_p10_p50_p90=spread["step"],
                gemm_us_p10_p50_p90=spread["gemm"],
                frac_fp4_peak=tfl / FP4_PEAK_TFLOPS, gemm_frac_fp4_peak=tfl_g / FP4_PEAK_TFLOPS,
                rel_error_vs_fp32_product=dict(mx_fp4=err_mx, two_level_w4a4=err_two))


def bench_quantize(torch, fp4, workloads, steps):
    """quantize_fp4 on its two hot uses: the decode weights (float32 [14336 x 4096] to the
    tiled E2M1 layout, done once per model load) and the prefill activations (bf16
    [2048 x 4096] to canonical E2M1). HBM-bound; GB/s of input + codes + scales."""
    out = {}
    _, w, _ = workloads.decode()
    wd = [torch.from_numpy(w).cuda()]
    wd.append(wd[0].clone())  # two copies (470 MB) so the Infinity Cache cannot hold the input
    del w
    n, k = wd[0].shape
    qs = [fp4.empty_qtensor(n, k, layout=fp4.LAYOUT_TILED) for _ in wd]
    fns = [(lambda x=x, q=q: fp4.quantize_fp4(x, layout=fp4.LAYOUT_TILED, out=q)) for x, q in zip(wd, qs)]
    for f in fns:
        f()
    timer = Timer(torch)
    reps = max(4, steps // 16)
    secs = timer.region(lambda: [f() for f in fns], reps) / (reps * len(fns))
    gw = capture(torch, fns)
    gw.replay()
    spread_w = replay_samples(torch, gw, len(fns), 8)
    nbytes = n * k * 4 + n * k // 2 + n * k // 16 + n * (k // 256) * 2
    out["weights_f32_tiled"] = dict(rows=n, k=k, per_call_s=secs, bytes=nbytes, inputs_rotated=len(fns),
                                    call_us_p10_p50_p90=pct_us(spread_w),
                                    gbs=nbytes / secs / 1e9, frac_hbm_peak=nbytes / secs / 1e9 / HBM_PEAK_GBS)
    del wd, qs, fns
    a, _, _ = workloads.prefill()
    a0 = torch.from_numpy(a).cuda().to(torch.bfloat16)
    m, k = a0.shape
    xs = [a0] + [a0.clone() for _ in range(ROTATE - 1)]
    qs = [fp4.empty_qtensor(m, k, layout=fp4.LAYOUT_CANONICAL) for _ in xs]
    fns = [(lambda x=x, q=q: fp4.quantize_fp4(x, layout=fp4.LAYOUT_CANONICAL, out=q)) for x, q in zip(xs, qs)]
    for f in fns:
        f()
    g = capture(torch, fns)
    g.replay()
    secs = run_steps(torch, timer, g, fns, max(ROTATE, steps)) / max(ROTATE, steps)
    spread_a = replay_samples(torch, g, len(fns), 8)
    nbytes = m * k * 2 + m * k // 2 + m * k // 16 + m * (k // 256) * 2
    out["activations_bf16_canonical"] = dict(rows=m, k=k, per_call_s=secs, bytes=nbytes, inputs_rotated=len(fns),
                                             call_us_p10_p50_p90=pct_us(spread_a),
                                             gbs=nbytes / secs / 1e9,
                                             frac_hbm_peak=nbytes / secs / 1e9 / HBM_PEAK_GBS)
    return out


def bench_dequantize(torch, fp4, workloads, steps):
    """dequantize_fp4 of the decode weights (14336 x 4096 E2M1, tiled) to bf16: codes,
    micro- and macro-scales read once, the bf16 matrix written once (GB/s of both). 8
    quantized copies rotate (268 MB) into two output buffers."""
    _, w, _ = workloads.decode()
    q0 = fp4.quantize_fp4(torch.from_numpy(w).cuda(), layout=fp4.LAYOUT_TILED)
    del w
    n, k = q0.rows, q0.k
    srcs = [q0] + [clone_q(fp4, q0) for _ in range(7)]
    outs = [torch.empty(n, k, dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    fns = [(lambda q=q, o=outs[i % 2]: fp4.dequantize_fp4(q, out=o)) for i, q in enumerate(srcs)]
    for f in fns:
        f()
    g = capture(torch, fns)
    g.replay()
    timer = Timer(torch)
    n_steps = max(len(fns), steps)
    secs = run_steps(torch, timer, g, fns, n_steps) / n_steps
    spread = replay_samples(torch, g, len(fns), 8)
    nbytes = n * k // 2 + n * k // 16 + n * (k // 256) * 2 + n * k * 2
    return {"tiled_to_bf16": dict(rows=n, k=k, per_call_s=secs, bytes=nbytes, inputs_rotated=len(fns),
                                  call_us_p10_p50_p90=pct_us(spread), gbs=nbytes / secs / 1e9,
                                  frac_hbm_peak=nbytes / secs / 1e9 / HBM_PEAK_GBS)}


def bench_repack(torch, fp4, workloads, steps):
    """repack_fp4 of the decode weights (14336 x 4096 E2M1), canonical -> tiled and back:
    codes, micro- and macro-scales read once and written once (GB/s of both). 16 source
    copies rotate (over 500 MB)."""
    _, w, _ = workloads.decode()
    can0 = fp4.quantize_fp4(torch.from_numpy(w).cuda(), layout=fp4.LAYOUT_CANONICAL)
    del w
    n, k = can0.rows, can0.k
    srcs = [can0] + [clone_q(fp4, can0) for _ in range(ROTATE - 1)]
    tils = [fp4.empty_qtensor(n, k, layout=fp4.LAYOUT_TILED) for _ in srcs]
    backs = [fp4.empty_qtensor(n, k, layout=fp4.LAYOUT_CANONICAL) for _ in srcs]
    nbytes = 2 * (n * k // 2 + n * k // 16 + n * (k // 256) * 2)
    timer = Timer(torch)
    out = {}
    for name, pairs in (("canonical_to_tiled", list(zip(srcs, tils))), ("tiled_to_canonical", list(zip(tils, backs)))):
        dst_layout = pairs[0][1].layout
        fns = [(lambda a=a, b=b, L=dst_layout: fp4.repack_fp4(a, L, out=b)) for a, b in pairs]
        for f in fns:
            f()
        g = capture(torch, fns)
        g.replay()
        n_steps = max(steps, len(fns))
        per = run_steps(torch, timer, g, fns, n_steps) / n_steps
        out[name] = dict(rows=n, k=k, per_call_s=per, bytes=nbytes, gbs=nbytes / per / 1e9,
                         frac_hbm_peak=nbytes / per / 1e9 / HBM_PEAK_GBS, inputs_rotated=len(fns),
                         call_us_p10_p50_p90=pct_us(replay_samples(torch, g, len(fns), 8)))
    torch.cuda.synchronize()
    out["round_trip_identical"] = bool(all(torch.equal(a.codes, b.codes) and torch.equal(a.micro, b.micro)
                                           and torch.equal(a.macro, b.macro) for a, b in zip(srcs, backs)))
    return out


def ceilings(torch, steps):
    """The two ceilings of the headline legs, measured on this device in this run: the HBM
    read floor at the decode weights' size (a plain streaming read of 16 rotated copies,
    512 workgroups of 256 threads, graph replays: the probes' best launch shape), and the
    sustained FP16 MFMA rate with register operands (2 waves per SIMD, 8 independent
    accumulators; no memory traffic, so an upper bound for a product kernel)."""
    import ctypes
    lib = probe_library()
    st = lambda: ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.zeros(1024, dtype=torch.int32, device="cuda")
    m, k, n = 8, 4096, 14336
    wbytes = n * k // 2 + n * k // 16 + n * (k // 256) * 2
    bufs = [torch.ones(wbytes // 4, dtype=torch.int32, device="cuda") for _ in range(ROTATE)]
    fns = [(lambda b=b: lib.probe_read(ctypes.c_void_p(b.data_ptr()), wbytes, ctypes.c_void_p(sink.data_ptr()),
                                       2 * cus, 256, st())) for b in bufs]
    for f in fns:
        assert f() == 0
    g = capture(torch, fns)
    g.replay()
    per = replay_samples(torch, g, ROTATE, max(16, steps // ROTATE))
    del bufs
    clocks = torch.zeros(2 * 2 * cus, dtype=torch.int64, device="cuda")
    blocks, chains, iters = 2 * cus, 8, 8192
    fn = lambda: lib.probe_mfma(0, chains, blocks, iters, ctypes.c_void_p(clocks.data_ptr()), st())
    timer = Timer(torch)
    for _ in range(8):
        assert fn() == 0
    t = float(np.median([timer.region(fn, 1) for _ in range(8)]))
    c = clocks.view(-1, 2).cpu().numpy().astype(np.float64)
    ghz = float(np.median(c[:, 0] / (c[:, 1] / 100e6))) / 1e9
    mfma_tflops = blocks * 4 * iters * chains * 16384 / t / 1e12
    return dict(read_floor_bytes=wbytes, read_floor_us_p10_p50_p90=pct_us(per),
                read_floor_gbs=wbytes / float(np.median(per)) / 1e9,
                mfma_f16_register_tflops=round(mfma_tflops, 1), mfma_probe_shader_ghz=round(ghz, 3))


def copy_probe(torch, mib=256, reps=4):
    """A plain device copy of known size, for scaling the FETCH_SIZE / WRITE_SIZE counters
    of a counter run to bytes (the copy moves exactly mib MiB each way)."""
    src = torch.ones(mib << 18, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    return dict(bytes_each_way=mib << 20, launches=reps)


def device_state():
    """Clocks and power cap of the GPU as rocm-smi reports them (read-only queries), or
    the error text when the tool is missing; recorded so that box-to-box differences can
    be attributed."""
    import subprocess
    out = {}
    for key, args in (("clocks", ["--showclocks"]), ("max_power", ["--showmaxpower"]),
                      ("power", ["--showpower"])):
        try:
            r = subprocess.run(["rocm-smi", *args, "--json"], capture_output=True, text=True, timeout=20)
            rec = json.loads(r.stdout) if r.returncode == 0 and r.stdout.strip() else {"error": r.stderr[-200:]}
            card = next(iter(rec.values())) if rec and "error" not in rec else rec
            out[key] = card
        except Exception as e:  # pragma: no cover - depends on the host
            out[key] = {"error": str(e)[:200]}
    return out


def probe_library():
    import ctypes
    path = os.path.join(ROOT, "block_scaled_fp4_e2m1_amd", "libfp4_probes.so")
    lib = ctypes.CDLL(path)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.probe_read.argtypes = [vp, i64, vp, i32, i32, vp]
    lib.probe_mfma.argtypes = [i32, i32, i32, i32, vp, vp]  # clocks: uint64 [2 x blocks]
    lib.probe_lds_read.argtypes = [i32, i32, vp, vp]
    lib.probe_valu.argtypes = [i32, i32, i32, vp, vp]
    lib.probe_mix.argtypes = [i32, i32, i32, vp, vp]
    for f in (lib.probe_read, lib.probe_mfma, lib.probe_lds_read, lib.probe_valu, lib.probe_mix):
        f.restype = i32
    return lib


def bench_probes(torch, fp4, steps):
    """Measured ceilings of this device, beside the spec peaks the roofline fractions use:
    the HBM read floor at the decode product's weight bytes and launch shapes (16 rotated
    copies, over 512 MB, so the Infinity Cache cannot hold them; graph replays, per-launch
    averages as the decode leg measures itself) and at 1 GiB; a device copy; the sustained
    FP16 MFMA rate and the LDS read bandwidth per compute unit, each with the shader clock
    the probe ran at (cycles from s_memtime against the 100 MHz real-time counter)."""
    import ctypes
    lib = probe_library()
    st = lambda: ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.zeros(1024, dtype=torch.int32, device="cuda")
    res = {"compute_units": cus, "device_state_before": device_state()}
    timer = Timer(torch)

    def pct(a):
        return [float(np.percentile(a, q)) for q in (10, 50, 90)]

    # read floor at the decode weights' size (codes + micro + macro) and launch shapes
    m, k, n = 8, 4096, 14336
    wbytes = n * k // 2 + n * k // 16 + n * (k // 256) * 2
    bufs = [torch.ones(wbytes // 4, dtype=torch.int32, device="cuda") for _ in range(ROTATE)]
    shapes = {"decode_gemv_shape_224x1024": (224, 1024), "cus_x_1024": (cus, 1024),
              "cus_x_512": (cus, 512), "2cus_x_256": (2 * cus, 256), "4cus_x_256": (4 * cus, 256)}
    reads = {}
    for name, (blocks, threads) in shapes.items():
        fns = [(lambda b=b: lib.probe_read(ctypes.c_void_p(b.data_ptr()), wbytes, ctypes.c_void_p(sink.data_ptr()),
                                           blocks, threads, st())) for b in bufs]
        for f in fns:
            assert f() == 0
        g = capture(torch, fns)
        g.replay()
        per = []
        for _ in range(max(8, steps // ROTATE)):
            per.append(timer.region(g.replay, 1) / ROTATE)
        per = np.array(per)
        reads[name] = dict(us_per_launch_p10_p50_p90=[x * 1e6 for x in pct(per)],
                           gbs_p50=wbytes / np.median(per) / 1e9)
    res["read_floor_decode_weights"] = dict(bytes=wbytes, rotated_copies=ROTATE, launch="HIP graph replay",
                                            shapes=reads)
    del bufs
    big = torch.ones(1 << 28, dtype=torch.int32, device="cuda")  # 1 GiB
    best = {}
    for blocks, threads in ((cus, 1024), (2 * cus, 512), (4 * cus, 256)):
        fn = lambda: lib.probe_read(ctypes.c_void_p(big.data_ptr()), big.numel() * 4,
                                    ctypes.c_void_p(sink.data_ptr()), blocks, threads, st())
        fn()
        best[f"{blocks}x{threads}"] = big.numel() * 4 / (timer.region(fn, 10) / 10) / 1e9
    res["read_1gib_gbs"] = best
    dst = torch.empty_like(big)
    dst.copy_(big)
    res["copy_1gib_gbs_read_plus_write"] = 2 * big.numel() * 4 / (timer.region(lambda: dst.copy_(big), 10) / 10) / 1e9
    del big, dst

    def clocked(fn, blocks, launches):
        """Runs fn `launches` times (the first ones bring the clocks up), returns the median
        launch time, and the shader clock of the last launch (median over workgroups)."""
        clocks = torch.zeros(2 * blocks, dtype=torch.int64, device="cuda")
        for _ in range(launches // 2):
            assert fn(clocks) == 0
        t = np.array([timer.region(lambda: fn(clocks), 1) for _ in range(launches // 2)])
        c = clocks.view(-1, 2).cpu().numpy().astype(np.float64)
        ghz = float(np.median(c[:, 0] / (c[:, 1] / 100e6))) / 1e9
        return float(np.median(t)), ghz, float(np.median(c[:, 0]))

    # MFMA: shapes x waves per SIMD (blocks of 4 waves per CU) x independent accumulators
    mf = {}
    for kind, kname, fl in ((0, "16x16x32_f16", 16384), (1, "32x32x16_f16", 32768), (2, "16x16x32_bf16", 16384)):
        for per_simd, chains in ((1, 8), (2, 8), (4, 8)):
            if kind == 1 and chains == 16:
                continue  # 16 accumulators of 16 registers
            blocks, iters = per_simd * cus, 16384 // per_simd * 8 // chains
            t, ghz, cyc = clocked(lambda c: lib.probe_mfma(kind, chains, blocks, iters, ctypes.c_void_p(c.data_ptr()),
                                                           st()), blocks, 16)
            flops = blocks * 4 * iters * chains * fl
            mf[f"{kname}_w{per_simd}_c{chains}"] = dict(
                tflops=round(flops / t / 1e12, 1), frac_of_spec=round(flops / t / 1e12 / BF16_PEAK_TFLOPS, 3),
                shader_ghz=round(ghz, 3), cycles_per_mfma_per_simd=round(cyc / (per_simd * iters * chains), 2))
    res["mfma"] = mf
    # VALU issue rates: 4 waves per SIMD, 8 independent chains per wave
    va = {}
    for kind, kname in enumerate(("cvt_scalef32_pk_f16_fp4", "pk_mul_f16", "perm_b32", "mul_f32",
                                  "cvt_scalef32_pk_f16_fp8", "and_or_merge", "cvt_scalef32_pk_f32_fp4+xor")):
        blocks, iters = 4 * cus, 4096
        t, ghz, cyc = clocked(lambda c: lib.probe_valu(kind, blocks, iters, ctypes.c_void_p(c.data_ptr()), st()),
                              blocks, 8)
        # instructions per SIMD: 4 waves x iters x 8; cycles from the wall time and the clock
        va[kname] = dict(cycles_per_wave_instruction=round(t * ghz * 1e9 / (4 * iters * 8), 2), shader_ghz=round(ghz, 3))
    res["valu"] = va
    # MFMA + independent VALU in one instruction stream: cycles per iteration of 8 MFMAs
    mx = {}
    for per_simd in (1, 2, 4):
        for nv in (0, 8, 16, 24, 32, 48):
            blocks, iters = per_simd * cus, 8192 // per_simd
            t, ghz, cyc = clocked(lambda c: lib.probe_mix(nv, blocks, iters, ctypes.c_void_p(c.data_ptr()), st()),
                                  blocks, 8)
            mx[f"w{per_simd}_valu{nv}"] = round(t * ghz * 1e9 / (per_simd * iters), 1)
    res["mix_cycles_per_8_mfma_per_simd"] = mx
    # LDS: two blocks (8 waves) per CU
    blocks, iters = 2 * cus, 8192
    t, ghz, cyc = clocked(lambda c: lib.probe_lds_read(blocks, iters, ctypes.c_void_p(c.data_ptr()), st()),
                          blocks, 20)
    lds_bytes = blocks * 4 * iters * 16 * 1024
    res["lds_read"] = dict(bytes_per_cu_per_s=lds_bytes / t / cus, shader_ghz=ghz,
                           bytes_per_clk_per_cu=lds_bytes / t / cus / (ghz * 1e9),
                           bytes_per_clk_per_cu_from_cycles=2 * 4 * iters * 16 * 1024 / cyc)
    res["device_state_after"] = device_state()
    torch.cuda.synchronize()
    return res


def _read_csv(path):
    import csv
    with open(path, newline="") as fh:
        return list(csv.DictReader(fh))


def summarize_stats(stats_csv, title, command):
    """Markdown summary of a rocprofv3 --stats kernel table (durations in ns)."""
    rows = _read_csv(stats_csv)
    lines = [f"# {title}", "", "Command (from the repository root, after `cd /tmp && export TMPDIR=/tmp`):", "",
             "```", command, "```", "",
             "| kernel | calls | average (us) | min (us) | max (us) | share of GPU time |",
             "|---|---|---|---|---|---|"]
    for r in rows:
        name = r["Name"]
        if len(name) > 110:
            name = name[:107] + "..."
        lines.append(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                     f"{float(r['Percentage']):.1f}% |")
    return "\n".join(lines) + "\n"


def summarize_traffic(fetch_csv, write_csv, kernel_substr, group, name, commands):
    """Per-launch HBM bytes of one kernel from two rocprofv3 --pmc runs (FETCH_SIZE, then
    WRITE_SIZE; values per dispatch), each scaled by what the same counter reads for the
    plain copy of known size in the same run."""
    out = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = [r for r in _read_csv(path) if r["Counter_Name"] == counter]
        # the probe's copies are the run's last copy dispatches
        copies = sorted((int(r["Dispatch_Id"]), float(r["Counter_Value"])) for r in rows
                        if "copyBuffer" in r["Kernel_Name"])
        kern = [float(r["Counter_Value"]) for r in rows if kernel_substr in r["Kernel_Name"]]
        if len(copies) < 4 or not kern:
            raise SystemExit(f"{path}: no probe copies or no {kernel_substr} dispatches")
        copy_v = float(np.median([v for _, v in copies[-4:]]))
        factor = (256 << 20) / copy_v
        out[counter] = dict(kernel_counter_median=float(np.median(kern)), dispatches=len(kern),
                            copy_counter_median=copy_v, bytes_per_unit=factor,
                            bytes_per_launch=float(np.median(kern)) * factor)
    total = out["FETCH_SIZE"]["bytes_per_launch"] + out["WRITE_SIZE"]["bytes_per_launch"]
    rec = {"kernel_group": group, "source_hash": source_hash(KERNEL_SOURCES[group]),
           "kernel": kernel_substr, "bytes_per_launch": round(total),
           "fetch_bytes_per_launch": round(out["FETCH_SIZE"]["bytes_per_launch"]),
           "write_bytes_per_launch": round(out["WRITE_SIZE"]["bytes_per_launch"]),
           "counters": out, "commands": commands}
    with open(os.path.join(ROOT, "profiles", f"{name}_traffic.json"), "w") as fh:
        json.dump(rec, fh, indent=1)
        fh.write("\n")
    return rec


def summarize_counters(csv_path, kernel_substr, title, command, simds=1024, xcds=8):
    """Markdown summary of one rocprofv3 --pmc pass (per-dispatch medians for one kernel)
    with the MFMA-busy fraction when the pass holds SQ_VALU_MFMA_BUSY_CYCLES and
    GRBM_GUI_ACTIVE: busy cycles summed over all SIMDs / (kernel cycles x SIMDs), where
    GRBM_GUI_ACTIVE is summed over the XCDs."""
    rows = [r for r in _read_csv(csv_path) if kernel_substr in r["Kernel_Name"]]
    if not rows:
        raise SystemExit(f"{csv_path}: no {kernel_substr} dispatches")
    vals = {}
    for r in rows:
        vals.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    med = {k: float(np.median(v)) for k, v in vals.items()}
    lines = [f"# {title}", "", "Command (from the repository root, after `cd /tmp && export TMPDIR=/tmp`):", "",
             "```", command, "```", "", f"Kernel: `{rows[0]['Kernel_Name'][:100]}`, "
             f"{len(vals[next(iter(vals))])} dispatches; per-dispatch medians:", "",
             "| counter | median |", "|---|---|"]
    lines += [f"| {k} | {v:.6g} |" for k, v in sorted(med.items())]
    if "SQ_VALU_MFMA_BUSY_CYCLES" in med and "GRBM_GUI_ACTIVE" in med:
        kcycles = med["GRBM_GUI_ACTIVE"] / xcds
        busy = med["SQ_VALU_MFMA_BUSY_CYCLES"] / (kcycles * simds)
        lines += ["", f"MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / {xcds} x {simds} SIMDs)"
                      f" = {busy:.3f}"]
        if "SQ_INSTS_MFMA" in med:
            lines += [f"cycles per MFMA instruction per SIMD = "
                      f"{med['SQ_VALU_MFMA_BUSY_CYCLES'] / med['SQ_INSTS_MFMA']:.2f}"]
        if "SQ_INSTS_VALU" in med and "SQ_INSTS_MFMA" in med:
            lines += [f"VALU instructions (MFMA included) per MFMA = "
                      f"{med['SQ_INSTS_VALU'] / med['SQ_INSTS_MFMA']:.2f}"]
    return "\n".join(lines) + "\n"


def bench_policy(torch, fp4, workloads, steps):
    """The 8-layer W4A4/W4A8 policy stack (512 x 5120 x 5120 per layer), per step the eight
    layers' activation passes and products; three copies of the stack (460 MB) rotate."""
    cfg = workloads.WORKLOADS["policy_stack"]
    m, k, n = cfg["m"], cfg["k"], cfg["n"]
    flags = workloads.policy_flags()
    layers, w32 = [], []
    for l in range(cfg["layers"]):
        w, x = workloads.policy_layer(l)
        act = fp4.fp4_policy_select(fp4.POLICY_AUTO, bool(flags[l]))
        w32.append(torch.from_numpy(w).cuda())
        layers.append((act, fp4.quantize_fp4(w32[-1], layout=fp4.LAYOUT_TILED),
                       torch.from_numpy(x).cuda().to(torch.bfloat16)))
    copies = [layers] + [[(act, clone_q(fp4, q), x.clone()) for act, q, x in layers]
                         for _ in range(STACK_COPIES - 1)]
    out = torch.empty(m, n, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(fp4.fp4_workspace_bytes(fp4.A4, m, n, k), dtype=torch.uint8, device="cuda")
    fns = [(lambda a=act, q=wq, x=x: fp4.gemm_w4aX(a, x, q, out=out, workspace=ws))
           for stack in copies for act, wq, x in stack]
    for f in fns:
        f()
    g = capture(torch, fns)
    g.replay()
    timer = Timer(torch)
    reps = max(2, -(-steps // STACK_COPIES))
    secs = timer.region(g.replay, reps)
    per = secs / (reps * STACK_COPIES)  # one step = one pass over the 8 layers
    spread = replay_samples(torch, g, STACK_COPIES, 8)
    flops = 2 * m * n * k * len(layers)

    # per precision: one A4 and one A8 layer alone, over its three copies
    def layer_time(act):
        i = next(j for j, (a_, _, _) in enumerate(layers) if a_ == act)
        lf = [fns[c * len(layers) + i] for c in range(STACK_COPIES)]
        gl = capture(torch, lf)
        gl.replay()
        return float(np.median(replay_samples(torch, gl, len(lf), 16)))
    # chained: x_{l+1} = layer_l(x_l), layer 0 fed its own input, the three stack copies
    # rotating as above (reported, not gated); the last output against the float32 chain
    # of the unquantized weights from the same input
    bufs = [torch.empty(m, n, dtype=torch.bfloat16, device="cuda") for _ in layers]
    chain = []
    for stack in copies:
        xin = stack[0][2]
        for l, (act, wq, _) in enumerate(stack):
            chain.append(lambda a=act, q=wq, xi=xin, o=bufs[l]: fp4.gemm_w4aX(a, xi, q, out=o, workspace=ws))
            xin = bufs[l]
    for f in chain:
        f()
    gc = capture(torch, chain)
    gc.replay()
    chain_spread = replay_samples(torch, gc, STACK_COPIES, 8)
    torch.cuda.synchronize()
    y = layers[0][2].float()
    for wl in w32:
        y = torch.matmul(y, wl.t().contiguous())
    chain_err = float(torch.linalg.norm(bufs[-1].float() - y) / torch.linalg.norm(y))
    del w32
    tfl = flops / per / 1e12
    return dict(layers=len(layers), flagged=[int(i) for i in np.nonzero(flags)[0]], per_step_s=per,
                stack_copies_rotated=STACK_COPIES, step_us_p10_p50_p90=pct_us(spread),
                chained=dict(step_us_p10_p50_p90=pct_us(chain_spread), rel_error_vs_fp32_chain=chain_err),
                kernels={"a4": fp4.fp4_product_kernel(fp4.A4, torch.bfloat16, m, n, k),
                         "a8": fp4.fp4_product_kernel(fp4.A8, torch.bfloat16, m, n, k)},
                tflops=tfl, frac_bf16_peak=tfl / BF16_PEAK_TFLOPS,
                layer_a4_s=layer_time(fp4.A4), layer_a8_s=layer_time(fp4.A8))


def bench_sensitive(torch, fp4, workloads, steps):
    """The 8-layer policy stack (512 x 5120 x 5120 per layer) under the two added policy
    modes: "sensitive-w8" (flagged layers W8A8: E4M3 weights and 8-bit activations, the
    rest W4A4) and "static" (flagged layers A8, the rest A4, both with activation macro-
    scales calibrated beforehand on a separate batch). Per step: every layer's activation
    pass and product. Also the time of one layer of each kind alone and, on the first
    flagged layer, each precision's relative Frobenius error against the float32 product
    of the unquantized inputs."""
    cfg = workloads.WORKLOADS["policy_stack"]
    m, k, n = cfg["m"], cfg["k"], cfg["n"]
    flags = workloads.policy_flags()
    out = torch.empty(m, n, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(fp4.fp4_workspace_bytes(fp4.A8, m, n, k), dtype=torch.uint8, device="cuda")
    res = {}
    timer = Timer(torch)
    single = {}
    acc_layer = int(np.nonzero(flags)[0][0])
    for mode, name in ((fp4.POLICY_SENSITIVE_W8, "sensitive_w8"), (fp4.POLICY_STATIC, "static")):
        fns, kinds, copy_fns = [], [], []
        for l in range(cfg["layers"]):
            w, x = workloads.policy_layer(l)
            code = fp4.fp4_policy_select(mode, bool(flags[l]))
            wd = torch.from_numpy(w).cuda()
            xd = torch.from_numpy(x).cuda().to(torch.bfloat16)
            if code == fp4.W8A8:
                wq = fp4.quantize_fp4(wd, elem=fp4.ELEM_E4M3, layout=fp4.LAYOUT_TILED)
                fns.append(lambda x=xd, q=wq: fp4.gemm_w8a8(x, q, out=out, workspace=ws))
                copy_fns.append(lambda x=xd, q=wq: [lambda x2=x.clone(), q2=clone_q(fp4, q):
                                                    fp4.gemm_w8a8(x2, q2, out=out, workspace=ws)
                                                    for _ in range(STACK_COPIES - 1)])
            elif code in (fp4.A4S, fp4.A8S):
                act = fp4.A8 if code == fp4.A8S else fp4.A4
                amax = torch.zeros(k // 256, dtype=torch.float32, device="cuda")
                calib = torch.from_numpy(workloads.policy_calibration(l, rows=cfg["calib_rows"])).cuda()
                macro = fp4.act_macro_calibrate(calib.to(torch.bfloat16), amax,
                                                fp4.ELEM_E4M3 if act == fp4.A8 else fp4.ELEM_E2M1)
                wq = fp4.quantize_fp4(wd, layout=fp4.LAYOUT_TILED)
                fns.append(lambda a=act, x=xd, q=wq, mc=macro: fp4.gemm_w4aX_static(a, x, mc, q, out=out,
                                                                                   workspace=ws))
                copy_fns.append(lambda a=act, x=xd, q=wq, mc=macro: [
                    lambda x2=x.clone(), q2=clone_q(fp4, q): fp4.gemm_w4aX_static(a, x2, mc, q2, out=out,
                                                                                 workspace=ws)
                    for _ in range(STACK_COPIES - 1)])
            else:
                wq = fp4.quantize_fp4(wd, layout=fp4.LAYOUT_TILED)
                fns.append(lambda a=code, x=xd, q=wq: fp4.gemm_w4aX(a, x, q, out=out, workspace=ws))
                copy_fns.append(lambda a=code, x=xd, q=wq: [
                    lambda x2=x.clone(), q2=clone_q(fp4, q): fp4.gemm_w4aX(a, x2, q2, out=out, workspace=ws)
                    for _ in range(STACK_COPIES - 1)])
            kinds.append(code)
            del wd
        # three copies of the stack rotate (layer l of copy c at index c * layers + l)
        extra = [mk() for mk in copy_fns]
        nl = len(fns)
        all_fns = fns + [extra[l][c] for c in range(STACK_COPIES - 1) for l in range(nl)]
        for f in all_fns:
            f()
        g = capture(torch, all_fns)
        g.replay()
        reps = max(2, -(-steps // STACK_COPIES))
        per = timer.region(g.replay, reps) / (reps * STACK_COPIES)
        spread = replay_samples(torch, g, STACK_COPIES, 8)
        tfl = 2 * m * n * k * nl / per / 1e12
        res[name] = dict(per_step_s=per, tflops=tfl, frac_bf16_peak=tfl / BF16_PEAK_TFLOPS,
                         stack_copies_rotated=STACK_COPIES, step_us_p10_p50_p90=pct_us(spread),
                         codes=[int(c) for c in kinds])
        for l, c in enumerate(kinds):
            if c not in single:
                lf = [all_fns[cc * nl + l] for cc in range(STACK_COPIES)]
                gl = capture(torch, lf)
                gl.replay()
                single[c] = float(np.median(replay_samples(torch, gl, len(lf), 16)))
    names = {fp4.W8A8: "w8a8", fp4.A4: "w4a4", fp4.A4S: "w4a4_static", fp4.A8S: "w4a8_static"}
    for c, t in single.items():
        res[f"layer_{names[c]}_s"] = t
        res[f"layer_{names[c]}_tflops"] = 2 * m * n * k / t / 1e12
    # accuracy on the first flagged layer against the float32 product of bf16 x and float32 W
    w, x = workloads.policy_layer(acc_layer)
    wd = torch.from_numpy(w).cuda()
    xd = torch.from_numpy(x).cuda().to(torch.bfloat16)
    ref = xd.float() @ wd.t()
    nref = torch.linalg.norm(ref).item()
    wq4 = fp4.quantize_fp4(wd, layout=fp4.LAYOUT_TILED)
    wq8 = fp4.quantize_fp4(wd, elem=fp4.ELEM_E4M3, layout=fp4.LAYOUT_TILED)
    amax = torch.zeros(k // 256, dtype=torch.float32, device="cuda")
    calib = torch.from_numpy(workloads.policy_calibration(acc_layer, rows=cfg["calib_rows"])).cuda()
    mac8 = fp4.act_macro_calibrate(calib.to(torch.bfloat16), amax, fp4.ELEM_E4M3)
    outs = {"w8a8": fp4.gemm_w8a8(xd, wq8, out_dtype=torch.float32),
            "w4a16": fp4.gemm_w4aX(fp4.A16, xd, wq4, out_dtype=torch.float32),
            "w4a8": fp4.gemm_w4aX(fp4.A8, xd, wq4, out_dtype=torch.float32),
            "w4a8_static": fp4.gemm_w4aX_static(fp4.A8, xd, mac8, wq4, out_dtype=torch.float32),
            "w4a4": fp4.gemm_w4aX(fp4.A4, xd, wq4, out_dtype=torch.float32)}
    res["rel_error_vs_fp32_product"] = {kk: torch.linalg.norm(v - ref).item() / nref for kk, v in outs.items()}
    res["accuracy_layer"] = acc_layer
    torch.cuda.synchronize()
    return res


def bench_moe(torch, fp4, workloads, steps):
    """The whole mixture-of-experts layer on the device, one HIP graph per step: routing of
    the float32 router logits, the gate/up grouped product (A4, rows gathered by token),
    the SiLU-gated down product (A4) and the weighted combine. Each stage is also timed in
    a graph of its own for the breakdown."""
    cfg = workloads.WORKLOADS["moe_w4a4"]
    E, H, I, T, K = cfg["experts"], cfg["hidden"], cfg["inter"], cfg["tokens"], cfg["top_k"]
    R = T * K
    w1q = fp4.empty_qtensor(E * 2 * I, H, layout=fp4.LAYOUT_TILED)
    w2q = fp4.empty_qtensor(E * H, I, layout=fp4.LAYOUT_TILED)
    for e in range(E):
        w1, w2 = workloads.moe_expert_weights(e)
        for wt, q in ((w1, w1q), (w2, w2q)):
            rows, k = wt.shape
            sub = fp4.QTensor(q.codes[e * rows * k // 2:(e + 1) * rows * k // 2],
                              q.micro[e * rows * k // 16:(e + 1) * rows * k // 16],
                              q.macro[e * rows * k // 256:(e + 1) * rows * k // 256],
                              rows, k, 0, fp4.LAYOUT_TILED)
            fp4.quantize_fp4(torch.from_numpy(wt).cuda(), layout=fp4.LAYOUT_TILED, out=sub)
    logits = torch.from_numpy(workloads.moe_router_logits()).cuda()
    xd = torch.from_numpy(workloads.moe_tokens()).cuda().to(torch.bfloat16)
    dev = xd.device
    routed = (torch.empty(T, K, dtype=torch.int32, device=dev),
              torch.empty(T, K, dtype=torch.float32, device=dev),
              torch.empty(E + 1, dtype=torch.int32, device=dev),
              torch.empty(R, dtype=torch.int32, device=dev),
              torch.empty(T, K, dtype=torch.int32, device=dev))
    _, wts, off, rt, tr = routed
    wsr = torch.empty(max(256, fp4.library().moe_route_workspace_bytes(T, E)), dtype=torch.uint8, device=dev)
    y1 = torch.empty(R, 2 * I, dtype=torch.bfloat16, device=dev)
    y2 = torch.empty(R, H, dtype=torch.bfloat16, device=dev)
    out = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
    ws1 = torch.empty(fp4.fp4_workspace_bytes(fp4.A4, T, 2 * I, H), dtype=torch.uint8, device=dev)
    ws2 = torch.empty(fp4.fp4_workspace_bytes(fp4.A4, R, H, I), dtype=torch.uint8, device=dev)

    stages = {
        "route": lambda: fp4.moe_route(logits, K, workspace=wsr, out=routed),
        "gate_up": lambda: fp4.grouped_gemm_w4aX(fp4.A4, xd, rt, off, E, R, w1q, out=y1, workspace=ws1),
        "gated_down": lambda: fp4.grouped_gemm_w4aX_gated(fp4.A4, y1, off, E, w2q, out=y2, workspace=ws2),
        "combine": lambda: fp4.moe_combine(y2, tr, wts, out=out),
    }

    def layer():
        for f in stages.values():
            f()
    layer()
    timer = Timer(torch)
    g = capture(torch, [layer])
    g.replay()
    per = timer.region(g.replay, steps) / steps
    spread = replay_samples(torch, g, 1, max(8, steps))
    parts = {}
    for name, f in stages.items():
        gs = capture(torch, [f])
        gs.replay()
        parts[name + "_s"] = timer.region(gs.replay, steps) / steps
    torch.cuda.synchronize()
    counts = np.diff(off.cpu().numpy())
    flops = 2 * R * (2 * I) * H + 2 * R * H * I
    gemm_s = parts["gate_up_s"] + parts["gated_down_s"]
    return dict(experts=E, top_k=K, tokens=T, hidden=H, inter=I, routed_rows=R,
                layer_per_step_s=per, layer_tflops=flops / per / 1e12,
                layer_us_p10_p50_p90=pct_us(spread),
                weight_bytes=int(w1q.codes.numel() + w1q.micro.numel() + 2 * w1q.macro.numel()
                                 + w2q.codes.numel() + w2q.micro.numel() + 2 * w2q.macro.numel()),
                gemm_tflops=flops / gemm_s / 1e12,
                frac_bf16_peak=flops / gemm_s / 1e12 / BF16_PEAK_TFLOPS,
                stages=parts,
                rows_per_expert=dict(min=int(counts.min()), max=int(counts.max()),
                                     mean=float(counts.mean()), histogram=count_histogram(counts, 8)))


def build_kv_cache(torch, fp4, workloads, cfg, layer, chunk=4096):
    """One layer's cache filled with max_tokens seeded tokens per sequence (device draws)."""
    B, Hkv, D, T = cfg["n_seq"], cfg["kv_heads"], cfg["head_dim"], cfg["max_tokens"]
    ch = workloads.kv_key_outliers(Hkv * D, 0.005, cfg["seed"])
    cache = fp4.KvCache(B, T, Hkv)
    for i, c0 in enumerate(range(0, T, chunk)):
        k = workloads.kv_rows_device(torch, B * chunk, Hkv * D, cfg["seed"], 100 * layer + 2 * i, outliers=ch)
        v = workloads.kv_rows_device(torch, B * chunk, Hkv * D, cfg["seed"], 100 * layer + 2 * i + 1)
        fp4.kv_cache_append(cache, k, v, torch.full((B,), c0, dtype=torch.int32, device="cuda"))
        del k, v
    return cache


def bench_attention(torch, fp4, workloads, steps):
    """One decode step of attention over the FP4 KV cache: append the step's token to every
    sequence, then attention over L + 1 tokens. Two layers' caches alternate so the 256 MB
    Infinity Cache cannot hold the working set."""
    cfg = workloads.WORKLOADS["decode_attention_fp4kv"]
    B, Hq, Hkv, D, T = cfg["n_seq"], cfg["q_heads"], cfg["kv_heads"], cfg["head_dim"], cfg["max_tokens"]
    lens = workloads.kv_lengths(B, cfg["min_len"], cfg["max_len"], cfg["seed"])
    caches = [build_kv_cache(torch, fp4, workloads, cfg, layer) for layer in range(2)]
    q = torch.from_numpy(workloads.kv_queries(B, Hq, D, cfg["seed"])).cuda().to(torch.bfloat16)
    rng = np.random.default_rng((cfg["seed"], 3))
    k1 = torch.from_numpy(rng.standard_normal((B, Hkv * D), dtype=np.float32)).cuda().to(torch.bfloat16)
    v1 = torch.from_numpy(rng.standard_normal((B, Hkv * D), dtype=np.float32)).cuda().to(torch.bfloat16)
    pos = torch.from_numpy(lens).cuda()
    lengths = torch.from_numpy(lens + 1).cuda()
    outs = [torch.empty(B, Hq, D, dtype=torch.bfloat16, device="cuda") for _ in caches]
    ws = torch.empty(fp4.library().attention_workspace_bytes(B, Hq, T), dtype=torch.uint8, device="cuda")

    def step(i):
        fp4.kv_cache_append(caches[i], k1, v1, pos)
        fp4.attention_decode_fp4kv(q, caches[i], lengths, out=outs[i], workspace=ws)

    def attn(i):
        fp4.attention_decode_fp4kv(q, caches[i], lengths, out=outs[i], workspace=ws)
    timer = Timer(torch)
    res, spread = {}, {}
    for name, fn in (("step", step), ("attention", attn)):
        fns = [lambda i=i: fn(i) for i in range(len(caches))]
        for f in fns:
            f()
        g = capture(torch, fns)
        g.replay()
        res[name] = run_steps(torch, timer, g, fns, steps) / steps
        spread[name] = pct_us(replay_samples(torch, g, len(fns), max(8, steps // len(fns))))
    torch.cuda.synchronize()
    tokens = int((lens.astype(np.int64) + 1).sum())
    per_token_head = 2 * (D // 2 + D // 16 + 1)  # K and V: codes, micro, macro (a pair's 2 B / 2)
    cache_bytes = tokens * Hkv * per_token_head
    io_bytes = 2 * B * Hq * D * 2  # q in, out
    total = cache_bytes + io_bytes
    return dict(n_seq=B, q_heads=Hq, kv_heads=Hkv, head_dim=D, max_tokens=T,
                context_min_mean_max=[int(lens.min() + 1), float(lens.mean() + 1), int(lens.max() + 1)],
                algorithmic_bytes=total, bf16_cache_bytes_equivalent=tokens * Hkv * 2 * D * 2,
                step_s=res["step"], attention_s=res["attention"],
                step_us_p10_p50_p90=spread["step"], attention_us_p10_p50_p90=spread["attention"],
                gbs_attention=total / res["attention"] / 1e9, gbs_step=total / res["step"] / 1e9,
                frac_hbm_attention=total / res["attention"] / 1e9 / HBM_PEAK_GBS,
                traffic_bytes_per_launch=load_traffic("attention_decode_fp4kv"),
                layers_rotated=len(caches))


def cpu_baseline(workloads, budget_s=12.0):
    """The oracle, as written, on a bounded sample of the decode workload: quantize rows of
    W, dequantize, float64 product with the 8 activation rows; GB/s of the same
    algorithmic traffic per processed weight row."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = os.cpu_count() or 1
    a, w, _ = workloads.decode()
    m, k, n = 8, 4096, 14336
    a64 = a.astype(np.float64)
    rows_done, t0 = 0, time.perf_counter()
    chunk = 512
    t_quant = 0.0
    while time.perf_counter() - t0 < budget_s and rows_done < n:
        sl = w[rows_done:rows_done + chunk].astype(np.float64)
        tq = time.perf_counter()
        q = oracle.quantize(sl)
        t_quant += time.perf_counter() - tq
        _ = oracle.gemm(a64, q, oracle.A16)
        rows_done += sl.shape[0]
    secs = time.perf_counter() - t0
    t_prod = secs - t_quant
    frac = rows_done / n
    nbytes = algorithmic_bytes_gemv(m, n, k) * frac
    cpu_model = platform.processor() or ""
    try:
        with open("/proc/cpuinfo") as fh:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")), cpu_model)
    except OSError:
        pass
    return {"value": nbytes / t_prod / 1e9, "unit": "GB/s", "cores": int(blas_threads),
            "kind": "oracle", "cpu_model": cpu_model, "host_cpus": os.cpu_count(),
            "quantize_s": round(t_quant, 3), "product_s": round(t_prod, 3),
            "sample": f"decode W4A16 product on {rows_done} of {n} weight rows "
                      f"(dequantize + float64 matmul {t_prod:.2f} s; the oracle's quantization "
                      f"of those rows took {t_quant:.2f} s more); numpy elementwise work is "
                      f"single-threaded, the float64 matmul uses {blas_threads} BLAS threads; "
                      f"host has {os.cpu_count()} CPUs"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=320)
    ap.add_argument("--warmup", type=int, default=32)
    ap.add_argument("--skip-secondary", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["decode", "prefill", "policy", "moe", "quantize", "dequantize", "attention", "mx",
                                       "sensitive", "probes", "repack", "ceilings"],
                    default=None,
                    help="run one workload only (for profiling); prints its record")
    ap.add_argument("--copy-probe", action="store_true",
                    help="with --only: end with 256 MiB device copies (counter calibration)")
    ap.add_argument("--summarize-stats", nargs=3, metavar=("STATS_CSV", "TITLE", "COMMAND"),
                    help="print a markdown summary of a rocprofv3 kernel-stats CSV and exit")
    ap.add_argument("--summarize-traffic", nargs=5,
                    metavar=("FETCH_CSV", "WRITE_CSV", "KERNEL", "GROUP", "NAME"),
                    help="write profiles/NAME_traffic.json from two counter runs and exit")
    ap.add_argument("--commands", nargs="*", default=[], help="commands recorded with --summarize-traffic")
    ap.add_argument("--summarize-counters", nargs=4, metavar=("PMC_CSV", "KERNEL", "TITLE", "COMMAND"),
                    help="print a markdown summary of one rocprofv3 --pmc pass for one kernel and exit")
    args = ap.parse_args()
    if args.summarize_stats:
        sys.stdout.write(summarize_stats(*args.summarize_stats))
        return
    if args.summarize_counters:
        sys.stdout.write(summarize_counters(*args.summarize_counters))
        return
    if args.summarize_traffic:
        rec = summarize_traffic(*args.summarize_traffic, commands=args.commands)
        print(json.dumps({k: rec[k] for k in ("kernel", "bytes_per_launch", "fetch_bytes_per_launch",
                                              "write_bytes_per_launch")}))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path).", file=sys.stderr)
        sys.exit(2)

    import torch
    import block_scaled_fp4_e2m1_amd as fp4
    import workloads
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if fp4.fp4_device_check() != 0:
        print("device is not gfx950", file=sys.stderr)
        sys.exit(1)

    if args.only:
        fn = {"decode": lambda: bench_decode(torch, fp4, workloads, args.steps, args.warmup),
              "prefill": lambda: bench_prefill(torch, fp4, workloads, args.steps),
              "policy": lambda: bench_policy(torch, fp4, workloads, args.steps),
              "moe": lambda: bench_moe(torch, fp4, workloads, args.steps),
              "quantize": lambda: bench_quantize(torch, fp4, workloads, args.steps),
              "dequantize": lambda: bench_dequantize(torch, fp4, workloads, args.steps),
              "attention": lambda: bench_attention(torch, fp4, workloads, args.steps),
              "mx": lambda: bench_mx(torch, fp4, workloads, args.steps),
              "sensitive": lambda: bench_sensitive(torch, fp4, workloads, args.steps),
              "probes": lambda: bench_probes(torch, fp4, args.steps),
              "repack": lambda: bench_repack(torch, fp4, workloads, args.steps),
              "ceilings": lambda: ceilings(torch, args.steps)}[args.only]
        rec = {args.only: fn()}
        if args.copy_probe:
            rec["copy_probe"] = copy_probe(torch)
        print(json.dumps(rec), flush=True)
        return

    state_before = device_state()
    dec = bench_decode(torch, fp4, workloads, args.steps, args.warmup)
    print(f"# decode done: {dec['per_launch_s'] * 1e6:.2f} us/launch", file=sys.stderr, flush=True)
    ceil = ceilings(torch, args.steps)
    print(f"# ceilings done: read floor {ceil['read_floor_gbs']:.0f} GB/s, "
          f"MFMA {ceil['mfma_f16_register_tflops']:.0f} TFLOP/s", file=sys.stderr, flush=True)
    secondary = {}
    if not args.skip_secondary:
        secondary["prefill_w4a4"] = bench_prefill(torch, fp4, workloads, max(8, args.steps // 8))
        print("# prefill done", file=sys.stderr, flush=True)
        secondary["policy_stack"] = bench_policy(torch, fp4, workloads, max(4, args.steps // 32))
        print("# policy done", file=sys.stderr, flush=True)
        secondary["moe_w4a4"] = bench_moe(torch, fp4, workloads, max(4, args.steps // 32))
        print("# moe done", file=sys.stderr, flush=True)
        secondary["quantize"] = bench_quantize(torch, fp4, workloads, args.steps)
        print("# quantize done", file=sys.stderr, flush=True)
        secondary["dequantize"] = bench_dequantize(torch, fp4, workloads, args.steps)
        print("# dequantize done", file=sys.stderr, flush=True)
        secondary["repack"] = bench_repack(torch, fp4, workloads, max(16, args.steps // 4))
        print("# repack done", file=sys.stderr, flush=True)
        secondary["decode_attention_fp4kv"] = bench_attention(torch, fp4, workloads, max(8, args.steps // 8))
        print("# attention done", file=sys.stderr, flush=True)
        secondary["prefill_mx_fp4"] = bench_mx(torch, fp4, workloads, max(8, args.steps // 8))
        print("# mx done", file=sys.stderr, flush=True)
        secondary["policy_stack_sensitive_static"] = bench_sensitive(torch, fp4, workloads,
                                                                     max(4, args.steps // 32))
        print("# sensitive done", file=sys.stderr, flush=True)
    state_after = device_state()
    cpu = None if args.no_cpu_baseline else cpu_baseline(workloads)
    # fractions of the measured ceilings beside the spec ones
    mfma_probe = ceil["mfma_f16_register_tflops"]
    for key in ("prefill_w4a4", "policy_stack"):
        if key in secondary:
            secondary[key]["frac_of_mfma_probe"] = secondary[key]["tflops"] / mfma_probe
    if "moe_w4a4" in secondary:
        secondary["moe_w4a4"]["frac_of_mfma_probe"] = secondary["moe_w4a4"]["gemm_tflops"] / mfma_probe

    traffic = load_traffic("gemv_decode_w4a16")
    achieved = dec["gbs"]
    rec = {
        "metric": METRIC,
        "value": round(dec["gbs"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": dec["per_launch_s"] * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "decode_w4a16: A bf16 [8 x 4096] . W^T, W two-level block FP4 "
                               "[14336 x 4096] (E2M1, E4M3 per 16, FP16 per 256), C bf16",
                   "m": 8, "k": 4096, "n": 14336, "weight_copies_rotated": ROTATE,
                   "launch": "HIP graph replay",
                   "launch_us_p10_p50_p90": dec["launch_us_p10_p50_p90"]},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "algorithmic_bytes_per_launch": dec["bytes"],
                     "measured_read_floor_gbs": round(ceil["read_floor_gbs"], 1),
                     "frac_of_read_floor": round(achieved / ceil["read_floor_gbs"], 4)},
        "ceilings": ceil,
        "device_state": {"before": state_before, "after": state_after},
        "cpu_baseline": cpu,
        "secondary": secondary,
    }
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
