#!/usr/bin/env python3
"""Benchmark: AWQ scale search + pack of one linear layer on one MI355X.

A step is one pass of the whole per-layer path on one synthetic layer: activation
statistics, scale family + fake quantisation + output-error loss for all 20 alphas,
argmin, final quantise-and-pack.  Inputs are resident in HBM before timing starts.
The default workload is the 4096 x 4096 layer with 4096 calibration tokens (4-bit,
zero-point, group 128, 20 alphas).

Prints one JSON line.  The loss product's live duration comes from HIP events that the
library records on its own stream around that launch (one launch per step, the whole
alpha grid in one pass).  On this layer the library takes the loss through G = X^T X
(formed once per step, also bracketed by events): the loss product is then dW_k G'^T
over the block upper triangle of G, and its flops are counted as executed.  The CPU baseline is the oracle, timed on a bounded row subset
of the same layer (the loss is a sum over rows) and scaled to the full layer.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import re
import sys
import time

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 MFMA
# fp32 vector ALU without packed fp32 instructions (the kernels are built without them):
# 256 CUs x 64 lanes per clock x 2 flops (FMA) x 2.4 GHz; packed math would double it.
FP32_VALU_PEAK_TFLOPS = 78.6


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--config", default="c2", help="workload name (c1 .. c5)")
    p.add_argument("--layer", type=int, default=0, help="layer index within the workload")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-variants", action="store_true",
                   help="skip timing the statistic / threshold / rotation / table variants")
    p.add_argument("--cpu-rows", type=int, default=4096,
                   help="rows of W in the oracle's timed sample")
    p.add_argument("--calib-copy-mib", type=int, default=0,
                   help="after timing, run one device-to-device copy of this many MiB (a kernel of "
                        "known traffic, used to scale the HBM byte counters)")
    p.add_argument("--traffic-summary", default=os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                             "profiles", "loss_gemm_c2_counters.md"),
                   help="rocprofv3 counter summary holding the HBM bytes per loss-product launch")
    return p.parse_args()


class HipEvent:
    """A raw hipEvent_t from the HIP runtime torch already loaded (same SONAME), so that
    the library can record it on its own launches and we can read the elapsed time."""

    _hip = None

    def __init__(self):
        import ctypes
        if HipEvent._hip is None:
            hip = ctypes.CDLL("libamdhip64.so.7")
            hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
            hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                ctypes.c_void_p]
            hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
            HipEvent._hip = hip
        self._ct = ctypes
        self.h = ctypes.c_void_p()
        if HipEvent._hip.hipEventCreate(ctypes.byref(self.h)) != 0:
            raise RuntimeError("hipEventCreate failed")

    @property
    def handle(self) -> int:
        return int(self.h.value)

    def record(self, stream_ptr: int):
        if HipEvent._hip.hipEventRecord(self.h, self._ct.c_void_p(stream_ptr)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, end: "HipEvent") -> float:
        f = self._ct.c_float()
        rc = HipEvent._hip.hipEventElapsedTime(self._ct.byref(f), self.h, end.h)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(f.value)


def cpu_baseline(layer, alphas, cfg, rows, repeats=2):
    """Time the oracle (as it stands) on rows [0, rows) of W with the full X, `repeats`
    times (the mean is reported)."""
    import numpy as np
    from oracle import awq_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()
                       if i.get("user_api") == "blas"] or [1])
    except Exception:  # noqa: BLE001
        threads = 1
    ocfg = O.QConfig(cfg.w_bit, cfg.group_size, cfg.zero_point)
    W, X = layer.W, layer.X
    M = W.shape[0]
    rows = min(rows, M)
    layer_s, total = 0.0, 0.0
    for _ in range(repeats):
        t0 = time.perf_counter()
        a = O.act_stats(X)
        t1 = time.perf_counter()
        res = O.search_scales(W[:rows], X, a, alphas, ocfg)
        O.quantize_pack(W[:rows], res["s_star"], ocfg)
        t2 = time.perf_counter()
        layer_s += ((t1 - t0) + (t2 - t1) * (M / rows)) / repeats
        total += t2 - t0
    cpu_model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    cpu_model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"value": 1.0 / layer_s, "unit": "layers/s", "cores": int(threads), "kind": "oracle",
            "cpu_model": cpu_model, "os_cpu_count": os.cpu_count(),
            "sample": (f"statistics over all {X.shape[0]} tokens, then the 20-alpha search and the "
                       f"pack on rows 0..{rows - 1} of {M}; search+pack time scaled by {M / rows:g} "
                       f"(the loss and the pack are sums/maps over rows); mean of {repeats} "
                       f"runs, {total:.1f} s in all")}


def cpu_oracle_widened(layer, cfg, rows_table=64, rows_clip=8, rows_w4=512):
    """The oracle (as it stands) timed on the widened rows, each on a bounded sample of the
    same workload and scaled to it (rows are independent in every one of them)."""
    import numpy as np
    from oracle import awq_oracle as O
    ocfg = O.QConfig(cfg.w_bit, cfg.group_size, cfg.zero_point)
    W, X = layer.W, layer.X
    M, K = W.shape
    out = {}

    def clock(fn):
        t0 = time.perf_counter()
        r = fn()
        return r, (time.perf_counter() - t0) * 1e3

    a, _ = clock(lambda: O.act_stats(X))
    for name, fn in [("stat_max_abs", lambda: O.act_stat_max_abs(X)),
                     ("stat_rms_ratio", lambda: O.act_stat_rms_ratio(X)),
                     ("stat_ema_mean_b512", lambda: O.act_stat_ema_mean(X, 512, 0.9)),
                     ("threshold_scales", lambda: O.threshold_scales(a, 70.0, 2.0)),
                     ("hadamard_rotate_X_b128", lambda: O.hadamard_rotate(X, 128))]:
        _, ms = clock(fn)
        out[name] = {"ms": ms, "sample": "full input"}
    table = np.stack([O.threshold_scales(a, p, f) for p in (50.0, 70.0, 85.0, 95.0, 99.0)
                      for f in (1.5, 2.0, 3.0, 4.0)])
    _, ms = clock(lambda: O.search_scale_table(W[:rows_table], X, table, ocfg))
    out["search_scale_table_20_threshold_rows"] = {
        "ms": ms * M / rows_table,
        "sample": f"rows 0..{rows_table - 1} of {M}, scaled by {M / rows_table:g}"}
    s_half = O.scale_family(a, np.array([0.5], np.float32))[0]
    ratios = np.array([1.0 - 0.025 * k for k in range(20)], np.float32)
    _, ms = clock(lambda: O.clip_search(W[:rows_clip], X, s_half, ocfg, ratios))
    out["clip_search_20_ratios"] = {
        "ms": ms * M / rows_clip, "sample": f"rows 0..{rows_clip - 1} of {M}, scaled by "
                                             f"{M / rows_clip:g}"}
    rng = np.random.default_rng(20250)
    M2, K2, g = 28672, 8192, cfg.group_size
    pk = rng.integers(0, 256, (rows_w4, K2 // 2), dtype=np.uint8)
    sc = rng.uniform(0.0005, 0.02, (rows_w4, K2 // g)).astype(np.float16)
    zr = rng.integers(0, 16, (rows_w4, K2 // g)).astype(np.float16)
    x16 = rng.standard_normal((16, K2)).astype(np.float16)
    for T in (1, 4, 16):
        _, ms = clock(lambda: O.w4a16_matmul(pk, sc, zr, x16[:T], g))
        out[f"w4a16_{M2}x{K2}_T{T}_folded"] = {
            "ms": ms * M2 / rows_w4,
            "sample": f"{rows_w4} of {M2} rows, scaled by {M2 / rows_w4:g}"}
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this build measures "
              "one GPU's share of the layer and has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import weight_only_quantization_act_amd as awq
    from synth import CONFIGS, alpha_grid, make_layer

    if not torch.cuda.is_available():
        print("bench.py needs a HIP GPU", file=sys.stderr)
        sys.exit(3)
    torch.cuda.set_device(0)
    spec = CONFIGS[args.config][args.layer]
    layer = make_layer(spec)
    M, K, N = spec.out_features, spec.in_features, spec.n_tokens
    cfg = awq.qconfig(spec.w_bit, spec.group_size, spec.zero_point)
    alphas = alpha_grid(spec.n_alpha)
    nA = len(alphas)

    Wd = torch.from_numpy(layer.W).cuda()
    Xd = torch.from_numpy(layer.X).cuda()
    ws_search = torch.empty(awq.awq_workspace_bytes(M, K, N, cfg, nA, 0), dtype=torch.uint8,
                            device="cuda")
    ws_stats = torch.empty(awq.awq_act_stats_workspace_bytes(N, K), dtype=torch.uint8,
                           device="cuda")
    stream = torch.cuda.current_stream()
    sptr = int(stream.cuda_stream)

    def step(ev=None):
        if ev is not None:
            ev["st0"].record(sptr)
        a = awq.awq_act_stats(Xd, workspace=ws_stats)
        if ev is not None:
            ev["st1"].record(sptr)
            awq.awq_set_profile_events(ev["g0"], ev["g1"], ev["f0"], ev["f1"], ev["r0"],
                                       ev["r1"])
        res = awq.awq_search_scales(Wd, Xd, a, alphas, cfg, workspace=ws_search)
        if ev is not None:
            ev["p0"].record(sptr)
        out = awq.awq_quantize_pack(Wd, res["s"], cfg)
        if ev is not None:
            ev["p1"].record(sptr)
        return res, out

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # the timed steps carry no events of their own; the per-kernel breakdown comes from a
    # second pass of the same steps with events around each part
    t_start, t_end = HipEvent(), HipEvent()
    torch.cuda.synchronize()
    t_start.record(sptr)
    for i in range(args.steps):
        res, out = step()
    t_end.record(sptr)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_ms(t_end)
    ms_per_step = total_ms / args.steps

    names = ("st0", "st1", "g0", "g1", "f0", "f1", "r0", "r1", "p0", "p1")
    evs = [{n: HipEvent() for n in names} for _ in range(args.steps)]
    for i in range(args.steps):
        res, out = step(evs[i])
    torch.cuda.synchronize()

    def avg(a, b):
        return float(np.mean([e[a].elapsed_ms(e[b]) for e in evs]))

    gram = awq.awq_loss_form(M, K, N, nA) == awq.AWQ_LOSS_GRAM
    gemm_ms, fq_ms = avg("g0", "g1"), avg("f0", "f1")
    stats_ms, pack_ms = avg("st0", "st1"), avg("p0", "p1")
    gram_ms = avg("r0", "r1") if gram else 0.0

    status = int(res["status"].cpu()[0])
    direct_flops = 2.0 * M * N * K * nA                     # the direct product dW_k X^T
    if gram:
        # one launch = all alphas; each half (128 channels) of a 256-channel column tile runs
        # over k from its own first channel on (the executed MFMA work)
        gemm_flops = nA * sum(2.0 * M * min(128, K - c0) * (K - c0) for c0 in range(0, K, 128))
        gram_flops = sum(2.0 * N * min(128, K - c0) * (K - c0) for c0 in range(0, K, 128))
    else:
        gemm_flops, gram_flops = direct_flops, 0.0
    gemm_tflops = gemm_flops / (gemm_ms * 1e-3) / 1e12
    g = spec.group_size
    stats_bytes = 2.0 * N * K + 4.0 * K
    fq_bytes = 2.0 * M * K + 4.0 * K * nA + 2.0 * M * K * nA
    pack_bytes = 2.0 * M * K + 4.0 * K + M * K / 2 + 4.0 * M * K / g

    # HBM bytes per launch from the committed counter summary, valid only for the kernel
    # source and workload it was measured on (null otherwise).
    traffic = None
    counters = None  # matrix-core busy fraction and clock from the same summary
    if os.path.exists(args.traffic_summary):
        kv = {}
        with open(args.traffic_summary) as f:
            for ln in f:
                m = re.match(r"^(kernel_source_sha|workload|hbm_bytes_per_launch|mfma_busy_frac|"
                             r"shader_clock_ghz): (\S+)\s*$", ln)
                if m:
                    kv[m.group(1)] = m.group(2)
        if kv.get("workload") == spec.name and kv.get("kernel_source_sha") == _kernel_sha():
            traffic = float(kv["hbm_bytes_per_launch"])
            if "mfma_busy_frac" in kv:
                counters = {"mfma_busy_frac": float(kv["mfma_busy_frac"]),
                            "shader_clock_GHz": float(kv["shader_clock_ghz"]),
                            "source": os.path.basename(args.traffic_summary)}

    line = {
        "metric": "AWQ layers/s at 4096x4096; loss-GEMM TFLOP/s & MFMA util; pack GB/s",
        "value": 1000.0 / ms_per_step,
        "unit": "layers/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic (seeded fp16 weights and calibration activations with outlier channels)",
        "config": {"workload": (f"{spec.name}: W {M}x{K} fp16, X {N} tokens x {K}, "
                                f"{spec.w_bit}-bit {'zero-point' if spec.zero_point else 'symmetric'}, "
                                f"group {g}, {nA} alphas"),
                   "out_features": M, "in_features": K, "n_tokens": N, "w_bit": spec.w_bit,
                   "group_size": g, "zero_point": spec.zero_point, "n_alpha": nA,
                   "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "achieved": gemm_tflops, "peak": MFMA_F16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": gemm_tflops / MFMA_F16_PEAK_TFLOPS,
                     "traffic": traffic,
                     "kernel": "k_loss_gemm" + ("<G form>" if gram else ""),
                     "flops_per_launch": gemm_flops, "avg_launch_ms": gemm_ms,
                     "mfma_counters": counters,
                     # the G form executes M K^2 (1 + 256/K) per alpha instead of 2 M K N: the
                     # direct product's flops over the Gram pass plus this launch, for scale
                     "form": "gram" if gram else "direct",
                     "direct_equivalent_TFLOP/s": direct_flops / ((gemm_ms + gram_ms) * 1e-3) / 1e12},
        "kernels": {
            "act_stats": {"ms": stats_ms, "GB/s": stats_bytes / (stats_ms * 1e-3) / 1e9,
                          "frac_hbm": stats_bytes / (stats_ms * 1e-3) / 1e9 / HBM_PEAK_GBS},
            "fake_quant": {"ms": fq_ms, "GB/s": fq_bytes / (fq_ms * 1e-3) / 1e9,
                           "frac_hbm": fq_bytes / (fq_ms * 1e-3) / 1e9 / HBM_PEAK_GBS},
            "loss_gemm": {"ms": gemm_ms, "TFLOP/s": gemm_tflops,
                          "frac_mfma": gemm_tflops / MFMA_F16_PEAK_TFLOPS,
                          "form": "gram" if gram else "direct",
                          "direct_equivalent_TFLOP/s":
                              direct_flops / ((gemm_ms + gram_ms) * 1e-3) / 1e12},
            **({"gram": {"ms": gram_ms, "TFLOP/s": gram_flops / (gram_ms * 1e-3) / 1e12,
                         "frac_mfma": gram_flops / (gram_ms * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS,
                         "kernels": "k_transpose_x + k_loss_gemm<G build> + k_gram_full_split"}} if gram else {}),
            "quant_pack": {"ms": pack_ms, "GB/s": pack_bytes / (pack_ms * 1e-3) / 1e9,
                           "frac_hbm": pack_bytes / (pack_ms * 1e-3) / 1e9 / HBM_PEAK_GBS},
        },
        "search_status": status,
    }
    if not args.no_variants:
        line["variants"] = time_variants(awq, torch, Wd, Xd, cfg, sptr, M, K, N)
        line["w4a16"] = time_w4a16(awq, torch, out, res["s"], Xd, cfg, sptr, M, K)
        line["large_layers"] = time_large_layers(awq, torch, alphas, sptr)
        line["small_layer"] = time_small_layer(awq, torch, sptr)
    line["ceilings"] = measure_ceilings(torch, sptr)
    if args.calib_copy_mib > 0:
        src = torch.ones(args.calib_copy_mib * (1 << 20) // 2, dtype=torch.float16, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        line["calib_copy_bytes"] = {"read": src.numel() * 2, "write": dst.numel() * 2}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(layer, alphas, cfg, args.cpu_rows)
        if not args.no_variants:
            line["cpu_oracle_widened"] = cpu_oracle_widened(layer, cfg)
    print(json.dumps(line), flush=True)


def measure_ceilings(torch, sptr, reps=20):
    """This box's practical ceilings, measured after the timed region: a 512 MiB
    device-to-device copy (read + write bytes over time) and a plain fp16 4096^3 product
    through torch.matmul (hipBLASLt), both on contiguous operands."""

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = HipEvent(), HipEvent()
        e0.record(sptr)
        for _ in range(reps):
            fn()
        e1.record(sptr)
        torch.cuda.synchronize()
        return e0.elapsed_ms(e1) / reps

    src = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    ms = timed(lambda: dst.copy_(src))
    copy_gbs = 2.0 * src.numel() / (ms * 1e-3) / 1e9
    del src, dst
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7)
    a = torch.randn((4096, 4096), device="cuda", generator=gen).half()
    b = torch.randn((4096, 4096), device="cuda", generator=gen).half()
    c = torch.empty((4096, 4096), device="cuda", dtype=torch.float16)
    ms = timed(lambda: torch.matmul(a, b, out=c))
    gemm_tf = 2.0 * 4096 ** 3 / (ms * 1e-3) / 1e12
    del a, b, c
    torch.cuda.empty_cache()
    return {"copy_GB/s": copy_gbs, "copy_frac_of_8TBps": copy_gbs / HBM_PEAK_GBS,
            "torch_matmul_fp16_4096^3_TFLOP/s": gemm_tf,
            "torch_matmul_frac_of_2.5PF": gemm_tf / MFMA_F16_PEAK_TFLOPS}


def time_variants(awq, torch, Wd, Xd, cfg, sptr, M, K, N, reps=20):
    """Average time per call of the widened entry points on the same layer, measured
    after the timed region (HIP events around `reps` back-to-back calls)."""

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = HipEvent(), HipEvent()
        e0.record(sptr)
        for _ in range(reps):
            fn()
        e1.record(sptr)
        torch.cuda.synchronize()
        return e0.elapsed_ms(e1) / reps

    out = {}
    x_bytes = 2.0 * N * K + 4.0 * K
    for name, mode, extra in [("stat_max_abs", awq.AWQ_STAT_MAX_ABS, ()),
                              ("stat_rms_ratio", awq.AWQ_STAT_RMS_RATIO, ()),
                              ("stat_ema_mean_b512", awq.AWQ_STAT_EMA_MEAN, (512, 0.9))]:
        ms = timed(lambda: awq.awq_act_stats_ex(Xd, mode, *extra))
        gbs = x_bytes / (ms * 1e-3) / 1e9
        out[name] = {"ms": ms, "GB/s": gbs, "frac_hbm": gbs / HBM_PEAK_GBS}
    a = awq.awq_act_stats(Xd)
    out["threshold_scales"] = {"ms": timed(lambda: awq.awq_threshold_scales(a, 70.0, 2.0)),
                               "in_features": K}
    Xr = torch.empty_like(Xd)
    ms = timed(lambda: awq.awq_hadamard_rotate(Xd, 128, out=Xr))
    gbs = 4.0 * N * K / (ms * 1e-3) / 1e9
    out["hadamard_rotate_X_b128"] = {"ms": ms, "GB/s": gbs, "frac_hbm": gbs / HBM_PEAK_GBS}
    table = torch.stack([awq.awq_threshold_scales(a, p, f) for p in (50.0, 70.0, 85.0, 95.0, 99.0)
                         for f in (1.5, 2.0, 3.0, 4.0)]).contiguous()
    ws = torch.empty(awq.awq_workspace_bytes(M, K, N, cfg, table.shape[0], 0), dtype=torch.uint8,
                     device="cuda")
    ms = timed(lambda: awq.awq_search_scale_table(Wd, Xd, table, cfg, workspace=ws))
    tf = 2.0 * M * N * K * table.shape[0] / (ms * 1e-3) / 1e12
    form = awq.awq_loss_form(M, K, N, table.shape[0])
    out["search_scale_table_20_threshold_rows"] = {
        "ms": ms, "direct_equivalent_TFLOP/s": tf,
        "form": "gram" if form == awq.AWQ_LOSS_GRAM else "direct"}
    ratios = [1.0 - 0.025 * k for k in range(20)]
    s_best = awq.awq_search_scales(Wd, Xd, a, [0.5], cfg)["s"]
    ws_clip = torch.empty(awq.awq_clip_workspace_bytes(M, K, N, cfg), dtype=torch.uint8,
                          device="cuda")
    ms = timed(lambda: awq.awq_clip_search(Wd, Xd, s_best, ratios, cfg, workspace=ws_clip))
    g = cfg.group_size
    tf = (2.0 * N * K * g + 2.0 * M * K * g * 20) / (ms * 1e-3) / 1e12
    # executed matrix-core work: the Gram sums once, and for the quadratic forms three fp16
    # passes (hi/lo splits of G and of d) over the tiles of G's upper block triangle that a
    # row tile of 16 reads (k-steps of 32 from its diagonal block on)
    rt, ks = g // 16, g // 32
    tiles = sum(ks - r // 2 for r in range(rt)) / (rt * ks)
    mfma_flops = 2.0 * N * K * g + 3 * 2.0 * M * K * g * 20 * tiles
    mfma_tf = mfma_flops / (ms * 1e-3) / 1e12
    out["clip_search_20_ratios"] = {
        "ms": ms, "gram_flops": 2.0 * N * K * g, "quadratic_flops": 2.0 * M * K * g * 20,
        "TFLOP/s": tf, "mfma_flops_executed": mfma_flops, "mfma_TFLOP/s": mfma_tf,
        "peak_TFLOP/s": MFMA_F16_PEAK_TFLOPS, "frac_mfma": mfma_tf / MFMA_F16_PEAK_TFLOPS,
        "bound": "alu",
        "limiter": "vector issue of the per-(row, ratio) quantisation (about 16 instructions "
                   "per element; SQ counters show the vector unit 60-65% busy, the matrix "
                   "cores about 30%)"}
    return out


def time_small_layer(awq, torch, sptr, reps=50):
    """The whole path (statistics, 20-alpha search, pack) of the 512 x 512 layer with 256
    tokens, symmetric 4-bit: launch-bound, so timed both as eager calls and as replays of
    the same calls captured in one HIP graph."""
    from synth import CONFIGS, alpha_grid, make_layer
    spec = CONFIGS["c1"][0]
    L = make_layer(spec)
    M, K, N = spec.out_features, spec.in_features, spec.n_tokens
    cfg = awq.qconfig(spec.w_bit, spec.group_size, spec.zero_point)
    alphas = alpha_grid(spec.n_alpha)
    Wd, Xd = torch.from_numpy(L.W).cuda(), torch.from_numpy(L.X).cuda()
    ws_s = torch.empty(awq.awq_workspace_bytes(M, K, N, cfg, len(alphas), 0), dtype=torch.uint8,
                       device="cuda")
    ws_a = torch.empty(awq.awq_act_stats_workspace_bytes(N, K), dtype=torch.uint8, device="cuda")

    def layer():
        return awq.quantize_layer(Wd, Xd, alphas, cfg, search_workspace=ws_s, stats_workspace=ws_a)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = HipEvent(), HipEvent()
        s = int(torch.cuda.current_stream().cuda_stream)
        e0.record(s)
        for _ in range(reps):
            fn()
        e1.record(s)
        torch.cuda.synchronize()
        return e0.elapsed_ms(e1) / reps

    eager_ms = timed(layer)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            layer()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer()
    graph_ms = timed(g.replay)
    del g
    return {"workload": f"c1: W {M}x{K}, X {N} tokens, {spec.w_bit}-bit symmetric, group "
                        f"{spec.group_size}, 20 alphas",
            "eager_us": eager_ms * 1e3, "eager_layers/s": 1000.0 / eager_ms,
            "graph_replay_us": graph_ms * 1e3, "graph_layers/s": 1000.0 / graph_ms}


def w4a16_bytes(M, K, g, T, with_s):
    """HBM bytes one W4A16 product must move: codes, fp16 step and zero per group, the
    activations, s if given, and the fp16 output."""
    return M * K / 2 + 4.0 * M * K / g + 2.0 * T * K + (4.0 * K if with_s else 0.0) + 2.0 * T * M


def time_large_layers(awq, torch, alphas, sptr, reps=2):
    """The whole 20-alpha search (statistics excluded) on the four large layer shapes, with
    seeded device-side weights and activations (1% of the channels scaled by 20).  With
    many more tokens than channels the library takes the loss through X^T X; the
    direct-equivalent rate divides the direct form's 2 M K N per alpha by the time."""
    shapes = [("c3 up", 11008, 4096, 16384, 4, 128, 1), ("c3 down", 4096, 11008, 16384, 4, 128, 1),
              ("c5", 13824, 5120, 32768, 3, 64, 1), ("c4", 28672, 8192, 65536, 4, 128, 1)]
    out = {}
    gen = torch.Generator(device="cuda")
    for name, M, K, N, b, g, zp in shapes:
        gen.manual_seed(20260 + M)
        W = (torch.randn((M, K), device="cuda", generator=gen) * 0.02).half()
        X = torch.randn((N, K), device="cuda", generator=gen)
        X[:, ::100] *= 20.0
        X = X.half()
        cfg = awq.qconfig(b, g, zp)
        a = awq.awq_act_stats(X)
        ws = torch.empty(awq.awq_workspace_bytes(M, K, N, cfg, len(alphas), 0),
                         dtype=torch.uint8, device="cuda")
        awq.awq_search_scales(W, X, a, alphas, cfg, workspace=ws)
        torch.cuda.synchronize()
        e0, e1 = HipEvent(), HipEvent()
        e0.record(sptr)
        for _ in range(reps):
            awq.awq_search_scales(W, X, a, alphas, cfg, workspace=ws)
        e1.record(sptr)
        torch.cuda.synchronize()
        ms = e0.elapsed_ms(e1) / reps
        direct = 2.0 * M * K * N * len(alphas)
        out[name] = {"M": M, "K": K, "N": N, "w_bit": b, "group_size": g, "search_ms": ms,
                     "form": "gram" if awq.awq_loss_form(M, K, N, len(alphas)) == awq.AWQ_LOSS_GRAM
                     else "direct",
                     "direct_equivalent_TFLOP/s": direct / (ms * 1e-3) / 1e12}
        del W, X, a, ws
        torch.cuda.empty_cache()
    return out


def time_w4a16(awq, torch, packed, s, Xd, cfg, sptr, M, K, reps=50):
    """The packed layer's W4A16 product at decode batches 1 and 4: on the layer just packed,
    and on a 28672 x 8192 packed layer (the 70B-class MLP shape) of seeded random codes."""

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = HipEvent(), HipEvent()
        e0.record(sptr)
        for _ in range(reps):
            fn()
        e1.record(sptr)
        torch.cuda.synchronize()
        return e0.elapsed_ms(e1) / reps

    out = {}
    codes, scales, zeros = packed
    g = cfg.group_size
    # the fold workspace of the s-given calls is allocated once, outside the timed loops
    ws = torch.empty(max(256, awq.awq_w4a16_workspace_bytes(16, max(K, 8192))),
                     dtype=torch.uint8, device="cuda")
    for T in (1, 4):
        x = Xd[:T].contiguous()
        ms = timed(lambda: awq.awq_w4a16_matmul(x, codes, scales, zeros, cfg, s=s, workspace=ws))
        b = w4a16_bytes(M, K, g, T, True)
        out[f"{M}x{K}_T{T}"] = {"us": ms * 1e3, "GB/s": b / (ms * 1e-3) / 1e9, "bytes": b,
                                "frac_hbm": b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
    M2, K2 = 28672, 8192
    gen = torch.Generator(device="cuda")
    gen.manual_seed(20250)
    c2 = torch.randint(0, 256, (M2, K2 // 2), dtype=torch.uint8, device="cuda", generator=gen)
    sc2 = (torch.rand((M2, K2 // g), device="cuda", generator=gen) * 0.02 + 0.0005).half()
    z2 = torch.randint(0, 16, (M2, K2 // g), device="cuda", generator=gen).half()
    s2 = torch.rand((K2,), device="cuda", generator=gen) * 3 + 0.5
    x2 = torch.randn((16, K2), device="cuda", generator=gen).half()
    for T in (1, 4, 16):
        x = x2[:T].contiguous()
        if T <= 4:
            ms = timed(lambda: awq.awq_w4a16_matmul(x, c2, sc2, z2, cfg, s=s2, workspace=ws))
            b = w4a16_bytes(M2, K2, g, T, True)
            out[f"{M2}x{K2}_T{T}"] = {"us": ms * 1e3, "GB/s": b / (ms * 1e-3) / 1e9, "bytes": b,
                                      "frac_hbm": b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
        # S^-1 already folded into the activations (the deployed form): no division
        ms = timed(lambda: awq.awq_w4a16_matmul(x, c2, sc2, z2, cfg))
        b = w4a16_bytes(M2, K2, g, T, False)
        out[f"{M2}x{K2}_T{T}_folded"] = {"us": ms * 1e3, "GB/s": b / (ms * 1e-3) / 1e9,
                                          "bytes": b,
                                          "frac_hbm": b / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
    return out


def _kernel_sha():
    import hashlib
    p = os.path.join(os.path.dirname(os.path.abspath(__file__)), "weight_only_quantization_act_amd",
                     "csrc", "loss_gemm.hip")
    with open(p, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


if __name__ == "__main__":
    main()
