#!/usr/bin/env python3
"""Benchmark: AWQ scale search + pack of one linear layer on one MI355X.

A step is one pass of the whole per-layer path on one synthetic layer: activation
statistics, scale family + fake quantisation + output-error loss for all 20 alphas,
argmin, final quantise-and-pack.  Inputs are resident in HBM before timing starts.
The default workload is the 4096 x 4096 layer with 4096 calibration tokens (4-bit,
zero-point, group 128, 20 alphas).

Prints one JSON line.  The loss product's live duration comes from HIP events that the
library records on its own stream around each of a step's loss-product launches (the grid
runs in the library's default passes, 6, 6, 6 and 2 points on this layer, so that each pass's
dW stays in the last-level cache).  On this layer the library takes the loss through G = X^T X
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
    p.add_argument("--alpha-batch", type=int, default=0,
                   help="grid points per pass of the search (0: the library's choice)")
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
            hip.hipGetLastError.argtypes = []
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
            # a failed query (an event never recorded) leaves its error pending in the
            # runtime, where the next unrelated call would report it: clear it here
            HipEvent._hip.hipGetLastError()
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


def pass_event_times(evs):
    """Sum the per-pass fake-quantisation and loss-product times of one search from the
    4 n events armed with awq_set_profile_pass_events; passes the search did not run were
    never recorded (their elapsed-time query fails).  Returns (fq_ms, loss_ms, passes)."""
    fq = loss = 0.0
    n = 0
    for p in range(len(evs) // 4):
        try:
            f = evs[4 * p].elapsed_ms(evs[4 * p + 1])
            g = evs[4 * p + 2].elapsed_ms(evs[4 * p + 3])
        except RuntimeError:
            break
        fq += f
        loss += g
        n += 1
    return fq, loss, n


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); this benchmark measures "
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
    ws_search = torch.empty(awq.awq_workspace_bytes(M, K, N, cfg, nA, args.alpha_batch), dtype=torch.uint8,
                            device="cuda")
    ws_stats = torch.empty(awq.awq_act_stats_workspace_bytes(N, K), dtype=torch.uint8,
                           device="cuda")
    stream = torch.cuda.current_stream()
    sptr = int(stream.cuda_stream)

    def step(ev=None, pev=None):
        if ev is not None:
            ev["st0"].record(sptr)
            awq.awq_set_stats_profile_events(ev["sk0"], ev["sk1"])
        a = awq.awq_act_stats(Xd, workspace=ws_stats)
        if ev is not None:
            ev["st1"].record(sptr)
            # the Gram pass from the one-shot hook; the fake quantisation and loss product of
            # every pass of the grid from the per-pass hook
            awq.awq_set_profile_events(None, None, None, None, ev["r0"], ev["r1"])
            awq.awq_set_profile_pass_events(pev)
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

    names = ("st0", "st1", "sk0", "sk1", "r0", "r1", "p0", "p1")
    evs = [{n: HipEvent() for n in names} for _ in range(args.steps)]
    pevs = [[HipEvent() for _ in range(4 * nA)] for _ in range(args.steps)]
    for i in range(args.steps):
        res, out = step(evs[i], pevs[i])
    torch.cuda.synchronize()

    def avg(a, b):
        return float(np.mean([e[a].elapsed_ms(e[b]) for e in evs]))

    gram = awq.awq_loss_form(M, K, N, nA) == awq.AWQ_LOSS_GRAM
    per_step = [pass_event_times(pe) for pe in pevs]
    passes = per_step[0][2]
    assert passes >= 1 and all(t[2] == passes for t in per_step), "per-pass events"
    fq_ms = float(np.mean([t[0] for t in per_step]))          # all passes of a step
    gemm_total_ms = float(np.mean([t[1] for t in per_step]))
    gemm_ms = gemm_total_ms / passes                           # average loss-product launch
    stats_ms, pack_ms = avg("st0", "st1"), avg("p0", "p1")
    stats_pass_ms = avg("sk0", "sk1")
    gram_ms = avg("r0", "r1") if gram else 0.0

    status = int(res["status"].cpu()[0])
    direct_flops = 2.0 * M * N * K * nA                     # the direct product dW_k X^T
    gemm_flops = loss_product_flops(M, K, N, nA, gram)
    gram_flops = gram_build_flops(N, K) if gram else 0.0
    gemm_tflops = gemm_flops / (gemm_total_ms * 1e-3) / 1e12
    g = spec.group_size
    # algorithmic bytes read and written by the streaming kernels
    stats_rw = (2.0 * N * K, 4.0 * K)
    # (W is read once by each pass's fake quantisation)
    fq_rw = (2.0 * M * K * passes + 4.0 * K * nA, 2.0 * M * K * nA)
    pack_rw = (2.0 * M * K + 4.0 * K, M * K / 2 + 4.0 * M * K / g)
    ceilings = measure_ceilings(awq, torch, sptr)

    # HBM bytes per launch from the committed counter summary, valid only for the kernel
    # source and workload it was measured on (null otherwise).
    traffic = None
    counters = None  # matrix-core busy fraction and clock from the same summary
    if os.path.exists(args.traffic_summary):
        kv = {}
        with open(args.traffic_summary) as f:
            for ln in f:
                m = re.match(r"^(kernel_source_sha|workload|launches_per_step|hbm_bytes_per_launch|"
                             r"mfma_busy_frac|shader_clock_ghz): (\S+)\s*$", ln)
                if m:
                    kv[m.group(1)] = m.group(2)
        if (kv.get("workload") == spec.name and kv.get("kernel_source_sha") == _kernel_sha()
                and kv.get("launches_per_step") == str(passes)):
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
                   "search_passes": passes,
                   "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "achieved": gemm_tflops, "peak": MFMA_F16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": gemm_tflops / MFMA_F16_PEAK_TFLOPS,
                     "traffic": traffic,
                     "kernel": "k_loss_gemm" + ("<G form>" if gram else ""),
                     "flops_per_launch": gemm_flops / passes, "avg_launch_ms": gemm_ms,
                     "launches_per_step": passes,
                     "mfma_counters": counters,
                     # the same rate against this device's matrix-core-only probe (same run)
                     "measured_ceiling": {
                         "TFLOP/s": ceilings["mfma_probe"]["TFLOP/s"],
                         "shader_clock_GHz": ceilings["mfma_probe"]["shader_clock_GHz"],
                         "frac": gemm_tflops / ceilings["mfma_probe"]["TFLOP/s"],
                         "source": "awq_probe_mfma"},
                     "form": "gram" if gram else "direct",
                     # the G form executes M K^2 (1 + 128/K) per alpha where the direct product
                     # would take 2 M K N: the ratio of the two is work saved, not a rate
                     "direct_over_executed_flops": direct_flops / (gemm_flops + gram_flops)},
        "kernels": {
            "act_stats": hbm_entry(*stats_rw, stats_pass_ms, ceilings, call_ms=stats_ms,
                                   timed="streaming pass (first of the two launches), library "
                                         "events"),
            "fake_quant": hbm_entry(*fq_rw, fq_ms, ceilings, launches=passes,
                                    timed="all launches of a step, library events"),
            "loss_gemm": {"ms": gemm_total_ms, "launches": passes, "TFLOP/s": gemm_tflops,
                          "frac_mfma": gemm_tflops / MFMA_F16_PEAK_TFLOPS,
                          "form": "gram" if gram else "direct"},
            **({"gram": {"ms": gram_ms, "build_flops": gram_flops,
                         "TFLOP/s": gram_flops / (gram_ms * 1e-3) / 1e12,
                         "frac_mfma": gram_flops / (gram_ms * 1e-3) / 1e12 / MFMA_F16_PEAK_TFLOPS,
                         "timed": "the whole Gram pass (transpose, build, combine, split) "
                                  "against the build's executed flops"}} if gram else {}),
            "quant_pack": hbm_entry(*pack_rw, pack_ms, ceilings,
                                    timed="one launch, events around the call"),
        },
        "search_status": status,
    }
    if not args.no_variants:
        line["variants"] = time_variants(awq, torch, Wd, Xd, cfg, sptr, M, K, N, ceilings)
        line["w4a16"] = time_w4a16(awq, torch, out, res["s"], Xd, cfg, sptr, M, K, ceilings)
        line["large_layers"] = time_large_layers(awq, torch, alphas, sptr, ceilings)
        line["small_layer"] = time_small_layer(awq, torch, sptr)
    line["ceilings"] = ceilings
    line["size_floor"] = measure_size_floor(awq, torch, Xd, Wd, sptr)
    # the short streaming calls as graph replays (kernel time, no per-launch dispatch gap)
    # against the same-size probes timed back to back; the statistics call is two launches
    sf = line["size_floor"]
    st_g, _ = graph_and_eager_ms(torch, lambda: awq.awq_act_stats(Xd, workspace=ws_stats), sptr, 20)
    pk_g, _ = graph_and_eager_ms(torch, lambda: awq.awq_quantize_pack(Wd, res["s"], cfg), sptr, 20)
    line["kernels"]["act_stats"]["graph_call_ms"] = st_g
    line["kernels"]["act_stats"]["frac_same_size_read_probe"] = sf["read_X_probe"]["ms"] / st_g
    line["kernels"]["quant_pack"]["graph_call_ms"] = pk_g
    line["kernels"]["quant_pack"]["frac_same_size_copy_probe"] = (
        sf["copy_W_probe"]["ms"] * (pack_rw[0] + pack_rw[1]) / (2.0 * M * K * 2.0) / pk_g)
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


def loss_product_flops(M, K, N, n_alpha, gram):
    """Matrix-core flops of the loss product over the whole grid (all passes), as executed.  G form:
    each half (128 channels) of a 256-channel tile row runs over k from its own first channel
    on, for 256-row tiles of dW (M a multiple of 256 here).  Direct form: 2 M K N per alpha."""
    if not gram:
        return 2.0 * M * K * N * n_alpha
    m_pad = -(-M // 256) * 256
    return n_alpha * sum(2.0 * m_pad * min(128, K - c0) * (K - c0) for c0 in range(0, K, 128))


def gram_build_flops(N, K):
    """Matrix-core flops of the Gram build as executed: every 256 x 256 tile of G's upper block
    triangle (the diagonal tiles whole) over the N tokens."""
    T = -(-K // 256)
    return T * (T + 1) / 2 * 2.0 * 256 * 256 * N


def measure_size_floor(awq, torch, Xd, Wd, sptr, reps=20):
    """Plain device operations on the headline layer's own tensors, for the size floor of the
    short statistics and pack launches: a full read of X (the read probe, and torch.sum over
    all elements with fp32 accumulation) and a copy of W (the copy probe and torch's copy,
    read + write of the same bytes).  At 32-64 MiB these operands fit the 256 MB last-level
    cache, so no HBM fraction is given for them."""

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
    ms = timed(lambda: torch.sum(Xd, dtype=torch.float32))
    b = Xd.numel() * 2.0
    out["read_X_torch_sum"] = {"ms": ms, "bytes": b, "GB/s": b / (ms * 1e-3) / 1e9}
    dst = torch.empty_like(Wd)
    ms = timed(lambda: dst.copy_(Wd))
    b = Wd.numel() * 4.0
    out["copy_W"] = {"ms": ms, "bytes": b, "GB/s": b / (ms * 1e-3) / 1e9}
    ms = timed(lambda: awq.awq_probe_read(Xd))
    b = Xd.numel() * 2.0
    out["read_X_probe"] = {"ms": ms, "bytes": b, "GB/s": b / (ms * 1e-3) / 1e9}
    ms = timed(lambda: awq.awq_probe_copy(Wd, dst))
    b = Wd.numel() * 4.0
    out["copy_W_probe"] = {"ms": ms, "bytes": b, "GB/s": b / (ms * 1e-3) / 1e9}
    return out


def measure_ceilings(awq, torch, sptr, reps=5):
    """This device's practical ceilings, measured after the timed region with the library's
    probes and torch:
      - matrix cores: awq_probe_mfma, blocks of eight waves issuing back-to-back fp16
        32x32x16 MFMAs on registers; the shader clock from the shader-clock and real-time
        counters;
      - LDS: awq_probe_lds, conflict-free 16-byte reads, bytes per shader clock per unit;
      - HBM: a streaming read (awq_probe_read) and write (awq_probe_write) of 1 GiB and a
        copy (awq_probe_copy, and torch's copy) of 512 MiB (read + write bytes over time),
        all larger than the 256 MB last-level cache;
      - a plain fp16 4096^3 product through torch.matmul (hipBLASLt)."""

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
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    wall_ghz = awq.awq_probe_wall_clock_khz(0) * 1e-6

    def clock_ghz(ticks):
        # shader-clock ticks over real-time ticks of each block's first wave (its own loop)
        t = ticks.cpu().double()
        return float((t[:, 0] / t[:, 1]).median()) * wall_ghz

    # matrix cores: four rounds of blocks (one block of eight waves fits a compute unit);
    # the rate comes from the kernel's events, not from the blocks' ticks, because the
    # older wave of a SIMD finishes its loop well before the younger one
    iters, blocks = 8000, 4 * n_cu
    ms = timed(lambda: awq.awq_probe_mfma(blocks, iters))
    ghz = clock_ghz(awq.awq_probe_mfma(blocks, iters))
    tfs = blocks * 8.0 * iters * 8 * 32768 / (ms * 1e-3) / 1e12
    out["mfma_probe"] = {"TFLOP/s": tfs, "frac_of_2.5PF": tfs / MFMA_F16_PEAK_TFLOPS,
                         "shader_clock_GHz": ghz,
                         "flop_per_clock_per_SIMD": tfs * 1e12 / (n_cu * 4 * ghz * 1e9),
                         "ms": ms, "blocks": blocks, "compute_units": n_cu}
    # LDS reads, same geometry
    iters = 2000
    ms = timed(lambda: awq.awq_probe_lds(blocks, iters))
    ghz = clock_ghz(awq.awq_probe_lds(blocks, iters))
    tbs = blocks * 8.0 * iters * 16 * 1024 / (ms * 1e-3) / 1e12
    out["lds_probe"] = {"TB/s": tbs, "shader_clock_GHz": ghz,
                        "bytes_per_clock_per_CU": tbs * 1e12 / (n_cu * ghz * 1e9), "ms": ms}
    # HBM: 1 GiB read, 1 GiB written, 512 MiB copied (1 GiB moved)
    buf = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    ms = timed(lambda: awq.awq_probe_read(buf))
    out["read_GB/s"] = buf.numel() / (ms * 1e-3) / 1e9
    ms = timed(lambda: awq.awq_probe_write(buf))
    out["write_GB/s"] = buf.numel() / (ms * 1e-3) / 1e9
    src, dst = buf[: 512 << 20], buf[512 << 20:]
    ms = timed(lambda: awq.awq_probe_copy(src, dst))
    out["copy_GB/s"] = 2.0 * src.numel() / (ms * 1e-3) / 1e9
    ms = timed(lambda: dst.copy_(src))
    out["torch_copy_GB/s"] = 2.0 * src.numel() / (ms * 1e-3) / 1e9
    del buf, src, dst
    for k in ("read", "write", "copy", "torch_copy"):
        out[f"{k}_frac_of_8TBps"] = out[f"{k}_GB/s"] / HBM_PEAK_GBS
    gen = torch.Generator(device="cuda")
    gen.manual_seed(7)
    a = torch.randn((4096, 4096), device="cuda", generator=gen).half()
    b = torch.randn((4096, 4096), device="cuda", generator=gen).half()
    c = torch.empty((4096, 4096), device="cuda", dtype=torch.float16)
    ms = timed(lambda: torch.matmul(a, b, out=c))
    gemm_tf = 2.0 * 4096 ** 3 / (ms * 1e-3) / 1e12
    del a, b, c
    torch.cuda.empty_cache()
    out["torch_matmul_fp16_4096^3_TFLOP/s"] = gemm_tf
    out["torch_matmul_frac_of_2.5PF"] = gemm_tf / MFMA_F16_PEAK_TFLOPS
    return out


def hbm_entry(rd, wr, ms, ceil, **extra):
    """A streaming kernel's rate: algorithmic bytes read (rd) and written (wr) over its time,
    as a fraction of 8 TB/s and of this device's measured ceiling for that mix of reads and
    writes.  The ceiling's time adds the read and write streams at the probes' rates and a
    turnaround cost for interleaving them, fitted so that an equal mix (a copy) takes the
    copy probe's time:  t = rd / read + wr / write + c min(rd, wr),
    c = 2 / copy - 1 / read - 1 / write (at least 0)."""
    b = rd + wr
    gbs = b / (ms * 1e-3) / 1e9
    r, w, cp = (ceil[k] * 1e9 for k in ("read_GB/s", "write_GB/s", "copy_GB/s"))
    turn = max(0.0, 2.0 / cp - 1.0 / r - 1.0 / w)
    t_ceil = rd / r + wr / w + turn * min(rd, wr)
    return {"ms": ms, "bytes": b, "GB/s": gbs, "frac_hbm_8TBps": gbs / HBM_PEAK_GBS,
            "ceiling_GB/s": b / t_ceil / 1e9, "frac_measured_ceiling": t_ceil / (ms * 1e-3),
            **extra}


def graph_and_eager_ms(torch, fn, sptr, reps):
    """(GPU time, host-inclusive time) per call of `fn`, in ms.  The GPU time comes from
    replays of `reps` calls captured in one HIP graph (HIP events around a replay), so the
    host's per-call marshalling and launch cost drop out; the eager figure is `reps` calls
    issued back to back, which for calls of a few microseconds is set by the host."""
    fn()
    torch.cuda.synchronize()
    e0, e1 = HipEvent(), HipEvent()
    e0.record(sptr)
    for _ in range(reps):
        fn()
    e1.record(sptr)
    torch.cuda.synchronize()
    eager = e0.elapsed_ms(e1) / reps
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(reps):
            fn()
    g.replay()
    torch.cuda.synchronize()
    best = None
    for _ in range(3):
        e0, e1 = HipEvent(), HipEvent()
        e0.record(sptr)
        g.replay()
        e1.record(sptr)
        torch.cuda.synchronize()
        ms = e0.elapsed_ms(e1) / reps
        best = ms if best is None else min(best, ms)
    del g
    return best, eager


def time_variants(awq, torch, Wd, Xd, cfg, sptr, M, K, N, ceil, reps=20):
    """Average time per call of the widened entry points on the same layer, measured
    after the timed region: the streaming calls as graph replays (with the eager per-call
    time beside them), the two searches as `reps` back-to-back calls (milliseconds each,
    so host overhead does not count)."""

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
    for name, mode, extra in [("stat_max_abs", awq.AWQ_STAT_MAX_ABS, ()),
                              ("stat_rms_ratio", awq.AWQ_STAT_RMS_RATIO, ()),
                              ("stat_ema_mean_b512", awq.AWQ_STAT_EMA_MEAN, (512, 0.9))]:
        ms, eager = graph_and_eager_ms(torch, lambda: awq.awq_act_stats_ex(Xd, mode, *extra),
                                       sptr, reps)
        out[name] = hbm_entry(2.0 * N * K, 4.0 * K, ms, ceil, eager_call_ms=eager,
                              timed="whole call (two launches), graph replay")
    a = awq.awq_act_stats(Xd)
    ms, eager = graph_and_eager_ms(torch, lambda: awq.awq_threshold_scales(a, 70.0, 2.0), sptr,
                                   reps)
    out["threshold_scales"] = {"ms": ms, "eager_call_ms": eager, "in_features": K,
                               "timed": "graph replay"}
    Xr = torch.empty_like(Xd)
    ms, eager = graph_and_eager_ms(torch, lambda: awq.awq_hadamard_rotate(Xd, 128, out=Xr), sptr,
                                   reps)
    out["hadamard_rotate_X_b128"] = hbm_entry(2.0 * N * K, 2.0 * N * K, ms, ceil,
                                              eager_call_ms=eager, timed="graph replay")
    table = torch.stack([awq.awq_threshold_scales(a, p, f) for p in (50.0, 70.0, 85.0, 95.0, 99.0)
                         for f in (1.5, 2.0, 3.0, 4.0)]).contiguous()
    ws = torch.empty(awq.awq_workspace_bytes(M, K, N, cfg, table.shape[0], 0), dtype=torch.uint8,
                     device="cuda")
    ms = timed(lambda: awq.awq_search_scale_table(Wd, Xd, table, cfg, workspace=ws))
    gram = awq.awq_loss_form(M, K, N, table.shape[0]) == awq.AWQ_LOSS_GRAM
    ex = loss_product_flops(M, K, N, table.shape[0], gram) + (gram_build_flops(N, K) if gram else 0)
    tfx = ex / (ms * 1e-3) / 1e12
    out["search_scale_table_20_threshold_rows"] = {
        "ms": ms, "executed_mfma_flops": ex, "TFLOP/s_whole_search": tfx,
        "frac_mfma_whole_search": tfx / MFMA_F16_PEAK_TFLOPS,
        "form": "gram" if gram else "direct"}
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


def time_large_layers(awq, torch, alphas, sptr, ceil, reps=2):
    """The whole 20-alpha search on the four large layer shapes, with seeded device-side
    weights and activations (1% of the channels scaled by 20).  The library's event hook
    times the Gram pass and the loss product of each search separately; their rates are
    executed matrix-core flops over kernel time.  On the 70B-class shape the statistics
    (over its 1 GiB of activations) and the pack (of its 448 MiB weight) are timed too."""
    shapes = [("c3 up", 11008, 4096, 16384, 4, 128, 1), ("c3 down", 4096, 11008, 16384, 4, 128, 1),
              ("c5", 13824, 5120, 32768, 3, 64, 1), ("c4", 28672, 8192, 65536, 4, 128, 1)]
    out = {}
    gen = torch.Generator(device="cuda")
    nA = len(alphas)

    def tf(flops, ms):
        v = flops / (ms * 1e-3) / 1e12
        return {"TFLOP/s": v, "frac_mfma": v / MFMA_F16_PEAK_TFLOPS}

    for name, M, K, N, b, g, zp in shapes:
        gen.manual_seed(20260 + M)
        W = (torch.randn((M, K), device="cuda", generator=gen) * 0.02).half()
        X = torch.randn((N, K), device="cuda", generator=gen)
        X[:, ::100] *= 20.0
        X = X.half()
        cfg = awq.qconfig(b, g, zp)
        a = awq.awq_act_stats(X)
        ws = torch.empty(awq.awq_workspace_bytes(M, K, N, cfg, nA, 0),
                         dtype=torch.uint8, device="cuda")
        awq.awq_search_scales(W, X, a, alphas, cfg, workspace=ws)
        torch.cuda.synchronize()
        gram = awq.awq_loss_form(M, K, N, nA) == awq.AWQ_LOSS_GRAM
        runs = []
        for _ in range(reps):
            ev = [HipEvent() for _ in range(8)]
            pev = [HipEvent() for _ in range(4 * nA)]
            ev[0].record(sptr)
            awq.awq_set_profile_events(None, None, None, None, ev[6], ev[7])
            awq.awq_set_profile_pass_events(pev)
            awq.awq_search_scales(W, X, a, alphas, cfg, workspace=ws)
            ev[1].record(sptr)
            runs.append((ev, pev))
        torch.cuda.synchronize()
        search_ms = float(sum(e[0].elapsed_ms(e[1]) for e, _ in runs) / reps)
        pt = [pass_event_times(pe) for _, pe in runs]
        gemm_ms = float(sum(t[1] for t in pt) / len(pt))
        fq_ms = float(sum(t[0] for t in pt) / len(pt))
        passes = pt[0][2]
        gflops = loss_product_flops(M, K, N, nA, gram)
        entry = {"M": M, "K": K, "N": N, "w_bit": b, "group_size": g, "search_ms": search_ms,
                 "form": "gram" if gram else "direct",
                 "passes": passes,
                 "loss_product": {"ms": gemm_ms, "flops": gflops, **tf(gflops, gemm_ms)},
                 "fake_quant": {"ms": fq_ms,
                                "GB/s": (2.0 * M * K * (nA + passes)) / (fq_ms * 1e-3) / 1e9}}
        bflops = 0.0
        if gram:
            gram_ms = float(sum(e[6].elapsed_ms(e[7]) for e, _ in runs) / reps)
            bflops = gram_build_flops(N, K)
            entry["gram_pass"] = {"ms": gram_ms, "build_flops": bflops, **tf(bflops, gram_ms)}
        entry["direct_over_executed_flops"] = 2.0 * M * K * N * nA / (gflops + bflops)
        if name == "c4":
            entry["act_stats"] = time_stats_and_pack(awq, torch, W, X, cfg, sptr, ceil)
        out[name] = entry
        del W, X, a, ws
        torch.cuda.empty_cache()
    return out


def time_stats_and_pack(awq, torch, W, X, cfg, sptr, ceil, reps=5):
    """Statistics over a 1 GiB activation tensor and the pack of a 448 MiB weight: sizes at
    which the HBM fraction of these streaming kernels is not set by launch overhead."""
    N, K = X.shape
    M = W.shape[0]
    ws = torch.empty(awq.awq_act_stats_workspace_bytes(N, K), dtype=torch.uint8, device="cuda")
    s = torch.ones(K, dtype=torch.float32, device="cuda") * 1.5
    awq.awq_act_stats(X, workspace=ws)
    awq.awq_quantize_pack(W, s, cfg)
    torch.cuda.synchronize()
    st, pk = [], []
    for _ in range(reps):
        e = [HipEvent() for _ in range(4)]
        awq.awq_set_stats_profile_events(e[0], e[1])
        awq.awq_act_stats(X, workspace=ws)
        e[2].record(sptr)
        awq.awq_quantize_pack(W, s, cfg)
        e[3].record(sptr)
        st.append(e)
    torch.cuda.synchronize()
    ms_s = float(sum(e[0].elapsed_ms(e[1]) for e in st) / reps)
    ms_p = float(sum(e[2].elapsed_ms(e[3]) for e in st) / reps)
    return {"stats_pass": hbm_entry(2.0 * N * K, 4.0 * K, ms_s, ceil),
            "quant_pack": hbm_entry(2.0 * M * K + 4.0 * K,
                                    M * K / 2 + 4.0 * M * K / cfg.group_size, ms_p, ceil)}


def time_w4a16(awq, torch, packed, s, Xd, cfg, sptr, M, K, ceil, reps=50):
    """The packed layer's W4A16 product at decode batches 1 and 4: on the layer just packed,
    and on a 28672 x 8192 packed layer (the 70B-class MLP shape) of seeded random codes.
    Kernel time from graph replays; the eager per-call time (host marshalling and launch
    included) is reported beside it."""
    out = {}
    codes, scales, zeros = packed
    g = cfg.group_size
    # the fold workspace of the s-given calls is allocated once, outside the timed loops
    ws = torch.empty(max(256, awq.awq_w4a16_workspace_bytes(16, max(K, 8192))),
                     dtype=torch.uint8, device="cuda")

    def entry(fn, b, out_bytes):
        ms, eager = graph_and_eager_ms(torch, fn, sptr, reps)
        e = hbm_entry(b - out_bytes, out_bytes, ms, ceil, eager_call_us=eager * 1e3)
        e["us"] = ms * 1e3
        return e

    for T in (1, 4):
        x = Xd[:T].contiguous()
        y = torch.empty((T, M), dtype=torch.float16, device="cuda")
        out[f"{M}x{K}_T{T}"] = entry(
            lambda: awq.awq_w4a16_matmul(x, codes, scales, zeros, cfg, s=s, out=y, workspace=ws),
            w4a16_bytes(M, K, g, T, True), 2.0 * T * M)
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
        y = torch.empty((T, M2), dtype=torch.float16, device="cuda")
        if T <= 4:
            out[f"{M2}x{K2}_T{T}"] = entry(
                lambda: awq.awq_w4a16_matmul(x, c2, sc2, z2, cfg, s=s2, out=y, workspace=ws),
                w4a16_bytes(M2, K2, g, T, True), 2.0 * T * M2)
        # S^-1 already folded into the activations (the deployed form): no division
        out[f"{M2}x{K2}_T{T}_folded"] = entry(
            lambda: awq.awq_w4a16_matmul(x, c2, sc2, z2, cfg, out=y),
            w4a16_bytes(M2, K2, g, T, False), 2.0 * T * M2)
    return out


def _kernel_sha():
    import hashlib
    p = os.path.join(os.path.dirname(os.path.abspath(__file__)), "weight_only_quantization_act_amd",
                     "csrc", "loss_gemm.hip")
    with open(p, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


if __name__ == "__main__":
    main()
