"""Helpers shared by the GPU parity tests (comparison rules, device transfer)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import weight_only_quantization_act_amd as awq
from oracle import awq_oracle as O

LOSS_RTOL = 1e-3   # per-alpha loss tolerance
GAP_RTOL = 1e-3    # the chosen alpha must agree when best and runner-up differ by more

requires_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a HIP GPU")


def dev(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda")


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().numpy()


def ocfg(cfg) -> O.QConfig:
    return O.QConfig(cfg.w_bit, cfg.group_size, cfg.zero_point)


def say(msg: str):
    print(msg, flush=True)


def check_search(res_gpu, res_orc, where=""):
    """Per-alpha losses within LOSS_RTOL; same argmin when the oracle's gap between the best
    and the runner-up exceeds GAP_RTOL; s_out equal to the chosen alpha's scales (to one
    fp32 ulp, the power being evaluated by two different libraries)."""
    lg = host(res_gpu["losses"])
    lo = res_orc["losses"]
    assert lg.shape == lo.shape
    fin = np.isfinite(lo)
    assert np.array_equal(np.isfinite(lg), fin), (where, lg, lo)
    rel = np.abs(lg[fin] - lo[fin]) / np.maximum(np.abs(lo[fin]), 1e-300)
    assert rel.max(initial=0.0) <= LOSS_RTOL, (where, rel.max(), lg, lo)
    bg = int(host(res_gpu["best"])[0])
    bo = int(res_orc["best"])
    if bo >= 0 and fin.sum() >= 2:
        srt = np.sort(lo[fin])
        gap = (srt[1] - srt[0]) / max(abs(srt[0]), 1e-300)
        if gap > GAP_RTOL:
            assert bg == bo, (where, bg, bo, gap, lo)
        else:
            # near tie: the GPU's pick must still be within tolerance of the best loss
            assert bg >= 0 and lo[bg] <= srt[0] * (1 + 2 * LOSS_RTOL), (where, bg, bo, lo)
    else:
        assert bg == bo, (where, bg, bo)
    s = host(res_gpu["s"])
    if bg >= 0:
        want = res_orc["s_table"][bg]
    else:
        want = np.ones_like(s)
    ulps = np.abs(s.view(np.int32).astype(np.int64) - want.view(np.int32).astype(np.int64))
    assert ulps.max(initial=0) <= 1, (where, ulps.max())
    return lg, lo, bg, bo


def check_pack(codes, scales, zeros, W16, s32, cfg, where=""):
    pk, sc, zr = O.quantize_pack(W16, s32, ocfg(cfg))
    cg, sg, zg = host(codes), host(scales), host(zeros)
    if not np.array_equal(cg, pk):
        bad = np.argwhere(cg != pk)
        r, c = bad[0]
        raise AssertionError(f"{where}: {len(bad)} code bytes differ, first at row {r} byte {c}: "
                             f"gpu {cg[r, c]:#04x} oracle {pk[r, c]:#04x}")
    assert np.array_equal(sg.view(np.uint16), sc.view(np.uint16)), (where, "scales differ")
    assert np.array_equal(zg.view(np.uint16), zr.view(np.uint16)), (where, "zeros differ")
