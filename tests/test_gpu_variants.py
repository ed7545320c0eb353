"""GPU variants of the statistic, the scale family and the inputs, through the C ABI,
against the CPU oracle.

  - statistics: max |x| and the EMA of batch means bit-exact; E|x| / sqrt(E x^2) within
    one fp32 ulp (its fp64 sum of squares is not exact, so the summation order can move
    the last bit); ragged token counts, batches that do not divide N, one token, NaN;
  - percentile-threshold scales bit-exact (ties, K not a power of two, the extremes
    0 and 100, the 32768-channel maximum; negative scores, +-0, subnormals, +-inf and
    NaN, which both sides order last);
  - the search over an explicit scale table: the same bars as the alpha-grid search;
  - the blockwise Hadamard rotation: equal fp16 values (+0 and -0 count as equal; both
    sides take the exact +-1 sums in fp64, one rounding for the normalisation and a
    correctly rounded cast), and the search on rotated weights and activations.
"""
import numpy as np
import pytest
import torch

import weight_only_quantization_act_amd as awq
from oracle import awq_oracle as O
from synth import CONFIGS, alpha_grid, make_layer, small_spec
from tests.gpu_util import check_search, dev, host, ocfg, requires_gpu, say

pytestmark = [pytest.mark.gpu, requires_gpu]

F16, F32 = np.float16, np.float32

STAT_CASES = [(1, 8, "normal"), (37, 136, "normal"), (300, 1000, "t4"), (513, 1001, "normal"),
              (4099, 2056, "t4")]


def _same_f32(g, o, max_ulp=0):
    g = np.asarray(g, F32)
    o = np.asarray(o, F32)
    assert g.shape == o.shape
    nan = np.isnan(o)
    assert np.array_equal(np.isnan(g), nan)
    d = np.abs(g[~nan].view(np.int32).astype(np.int64) - o[~nan].view(np.int32).astype(np.int64))
    assert d.max(initial=0) <= max_ulp, d.max(initial=0)


# ----------------------------------------------------------------------------- statistics
@pytest.mark.parametrize("N,K,dist", STAT_CASES)
def test_stat_max_abs(N, K, dist):
    say(f"max|x| N={N} K={K}")
    L = make_layer(small_spec("m", 8, K, N, x_dist=dist, outlier_count=max(1, K // 100)))
    g = host(awq.awq_act_stats_ex(dev(L.X), awq.AWQ_STAT_MAX_ABS))
    _same_f32(g, O.act_stat_max_abs(L.X))


@pytest.mark.parametrize("N,K,dist", STAT_CASES)
def test_stat_rms_ratio(N, K, dist):
    say(f"rms ratio N={N} K={K}")
    L = make_layer(small_spec("r", 8, K, N, x_dist=dist, outlier_count=max(1, K // 100)))
    X = L.X.copy()
    X[:, 3] = 0                               # an all-zero channel gets 0
    g = host(awq.awq_act_stats_ex(dev(X), awq.AWQ_STAT_RMS_RATIO))
    o = O.act_stat_rms_ratio(X)
    assert g[3] == 0.0 and o[3] == 0.0
    _same_f32(g, o, max_ulp=1)


@pytest.mark.parametrize("N,K,batch", [(1, 8, 1), (300, 1000, 64), (1000, 512, 7),
                                       (4099, 2056, 512), (257, 136, 5000), (2048, 1024, 2048)])
def test_stat_ema_mean(N, K, batch):
    say(f"ema N={N} K={K} batch={batch}")
    L = make_layer(small_spec("e", 8, K, N, outlier_count=max(1, K // 100)))
    for mom in (0.9, 0.0, 0.5):
        g = host(awq.awq_act_stats_ex(dev(L.X), awq.AWQ_STAT_EMA_MEAN, batch, mom))
        _same_f32(g, O.act_stat_ema_mean(L.X, batch, mom))


def test_stats_nan_propagates():
    L = make_layer(small_spec("n", 8, 256, 700))
    X = L.X.copy()
    X[650, 17] = np.nan
    Xd = dev(X)
    for mode, ref in [(awq.AWQ_STAT_MAX_ABS, O.act_stat_max_abs(X)),
                      (awq.AWQ_STAT_RMS_RATIO, O.act_stat_rms_ratio(X)),
                      (awq.AWQ_STAT_EMA_MEAN, O.act_stat_ema_mean(X, 100, 0.9))]:
        g = host(awq.awq_act_stats_ex(Xd, mode, 100, 0.9))
        _same_f32(g, ref, max_ulp=1 if mode == awq.AWQ_STAT_RMS_RATIO else 0)


def test_stats_mean_mode_matches_plain_entry():
    L = make_layer(small_spec("p", 8, 1000, 513))
    Xd = dev(L.X)
    a = host(awq.awq_act_stats(Xd))
    b = host(awq.awq_act_stats_ex(Xd, awq.AWQ_STAT_MEAN_ABS))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_stats_variants_headline_layer():
    L = make_layer(CONFIGS["c2"][0])
    Xd = dev(L.X)
    say("stat variants c2 4096x4096")
    _same_f32(host(awq.awq_act_stats_ex(Xd, awq.AWQ_STAT_MAX_ABS)), O.act_stat_max_abs(L.X))
    _same_f32(host(awq.awq_act_stats_ex(Xd, awq.AWQ_STAT_RMS_RATIO)), O.act_stat_rms_ratio(L.X), 1)
    _same_f32(host(awq.awq_act_stats_ex(Xd, awq.AWQ_STAT_EMA_MEAN, 512, 0.9)),
              O.act_stat_ema_mean(L.X, 512, 0.9))


# ----------------------------------------------------------------------------- threshold
def _scores(rng, K, kind):
    if kind == "lognormal":
        return np.exp(rng.normal(0.0, 1.0, K)).astype(F32)
    if kind == "ties":                          # few distinct values: many exact ties
        return rng.integers(0, 5, K).astype(F32) * F32(0.25)
    if kind == "constant":
        return np.full(K, 1.5, F32)
    if kind == "special":                       # signs, +-0, subnormals, +-inf, NaN
        v = rng.normal(0.0, 1.0, K).astype(F32)
        pool = np.array([0.0, -0.0, 1e-42, -1e-42, np.inf, -np.inf, np.nan, 2.0], F32)
        pick = rng.random(K) < 0.3
        v[pick] = pool[rng.integers(0, pool.size, int(pick.sum()))]
        return v
    raise ValueError(kind)


@pytest.mark.parametrize("K", [1, 2, 7, 128, 1000, 4096, 11008, 32768])
@pytest.mark.parametrize("kind", ["lognormal", "ties", "constant", "special"])
def test_threshold_scales(K, kind):
    say(f"threshold K={K} {kind}")
    rng = np.random.default_rng(K * 7 + len(kind))
    a = _scores(rng, K, kind)
    ad = dev(a)
    for p, f in [(70.0, 2.0), (85.0, 2.0), (0.0, 1.5), (100.0, 3.0), (99.9, 4.0), (33.3, 0.5)]:
        g = host(awq.awq_threshold_scales(ad, p, f))
        o = O.threshold_scales(a, p, f)
        assert np.array_equal(g.view(np.uint32), o.view(np.uint32)), (K, kind, p, f)


def test_threshold_scales_from_gpu_statistic():
    """Threshold on the GPU statistic of a layer with outlier channels, compared with the
    oracle's threshold on the oracle's statistic (the two statistics are bit-equal)."""
    L = make_layer(small_spec("t", 8, 4096, 1024, outlier_count=40))
    a = awq.awq_act_stats(dev(L.X))
    g = host(awq.awq_threshold_scales(a, 99.0, 2.0))
    o = O.threshold_scales(O.act_stats(L.X), 99.0, 2.0)
    assert np.array_equal(g, o)
    assert 1 <= (g == 2.0).sum() <= 41     # above the 99th percentile of 4096 values


# ----------------------------------------------------------------------------- scale table
@pytest.mark.parametrize("M,K,N,w_bit,g,zp", [(256, 256, 256, 4, 128, 1),
                                              (300, 384, 700, 4, 128, 1),
                                              (77, 160, 33, 3, 32, 1),
                                              (520, 512, 1, 4, 64, 0),
                                              (200, 256, 4000, 4, 128, 1)])  # loss via X^T X
def test_search_scale_table(M, K, N, w_bit, g, zp):
    say(f"table search M={M} K={K} N={N}")
    L = make_layer(small_spec("q", M, K, N, w_bit=w_bit, group_size=g, zero_point=zp,
                              outlier_count=max(1, K // 100), seed=M + K))
    cfg = awq.qconfig(w_bit, g, zp)
    a = O.act_stats(L.X)
    rows = [O.scale_family(a, alpha_grid(6))]
    rows += [O.threshold_scales(a, p, f)[None, :] for p, f in [(70, 2.0), (90, 4.0), (99, 8.0)]]
    table = np.ascontiguousarray(np.concatenate(rows, axis=0), dtype=F32)
    res = awq.awq_search_scale_table(dev(L.W), dev(L.X), dev(table), cfg)
    torch.cuda.synchronize()
    orc = O.search_scale_table(L.W, L.X, table, ocfg(cfg))
    check_search(res, orc, f"table {M}x{K}x{N}")
    assert int(host(res["status"])[0]) == awq.AWQ_OK


def test_scale_table_equals_alpha_grid_search():
    """A table holding a^alpha (numpy's power) gives the alpha-grid search's losses."""
    L = make_layer(small_spec("g", 512, 512, 600, outlier_count=5))
    cfg = awq.qconfig(4, 128, 1)
    alphas = alpha_grid(20)
    Wd, Xd = dev(L.W), dev(L.X)
    a = awq.awq_act_stats(Xd)
    grid = awq.awq_search_scales(Wd, Xd, a, alphas, cfg)
    tab = O.scale_family(host(a), alphas)
    torch.cuda.synchronize()
    res = awq.awq_search_scale_table(Wd, Xd, dev(tab), cfg)
    # the library's power may differ from numpy's by one fp32 ulp, hence rtol, not bits
    lg, lt = host(grid["losses"]), host(res["losses"])
    assert np.allclose(lg, lt, rtol=1e-6, atol=0)
    assert int(host(grid["best"])[0]) == int(host(res["best"])[0])


# ----------------------------------------------------------------------------- Hadamard
def _check_rotation(g, o, where):
    g = np.asarray(g, F16).astype(np.float64)
    o = np.asarray(o, F16).astype(np.float64)
    assert g.shape == o.shape
    diff = ~((g == o) | (np.isnan(g) & np.isnan(o)))
    if diff.any():
        r = np.argwhere(diff)[0]
        raise AssertionError(f"{where}: {int(diff.sum())} values differ, first at {tuple(r)}: "
                             f"gpu {g[tuple(r)]!r} oracle {o[tuple(r)]!r}")


@pytest.mark.parametrize("block", [2, 4, 8, 16, 32, 64, 128, 256, 512])
def test_hadamard_blocks(block):
    rows, K = 37, 1024
    say(f"hadamard block={block}")
    L = make_layer(small_spec("h", rows, K, 8, outlier_count=10))
    A = L.W * F16(64)                                  # a typical fp16 spread
    A[0, :] = L.X[0]                                   # activation-like row with outliers
    g = host(awq.awq_hadamard_rotate(dev(A), block))
    _check_rotation(g, O.hadamard_rotate(A, block), f"block {block}")


@pytest.mark.parametrize("rows,K,block", [(1, 8, 8), (3, 24, 8), (257, 640, 128), (4099, 512, 512),
                                         (5, 11008, 256)])
def test_hadamard_shapes_and_in_place(rows, K, block):
    say(f"hadamard {rows}x{K} block={block}")
    rng = np.random.default_rng(rows + K)
    A = rng.standard_t(4, (rows, K)).astype(F16)
    o = O.hadamard_rotate(A, block)
    Ad = dev(A)
    g = host(awq.awq_hadamard_rotate(Ad, block))
    _check_rotation(g, o, "out of place")
    awq.awq_hadamard_rotate(Ad, block, out=Ad)         # in place
    _check_rotation(host(Ad), o, "in place")


def test_hadamard_headline_activations():
    L = make_layer(CONFIGS["c2"][0])
    say("hadamard c2 X 4096x4096 block 128")
    g = host(awq.awq_hadamard_rotate(dev(L.X), 128))
    _check_rotation(g, O.hadamard_rotate(L.X, 128), "c2 X")


def test_hadamard_spreads_outliers_and_search_on_rotated_layer():
    """Rotating W and X by the same orthogonal blocks keeps W X^T and flattens the
    per-channel statistic; the search then runs on the rotated layer."""
    L = make_layer(small_spec("o", 512, 1024, 700, outlier_count=8))
    cfg = awq.qconfig(4, 128, 1)
    alphas = alpha_grid(20)
    Wr_d = awq.awq_hadamard_rotate(dev(L.W), 128)
    Xr_d = awq.awq_hadamard_rotate(dev(L.X), 128)
    Wr_o, Xr_o = O.hadamard_rotate(L.W, 128), O.hadamard_rotate(L.X, 128)
    _check_rotation(host(Wr_d), Wr_o, "W")
    _check_rotation(host(Xr_d), Xr_o, "X")
    a0, ar = O.act_stats(L.X), O.act_stats(Xr_o)
    assert ar.max() / np.median(ar) < a0.max() / np.median(a0) / 4
    a = awq.awq_act_stats(Xr_d)
    res = awq.awq_search_scales(Wr_d, Xr_d, a, alphas, cfg)
    torch.cuda.synchronize()
    # oracle inputs come from the oracle's own rotation
    orc = O.search_scales(Wr_o, Xr_o, O.act_stats(Xr_o), alphas, ocfg(cfg))
    check_search(res, orc, "rotated")
