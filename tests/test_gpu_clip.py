"""Clip search and the clipped pack on the GPU (through the C ABI) against the oracle.

Group errors: the GPU takes e = d^T (X_j^T X_j) d, the Gram sums on the matrix cores in
fp32 over at most 256 tokens (within 2^-16 of the sum of |products|) and added in fp64, then
an fp32 quadratic form over fp16 hi + lo splits of G and of d; the oracle takes the group's
partial product directly in fp64.  Bar: |e_gpu - e| <= 1e-3 e for every group error (an
error the oracle finds exactly 0 must be exactly 0 on the GPU too), and the same ratio
wherever the oracle's best and runner-up differ by more than 1e-3 relative; elsewhere the
GPU's choice must be within 2e-3 of the best.  The clipped pack is bit-exact.
"""
import numpy as np
import pytest
import torch

import weight_only_quantization_act_amd as awq
from oracle import awq_oracle as O
from synth import CONFIGS, make_layer, row_subset, small_spec
from tests.gpu_util import dev, host, ocfg, requires_gpu, say

pytestmark = [pytest.mark.gpu, requires_gpu]

F16, F32, F64 = np.float16, np.float32, np.float64
RATIOS = (1.0 - np.arange(11) * 0.05).astype(F32)          # 1.0, 0.95, ..., 0.5
CLIP_RTOL = 1e-3
CLIP_STOL = 2.0 ** -18


def _conditioning(W16, X16, s32, cfg, ratios, rows):
    """S[k][m][j] = sum_t (sum_{i in j} |d_i| |x_{t,i}|)^2: the group error with every term's
    sign made positive, the scale of a rounding error committed on the terms."""
    g = cfg.group_size
    K = W16.shape[1]
    Xa = np.abs(X16.astype(F64))
    out = np.empty((len(ratios), len(rows), K // g))
    for k, r in enumerate(ratios):
        d = np.abs(O.delta_weight(W16[rows], s32, cfg, clip=np.full((len(rows), K // g), r, F32)))
        for j in range(K // g):
            y = d[:, j * g:(j + 1) * g] @ Xa[:, j * g:(j + 1) * g].T
            out[k, :, j] = np.sum(y * y, axis=1)
    return out


def _check_clip(res, W16, X16, s32, cfg, ratios, rows, where):
    orc = O.clip_search(W16[rows], X16, s32, cfg, ratios)
    eo = orc["errors"]
    eg = host(res["errors"])[:, rows, :].astype(F64)
    S = _conditioning(W16, X16, s32, cfg, ratios, rows)
    pos = eo > 0
    err = np.abs(eg - eo)
    rel = np.where(pos, err / np.where(pos, eo, 1.0), 0.0)
    cond = np.where(S > 0, err / np.where(S > 0, S, 1.0), 0.0)
    tol = CLIP_RTOL * eo + CLIP_STOL * S
    bad = (err > tol) | (~pos & (eg != eo))
    say(f"  {where}: group errors max rel err {rel.max(initial=0.0):.2e}, beyond 1e-3 relative: "
        f"{int((rel > CLIP_RTOL).sum())} of {eo.size}; max |err| / S {cond.max(initial=0.0):.2e}")
    if bad.any():
        k, m, j = np.argwhere(bad)[0]
        raise AssertionError(f"{where}: {int(bad.sum())} group errors off, first ratio {k} row "
                             f"{rows[m]} group {j}: gpu {eg[k, m, j]!r} oracle {eo[k, m, j]!r} "
                             f"S {S[k, m, j]!r}")
    bg = host(res["best"])[rows]
    bo = orc["best"]
    srt = np.sort(eo, axis=0)
    gap = ((srt[1] - srt[0]) / np.maximum(srt[0], 1e-300) if len(ratios) > 1
           else np.full(eo.shape[1:], np.inf))
    clear = gap > 1e-3
    assert np.array_equal(bg[clear], bo[clear]), (where, int((bg[clear] != bo[clear]).sum()))
    mm, jj = np.nonzero(~clear)
    if mm.size:
        chosen = eo[bg[mm, jj], mm, jj]
        assert np.all(chosen <= srt[0][mm, jj] * (1 + 2e-3) + tol[bg[mm, jj], mm, jj]), where
    cg = host(res["clip"])[rows]
    assert np.array_equal(cg, ratios[bg]), where
    return int(clear.sum()), int(bg.size)


CASES = [
    # M, K, N, w_bit, g, zp
    (40, 256, 300, 4, 128, 1),
    (33, 512, 129, 4, 64, 0),
    (70, 320, 50, 3, 32, 1),
    (17, 128, 1, 4, 128, 1),      # one token
    (128, 1024, 700, 4, 128, 0),
    (8, 128, 20000, 4, 128, 1),   # 64 token splits of 320: several fp32 sums per split
]


@pytest.mark.parametrize("M,K,N,w_bit,g,zp", CASES)
def test_clip_search_parity(M, K, N, w_bit, g, zp):
    say(f"clip M={M} K={K} N={N} b={w_bit} g={g} zp={zp}")
    L = make_layer(small_spec("c", M, K, N, w_bit=w_bit, group_size=g, zero_point=zp,
                              outlier_count=max(1, K // 100), seed=M + K + N))
    rng = np.random.default_rng(M * K)
    s = np.exp(rng.uniform(-1.0, 2.0, K)).astype(F32)
    cfg = awq.qconfig(w_bit, g, zp)
    res = awq.awq_clip_search(dev(L.W), dev(L.X), dev(s), RATIOS, cfg, want_errors=True)
    torch.cuda.synchronize()
    clear, total = _check_clip(res, L.W, L.X, s, ocfg(cfg), RATIOS, np.arange(M),
                               f"{M}x{K}x{N}")
    say(f"  decided by a clear margin: {clear} of {total}")


@pytest.mark.parametrize("n_ratio,M,K,N,g", [(1, 37, 256, 90, 128), (64, 23, 192, 140, 64),
                                              (7, 161, 96, 70, 32)])
def test_clip_ratio_counts(n_ratio, M, K, N, g):
    """One ratio, the largest grid (64), and a grid that leaves a partial 16-pair slice,
    on layers whose 128-channel Gram spans run past in_features (K = 192 and 96)."""
    say(f"clip n_ratio={n_ratio} M={M} K={K} N={N} g={g}")
    L = make_layer(small_spec("r", M, K, N, group_size=g, outlier_count=2, seed=n_ratio + M))
    rng = np.random.default_rng(n_ratio)
    s = np.exp(rng.uniform(-1.0, 1.0, K)).astype(F32)
    ratios = (1.0 - np.arange(n_ratio) * (0.6 / max(1, n_ratio - 1))).astype(F32)
    cfg = awq.qconfig(4, g, 1)
    res = awq.awq_clip_search(dev(L.W), dev(L.X), dev(s), ratios, cfg, want_errors=True)
    torch.cuda.synchronize()
    _check_clip(res, L.W, L.X, s, ocfg(cfg), ratios, np.arange(M), f"n={n_ratio}")


def test_clip_wide_dynamic_range():
    """Rows whose magnitudes span 2^-12 .. 2^4 in one block and scales spanning four decades:
    the power of two shared by a block's rows and the scaled Gram matrix keep every group
    error within the same bound."""
    M, K, N, g = 48, 256, 400, 128
    L = make_layer(small_spec("w", M, K, N, outlier_count=3, seed=11))
    rng = np.random.default_rng(12)
    W = (L.W.astype(F64) * np.exp2(rng.uniform(-12, 4, M))[:, None]).astype(F16)
    s = np.exp(rng.uniform(np.log(1e-2), np.log(1e2), K)).astype(F32)
    cfg = awq.qconfig(4, g, 1)
    res = awq.awq_clip_search(dev(W), dev(L.X), dev(s), RATIOS, cfg, want_errors=True)
    torch.cuda.synchronize()
    clear, total = _check_clip(res, W, L.X, s, ocfg(cfg), RATIOS, np.arange(M), "wide range")
    say(f"  decided by a clear margin: {clear} of {total}")


def test_clip_degenerate():
    cfg = awq.qconfig(4, 128, 1)
    L = make_layer(small_spec("z", 8, 256, 64))
    W = L.W.copy()
    W[3] = 0                                             # zero rows: every ratio scores 0
    s = np.ones(256, F32)
    res = awq.awq_clip_search(dev(W), dev(L.X), dev(s), RATIOS, cfg, want_errors=True)
    torch.cuda.synchronize()
    assert np.all(host(res["errors"])[:, 3, :] == 0)
    assert np.all(host(res["best"])[3] == 0) and np.all(host(res["clip"])[3] == 1.0)
    X = L.X.copy()
    X[10, 5] = np.nan                                    # group 0's Gram matrix is NaN
    res = awq.awq_clip_search(dev(L.W), dev(X), dev(s), RATIOS, cfg)
    torch.cuda.synchronize()
    orc = O.clip_search(L.W, X, s, ocfg(cfg), RATIOS)
    assert np.all(host(res["best"])[:, 0] == -1) and np.all(orc["best"][:, 0] == -1)
    assert np.all(host(res["clip"])[:, 0] == 1.0)
    single = awq.awq_clip_search(dev(L.W), dev(L.X), dev(s), np.array([0.8], F32), cfg)
    torch.cuda.synchronize()
    assert np.all(host(single["best"]) == 0) and np.all(host(single["clip"]) == F32(0.8))


@pytest.mark.parametrize("w_bit,g,zp", [(4, 128, 1), (4, 64, 0), (3, 32, 1)])
def test_pack_clipped_bit_exact(w_bit, g, zp):
    """The clipped pack against the oracle's clipped quantiser, with ratios drawn on the
    host (including 1 and the grid's low end), and ratio 1 against the plain pack."""
    M, K = 300, 512
    say(f"pack clipped b={w_bit} g={g} zp={zp}")
    L = make_layer(small_spec("p", M, K, 8, w_bit=w_bit, group_size=g, zero_point=zp,
                              outlier_count=5))
    rng = np.random.default_rng(g + zp)
    s = np.exp(rng.uniform(-1.0, 2.0, K)).astype(F32)
    clip = RATIOS[rng.integers(0, len(RATIOS), (M, K // g))]
    cfg = awq.qconfig(w_bit, g, zp)
    c, sc, z = awq.awq_quantize_pack_clipped(dev(L.W), dev(s), dev(clip), cfg)
    pk, so, zo = O.quantize_pack(L.W, s, ocfg(cfg), clip=clip)
    assert np.array_equal(host(c), pk)
    assert np.array_equal(host(sc).view(np.uint16), so.view(np.uint16))
    assert np.array_equal(host(z).view(np.uint16), zo.view(np.uint16))
    ones = np.ones((M, K // g), F32)
    c1, s1, z1 = awq.awq_quantize_pack_clipped(dev(L.W), dev(s), dev(ones), cfg)
    c0, s0, z0 = awq.awq_quantize_pack(dev(L.W), dev(s), cfg)
    assert torch.equal(c1, c0) and torch.equal(s1, s0) and torch.equal(z1, z0)


def test_clip_headline_layer_sampled_rows():
    """The 4096 x 4096 layer with 4096 tokens and a 20-ratio grid, in the configuration the
    benchmark times, after the GPU scale search; the oracle rescores 24 seeded rows."""
    spec = CONFIGS["c2"][0]
    L = make_layer(spec)
    cfg = awq.qconfig(spec.w_bit, spec.group_size, spec.zero_point)
    ratios = (1.0 - np.arange(20) * 0.025).astype(F32)
    say("clip c2 4096x4096x4096 (GPU)")
    Wd, Xd = dev(L.W), dev(L.X)
    from synth import alpha_grid
    a = awq.awq_act_stats(Xd)
    srch = awq.awq_search_scales(Wd, Xd, a, alpha_grid(20), cfg)
    s = srch["s"]
    res = awq.awq_clip_search(Wd, Xd, s, ratios, cfg, want_errors=True)
    torch.cuda.synchronize()
    rows = row_subset(spec, 24)
    say("clip c2 (oracle, 24 rows)")
    clear, total = _check_clip(res, L.W, L.X, host(s), ocfg(cfg), ratios, rows, "c2")
    say(f"  decided by a clear margin: {clear} of {total}")
