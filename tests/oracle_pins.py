"""Pins that tie the CPU oracle to what the pages and the mathematics fix.

Every pin is a plain function that raises AssertionError (or any exception) when the
oracle disagrees.  They reach the oracle only through module attributes of
`oracle.awq_oracle`, so tests/test_oracle_mutations.py can plant a mistake in one oracle
function and check that at least one pin notices.

Pages (title, site):
  [AWQ-notes]  "AWQ" -- lizn-zn.github.io scholia-log, inference-quantization notes
  [AWQ-tut]    "AWQ量化" tutorial -- aiqz.cc
  [AWQ-blog]   "AWQ量化技术解析：激活感知的权重量化革命" -- kwkr.cn
  [GPTQ-AWQ]   "大模型的开发应用（十八）：大模型量化：GPTQ与AWQ" -- ewbang.com
  [AutoAWQ-70B] "AWQ 量化全流程拆解：将 70B 大模型塞进单张消费级 GPU" -- lnrq.cn
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np

from oracle import awq_oracle as O

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
F16, F32, F64 = np.float16, np.float32, np.float64


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _cfg(b=4, g=128, zp=1):
    return O.QConfig(w_bit=b, group_size=g, zero_point=zp)


# ---------------------------------------------------------------- output error (A4)
def pin_output_error_scaling():
    """[AWQ-notes §1.1] equal weight errors (0.1) give output errors 0.001 and 2.0 for
    activations 0.01 and 20: the loss is (dW * x)^2 per product."""
    ex = _golden("awq_notes_examples.json")["output_error_scaling"]
    for case in ex["cases"]:
        dW = np.array([[0.0, ex["weight_error"], 0.0]], dtype=F64)
        X = np.array([[0.0, case["activation"], 0.0],
                      [0.0, 0.0, 0.0]], dtype=F16)
        x16 = float(X[0, 1])
        loss = O.output_error_loss(dW, X)
        assert math.isclose(loss, (ex["weight_error"] * x16) ** 2, rel_tol=1e-12)
        assert math.isclose(math.sqrt(loss), case["output_error"], rel_tol=2e-3)


def pin_loss_bruteforce_tiny():
    """Triple loop over (row, token, channel) on tiny layers equals the oracle's loss
    [AWQ-notes §1.1 Delta Y = Delta W X, §4.1 squared Frobenius norm]."""
    rng = np.random.default_rng(11)
    for (M, K, N) in [(3, 8, 5), (5, 16, 2), (1, 4, 7), (8, 8, 8)]:
        dW = rng.standard_normal((M, K))
        X = rng.standard_normal((N, K)).astype(F16)
        want = 0.0
        for r in range(M):
            for t in range(N):
                acc = 0.0
                for i in range(K):
                    acc += dW[r, i] * float(X[t, i])
                want += acc * acc
        got = O.output_error_loss(dW, X)
        assert math.isclose(got, want, rel_tol=1e-12), (M, K, N, got, want)


def pin_loss_equals_printed_objective():
    """The Delta W route equals ||W X - Q(WS)S^-1 X||_F^2 written literally
    [AWQ-notes §4.1; GPTQ-AWQ §3 二.1]."""
    rng = np.random.default_rng(12)
    M, K, N = 16, 64, 24
    W = (0.02 * rng.standard_normal((M, K))).astype(F16)
    X = rng.standard_normal((N, K)).astype(F16)
    s = np.exp(rng.uniform(-1, 2, K)).astype(F32)
    cfg = _cfg(4, 32, 1)
    What = O.fake_quant_weight(W, s, cfg)
    a = O.output_error_loss(W.astype(F64) - What, X)
    b = O.layer_output_error(W, What, X)
    assert a > 0
    assert math.isclose(a, b, rel_tol=1e-9), (a, b)


def pin_row_separability():
    """The loss is a sum of per-row terms [GPTQ-AWQ §1.4 OBC: the objective splits into
    one term per output row], so any row subset's loss adds up exactly."""
    rng = np.random.default_rng(13)
    M, K, N = 12, 64, 10
    W = (0.02 * rng.standard_normal((M, K))).astype(F16)
    X = rng.standard_normal((N, K)).astype(F16)
    s = np.exp(rng.uniform(-1, 1, K)).astype(F32)
    cfg = _cfg(4, 64, 1)
    full = O.output_error_loss(O.delta_weight(W, s, cfg), X)
    parts = sum(O.output_error_loss(O.delta_weight(W[r:r + 1], s, cfg), X) for r in range(M))
    assert math.isclose(full, parts, rel_tol=1e-12)


def pin_identity_reparameterisation():
    """With Q replaced by the identity, (W S)(S^-1 X) = W X, so the loss is zero up to
    rounding for any positive scales [AWQ-notes §2.1]."""
    rng = np.random.default_rng(14)
    M, K, N = 8, 64, 16
    W = (0.02 * rng.standard_normal((M, K))).astype(F16)
    X = rng.standard_normal((N, K)).astype(F16)
    ref = O.output_error_loss(W.astype(F64), X)
    for _ in range(3):
        s = np.exp(rng.uniform(-3, 3, K)).astype(F32)
        loss = O.output_error_loss(O.delta_weight(W, s, _cfg(4, 32, 1), identity_quantizer=True), X)
        assert loss <= 1e-12 * ref, (loss, ref)
    # and a real quantiser is not the identity
    s = np.ones(K, dtype=F32)
    assert O.output_error_loss(O.delta_weight(W, s, _cfg(4, 32, 1)), X) > 1e-8 * ref


# ---------------------------------------------------------------- quantiser (A3)
def pin_step_nonlinearity():
    """[AWQ-notes §2.2] step 1: Q(0.4) = 0, while scaling by 2 first gives Q(0.8)/2 = 0.5.
    Group [0.4, 7.0], symmetric 4 bits -> step max/7 = 1."""
    ex = _golden("awq_notes_examples.json")["step_nonlinearity"]
    W = np.array([[ex["w"], 7.0]], dtype=F16)
    cfg = _cfg(4, 2, 0)
    codes, step, zero = O.quantize(W, np.ones(2, F32), cfg)
    assert step[0, 0] == F32(ex["step"])
    What = O.fake_quant_weight(W, np.ones(2, F32), cfg)
    assert What[0, 0] == ex["q_unscaled"]
    s = np.array([ex["scale"], 1.0], dtype=F32)
    What2 = O.fake_quant_weight(W, s, cfg)
    assert What2[0, 0] == ex["q_scaled_then_divided"]


def pin_worked_group_example():
    """[AWQ-notes §3.1] group max 1.0 -> step 1/7; w = 0.05 at x = 10 quantises to 0
    (output error -0.5); with s = 4: w' = 0.2, x' = 2.5, code 1, e' ~ -0.057,
    output error ~ -0.143, effective step ~ 0.036.  Symmetric INT4."""
    ex = _golden("awq_notes_examples.json")["worked_group"]
    tol = ex["tol_abs"]
    W = np.array([[ex["w_max"], ex["w"], 0.0, -0.3]], dtype=F16)
    X = np.zeros((1, 4), dtype=F16)
    X[0, 1] = ex["x"]
    cfg = _cfg(4, 4, 0)
    one = np.ones(4, F32)
    codes, step, zero = O.quantize(W, one, cfg)
    num, den = ex["step_exact_fraction"]
    assert step[0, 0] == F32(num / den)
    assert abs(float(step[0, 0]) - ex["step"]) < tol
    assert int(codes[0, 1]) - int(zero[0, 0]) == ex["code_unscaled"]
    What = O.fake_quant_weight(W, one, cfg)
    dy = (What[0, 1] - float(W[0, 1])) * float(X[0, 1])
    assert abs(dy - ex["dy_unscaled"]) < tol
    loss0 = O.output_error_loss(W.astype(F64) - What, X)
    assert math.isclose(loss0, dy * dy, rel_tol=1e-9)

    s = np.array([1.0, ex["scale"], 1.0, 1.0], dtype=F32)
    codes4, step4, zero4 = O.quantize(W, s, cfg)
    assert step4[0, 0] == step[0, 0]            # group max still set by the 1.0 weight
    assert int(codes4[0, 1]) - int(zero4[0, 0]) == ex["code_scaled"]
    w_scaled = float(W[0, 1]) * ex["scale"]
    assert abs(w_scaled - ex["w_scaled"]) < tol
    assert abs(ex["x"] / ex["scale"] - ex["x_scaled"]) < tol
    d = O.dequantize_scaled(codes4, step4, zero4, 4)
    e_scaled = float(d[0, 1]) - w_scaled
    assert abs(e_scaled - ex["e_scaled"]) < tol
    What4 = O.fake_quant_weight(W, s, cfg)
    dy4 = (What4[0, 1] - float(W[0, 1])) * float(X[0, 1])
    assert abs(dy4 - ex["dy_scaled"]) < tol
    assert math.isclose(dy4, e_scaled * ex["x_scaled"], rel_tol=1e-6)
    assert abs(float(step4[0, 0]) / ex["scale"] - ex["step_eff"]) < tol
    loss4 = O.output_error_loss(W.astype(F64) - What4, X)
    assert loss4 < loss0


def pin_over_scaling():
    """[AWQ-notes §3.3] scaling the 0.05 weight by 40 makes it the group maximum (2.0), the
    step grows to 2/7 ~ 0.286 and the unscaled weights see a coarser grid."""
    ex = _golden("awq_notes_examples.json")["over_scaling"]
    W = np.array([[ex["w_max"], ex["w"], 0.35, -0.6]], dtype=F16)
    cfg = _cfg(4, 4, 0)
    one = np.ones(4, F32)
    s = np.array([1.0, ex["scale"], 1.0, 1.0], dtype=F32)
    _, step1, _ = O.quantize(W, one, cfg)
    _, step40, _ = O.quantize(W, s, cfg)
    assert abs(float(step40[0, 0]) - ex["step_new"]) < ex["tol_abs"]
    num, den = ex["step_new_fraction"]
    assert abs(float(step40[0, 0]) - num / den) < 2e-4       # fp16 0.05 * 40 = 2.0001
    err1 = np.abs(O.fake_quant_weight(W, one, cfg) - W.astype(F64))[0, [0, 2, 3]]
    err40 = np.abs(O.fake_quant_weight(W, s, cfg) - W.astype(F64))[0, [0, 2, 3]]
    assert err40.max() > err1.max() + 0.05


def pin_nearest_code_bruteforce():
    """Every code is the nearest point of the group's grid {(c - z) * step} to v, ties to
    the even level, found by exhaustive search in exact rational arithmetic
    [AWQ-notes §2.3 (nearest rounding to a uniform grid); AWQ-tut Python 演示 uses
    numpy's round, which breaks ties to even]."""
    rng = np.random.default_rng(15)
    cases = []
    for b in (2, 3, 4):
        for zp in (0, 1):
            for g in (2, 4, 8):
                for _ in range(12):
                    W = (rng.standard_normal((2, 2 * g)) * rng.uniform(0.01, 3)).astype(F16)
                    s = np.exp(rng.uniform(-1, 1, 2 * g)).astype(F32)
                    cases.append((W, s, b, g, zp))
    # exact ties: step 1, values at half-integers
    cases.append((np.array([[7.0, 2.5, -1.5, 0.5]], F16), np.ones(4, F32), 4, 4, 0))
    cases.append((np.array([[15.0, 2.5, 3.5, 0.5]], F16), np.ones(4, F32), 4, 4, 1))
    checked = 0
    for W, s, b, g, zp in cases:
        cfg = _cfg(b, g, zp)
        codes, step, zero = O.quantize(W, s, cfg)
        v = W.astype(F32) * s[None, :]
        top = 2 ** b - 1
        lo_c = 0 if zp else (2 ** (b - 1) - (2 ** (b - 1) - 1))
        for r in range(W.shape[0]):
            for i in range(W.shape[1]):
                gi = i // g
                st = Fraction(float(step[r, gi]))
                z = int(zero[r, gi])
                vi = Fraction(float(v[r, i]))
                best, best_d = None, None
                for c in range(lo_c, top + 1):
                    dist = abs(vi - (c - z) * st)
                    if best is None or dist < best_d or (dist == best_d and (c - z) % 2 == 0):
                        best, best_d = c, dist
                ratio = vi / st
                near_half = abs(abs(ratio - math.floor(ratio)) - Fraction(1, 2)) < Fraction(1, 2 ** 20) * max(1, abs(ratio))
                if near_half and ratio.denominator != 2:
                    continue  # fp32 quotient may land on the other side of a near-tie
                assert int(codes[r, i]) == best, (W[r], s, b, g, zp, i, int(codes[r, i]), best)
                checked += 1
    assert checked > 1000


def pin_group_endpoints():
    """The group's extreme weights land on the end levels: symmetric -> +-qmax for the
    largest |v| (step = max|v| / qmax, AWQ-tut 量化基础); zero-point -> the minimum maps
    to code 0 and the maximum to the top code (or one below when both ends round inward).
    Groups run along the input dimension: one step per (row, block of g input channels)
    [AWQ-notes §3.2]."""
    rng = np.random.default_rng(16)
    M, K, g = 6, 48, 16
    W = (rng.standard_normal((M, K)) * 0.02).astype(F16)
    s = np.exp(rng.uniform(-0.5, 0.5, K)).astype(F32)
    v = W.astype(F32) * s[None, :]
    for b in (3, 4):
        codes, step, zero = O.quantize(W, s, _cfg(b, g, 0))
        assert step.shape == (M, K // g)
        qmax = 2 ** (b - 1) - 1
        for r in range(M):
            for j in range(K // g):
                seg = v[r, j * g:(j + 1) * g]
                k = int(np.argmax(np.abs(seg)))
                assert abs(int(codes[r, j * g + k]) - int(zero[r, j])) == qmax
                assert step[r, j] == F32(np.abs(seg).max() / F32(qmax))
        codes, step, zero = O.quantize(W, s, _cfg(b, g, 1))
        top = 2 ** b - 1
        for r in range(M):
            for j in range(K // g):
                seg = v[r, j * g:(j + 1) * g]
                assert int(codes[r, j * g + int(np.argmin(seg))]) == 0
                assert int(codes[r, j * g + int(np.argmax(seg))]) in (top - 1, top)
                assert step[r, j] == F32((F32(seg.max()) - F32(seg.min())) / F32(top))


def pin_error_bound_and_variance():
    """|v - Q(v)| <= step/2 without clipping [AWQ-notes §2.3], and the rounding error of a
    large random group is close to uniform, mean square ~ step^2/12 [AWQ-tut 误差分析]."""
    rng = np.random.default_rng(17)
    M, K, g = 64, 4096, 128
    W = (rng.standard_normal((M, K)) * 0.02).astype(F16)
    s = np.ones(K, F32)
    for zp in (0, 1):
        codes, step, zero = O.quantize(W, s, _cfg(4, g, zp))
        d = O.dequantize_scaled(codes, step, zero, g)
        e = (W.astype(F32) - d).astype(F64)
        st = np.repeat(step.astype(F64), g, axis=1)
        ratio = np.abs(e) / st
        if zp == 0:
            assert ratio.max() <= 0.5 * (1 + 1e-5)
        else:
            # only the top end can clip (both end roundings inward): bounded by one step
            assert ratio.max() <= 1.0 + 1e-5
            assert np.mean(ratio > 0.5 + 1e-5) < 2e-3
        ms = np.mean((e / st) ** 2)
        assert abs(ms - 1 / 12) < 0.03 / 12, ms


def pin_per_weight_scale_no_gain():
    """With one step per weight, scaling a weight by s scales its own step by s, so the
    effective step step'/s stays put [AWQ-notes §3.2]."""
    rng = np.random.default_rng(18)
    W = (rng.standard_normal((4, 16)) * 0.02).astype(F16)
    for zp in (0, 1):
        cfg = _cfg(4, 1, zp)
        _, step1, _ = O.quantize(W, np.ones(16, F32), cfg)
        for sval in (2.0, 4.0, 37.5):
            s = np.full(16, sval, F32)
            _, steps, _ = O.quantize(W, s, cfg)
            eff = steps.astype(F64) / sval
            assert np.allclose(eff, step1.astype(F64), rtol=1e-6, atol=0)


def pin_symmetric_clip_equivalence():
    """Symmetric codes never need the extra negative level, so clamping to +-(2^(b-1)-1)
    [AWQ-tut Python 演示] and clipping to [-8, 7] for 4 bits [AWQ-blog §2.1] agree:
    code 0 (= -8 after the offset) never occurs."""
    rng = np.random.default_rng(19)
    W = (rng.standard_normal((64, 1024)) * rng.uniform(0.001, 2)).astype(F16)
    s = np.exp(rng.uniform(-2, 2, 1024)).astype(F32)
    codes, _, zero = O.quantize(W, s, _cfg(4, 128, 0))
    assert codes.min() >= 1 and codes.max() <= 15
    assert np.all(zero == 8)


def pin_zero_group():
    """An all-zero group quantises to zero exactly (step replaced by 1; code = zero point)."""
    W = np.zeros((2, 8), F16)
    W[1, 4:] = 0.5
    for zp in (0, 1):
        codes, step, zero = O.quantize(W, np.ones(8, F32), _cfg(4, 4, zp))
        assert step[0, 0] == 1 and step[0, 1] == 1 and step[1, 0] == 1
        assert np.all(codes[0] == zero[0, 0])
        assert np.all(O.fake_quant_weight(W, np.ones(8, F32), _cfg(4, 4, zp))[0] == 0)


# ---------------------------------------------------------------- statistics (A1), scales (A2)
def pin_stats_closed_forms():
    """a_i = E|x_i| over tokens [AWQ-notes §1.2; AWQ-tut 激活感知]: exact for columns of
    constant magnitude and random sign; statistically sqrt(2/pi) for N(0,1) and 1 for
    Student-t with 4 degrees of freedom."""
    rng = np.random.default_rng(20)
    N, K = 96, 5
    mags = np.array([0.5, 3.0, 0.0, 17.25, 1e-3], F16)
    X = (np.sign(rng.standard_normal((N, K))) * mags[None, :].astype(F64)).astype(F16)
    a = O.act_stats(X)
    assert a.shape == (K,)
    assert np.array_equal(a, mags.astype(F32))
    n = 2_000_000
    xn = rng.standard_normal((n, 1)).astype(F16)
    an = float(O.act_stats(xn)[0])
    assert abs(an - math.sqrt(2 / math.pi)) < 4 * math.sqrt(1 - 2 / math.pi) / math.sqrt(n) + 2e-4
    xt = rng.standard_t(4.0, (n, 1)).astype(F16)
    at = float(O.act_stats(xt)[0])
    assert abs(at - 1.0) < 4 / math.sqrt(n) + 2e-4


def pin_stats_over_tokens():
    """The mean runs over tokens (rows of X^T), one value per input channel, and uses the
    magnitude, not the signed value."""
    X = np.array([[1.0, -2.0, 0.0], [-3.0, -2.0, 4.0]], F16)
    a = O.act_stats(X)
    assert np.array_equal(a, np.array([2.0, 2.0, 2.0], F32))


def pin_scale_family_closed_forms():
    """s = a^alpha [AWQ-notes §4.1]: alpha = 0 gives exactly 1 (no scaling, plain
    round-to-nearest), alpha = 1 gives a, alpha = 1/2 gives the float32 square root;
    every s is positive (a channel with a = 0 keeps s = 1) [AWQ-notes §2.1]."""
    rng = np.random.default_rng(21)
    a = np.concatenate([np.exp(rng.uniform(-5, 5, 200)), [0.0, 1.0, 65504.0]]).astype(F32)
    s = O.scale_family(a, np.array([0.0, 0.5, 1.0], F32))
    assert np.all(s[0] == 1.0)
    assert np.array_equal(s[1][a > 0], np.sqrt(a[a > 0]))
    assert np.array_equal(s[2][a > 0], a[a > 0])
    assert np.all(s > 0)
    third = O.scale_family(np.array([8.0, 27.0], F32), np.array([F32(1 / 3)], F32))
    assert np.allclose(third[0], [2.0, 3.0], rtol=1e-6)


def pin_alpha_zero_is_rtn():
    """At alpha = 0 the search evaluates plain round-to-nearest of W itself: the codes
    equal those of W with unit scales and the loss is that of the unscaled quantiser
    [AWQ-notes §4.1]."""
    rng = np.random.default_rng(22)
    M, K, N = 8, 256, 12
    W = (rng.standard_normal((M, K)) * 0.02).astype(F16)
    X = rng.standard_normal((N, K)).astype(F16)
    a = O.act_stats(X)
    cfg = _cfg(4, 128, 1)
    s0 = O.scale_family(a, np.array([0.0], F32))[0]
    c0, st0, z0 = O.quantize(W, s0, cfg)
    c1, st1, z1 = O.quantize(W, np.ones(K, F32), cfg)
    assert np.array_equal(c0, c1) and np.array_equal(st0, st1)
    res = O.search_scales(W, X, a, np.array([0.0, 0.5], F32), cfg)
    assert res["losses"][0] == O.output_error_loss(O.delta_weight(W, np.ones(K, F32), cfg), X)


# ---------------------------------------------------------------- search and select (A5)
def pin_salient_channel_search():
    """A layer with one strongly activated input channel whose weights are small: scaling
    it up (alpha > 0) lowers the output error [AWQ-notes §3.1], while pushing the scale
    until it sets the group range makes things worse again [AWQ-notes §3.3], so the best
    alpha is interior."""
    rng = np.random.default_rng(23)
    M, K, N = 32, 128, 64
    W = (rng.standard_normal((M, K)) * 0.02).astype(F16)
    W[:, 5] = (W[:, 5].astype(F32) * 0.1).astype(F16)
    X = rng.standard_normal((N, K))
    X[:, 5] *= 60.0
    X = X.astype(F16)
    a = O.act_stats(X)
    alphas = (np.arange(20) / 19).astype(F32)
    res = O.search_scales(W, X, a, alphas, _cfg(4, 128, 0))
    L = res["losses"]
    k = res["best"]
    assert 0 < k < len(alphas) - 1, L
    assert L[k] < L[0] and L[k] < L[-1]
    assert L[k] == L.min()
    assert np.array_equal(res["s_star"], res["s_table"][k])


def pin_select_rules():
    """argmin over finite losses, first index on ties; none finite -> -1 (reading of the
    troubleshooting advice to look for inf in the statistics, AWQ-blog §3.1)."""
    assert O.select_best(np.array([3.0, 1.0, 1.0, 2.0])) == 1
    assert O.select_best(np.array([np.nan, 2.0, 1.0])) == 2
    assert O.select_best(np.array([1.0, np.inf, np.nan, 0.5])) == 3
    assert O.select_best(np.array([np.inf, np.nan])) == -1
    assert O.select_best(np.array([5.0, 4.0, 6.0])) == 1


def pin_nonfinite_search():
    """A NaN in the activations makes every loss non-finite: no alpha is chosen and the
    scales fall back to 1."""
    rng = np.random.default_rng(24)
    W = (rng.standard_normal((4, 128)) * 0.02).astype(F16)
    X = rng.standard_normal((8, 128)).astype(F16)
    X[3, 7] = np.nan
    a = O.act_stats(X)
    res = O.search_scales(W, X, a, np.array([0.0, 0.5, 1.0], F32), _cfg(4, 128, 1))
    assert not np.isfinite(res["losses"]).any()
    assert res["best"] == -1 and np.all(res["s_star"] == 1.0)


# ---------------------------------------------------------------- pack (A6)
def pin_pack_layout():
    """Two 4-bit codes per byte, even input channel in the low nibble [AWQ-blog §4.2];
    round trip; 4-bit codes take a quarter of the fp16 bytes, a saving of 1 - b/16
    [AWQ-tut 部署实践]."""
    codes = np.array([[1, 2, 15, 0, 7, 8]], np.uint8)
    packed = O.pack_nibbles(codes)
    assert packed.tolist() == [[0x21, 0x0F, 0x87]]
    rng = np.random.default_rng(25)
    c = rng.integers(0, 16, (7, 64)).astype(np.uint8)
    assert np.array_equal(O.unpack_nibbles(O.pack_nibbles(c)), c)
    fig = _golden("deployment_figures.json")["memory_saving"]
    W = (rng.standard_normal((7, 128)) * 0.02).astype(F16)
    p, sc, zr = O.quantize_pack(W, np.ones(128, F32), _cfg(fig["w_bit"], 128, 1))
    assert p.dtype == np.uint8 and p.shape == (7, 64)
    assert 1 - p.nbytes / W.nbytes == fig["saving"]
    cc, st, zz = O.quantize(W, np.ones(128, F32), _cfg(4, 128, 1))
    assert np.array_equal(O.unpack_nibbles(p), cc)
    assert np.array_equal(sc, st.astype(F16)) and np.array_equal(zr.astype(np.int32), zz)


def pin_group_metadata_overhead():
    """fp16 step + fp16 zero per group is 4 bytes; at g = 128 a 70B-parameter model then
    carries about 2.2 GB of metadata [AutoAWQ-70B §四]."""
    fig = _golden("deployment_figures.json")["group_metadata_overhead"]
    W = np.zeros((2, 256), F16)
    _, sc, zr = O.quantize_pack(W, np.ones(256, F32), _cfg(4, fig["group_size"], 1))
    per_group = (sc.nbytes + zr.nbytes) / sc.size
    total = fig["params"] / fig["group_size"] * per_group
    assert abs(total - fig["overhead_bytes"]) <= fig["rel_tol"] * fig["overhead_bytes"]




def pin_stored_step_overflow():
    """The step is stored as FP16 [AWQ-blog §2.1].  IEEE binary16's largest finite value is
    (2 - 2^-10) 2^15 = 65504 and the next representable magnitude would be 2^16, so round
    to nearest even sends every value from the midpoint 65520 up to infinity and keeps
    65519.99... at 65504.  A symmetric 4-bit group whose largest |w s| is 7 x 65520 has a
    step of exactly 65520 and overflows; one fp16 spacing less in w does not."""
    with np.errstate(over="ignore"):
        assert F16(F32(65519.996)) == F16(65504.0) and np.isinf(F16(F32(65520.0)))
    w = np.zeros((2, 128), F16)
    w[0, 5] = 57344.0                       # 1792 x 32, exact in fp16
    w[1, 5] = 57312.0                       # one fp16 spacing (32) lower
    s = np.ones(128, F32)
    s[5] = F32(8.0 - 2.0 ** -9)             # 57344 s = 458640 = 7 x 65520 exactly
    cfg = _cfg(4, 128, 0)
    codes, step, zero = O.quantize(w, s, cfg)
    assert step[0, 0] == F32(65520.0) and step[1, 0] < F32(65520.0)
    _, sc, _ = O.quantize_pack(w, s, cfg)
    assert np.isinf(sc[0, 0]) and sc[1, 0] == F16(65472.0)   # 65483.4 to the nearest 32
    assert O.stored_step_overflows(sc) and O.stored_step_overflows(sc[:1])
    assert not O.stored_step_overflows(sc[1:])
    assert codes[0, 5] == 15 and codes[1, 5] == 15          # the codes are unaffected
    ordinary = O.quantize_pack((np.ones((3, 128)) * 0.02).astype(F16), np.ones(128, F32),
                               _cfg(4, 128, 1))[1]
    assert not O.stored_step_overflows(ordinary)


# ---------------------------------------------------------------- statistic / scale variants
def pin_max_abs_stat():
    """max |x| per channel over tokens [GPTQ-AWQ §3 二.2]: exact on constructed columns."""
    X = np.array([[1.0, -2.0, 0.0], [-3.0, 0.5, 0.0], [2.5, -0.25, 0.0]], F16)
    assert np.array_equal(O.act_stat_max_abs(X), np.array([3.0, 2.0, 0.0], F32))


def pin_rms_ratio_stat():
    """E|x| / sqrt(E x^2) [AWQ-blog §1.2]: 1 for constant magnitude, sqrt(2/pi) for N(0,1),
    1/sqrt(2) for Student-t(4), 0 for an all-zero channel."""
    rng = np.random.default_rng(31)
    N = 64
    X = (np.sign(rng.standard_normal((N, 3))) * np.array([0.5, 7.25, 0.0])).astype(F16)
    r = O.act_stat_rms_ratio(X)
    assert r[0] == 1.0 and r[1] == 1.0 and r[2] == 0.0
    n = 2_000_000
    rn = float(O.act_stat_rms_ratio(rng.standard_normal((n, 1)).astype(F16))[0])
    assert abs(rn - math.sqrt(2 / math.pi)) < 2e-3
    rt = float(O.act_stat_rms_ratio(rng.standard_t(4.0, (n, 1)).astype(F16))[0])
    assert abs(rt - 1 / math.sqrt(2)) < 1e-2


def pin_ema_stat():
    """EMA of batch means with momentum 0.9 from 0 [AWQ-blog §2.1]: equal batch means m
    give (1 - 0.9^n) m; two batches give 0.1 (0.9 m1 + m2); one batch gives 0.1 m."""
    mom = _golden("deployment_figures.json")["ema_statistics"]["momentum"]
    m = 3.0
    X = np.full((40, 2), m, F16)
    X[:, 1] = -m
    e = O.act_stat_ema_mean(X, 8, mom)          # 5 batches of 8 tokens
    assert np.allclose(e, (1 - mom ** 5) * m, rtol=1e-6)
    X2 = np.concatenate([np.full((10, 1), 1.0, F16), np.full((10, 1), 4.0, F16)])
    e2 = O.act_stat_ema_mean(X2, 10, mom)
    assert np.allclose(e2, (1 - mom) * (mom * 1.0 + 4.0), rtol=1e-6)
    assert np.allclose(O.act_stat_ema_mean(X2, 20, mom), (1 - mom) * 2.5, rtol=1e-6)
    # a short last batch averages over its own tokens
    X3 = np.concatenate([np.full((8, 1), 2.0, F16), np.full((3, 1), 5.0, F16)])
    assert np.allclose(O.act_stat_ema_mean(X3, 8, mom), (1 - mom) * (mom * 2.0 + 5.0), rtol=1e-6)


def pin_percentile_threshold():
    """The threshold is the linear-interpolation percentile (checked against numpy's
    routine), and with the tutorial's demo layout [AWQ-tut Python 演示: 70th percentile,
    factor 2, 128 channels half at base activation 0.3 and half at 5.0] the protected
    channels are exactly the top 30% by rank, all from the high half, scaled by 2."""
    rng = np.random.default_rng(32)
    for K in (5, 64, 1000):
        a = np.abs(rng.standard_normal(K)).astype(F32)
        for p in (0, 37.5, 70, 85, 99, 100):
            assert math.isclose(O.percentile_linear(a, p),
                                float(np.percentile(a.astype(F64), p, method="linear")),
                                rel_tol=1e-12, abs_tol=1e-15)
    demo = _golden("deployment_figures.json")["protection_demo"]
    K = demo["n_channels"]
    base = np.ones(K)
    base[: K // 2] = demo["low_base"]
    base[K // 2:] = demo["high_base"]
    X = (rng.standard_normal((256, K)) * demo["noise"] + base).astype(F16)
    a = O.act_stats(X)
    s = O.threshold_scales(a, demo["percentile"], demo["factor"])
    prot = s == F32(demo["factor"])
    pos = demo["percentile"] / 100 * (K - 1)
    assert prot.sum() == K - (math.floor(pos) + 1)
    assert np.all(prot[: K // 2] == 0)
    assert np.all(s[~prot] == 1.0)
    ranks = np.argsort(np.argsort(a))
    assert np.array_equal(prot, ranks > math.floor(pos))


def pin_scale_table_search():
    """Searching an explicit table equals searching the alpha family it came from; a
    table of all-ones scales gives the plain quantiser's loss."""
    rng = np.random.default_rng(33)
    W = (rng.standard_normal((16, 256)) * 0.02).astype(F16)
    X = rng.standard_normal((40, 256)).astype(F16)
    X[:, 3] *= 30
    a = O.act_stats(X)
    al = (np.arange(6) / 5).astype(F32)
    cfg = _cfg(4, 128, 1)
    r1 = O.search_scales(W, X, a, al, cfg)
    r2 = O.search_scale_table(W, X, O.scale_family(a, al), cfg)
    assert np.array_equal(r1["losses"], r2["losses"]) and r1["best"] == r2["best"]
    r3 = O.search_scale_table(W, X, np.ones((1, 256), F32), cfg)
    assert r3["losses"][0] == r1["losses"][0]


def pin_hadamard_example():
    """[AWQ-notes §5.1] the normalised 4x4 Hadamard maps [0.1, 0.2, 20, 0.1] to about
    [10.2, 9.9, -9.9, -10.0] and keeps the squared norm 400.06."""
    ex = _golden("awq_notes_examples.json")["hadamard_rotation"]
    x = np.array([ex["before"]], F16)
    y = O.hadamard_rotate(x, 4).astype(F64)[0]
    assert np.allclose(y, ex["after"], atol=ex["tol_abs"])
    assert abs(float(np.sum(y * y)) - ex["squared_norm"]) < 0.2
    assert abs(float(np.sum(x.astype(F64) ** 2)) - ex["squared_norm"]) < 0.2


def pin_hadamard_orthogonal():
    """H_n is the Sylvester matrix (checked against scipy's construction), H H^T = n I, the
    normalised block rotation is an involution, and with Q = identity the reparameterised
    layer computes the same output: (W R)(X R)^T = W X^T [AWQ-notes §5.1]."""
    from scipy.linalg import hadamard as scipy_hadamard
    for n in (1, 2, 4, 16, 128):
        H = O.hadamard_matrix(n)
        assert np.array_equal(H, scipy_hadamard(n).astype(F64))
        assert np.array_equal(H @ H.T, n * np.eye(n))
    rng = np.random.default_rng(34)
    A = (rng.standard_normal((6, 256)) * 0.5).astype(F16)
    twice = O.hadamard_rotate(O.hadamard_rotate(A, 64), 64)
    assert np.allclose(twice.astype(F64), A.astype(F64), atol=4e-3, rtol=4e-3)
    W = rng.standard_normal((5, 128))
    X = rng.standard_normal((7, 128))
    R = O.hadamard_matrix(128) / np.sqrt(128.0)
    assert np.allclose((W @ R) @ (X @ R).T, W @ X.T, atol=1e-10)
    x = np.zeros((1, 128), F16)
    x[0, 5] = 16.0                                  # one outlier spreads evenly
    y = O.hadamard_rotate(x, 128).astype(F64)
    assert np.allclose(np.abs(y), 16.0 / np.sqrt(128.0), rtol=1e-3)


def pin_w4a16_bruteforce():
    """The W4A16 product read byte by byte in plain Python loops (channel i of row m in
    byte i // 2, low nibble for even i [AWQ-blog §4.2]; weight (c - z) * step of its
    group [AWQ-blog §1.2]) equals the oracle's vectorised product, and a unit activation
    returns one column of the dequantised weights."""
    rng = np.random.default_rng(40)
    M, K, T, g = 3, 64, 2, 32
    packed = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    scales = (rng.uniform(0.001, 0.05, (M, K // g))).astype(np.float16)
    zeros = rng.integers(0, 16, (M, K // g)).astype(np.float16)
    X = rng.standard_normal((T, K)).astype(np.float16)
    y = O.w4a16_matmul(packed, scales, zeros, X, g)
    for t in range(T):
        for m in range(M):
            acc = 0.0
            for i in range(K):
                byte = int(packed[m, i // 2])
                c = (byte >> 4) if (i % 2) else (byte & 15)
                w = (c - float(zeros[m, i // g])) * float(scales[m, i // g])
                acc += w * float(X[t, i])
            assert math.isclose(acc, y[t, m], rel_tol=1e-12, abs_tol=1e-12), (t, m)
    e = np.zeros((1, K), np.float16)
    e[0, 37] = 1.0
    col = O.w4a16_matmul(packed, scales, zeros, e, g)[0]
    byte = packed[:, 18].astype(int)
    want = ((byte >> 4) - zeros[:, 1].astype(F64)) * scales[:, 1].astype(F64)
    assert np.array_equal(col, want)


def pin_w4a16_reproduces_layer():
    """Quantise-and-pack W S, fold S^-1 into the activations [AWQ-notes §4.3], and the
    packed product gives back x W^T to within the quantiser's error: every weight is off by
    at most half a step (pinned above) plus the fp16 rounding of the stored step, and every
    folded activation by the fp16 rounding of x / s."""
    rng = np.random.default_rng(41)
    M, K, T = 24, 256, 5
    W = (rng.standard_normal((M, K)) * 0.02).astype(np.float16)
    X = rng.standard_normal((T, K)).astype(np.float16)
    X[:, 9] *= 40
    for cfg in (_cfg(4, 128, 1), _cfg(4, 64, 0), _cfg(3, 32, 1)):
        s = O.scale_family(O.act_stats(X), np.array([0.5], F32))[0]
        packed, scales, zeros = O.quantize_pack(W, s, cfg)
        y = O.w4a16_matmul(packed, scales, zeros, X, cfg.group_size, s32=s)
        exact = X.astype(F64) @ W.astype(F64).T
        _, step32, _ = O.quantize(W, s, cfg)
        half = np.repeat(step32.astype(F64), cfg.group_size, axis=1) * (0.5 + 16 * 2.0 ** -11)
        xt = np.abs(X.astype(F64) / s.astype(F64)[None, :])
        ws = np.abs(W.astype(F64) * s.astype(F64)[None, :])
        bound = xt @ half.T * (1 + 2.0 ** -10) + xt @ ws.T * 2.0 ** -10
        assert np.all(np.abs(y - exact) <= bound), float(np.max(np.abs(y - exact) / bound))
        # and the bound is not vacuous: the error is a real fraction of it
        assert np.max(np.abs(y - exact) / bound) > 0.05


def pin_clip_ratio_one_and_range():
    """Ratio 1 is the plain quantiser bit for bit; a ratio below 1 shrinks the range by
    hand-checkable amounts and clamps the values beyond it [AWQ-notes §2.3 (Q rounds and
    clips)]."""
    rng = np.random.default_rng(50)
    W = (rng.standard_normal((6, 256)) * 0.05).astype(np.float16)
    s = np.exp(rng.uniform(-1, 1, 256)).astype(F32)
    for cfg in (_cfg(4, 128, 1), _cfg(4, 64, 0), _cfg(3, 32, 1)):
        ones = np.ones((6, 256 // cfg.group_size), F32)
        a, b = O.quantize(W, s, cfg), O.quantize(W, s, cfg, clip=ones)
        assert all(np.array_equal(x, y) for x, y in zip(a, b))
    # zero-point, 4 bits: v in [-1, 2]; ratio 0.5 -> hi 1.0, lo -0.5, step 0.1, zero 5
    v = np.linspace(-1.0, 2.0, 32).astype(np.float16)[None, :]
    c, st, z = O.quantize(v, np.ones(32, F32), _cfg(4, 32, 1), clip=np.full((1, 1), 0.5, F32))
    assert st[0, 0] == F32(F32(1.5) / F32(15)) and z[0, 0] == 5
    deq = O.dequantize_scaled(c, st, z, 32)[0]
    assert deq[-1] == F32(10 * st[0, 0]) and deq[0] == F32(-5 * st[0, 0])
    inside = np.abs(v[0].astype(F32) - F32(0.25)) <= F32(0.7)
    assert np.all(np.abs(deq[inside] - v[0].astype(F32)[inside]) <= st[0, 0] / 2 + 1e-7)
    # symmetric, 4 bits: max|v| = 2 -> ratio 0.5 -> 1.0, step 1/7, 2.0 clamps to 7 steps
    c, st, z = O.quantize(v, np.ones(32, F32), _cfg(4, 32, 0), clip=np.full((1, 1), 0.5, F32))
    assert st[0, 0] == F32(F32(1.0) / F32(7))
    assert O.dequantize_scaled(c, st, z, 32)[0, -1] == F32(7 * st[0, 0])


def pin_clip_group_error_identities():
    """The group error equals the quadratic form d^T (X_G^T X_G) d of the group's weight
    error, and when the groups' activations have disjoint token supports (no cross terms)
    the group errors add up to the layer's output-error loss [AWQ-notes §1.1]."""
    rng = np.random.default_rng(51)
    M, K, g = 5, 256, 64
    cfg = _cfg(4, g, 1)
    W = (rng.standard_normal((M, K)) * 0.03).astype(np.float16)
    X = rng.standard_normal((40, K)).astype(np.float16)
    s = np.exp(rng.uniform(-0.5, 0.5, K)).astype(F32)
    ratios = np.array([1.0, 0.9, 0.75], F32)
    e = O.clip_group_errors(W, X, s, cfg, ratios)
    for k, r in enumerate(ratios):
        d = O.delta_weight(W, s, cfg, clip=np.full((M, K // g), r, F32))
        for j in range(K // g):
            Xg = X[:, j * g:(j + 1) * g].astype(F64)
            Gram = Xg.T @ Xg
            dj = d[:, j * g:(j + 1) * g]
            q = np.einsum("mi,ij,mj->m", dj, Gram, dj)
            assert np.allclose(e[k, :, j], q, rtol=1e-10, atol=0)
    Xd = np.zeros((4 * 10, K), np.float16)
    for j in range(K // g):
        Xd[10 * j:10 * (j + 1), j * g:(j + 1) * g] = X[10 * j:10 * (j + 1), j * g:(j + 1) * g]
    e = O.clip_group_errors(W, Xd, s, cfg, ratios)
    for k, r in enumerate(ratios):
        d = O.delta_weight(W, s, cfg, clip=np.full((M, K // g), r, F32))
        assert math.isclose(float(e[k].sum()), O.output_error_loss(d, Xd), rel_tol=1e-12)


def pin_clip_search_choices():
    """With identity activations (the group error is the squared weight error): a group
    on the unclipped grid keeps ratio 1 (error 0); a group of even integers up to 6 with
    one 15 is reproduced exactly at ratio 14/15 except the 15, which clips to 14, so that
    ratio wins (error 1 against about 2.9 unclipped); equal ratios tie to the first."""
    g = 32
    cfg = _cfg(4, g, 0)
    on_grid = (np.arange(-7, 8, dtype=F64)[np.arange(g) % 15] * 0.25).astype(np.float16)
    ev = np.array([2.0, -2.0, 4.0, -4.0, 6.0, -6.0] * 6)[: g - 1]
    outl = np.concatenate([ev, [15.0]]).astype(np.float16)
    W = np.stack([on_grid, outl])
    X = np.eye(g, dtype=np.float16)
    s = np.ones(g, F32)
    ratios = np.array([1.0, 14.0 / 15.0, 0.5], F32)
    r = O.clip_search(W, X, s, cfg, ratios)
    e = r["errors"]
    assert r["best"][0, 0] == 0 and e[0, 0, 0] == 0.0 and e[1, 0, 0] > 0
    assert r["best"][1, 0] == 1 and e[1, 1, 0] < e[0, 1, 0] / 2
    assert abs(e[1, 1, 0] - 1.0) < 1e-3               # only the 15 -> 14 error remains
    assert r["clip"][1, 0] == ratios[1]
    tie = O.clip_search(W, X, s, cfg, np.array([1.0, 1.0, 0.5], F32))
    assert tie["best"][0, 0] == 0


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_") and callable(v)]
