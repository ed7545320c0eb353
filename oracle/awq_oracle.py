"""Plain CPU oracle for AWQ's per-layer activation-aware scale search and 4-bit packing.

TEST INFRASTRUCTURE ONLY.  This module is the checker that the GPU library is compared
against.  Only the test suite, the package smoke check and the benchmark's CPU-baseline
leg may import it; the library itself never does, and nothing here is shared with the HIP
kernels (no common code, tables or constants).

It is written for a reader holding the source pages, step by step in their order, with
no blocking, fusion or reordering beyond a numpy primitive per step:

  pages cited (title, site):
    [AWQ-notes]  "AWQ" -- lizn-zn.github.io scholia-log, inference-quantization notes
    [AWQ-tut]    "AWQ量化" tutorial -- aiqz.cc
    [AWQ-blog]   "AWQ量化技术解析：激活感知的权重量化革命" -- kwkr.cn
    [GPTQ-AWQ]   "大模型的开发应用（十八）：大模型量化：GPTQ与AWQ" -- ewbang.com
    [AutoAWQ-70B] "AWQ 量化全流程拆解：将 70B 大模型塞进单张消费级 GPU" -- lnrq.cn

Precision: statistics, scale powers, the de-scaling division and the loss are float64; the
quantiser itself is float32 with one IEEE rounding per operation (numpy float32 `*`, `/`,
`-` are single correctly rounded operations, never fused) and round-half-to-even
(`np.rint`), which is the elementwise sequence the GPU side must reproduce bit for bit.

Readings taken where the pages leave a step open (each repeated at its function):
  statistic     mean |x| over all calibration tokens (not max, not EMA)
  a_i == 0      s_i := 1
  groups        `group_size` consecutive input channels of one output row share a step
  symmetric     step = max|v| / (2^(b-1)-1), codes clamped to +-(2^(b-1)-1), stored with
                offset 2^(b-1) so that dequantisation is (c - z) * step in both modes
  zero-point    min-max over the group extended to include 0; z = rint(-min/step)
  zero step     a group whose step computes to 0 uses step 1 (it quantises to 0 exactly)
  step in loss  the float32 step (fp16 rounding of the step happens only when packing)
  loss          sum of squares of the output error, via Delta Y = Delta W X
  argmin        over finite losses, first index on ties; none finite -> index -1, s := 1
  packing       two 4-bit slots per byte, even input channel in the low nibble; a step
                that overflows its fp16 storage is reported (stored_step_overflows)
  W4A16 product y = x~ W_dequant^T with x~ = fl16(fl32(x / s)) when s is given, fp64
  clipping      per (row, group) ratio rho multiplies the group's range (hi, lo or max|v|)
                in float32 before the step; chosen by the group's own output error
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

F32 = np.float32
F64 = np.float64


@dataclasses.dataclass(frozen=True)
class QConfig:
    """Quantiser settings: the `w_bit`, `q_group_size` and `zero_point` keys of AutoAWQ's
    quant_config [AutoAWQ-70B §三; GPTQ-AWQ §3 "关键参数"]."""

    w_bit: int = 4
    group_size: int = 128
    zero_point: int = 1


# --------------------------------------------------------------------------------------
# A1  activation statistics
# --------------------------------------------------------------------------------------
def act_stats(X16: np.ndarray, channel_chunk: int = 1024) -> np.ndarray:
    """Per-input-channel mean activation magnitude, a_i = (1/N) sum_t |x_{t,i}|.

    [AWQ-notes §1.2 (a_i as the expectation of |x_i|); AWQ-tut 激活感知 (importance
    score as the average absolute activation over N calibration samples)].

    X16: float16 [N tokens][K channels].  Sums are float64 (for fp16 inputs they are exact
    while every partial sum stays below 2^29), divided by N in float64, then rounded to
    float32.  Processed in channel chunks only to bound memory.
    """
    X16 = np.asarray(X16)
    N, K = X16.shape
    if N <= 0:
        raise ValueError("act_stats needs at least one token")
    out = np.empty(K, dtype=F32)
    for c0 in range(0, K, channel_chunk):
        c1 = min(K, c0 + channel_chunk)
        col = np.abs(X16[:, c0:c1].astype(F64))
        out[c0:c1] = (col.sum(axis=0) / F64(N)).astype(F32)
    return out


# --------------------------------------------------------------------------------------
# A2  scale family
# --------------------------------------------------------------------------------------
def scale_family(a32: np.ndarray, alphas32: np.ndarray) -> np.ndarray:
    """s_{k,i} = a_i ** alpha_k for every grid point alpha_k  ->  float32 [n_alpha][K].

    [AWQ-notes §4.1 (s_i = a_i^alpha; alpha = 0 means no scaling); GPTQ-AWQ §3 二.2
    (grid search of alpha over [0, 1])].  The power is taken in float64 and rounded to
    float32.  Reading: a channel with a_i == 0 gets s_i = 1 (the pages require s_i > 0,
    AWQ-notes §2.1).
    """
    a32 = np.asarray(a32, dtype=F32)
    alphas32 = np.asarray(alphas32, dtype=F32)
    s = np.empty((alphas32.size, a32.size), dtype=F32)
    a64 = a32.astype(F64)
    for k, alpha in enumerate(alphas32):
        p = np.power(a64, F64(alpha))
        row = p.astype(F32)
        row[a32 == 0] = F32(1.0)
        s[k] = row
    return s


# --------------------------------------------------------------------------------------
# A3  group quantiser Q applied to the scaled weight W * diag(s)
# --------------------------------------------------------------------------------------
def quantize(W16: np.ndarray, s32: np.ndarray, cfg: QConfig, clip=None):
    """Group-wise uniform quantisation of v = W * s (float32, one rounding per op).

    [AWQ-tut 量化基础 (q = round(W/step), step = max|W| / (2^(b-1)-1));
     AWQ-tut 缩放保护 (scale the channel, quantise, divide back);
     GPTQ-AWQ §3 一.2 (w' = Round(w*s/step'));
     AWQ-notes §2.3 (Q(w) = step * round(w/step)); AWQ-notes §3.2 (one step shared by a
     group of 128 weights); AWQ-blog §2.1 (symmetric INT4 code = round(clip(W/s,-8,7)))]

    Returns (codes uint8 [M][K], step float32 [M][K/g], zero int32 [M][K/g]).
    Symmetric:  step = max_G|v| / qmax, qmax = 2^(b-1)-1; q = clamp(rint(v/step), +-qmax);
                code = q + 2^(b-1), zero = 2^(b-1).
    Zero-point: hi = max(max_G v, 0), lo = min(min_G v, 0), step = (hi - lo) / (2^b - 1);
                zero = clamp(rint(-lo/step), 0, 2^b-1); code = clamp(rint(v/step) + zero).
    A step that computes to 0 is replaced by 1.

    clip (optional, float32 [M][K/g], each in (0, 1]) shrinks a group's range before the
    step is taken -- hi and lo (zero-point) or max|v| (symmetric) are multiplied by the
    ratio in float32 -- and values beyond the shrunk range are clipped by the clamp
    [AWQ-notes closing note (the practical algorithm may add clipping); AWQ-notes §2.3
    (Q includes rounding and clipping)].  Ratio 1 is the plain quantiser.
    """
    W16 = np.asarray(W16)
    M, K = W16.shape
    g = cfg.group_size
    b = cfg.w_bit
    if K % g != 0:
        raise ValueError("in_features must be a multiple of group_size")
    v = W16.astype(F32) * np.asarray(s32, dtype=F32)[None, :]
    vg = v.reshape(M, K // g, g)
    if cfg.zero_point:
        top = F32(2 ** b - 1)
        hi = np.maximum(vg.max(axis=2, initial=-np.inf), F32(0.0))
        lo = np.minimum(vg.min(axis=2, initial=np.inf), F32(0.0))
        if clip is not None:
            r = np.asarray(clip, dtype=F32).reshape(M, K // g)
            hi = (hi * r).astype(F32)
            lo = (lo * r).astype(F32)
        step = ((hi - lo) / top).astype(F32)
        step[step == 0] = F32(1.0)
        zero = np.clip(np.rint(-lo / step), F32(0.0), top)
        q = np.rint(vg / step[:, :, None]) + zero[:, :, None]
        codes = np.clip(q, F32(0.0), top)
    else:
        qmax = F32(2 ** (b - 1) - 1)
        mag = np.abs(vg).max(axis=2, initial=F32(0.0))
        if clip is not None:
            mag = (mag * np.asarray(clip, dtype=F32).reshape(M, K // g)).astype(F32)
        step = (mag / qmax).astype(F32)
        step[step == 0] = F32(1.0)
        q = np.clip(np.rint(vg / step[:, :, None]), -qmax, qmax)
        zero = np.full(step.shape, F32(2 ** (b - 1)), dtype=F32)
        codes = q + zero[:, :, None]
    with np.errstate(invalid="ignore"):   # non-finite inputs give unspecified codes
        return (codes.reshape(M, K).astype(np.uint8), step.astype(F32),
                zero.astype(np.int32))


def dequantize_scaled(codes: np.ndarray, step: np.ndarray, zero: np.ndarray,
                      group_size: int) -> np.ndarray:
    """(code - zero) * step in float32: the quantised value of the *scaled* weight
    [AWQ-notes §2.3; GPTQ-AWQ §3 一.2 (dequantisation is step' * w')]."""
    M, K = codes.shape
    cg = codes.reshape(M, K // group_size, group_size).astype(F32)
    d = (cg - zero.astype(F32)[:, :, None]) * step[:, :, None]
    return d.reshape(M, K).astype(F32)


def fake_quant_weight(W16: np.ndarray, s32: np.ndarray, cfg: QConfig,
                      identity_quantizer: bool = False, clip=None) -> np.ndarray:
    """Q(W S) S^-1 in float64: quantise the scaled weight, then divide each input channel
    by its scale [AWQ-tut 缩放保护 (W_hat = Q(s W)/s); AWQ-notes §2.2, §4.1].

    identity_quantizer=True replaces Q by the identity (used to check that the scaling
    itself is an exact reparameterisation, AWQ-notes §2.1)."""
    s64 = np.asarray(s32, dtype=F32).astype(F64)
    if identity_quantizer:
        d = (W16.astype(F32) * np.asarray(s32, dtype=F32)[None, :]).astype(F64)
    else:
        codes, step, zero = (quantize(W16, s32, cfg) if clip is None
                             else quantize(W16, s32, cfg, clip=clip))
        d = dequantize_scaled(codes, step, zero, cfg.group_size).astype(F64)
    return d / s64[None, :]


def delta_weight(W16: np.ndarray, s32: np.ndarray, cfg: QConfig,
                 identity_quantizer: bool = False, clip=None) -> np.ndarray:
    """Delta W = W - Q(W S) S^-1 (float64) [AWQ-notes §1.1, weight error of the quantised
    layer; the sign does not matter for the squared loss]."""
    if clip is None:
        return W16.astype(F64) - fake_quant_weight(W16, s32, cfg, identity_quantizer)
    return W16.astype(F64) - fake_quant_weight(W16, s32, cfg, identity_quantizer, clip=clip)


# --------------------------------------------------------------------------------------
# A4  output-error loss
# --------------------------------------------------------------------------------------
def output_error_loss(dW64: np.ndarray, X16: np.ndarray, row_block: int = 1024) -> float:
    """|| Delta W X ||_F^2 = sum over rows r and tokens t of (sum_i dW[r,i] x_{t,i})^2.

    [AWQ-notes §1.1 (output error Delta Y = Delta W X); AWQ-notes §4.1 (squared Frobenius
    objective); AWQ-tut GPTQ对比 (expected squared output error)].  X16 is [tokens][K],
    i.e. the pages' X transposed, so the product is dW @ X16^T.  float64 throughout; rows
    in blocks only to bound memory (the sum is over rows, so blocking changes nothing but
    rounding order).
    """
    X64 = np.asarray(X16, dtype=F64)     # no copy when the caller already passes fp64
    total = F64(0.0)
    for r0 in range(0, dW64.shape[0], row_block):
        Y = dW64[r0:r0 + row_block] @ X64.T
        total += F64(np.sum(Y * Y))
    return float(total)


def layer_output_error(W16, What64, X16) -> float:
    """The objective exactly as printed, || W X - W_hat X ||_F^2, without forming Delta W
    first [AWQ-notes §4.1; GPTQ-AWQ §3 二.1].  Used to confirm the Delta W route."""
    X64 = np.asarray(X16).astype(F64)
    Y = W16.astype(F64) @ X64.T
    Yq = What64 @ X64.T
    return float(np.sum((Y - Yq) ** 2))


# --------------------------------------------------------------------------------------
# A5  selection
# --------------------------------------------------------------------------------------
def select_best(losses: np.ndarray) -> int:
    """Index of the smallest finite loss, the first one on ties; -1 if none is finite
    [AWQ-notes §4.1 (argmin over the restricted family); AWQ-notes reference note (the
    practical search runs over a restricted parametrisation)]."""
    losses = np.asarray(losses, dtype=F64)
    finite = np.isfinite(losses)
    if not finite.any():
        return -1
    masked = np.where(finite, losses, np.inf)
    return int(np.argmin(masked))


def search_scales(W16, X16, a32, alphas32, cfg: QConfig):
    """Grid search: for each alpha, s = a^alpha, loss = ||Delta W(s) X||^2; pick the argmin.

    [AWQ-notes §4.1; GPTQ-AWQ §3 二.1-二.2].  Returns a dict with
    s_table [n_alpha][K], losses [n_alpha] (float64), best (int), s_star [K] (float32)."""
    s_table = scale_family(a32, alphas32)
    losses = np.empty(len(alphas32), dtype=F64)
    X64 = np.asarray(X16, dtype=F64)     # exact widening, done once for all grid points
    for k in range(len(alphas32)):
        losses[k] = output_error_loss(delta_weight(W16, s_table[k], cfg), X64)
    best = select_best(losses)
    if best >= 0:
        s_star = s_table[best].copy()
    else:
        s_star = np.ones(np.asarray(a32).size, dtype=F32)
    return {"s_table": s_table, "losses": losses, "best": best, "s_star": s_star}


# --------------------------------------------------------------------------------------
# A6  quantise + pack
# --------------------------------------------------------------------------------------
def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """Two 4-bit codes per byte, input channel 2j in the low nibble and 2j+1 in the high
    nibble  ->  uint8 [M][K/2] [AWQ-blog §4.2 (two 4-bit values packed per byte)]."""
    codes = np.asarray(codes, dtype=np.uint8)
    lo = codes[:, 0::2].astype(np.uint16)
    hi = codes[:, 1::2].astype(np.uint16)
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    """Inverse of pack_nibbles."""
    packed = np.asarray(packed, dtype=np.uint8)
    M, H = packed.shape
    out = np.empty((M, 2 * H), dtype=np.uint8)
    out[:, 0::2] = packed & 0x0F
    out[:, 1::2] = packed >> 4
    return out


def quantize_pack(W16, s32, cfg: QConfig, clip=None):
    """Codes of Q(W S) packed two per byte, plus the per-group step as fp16 and the zero
    point as fp16 (an integer value) [AWQ-blog §1.2 (int4 codes with an fp16 scale,
    W = code * scale); AWQ-blog §2.1 (store the scale as FP16); AutoAWQ-70B §三
    (zero_point=True, group 128, 4 bits) and §四 (per-group metadata cost at g = 128)].

    The packed codes are of the *scaled* weight: S^-1 is folded into the preceding op
    [AWQ-notes §4.3].  Returns (packed uint8 [M][K/2], scales fp16 [M][K/g],
    zeros fp16 [M][K/g])."""
    codes, step, zero = (quantize(W16, s32, cfg) if clip is None
                         else quantize(W16, s32, cfg, clip=clip))
    with np.errstate(over="ignore"):  # a step of 65520 or more becomes fp16 infinity
        scales = step.astype(np.float16)
    return pack_nibbles(codes), scales, zero.astype(np.float16)


def stored_step_overflows(scales16) -> bool:
    """Whether a packed layer holds a step that is not finite in its fp16 storage.

    Reading of [AWQ-blog §2.1] (the step is stored as FP16) and §1.2 (the weight is
    dequantised as code times that scale): a group whose float32 step rounds to fp16
    infinity (round to nearest even, so every step of 65520 or more, fp16's largest finite
    value being 65504) cannot be dequantised from the stored format, and the pack reports
    the layer instead of returning such a step silently."""
    return not bool(np.all(np.isfinite(np.asarray(scales16, dtype=np.float16))))


def run_layer(W16, X16, alphas32, cfg: QConfig):
    """The whole path for one linear layer: statistics -> search -> pack."""
    a32 = act_stats(X16)
    res = search_scales(W16, X16, a32, alphas32, cfg)
    packed, scales, zeros = quantize_pack(W16, res["s_star"], cfg)
    res.update({"a": a32, "packed": packed, "scales": scales, "zeros": zeros})
    return res


# --------------------------------------------------------------------------------------
# Clip search after the scale search
# --------------------------------------------------------------------------------------
def clip_group_errors(W16, X16, s32, cfg: QConfig, ratios32) -> np.ndarray:
    """e[k][m][j]: the output error that group j of row m contributes on its own when every
    group's range is shrunk by ratio k, i.e. sum over tokens t of
    (sum_{i in group j} dW_k[m][i] x_{t,i})^2 with dW_k = W - Q_k(W S) S^-1
    [AWQ-notes §1.1 (output error of the weight error), closing note (clipping is searched
    with the same kind of objective as the scales)].  Reading: the per-group objective is
    the group's own partial product, so each (row, group) picks its ratio independently.
    fp64 [n_ratio][M][K/g]."""
    X64 = np.asarray(X16, dtype=F64)
    W16 = np.asarray(W16)
    M, K = W16.shape
    g = cfg.group_size
    ng = K // g
    out = np.empty((len(ratios32), M, ng), dtype=F64)
    for k, r in enumerate(np.asarray(ratios32, dtype=F32)):
        dW = delta_weight(W16, s32, cfg, clip=np.full((M, ng), r, dtype=F32))
        for j in range(ng):
            Y = dW[:, j * g:(j + 1) * g] @ X64[:, j * g:(j + 1) * g].T
            out[k, :, j] = np.sum(Y * Y, axis=1)
    return out


def clip_search(W16, X16, s32, cfg: QConfig, ratios32):
    """For every (row, group) the ratio with the smallest group error (first on ties, so
    the least clipping when the grid runs from 1 downwards; ratio 1 when no error is
    finite).  Returns errors [n_ratio][M][K/g], best index [M][K/g] and the chosen
    ratios float32 [M][K/g]."""
    ratios32 = np.asarray(ratios32, dtype=F32)
    e = clip_group_errors(W16, X16, s32, cfg, ratios32)
    fin = np.isfinite(e)
    masked = np.where(fin, e, np.inf)
    best = np.argmin(masked, axis=0).astype(np.int32)
    best[~fin.any(axis=0)] = -1
    clip = np.where(best >= 0, ratios32[np.maximum(best, 0)], F32(1.0)).astype(F32)
    return {"errors": e, "best": best, "clip": clip}


# --------------------------------------------------------------------------------------
# Consumer of the packed format: the W4A16 product at inference
# --------------------------------------------------------------------------------------
def fold_inverse_scales(X16: np.ndarray, s32: np.ndarray) -> np.ndarray:
    """x~ = x / s: the S^-1 that the pages fold into the preceding operation
    [AWQ-notes §4.3].  Reading: one fp32 division per element, then rounded to fp16, the
    dtype the preceding operation would emit."""
    X32 = np.asarray(X16).astype(F32)
    return (X32 / np.asarray(s32, dtype=F32)[None, :]).astype(np.float16)


def dequantize_packed(packed: np.ndarray, scales16: np.ndarray, zeros16: np.ndarray,
                      group_size: int) -> np.ndarray:
    """W_dequant = (c - z) * step for every weight, from the packed codes and the stored
    fp16 step and zero of its group [AWQ-blog §1.2 (W_dequant = W_int4 x scale_fp16);
    GPTQ-AWQ §3 (weights stay 4-bit and are dequantised on the fly for fp16 compute)].
    fp64, where it is exact ((c - z) is a small integer and the step an fp16)."""
    codes = unpack_nibbles(packed).astype(F64)
    M, K = codes.shape
    step = np.asarray(scales16, dtype=np.float16).astype(F64)
    zero = np.asarray(zeros16, dtype=np.float16).astype(F64)
    cg = codes.reshape(M, K // group_size, group_size)
    return ((cg - zero[:, :, None]) * step[:, :, None]).reshape(M, K)


def w4a16_matmul(packed, scales16, zeros16, X16, group_size: int, s32=None) -> np.ndarray:
    """y[t][m] = sum_i W_dequant[m][i] * x~[t][i] for fp16 activations X [T][K]: the
    product the packed layer serves at inference, with x~ = X when S^-1 has already been
    folded into the preceding operation and x~ = fold_inverse_scales(X, s) otherwise
    [AutoAWQ-70B §四 (GEMM kernels for batches, GEMV for single requests);
    AWQ-blog §4.2 (dequantisation fused into the product)].  fp64 [T][M]."""
    Xt = np.asarray(X16) if s32 is None else fold_inverse_scales(X16, s32)
    Wd = dequantize_packed(packed, scales16, zeros16, group_size)
    return Xt.astype(F64) @ Wd.T


# --------------------------------------------------------------------------------------
# Variants of the statistic and of the scale family (widening beyond the mean |x| / a^alpha
# path).  Each is a separate reading of a page; the search itself is unchanged.
# --------------------------------------------------------------------------------------
def act_stat_max_abs(X16: np.ndarray) -> np.ndarray:
    """a_i = max_t |x_{t,i}| [GPTQ-AWQ §3 二.2 (s = (max|A|)^alpha)].  Exact in fp32."""
    X16 = np.asarray(X16)
    if X16.shape[0] <= 0:
        raise ValueError("needs at least one token")
    return np.abs(X16).max(axis=0).astype(F32)


def act_stat_rms_ratio(X16: np.ndarray, channel_chunk: int = 1024) -> np.ndarray:
    """a_i = E|x_i| / sqrt(E[x_i^2]) [AWQ-blog §1.2 (importance score)], fp64, rounded to
    fp32.  Reading: a channel whose E[x^2] is 0 gets a_i = 0."""
    X16 = np.asarray(X16)
    N, K = X16.shape
    if N <= 0:
        raise ValueError("needs at least one token")
    out = np.empty(K, dtype=F32)
    for c0 in range(0, K, channel_chunk):
        c1 = min(K, c0 + channel_chunk)
        col = X16[:, c0:c1].astype(F64)
        m1 = np.abs(col).sum(axis=0) / F64(N)
        m2 = (col * col).sum(axis=0) / F64(N)
        with np.errstate(invalid="ignore", divide="ignore"):
            r = np.where(m2 > 0, m1 / np.sqrt(m2), F64(0.0))
        out[c0:c1] = r.astype(F32)
    return out


def act_stat_ema_mean(X16: np.ndarray, batch_tokens: int, momentum: float = 0.9) -> np.ndarray:
    """Exponential moving average of the per-batch mean |x| over consecutive batches of
    `batch_tokens` tokens: e <- momentum * e + (1 - momentum) * mean_batch |x|, starting
    from e = 0 [AWQ-blog §2.1 (calibration statistics pseudo-code, momentum 0.9)].
    Reading: batches are consecutive token ranges, the last may be shorter; fp64
    throughout, rounded to fp32 at the end.  (The page's running max of amax|x| over
    batches is the global max, i.e. act_stat_max_abs.)"""
    X16 = np.asarray(X16)
    N, K = X16.shape
    if N <= 0 or batch_tokens <= 0:
        raise ValueError("needs tokens and a positive batch size")
    mom = F64(momentum)
    keep = F64(1.0) - mom
    e = np.zeros(K, dtype=F64)
    for t0 in range(0, N, batch_tokens):
        blk = X16[t0:t0 + batch_tokens].astype(F64)
        m = np.abs(blk).sum(axis=0) / F64(blk.shape[0])
        e = mom * e + keep * m
    return e.astype(F32)


def percentile_linear(a32: np.ndarray, percentile: float) -> float:
    """The p-th percentile with linear interpolation between order statistics, in fp64:
    position (p/100)(K-1) in the sorted values [AWQ-tut 显著识别 (threshold at a high
    percentile of the importance scores)]."""
    v = np.sort(np.asarray(a32, dtype=F32)).astype(F64)
    pos = F64(percentile) / F64(100.0) * F64(v.size - 1)
    lo = int(np.floor(pos))
    hi = min(lo + 1, v.size - 1)
    frac = pos - F64(lo)
    return float(v[lo] + frac * (v[hi] - v[lo]))


def threshold_scales(a32: np.ndarray, percentile: float, factor: float) -> np.ndarray:
    """Fixed-factor protection: s_i = factor for channels whose statistic exceeds the
    percentile threshold, 1 otherwise [AWQ-tut 显著识别 (indicator 1_i = [a_i > tau]),
    缩放保护 (protect by a factor s > 1), Python 演示 (70th percentile, factor 2)]."""
    tau = percentile_linear(a32, percentile)
    a64 = np.asarray(a32, dtype=F32).astype(F64)
    return np.where(a64 > tau, F32(factor), F32(1.0)).astype(F32)


def search_scale_table(W16, X16, s_table32, cfg: QConfig):
    """The search of search_scales over an explicit table of candidate scale vectors."""
    s_table32 = np.asarray(s_table32, dtype=F32)
    losses = np.empty(s_table32.shape[0], dtype=F64)
    X64 = np.asarray(X16, dtype=F64)
    for k in range(s_table32.shape[0]):
        losses[k] = output_error_loss(delta_weight(W16, s_table32[k], cfg), X64)
    best = select_best(losses)
    s_star = s_table32[best].copy() if best >= 0 else np.ones(s_table32.shape[1], F32)
    return {"s_table": s_table32, "losses": losses, "best": best, "s_star": s_star}


def hadamard_matrix(n: int) -> np.ndarray:
    """Sylvester Hadamard matrix H_n (n a power of two): H_1 = [1],
    H_2m = [[H_m, H_m], [H_m, -H_m]] (fp64)."""
    if n < 1 or n & (n - 1):
        raise ValueError("n must be a power of two")
    H = np.ones((1, 1), dtype=F64)
    while H.shape[0] < n:
        H = np.block([[H, H], [H, -H]])
    return H


def hadamard_rotate(A16: np.ndarray, block: int) -> np.ndarray:
    """Rotate every row of A (fp16 [rows][K]) by the block-diagonal orthogonal matrix whose
    blocks are H_block / sqrt(block) along K [AWQ-notes §5.1 (WX = (WR)(R^T X) for
    orthogonal R; normalised Hadamard spreads an outlier), §5.2 (structured fast
    rotation)].  The product with the +-1 matrix H is taken first, in fp64, where it is
    exact for fp16 inputs (sums of at most 512 multiples of 2^-24 below 2^16 fit in 53
    bits, whatever order or fused operations the matmul uses); the normalisation
    1/sqrt(block) is then the one rounding, and the cast to fp16 rounds to nearest even."""
    A = np.asarray(A16).astype(F64)
    R, K = A.shape
    if K % block:
        raise ValueError("block must divide in_features")
    S = A.reshape(R, K // block, block) @ hadamard_matrix(block)
    out = (S * (F64(1.0) / np.sqrt(F64(block)))).reshape(R, K)
    return out.astype(np.float16)
