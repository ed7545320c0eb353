"""Each planted mistake in the CPU oracle must be caught by at least one pin.

The mistakes are planted in the oracle (on the CPU, via monkeypatch), never in the GPU
path.  They are the plausible slips of writing this method down: a wrong rounding mode,
a dropped zero point, a multiplied instead of divided scale, a transposed operand, a wrong
axis, a missing square, argmax for argmin, and so on.
"""
import numpy as np
import pytest

from oracle import awq_oracle as O
from tests import oracle_pins

F16, F32, F64 = np.float16, np.float32, np.float64

_orig_quantize = O.quantize
_orig_fake = O.fake_quant_weight
_orig_stats = O.act_stats
_orig_loss = O.output_error_loss
_orig_scale = O.scale_family
_orig_select = O.select_best
_orig_dequant = O.dequantize_scaled
_orig_pack = O.pack_nibbles


def _quantize_with(rounder=np.rint, sym_levels=None, drop_zero=False, group_rows=False,
                   no_zero_step_fix=False, no_include_zero=False):
    """A re-statement of the quantiser with one knob turned wrong."""

    def q(W16, s32, cfg):
        M, K = W16.shape
        g, b = cfg.group_size, cfg.w_bit
        v = W16.astype(F32) * np.asarray(s32, F32)[None, :]
        if group_rows:                      # groups along the output dimension
            v = v.T.copy()
            M, K = K, M
            if K % g:
                raise ValueError
        vg = v.reshape(M, K // g, g)
        if cfg.zero_point:
            top = F32(2 ** b - 1)
            hi, lo = vg.max(axis=2), vg.min(axis=2)
            if not no_include_zero:
                hi, lo = np.maximum(hi, F32(0)), np.minimum(lo, F32(0))
            step = ((hi - lo) / top).astype(F32)
            if not no_zero_step_fix:
                step[step == 0] = F32(1)
            zero = np.clip(rounder(-lo / step), 0, top)
            if drop_zero:
                zero = np.zeros_like(zero)
            codes = np.clip(rounder(vg / step[:, :, None]) + zero[:, :, None], 0, top)
        else:
            qmax = F32(sym_levels(b) if sym_levels else 2 ** (b - 1) - 1)
            step = (np.abs(vg).max(axis=2) / qmax).astype(F32)
            if not no_zero_step_fix:
                step[step == 0] = F32(1)
            qq = np.clip(rounder(vg / step[:, :, None]), -qmax, qmax)
            zero = np.full(step.shape, F32(2 ** (b - 1)))
            if drop_zero:
                zero = np.zeros_like(zero)
            codes = qq + zero[:, :, None]
        codes = codes.reshape(M, K)
        if group_rows:
            codes = codes.T
            step = np.repeat(step.T, 1, axis=0)
            zero = zero.T
            # shapes no longer match the (row, input-group) layout; keep them as produced
        with np.errstate(invalid="ignore"):
            return codes.astype(np.uint8), step.astype(F32), zero.astype(np.int32)

    return q


def _half_up(x):
    return np.floor(x + F32(0.5)).astype(F32)


def _fake_multiply(W16, s32, cfg, identity_quantizer=False):
    s64 = np.asarray(s32, F32).astype(F64)
    if identity_quantizer:
        d = (W16.astype(F32) * np.asarray(s32, F32)[None, :]).astype(F64)
    else:
        c, st, z = O.quantize(W16, s32, cfg)
        d = O.dequantize_scaled(c, st, z, cfg.group_size).astype(F64)
    return d * s64[None, :]


def _fake_no_unscale(W16, s32, cfg, identity_quantizer=False):
    c, st, z = O.quantize(W16, s32, cfg)
    return O.dequantize_scaled(c, st, z, cfg.group_size).astype(F64)


def _stats_signed(X16, channel_chunk=1024):
    X = np.asarray(X16).astype(F64)
    return (X.sum(axis=0) / X.shape[0]).astype(F32)


def _stats_max(X16, channel_chunk=1024):
    X = np.asarray(X16).astype(F64)
    return np.abs(X).max(axis=0).astype(F32)


def _stats_wrong_axis(X16, channel_chunk=1024):
    X = np.asarray(X16).astype(F64)
    m = np.abs(X).mean(axis=1).astype(F32)
    K = X.shape[1]
    return np.resize(m, K)


def _loss_untransposed(dW64, X16, row_block=1024):
    X64 = np.asarray(X16).astype(F64)
    Y = dW64 @ X64          # wrong orientation: only conforms when N == K
    return float(np.sum(Y * Y))


def _loss_no_square(dW64, X16, row_block=1024):
    X64 = np.asarray(X16).astype(F64)
    return float(np.sum(np.abs(dW64 @ X64.T)))


def _loss_weight_space(dW64, X16, row_block=1024):
    return float(np.sum(dW64 * dW64))


def _scale_linear(a32, alphas32):
    a32 = np.asarray(a32, F32)
    out = np.empty((len(alphas32), a32.size), F32)
    for k, al in enumerate(alphas32):
        r = (a32.astype(F64) * F64(al)).astype(F32)
        r[a32 == 0] = 1
        out[k] = r
    return out


def _scale_swapped(a32, alphas32):
    a32 = np.asarray(a32, F32)
    out = np.empty((len(alphas32), a32.size), F32)
    for k, al in enumerate(alphas32):
        out[k] = np.power(F64(al), a32.astype(F64)).astype(F32)
    return out


def _scale_zero_kept(a32, alphas32):
    a32 = np.asarray(a32, F32)
    out = np.empty((len(alphas32), a32.size), F32)
    for k, al in enumerate(alphas32):
        out[k] = np.power(a32.astype(F64), F64(al)).astype(F32)
    return out


def _select_argmax(losses):
    losses = np.asarray(losses, F64)
    if not np.isfinite(losses).any():
        return -1
    return int(np.argmax(np.where(np.isfinite(losses), losses, -np.inf)))


def _select_last_tie(losses):
    losses = np.asarray(losses, F64)
    if not np.isfinite(losses).any():
        return -1
    m = np.where(np.isfinite(losses), losses, np.inf)
    return int(len(m) - 1 - np.argmin(m[::-1]))


def _select_nan_blind(losses):
    return int(np.argmin(np.asarray(losses, F64)))


def _dequant_no_zero(codes, step, zero, group_size):
    M, K = codes.shape
    cg = codes.reshape(M, K // group_size, group_size).astype(F32)
    return (cg * step[:, :, None]).reshape(M, K).astype(F32)


def _pack_swapped(codes):
    codes = np.asarray(codes, np.uint8)
    return (codes[:, 1::2].astype(np.uint16) | (codes[:, 0::2].astype(np.uint16) << 4)).astype(np.uint8)


MUTANTS = {
    "round_floor": ("quantize", _quantize_with(rounder=np.floor)),
    "round_half_up": ("quantize", _quantize_with(rounder=_half_up)),
    "round_trunc": ("quantize", _quantize_with(rounder=np.trunc)),
    "sym_levels_2b_minus_1": ("quantize", _quantize_with(sym_levels=lambda b: 2 ** b - 1)),
    "sym_levels_2b1": ("quantize", _quantize_with(sym_levels=lambda b: 2 ** (b - 1))),
    "zero_point_dropped": ("quantize", _quantize_with(drop_zero=True)),
    "groups_along_rows": ("quantize", _quantize_with(group_rows=True)),
    "zero_step_unfixed": ("quantize", _quantize_with(no_zero_step_fix=True)),
    "range_without_zero": ("quantize", _quantize_with(no_include_zero=True)),
    "unscale_multiplies": ("fake_quant_weight", _fake_multiply),
    "unscale_missing": ("fake_quant_weight", _fake_no_unscale),
    "stats_signed_mean": ("act_stats", _stats_signed),
    "stats_max": ("act_stats", _stats_max),
    "stats_wrong_axis": ("act_stats", _stats_wrong_axis),
    "loss_untransposed": ("output_error_loss", _loss_untransposed),
    "loss_not_squared": ("output_error_loss", _loss_no_square),
    "loss_weight_space": ("output_error_loss", _loss_weight_space),
    "scale_linear_in_alpha": ("scale_family", _scale_linear),
    "scale_base_exponent_swapped": ("scale_family", _scale_swapped),
    "scale_zero_channel_kept": ("scale_family", _scale_zero_kept),
    "select_argmax": ("select_best", _select_argmax),
    "select_last_on_tie": ("select_best", _select_last_tie),
    "select_nan_blind": ("select_best", _select_nan_blind),
    "dequant_without_zero": ("dequantize_scaled", _dequant_no_zero),
    "nibbles_swapped": ("pack_nibbles", _pack_swapped),
}


def _max_signed(X16):
    return np.asarray(X16).max(axis=0).astype(F32)


def _rms_no_sqrt(X16, channel_chunk=1024):
    X = np.asarray(X16).astype(F64)
    m1 = np.abs(X).mean(axis=0)
    m2 = (X * X).mean(axis=0)
    with np.errstate(all="ignore"):
        return np.where(m2 > 0, m1 / m2, 0.0).astype(F32)


def _ema_swapped(X16, batch_tokens, momentum=0.9):
    X16 = np.asarray(X16)
    e = np.zeros(X16.shape[1])
    for t0 in range(0, X16.shape[0], batch_tokens):
        m = np.abs(X16[t0:t0 + batch_tokens].astype(F64)).mean(axis=0)
        e = (1 - momentum) * e + momentum * m
    return e.astype(F32)


def _percentile_no_interp(a32, percentile):
    v = np.sort(np.asarray(a32, F32)).astype(F64)
    return float(v[int(percentile / 100 * (v.size - 1))])


def _percentile_wrong_pos(a32, percentile):
    v = np.sort(np.asarray(a32, F32)).astype(F64)
    pos = min(percentile / 100 * v.size, v.size - 1)
    lo = int(np.floor(pos)); hi = min(lo + 1, v.size - 1)
    return float(v[lo] + (pos - lo) * (v[hi] - v[lo]))


def _threshold_inverted(a32, percentile, factor):
    tau = O.percentile_linear(a32, percentile)
    return np.where(np.asarray(a32, F64) < tau, F32(factor), F32(1.0)).astype(F32)


def _hadamard_wrong_sign(n):
    H = np.ones((1, 1))
    while H.shape[0] < n:
        H = np.block([[H, H], [-H, H]])
    return H


def _hadamard_rotate_unnormalised(A16, block):
    A = np.asarray(A16).astype(F64)
    R, K = A.shape
    return (A.reshape(R, K // block, block) @ O.hadamard_matrix(block)).reshape(R, K).astype(np.float16)


def _dequant_packed_no_zero(packed, scales16, zeros16, group_size):
    codes = O.unpack_nibbles(packed).astype(F64)
    M, K = codes.shape
    st = np.asarray(scales16, np.float16).astype(F64)
    return (codes.reshape(M, K // group_size, group_size) * st[:, :, None]).reshape(M, K)


def _dequant_packed_tiled(packed, scales16, zeros16, group_size):
    codes = O.unpack_nibbles(packed).astype(F64)
    st = np.tile(np.asarray(scales16, np.float16).astype(F64), (1, group_size))
    z = np.tile(np.asarray(zeros16, np.float16).astype(F64), (1, group_size))
    return (codes - z) * st


def _unpack_swapped(packed):
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty((packed.shape[0], 2 * packed.shape[1]), dtype=np.uint8)
    out[:, 0::2] = packed >> 4
    out[:, 1::2] = packed & 0x0F
    return out


def _fold_multiplies(X16, s32):
    return (np.asarray(X16).astype(F32) * np.asarray(s32, F32)[None, :]).astype(np.float16)


def _quantize_clip_divides(W16, s32, cfg, clip=None):
    if clip is None:
        return _orig_quantize(W16, s32, cfg)
    return _orig_quantize(W16, s32, cfg, clip=1.0 / np.asarray(clip, F32))


def _quantize_clip_ignored(W16, s32, cfg, clip=None):
    return _orig_quantize(W16, s32, cfg)


def _clip_errors_whole_row(W16, X16, s32, cfg, ratios32):
    X64 = np.asarray(X16, F64)
    M, K = np.asarray(W16).shape
    ng = K // cfg.group_size
    out = np.empty((len(ratios32), M, ng))
    for k, r in enumerate(np.asarray(ratios32, F32)):
        dW = O.delta_weight(W16, s32, cfg, clip=np.full((M, ng), r, F32))
        Y = dW @ X64.T
        out[k] = (np.sum(Y * Y, axis=1) / ng)[:, None]
    return out


_orig_clip_errors = O.clip_group_errors


def _clip_search_argmax(W16, X16, s32, cfg, ratios32):
    ratios32 = np.asarray(ratios32, F32)
    e = _orig_clip_errors(W16, X16, s32, cfg, ratios32)
    best = np.argmax(e, axis=0).astype(np.int32)
    return {"errors": e, "best": best, "clip": ratios32[best]}


MUTANTS.update({
    "clip_divides_range": ("quantize", _quantize_clip_divides),
    "clip_ignored": ("quantize", _quantize_clip_ignored),
    "clip_error_whole_row": ("clip_group_errors", _clip_errors_whole_row),
    "clip_search_argmax": ("clip_search", _clip_search_argmax),
})

MUTANTS.update({
    "w4a16_zero_not_subtracted": ("dequantize_packed", _dequant_packed_no_zero),
    "w4a16_groups_tiled": ("dequantize_packed", _dequant_packed_tiled),
    "unpack_nibbles_swapped": ("unpack_nibbles", _unpack_swapped),
    "fold_multiplies_by_s": ("fold_inverse_scales", _fold_multiplies),
})

MUTANTS.update({
    "max_signed": ("act_stat_max_abs", _max_signed),
    "rms_ratio_without_sqrt": ("act_stat_rms_ratio", _rms_no_sqrt),
    "ema_momentum_swapped": ("act_stat_ema_mean", _ema_swapped),
    "percentile_no_interpolation": ("percentile_linear", _percentile_no_interp),
    "percentile_position_K": ("percentile_linear", _percentile_wrong_pos),
    "threshold_inverted": ("threshold_scales", _threshold_inverted),
    "hadamard_wrong_recursion": ("hadamard_matrix", _hadamard_wrong_sign),
    "hadamard_unnormalised": ("hadamard_rotate", _hadamard_rotate_unnormalised),
})


def _overflow_nan_only(scales16):
    return bool(np.isnan(np.asarray(scales16, np.float16)).any())


def _overflow_strict_fp32(scales16):
    # compares against fp16's largest finite value as if the step were still fp32
    return bool((np.asarray(scales16, np.float16).astype(F32) > F32(65504.0)).any() is False)


_orig_quantize_pack = O.quantize_pack


def _pack_saturating(W16, s32, cfg, clip=None):
    codes, step, zero = (O.quantize(W16, s32, cfg) if clip is None
                         else O.quantize(W16, s32, cfg, clip=clip))
    sat = np.minimum(step, F32(65504.0)).astype(np.float16)
    return O.pack_nibbles(codes), sat, zero.astype(np.float16)


MUTANTS.update({
    "overflow_sees_only_nan": ("stored_step_overflows", _overflow_nan_only),
    "overflow_inverted": ("stored_step_overflows", _overflow_strict_fp32),
    "pack_step_saturates": ("quantize_pack", _pack_saturating),
})


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(O, attr, fn)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except Exception as e:  # noqa: BLE001 - any failure counts as detection
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"no pin detects mutant {name}"
