"""W4A16 product of a packed layer on the GPU (through the C ABI) against the fp64 oracle.

Bar, derived from the kernels' arithmetic: the folded activations x~ = fp16(fp32(x / s))
are formed identically on both sides; every (c - z) and every fp16 x fp16 product is
exact in fp32.  In the vector kernel a result passes through at most 32 dot-product
roundings in a lane, one multiplication by the step and the chunk sum (at most 1024
additions, bounded by their magnitudes); in the matrix-core kernel through the MFMA's
own sums, one fused multiply-add per group (at most 64 per wave) and at most 15 wave
additions.  Both stay within 256 * 2^-24 * sum_i |w_i x~_i| of the exact sum; the final
fp16 rounding adds at most one fp16 ulp.  A wrong nibble, group, zero or token would
break this by orders of magnitude.  With S^-1 folded (s = None) and two or more tokens
the library takes the matrix-core kernel, otherwise the vector kernel.
"""
import numpy as np
import pytest
import torch

import weight_only_quantization_act_amd as awq
from oracle import awq_oracle as O
from synth import CONFIGS, alpha_grid, make_layer, row_subset, small_spec
from tests.gpu_util import dev, host, ocfg, requires_gpu, say

pytestmark = [pytest.mark.gpu, requires_gpu]

F16, F32, F64 = np.float16, np.float32, np.float64


def _random_packed(rng, M, K, g, sym=False):
    packed = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    scales = rng.uniform(0.0005, 0.02, (M, K // g)).astype(F16)
    if sym:
        zeros = np.full((M, K // g), 8, F16)
    else:
        zeros = rng.integers(0, 16, (M, K // g)).astype(F16)
    return packed, scales, zeros


def _check(y_gpu, packed, scales, zeros, X, g, s=None, where=""):
    y_ref = O.w4a16_matmul(packed, scales, zeros, X, g, s32=s)
    Xt = np.asarray(X) if s is None else O.fold_inverse_scales(X, s)
    Wd = O.dequantize_packed(packed, scales, zeros, g)
    mag = np.abs(Xt.astype(F64)) @ np.abs(Wd).T
    E = 256 * 2.0 ** -24 * mag
    ulp = np.spacing((np.abs(y_ref) + E).astype(F16)).astype(F64)
    yg = np.asarray(y_gpu).astype(F64)
    assert yg.shape == y_ref.shape
    err = np.abs(yg - y_ref)
    bad = err > E + ulp
    if bad.any():
        t, m = np.argwhere(bad)[0]
        raise AssertionError(f"{where}: {int(bad.sum())} outputs off, first y[{t}][{m}] gpu "
                             f"{yg[t, m]!r} oracle {y_ref[t, m]!r} bound {(E + ulp)[t, m]!r}")
    return float(np.max(err / (E + ulp)))


CASES = [
    # M, K, T, g, with_s
    (64, 128, 1, 128, False),
    (300, 4096, 1, 128, True),      # ragged rows
    (257, 4096, 3, 64, False),
    (1000, 11008, 2, 128, True),    # 344 chunks: a 384-thread block on the 1024 bound
    (77, 8192, 4, 32, True),
    (129, 512, 5, 128, False),      # two passes of tokens (4 + 1)
    (40, 1024, 9, 64, True),        # three passes
    (9, 32768, 2, 128, False),      # the largest K: 1024 threads
    (33, 32, 1, 32, True),          # a single chunk
    (70, 4096, 4, 128, True),       # s given, several tokens: the fold, then the matrix cores
    (48, 1024, 21, 64, True),       # the same over two token passes
    # folded activations, several tokens: the matrix-core kernel
    (100, 1024, 16, 32, False),
    (50, 2048, 16, 64, False),
    (300, 4096, 7, 128, False),
    (65, 640, 17, 128, False),      # 16 + 1 tokens: two passes
    (200, 11008, 33, 128, False),   # three passes, 86 groups over the waves
    (3, 32768, 4, 32, False),       # 1024 groups of 32
]


@pytest.mark.parametrize("M,K,T,g,with_s", CASES)
def test_w4a16_random_codes(M, K, T, g, with_s):
    say(f"w4a16 M={M} K={K} T={T} g={g} s={with_s}")
    rng = np.random.default_rng(M * 31 + K + T)
    packed, scales, zeros = _random_packed(rng, M, K, g, sym=(g == 64))
    X = rng.standard_normal((T, K)).astype(F16)
    s = np.exp(rng.uniform(-1.0, 2.0, K)).astype(F32) if with_s else None
    cfg = awq.qconfig(4, g, 1)
    y = awq.awq_w4a16_matmul(dev(X), dev(packed), dev(scales), dev(zeros), cfg,
                             s=dev(s) if with_s else None)
    r = _check(host(y), packed, scales, zeros, X, g, s, f"{M}x{K}x{T}")
    say(f"  max err / bound {r:.3f}")
    if with_s and T >= 2:
        # the default call folds x / s into a workspace and takes the matrix-core kernel;
        # an empty workspace keeps the vector kernel, which must meet the same bound
        y2 = awq.awq_w4a16_matmul(dev(X), dev(packed), dev(scales), dev(zeros), cfg, s=dev(s),
                                  workspace=torch.empty(0, dtype=torch.uint8, device="cuda"))
        _check(host(y2), packed, scales, zeros, X, g, s, f"{M}x{K}x{T} vector kernel")
        # the fold is the oracle's x~ bit for bit: the same kernel on the oracle's x~ gives
        # the same bits
        y3 = awq.awq_w4a16_matmul(dev(O.fold_inverse_scales(X, s)), dev(packed), dev(scales),
                                  dev(zeros), cfg)
        assert np.array_equal(host(y).view(np.uint16), host(y3).view(np.uint16))


def test_w4a16_degenerate():
    cfg = awq.qconfig(4, 128, 1)
    rng = np.random.default_rng(5)
    packed, scales, zeros = _random_packed(rng, 16, 256, 128)
    # zero tokens: nothing to do
    y0 = awq.awq_w4a16_matmul(torch.empty((0, 256), dtype=torch.float16, device="cuda"),
                              dev(packed), dev(scales), dev(zeros), cfg)
    assert y0.shape == (0, 16)
    # all codes equal to their zero: y = 0 exactly, whatever x is
    z = rng.integers(0, 16, (16, 2)).astype(F16)
    codes = np.repeat(z.astype(np.uint8), 128, axis=1)
    pk = O.pack_nibbles(codes)
    X = (rng.standard_normal((3, 256)) * 100).astype(F16)
    y = host(awq.awq_w4a16_matmul(dev(X), dev(pk), dev(scales), dev(z), cfg))
    assert np.all(y == 0)
    # zero activations
    y = host(awq.awq_w4a16_matmul(dev(np.zeros((2, 256), F16)), dev(packed), dev(scales),
                                  dev(zeros), cfg))
    assert np.all(y == 0)
    # in_features = 0: every output is the empty sum
    e8 = torch.empty((4, 0), dtype=torch.uint8, device="cuda")
    e16 = torch.empty((4, 0), dtype=torch.float16, device="cuda")
    y = awq.awq_w4a16_matmul(torch.empty((2, 0), dtype=torch.float16, device="cuda"), e8, e16,
                             e16, cfg)
    assert torch.all(y == 0)


def test_w4a16_deterministic():
    rng = np.random.default_rng(6)
    packed, scales, zeros = _random_packed(rng, 512, 4096, 128)
    X = dev(rng.standard_normal((4, 4096)).astype(F16))
    cfg = awq.qconfig(4, 128, 1)
    for T in (1, 4):
        a = host(awq.awq_w4a16_matmul(X[:T], dev(packed), dev(scales), dev(zeros), cfg)).copy()
        b = host(awq.awq_w4a16_matmul(X[:T], dev(packed), dev(scales), dev(zeros), cfg))
        assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
    # a token's result does not depend on the other tokens of the batch (per-column sums)
    y16 = host(awq.awq_w4a16_matmul(dev(rng.standard_normal((16, 4096)).astype(F16)),
                                    dev(packed), dev(scales), dev(zeros), cfg))
    Xb = rng.standard_normal((16, 4096)).astype(F16)
    yb = host(awq.awq_w4a16_matmul(dev(Xb), dev(packed), dev(scales), dev(zeros), cfg))
    yb3 = host(awq.awq_w4a16_matmul(dev(Xb[3:5]), dev(packed), dev(scales), dev(zeros), cfg))
    assert np.array_equal(yb[3:5].view(np.uint16), yb3.view(np.uint16))
    assert y16.shape == (16, 512)


@pytest.mark.parametrize("name,w_bit,g,zp", [("c1", 4, 128, 0), ("q3", 3, 64, 1)])
def test_w4a16_end_to_end_layer(name, w_bit, g, zp):
    """The whole path on the GPU (statistics, search, pack), then the packed layer times the
    calibration activations with S^-1 folded in; the oracle runs the same path on the CPU.
    The product also reproduces X W^T to within the quantiser's error."""
    if name == "c1":
        L = make_layer(CONFIGS["c1"][0])
    else:
        L = make_layer(small_spec("q3", 384, 512, 300, w_bit=3, group_size=64, zero_point=1,
                                  outlier_count=5))
    say(f"w4a16 end to end {name}")
    cfg = awq.qconfig(w_bit, g, zp)
    alphas = alpha_grid(20)
    Wd, Xd = dev(L.W), dev(L.X)
    res = awq.quantize_layer(Wd, Xd, alphas, cfg)
    Xq = L.X[:7]
    y = awq.awq_w4a16_matmul(dev(Xq), res["codes"], res["scales"], res["zeros"], cfg, s=res["s"])
    torch.cuda.synchronize()
    orc = O.run_layer(L.W, L.X, alphas, ocfg(cfg))
    assert np.array_equal(host(res["codes"]), orc["packed"])
    _check(host(y), orc["packed"], orc["scales"], orc["zeros"], Xq, g, orc["s_star"], name)
    exact = Xq.astype(F64) @ L.W.astype(F64).T
    rel = np.linalg.norm(host(y).astype(F64) - exact) / np.linalg.norm(exact)
    assert rel < 0.2, rel


@pytest.mark.parametrize("cfg_name", ["c2", "c4"])
def test_w4a16_full_size_sampled_rows(cfg_name):
    """The headline and the 70B-class layer shapes at decode batch 1 and 4, in the launch
    configuration the benchmark times; the oracle recomputes a seeded sample of 512 output
    rows (each output is an independent row product)."""
    spec = CONFIGS[cfg_name][0]
    M, K, g = spec.out_features, spec.in_features, spec.group_size
    say(f"w4a16 full size {cfg_name} {M}x{K}")
    rng = np.random.default_rng(spec.seed_base + 7)
    packed, scales, zeros = _random_packed(rng, M, K, g)
    X = rng.standard_normal((4, K)).astype(F16)
    s = np.exp(rng.uniform(-1.0, 2.0, K)).astype(F32)
    cfg = awq.qconfig(4, g, 1)
    Pd, Sd, Zd, sd = dev(packed), dev(scales), dev(zeros), dev(s)
    rows = row_subset(spec, 512)
    for T in (1, 4):
        y = host(awq.awq_w4a16_matmul(dev(X[:T]), Pd, Sd, Zd, cfg, s=sd))
        _check(y[:, rows], packed[rows], scales[rows], zeros[rows], X[:T], g, s,
               f"{cfg_name} T={T}")
    X16 = rng.standard_normal((16, K)).astype(F16)
    for T in (1, 4, 16):                                 # S^-1 folded into x
        y = host(awq.awq_w4a16_matmul(dev(X16[:T]), Pd, Sd, Zd, cfg))
        _check(y[:, rows], packed[rows], scales[rows], zeros[rows], X16[:T], g, None,
               f"{cfg_name} folded T={T}")
