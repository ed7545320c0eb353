"""C ABI on the host: the library loads, exports every declared entry point, and rejects
bad arguments with the documented status codes before touching the GPU.

Every call below fails a host-side check that runs before any HIP call, so these tests
run without a GPU.  Pointer values are fake (never dereferenced)."""
import ctypes
import os
import re

import pytest

import weight_only_quantization_act_amd as awq
from weight_only_quantization_act_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "awq_act.h")

# the numbering of the planned boundary (OK .. NONFINITE = 0 .. 8), then the two codes
# added to it: ALIGN and SCALE_OVERFLOW
E = {"OK": 0, "NULL": 1, "SHAPE": 2, "CONFIG": 3, "ALPHA": 4, "WORKSPACE": 5, "DEVICE": 6,
     "HIP": 7, "NONFINITE": 8, "ALIGN": 9, "SCALE_OVERFLOW": 10}
WARNINGS = ("NONFINITE", "SCALE_OVERFLOW")

P = ctypes.c_void_p(0x10000)     # aligned fake device pointer (never dereferenced)
P_ODD = ctypes.c_void_p(0x10002)  # misaligned


@pytest.fixture(scope="module")
def L():
    return awq.lib()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+char\s*\*|int|size_t)\s+(awq_\w+)\s*\(",
                                 text, flags=re.M)))


def test_exports_every_declared_symbol(L):
    names = _declared_functions()
    assert len(names) == 29, names
    for n in names:
        assert hasattr(L, n), f"{n} declared in awq_act.h but not exported"
    assert set(names) == set(_lib._SIGNATURES)


def test_status_strings_and_enum(L):
    text = open(HEADER).read()
    for name, val in E.items():
        key = "AWQ_OK" if name == "OK" else (f"AWQ_W_{name}" if name in WARNINGS else f"AWQ_E_{name}")
        assert re.search(rf"\b{key}\s*=\s*{val}\b", text), key
        s = awq.status_str(val)
        assert s.startswith(key)
    assert "unknown" in awq.status_str(12345)


def _cfg(b=4, g=128, zp=1):
    return ctypes.byref(awq.qconfig(b, g, zp))


def _search(L, W=P, X=P, a=P, M=256, K=256, N=64, cfg=None, alphas=(0.0, 0.5, 1.0),
            n_alpha=None, s=P, losses=P, best=P, status=P, ws=P, ws_bytes=1 << 40):
    al = (ctypes.c_float * max(1, len(alphas)))(*alphas)
    n = len(alphas) if n_alpha is None else n_alpha
    return L.awq_search_scales(W, X, a, M, K, N, cfg if cfg is not None else _cfg(), al, n, s,
                               losses, best, status, ws, ws_bytes, None)


def test_search_validation(L):
    assert _search(L, W=None) == E["NULL"]
    assert _search(L, X=None) == E["NULL"]
    assert _search(L, s=None) == E["NULL"]
    assert _search(L, ws=None) == E["WORKSPACE"]
    assert _search(L, cfg=_cfg(5)) == E["CONFIG"]
    assert _search(L, cfg=_cfg(1)) == E["CONFIG"]
    assert _search(L, cfg=_cfg(4, 96)) == E["CONFIG"]
    assert _search(L, cfg=_cfg(4, 128, 2)) == E["CONFIG"]
    assert _search(L, K=200) == E["SHAPE"]           # not a multiple of 128
    assert _search(L, M=-1) == E["SHAPE"]
    assert _search(L, N=0) == E["SHAPE"]
    assert _search(L, M=1 << 20, K=1 << 12) == E["SHAPE"]  # M*K >= 2^31
    assert _search(L, N=1 << 20, K=1 << 12) == E["SHAPE"]
    assert _search(L, alphas=(), n_alpha=0) == E["ALPHA"]
    assert _search(L, alphas=tuple([0.5] * 65)) == E["ALPHA"]
    assert _search(L, alphas=(0.0, 1.5)) == E["ALPHA"]
    assert _search(L, alphas=(-0.1,)) == E["ALPHA"]
    assert _search(L, alphas=(float("nan"),)) == E["ALPHA"]
    need1 = awq.awq_workspace_bytes(256, 256, 64, awq.qconfig(), 3, 1)
    assert _search(L, ws_bytes=need1 - 1) == E["WORKSPACE"]
    assert _search(L, W=P_ODD) == E["ALIGN"]
    assert _search(L, X=P_ODD) == E["ALIGN"]
    assert _search(L, losses=ctypes.c_void_p(0x10004)) == E["ALIGN"]
    assert _search(L, ws=ctypes.c_void_p(0x10010)) == E["ALIGN"]


def test_workspace_query(L):
    cfg = awq.qconfig(4, 128, 1)
    M = K = 4096
    N = 2048                                     # the direct form
    assert awq.awq_loss_form(M, K, N, 20) == awq.AWQ_LOSS_DIRECT
    full = awq.awq_workspace_bytes(M, K, N, cfg, 20, 20)
    one = awq.awq_workspace_bytes(M, K, N, cfg, 20, 1)
    tiles = (M // 256) * (N // 256)
    fixed = 20 * K * 4 + 20 * tiles * 8          # both already multiples of 256
    assert one == fixed + M * K * 2
    assert full == fixed + 20 * M * K * 2
    assert awq.awq_workspace_bytes(M, K, N, cfg, 20, 99) == full
    assert awq.awq_workspace_bytes(M, K, N, cfg, 20, 7) == fixed + 7 * M * K * 2
    # the G form: tiles over K, then X^T (fp16 [K][N]), the fp32 split partials of the 136
    # tiles of G's upper block triangle, fp16 G', fp32 diagonal, the partials' tile maxima,
    # and the exponent, each 256-byte aligned.  The 4096 tokens go in two splits (2752 and
    # 1344): on 136 tiles one split leaves 120 of 256 compute units idle, and with two
    # uneven splits the short blocks run on the units the long ones leave free.
    N = 4096
    assert awq.awq_loss_form(M, K, N, 20) == awq.AWQ_LOSS_GRAM
    tiles = (M // 256) * (K // 256)
    splits = 2
    fixed = (20 * K * 4 + 20 * tiles * 8 + K * N * 2 + splits * 136 * 256 * 256 * 4 + K * K * 2
             + K * 4 + 1280 + 256)
    assert awq.awq_workspace_bytes(M, K, N, cfg, 20, 1) == fixed + M * K * 2
    assert awq.awq_workspace_bytes(M, K, N, cfg, 20, 20) == fixed + 20 * M * K * 2
    # more tokens than one split (8192) holds: at least three splits; the plan takes four
    # (three of 5760 tokens and one of 2720: the busiest compute unit then runs 11520
    # tokens' worth of tiles, against 13440 with three equal splits)
    N = 20000
    ld = 20000                                    # already a multiple of 8
    splits, pairs = 4, 136
    fixed = (20 * K * 4 + 20 * tiles * 8 + K * ld * 2 + splits * pairs * 256 * 256 * 4
             + K * K * 2 + K * 4 + ((splits * pairs * 4 + 255) // 256) * 256 + 256)
    assert awq.awq_workspace_bytes(M, K, N, cfg, 20, 1) == fixed + M * K * 2
    assert awq.awq_workspace_bytes(M, K, N, cfg, 0, 0) == 0
    assert awq.awq_workspace_bytes(M, 100, N, cfg, 20, 0) == 0
    assert awq.awq_workspace_bytes(0, K, N, cfg, 3, 0) == ((3 * K * 4 + 255) // 256) * 256
    s = awq.awq_act_stats_workspace_bytes(4096, 4096)
    assert s > 0 and s % 256 == 0
    assert awq.awq_act_stats_workspace_bytes(0, 16) == 0


def test_stats_validation(L):
    ws = awq.awq_act_stats_workspace_bytes(64, 256)
    f = L.awq_act_stats
    assert f(None, 64, 256, P, P, ws, None) == E["NULL"]
    assert f(P, 64, 256, None, P, ws, None) == E["NULL"]
    assert f(P, 64, 256, P, None, ws, None) == E["WORKSPACE"]
    assert f(P, 0, 256, P, P, ws, None) == E["SHAPE"]
    assert f(P, 64, -3, P, P, ws, None) == E["SHAPE"]
    assert f(P, 64, 256, P, P, ws - 1, None) == E["WORKSPACE"]
    assert f(P_ODD, 64, 256, P, P, ws, None) == E["ALIGN"]
    assert f(P, 64, 256, ctypes.c_void_p(0x10001), P, ws, None) == E["ALIGN"]


def test_pack_and_fake_quant_validation(L):
    f = L.awq_quantize_pack
    assert f(None, P, 8, 128, _cfg(), P, P, P, None) == E["NULL"]
    assert f(P, P, 8, 128, _cfg(), P, P, None, None) == E["NULL"]
    assert f(P, P, 8, 128, _cfg(4, 48), P, P, P, None) == E["CONFIG"]
    assert f(P, P, 8, 96, _cfg(4, 64), P, P, P, None) == E["SHAPE"]
    assert f(P, P_ODD, 8, 128, _cfg(), P, P, P, None) == E["ALIGN"]
    assert f(P, P, 8, 128, _cfg(), ctypes.c_void_p(0x10002), P, P, None) == E["ALIGN"]
    g = L.awq_fake_quant_delta
    assert g(None, P, 8, 128, _cfg(), P, None) == E["NULL"]
    assert g(P, P, 8, 100, _cfg(4, 32), P, None) == E["SHAPE"]
    assert g(P, P, 8, 128, _cfg(3, 128, 3), P, None) == E["CONFIG"]
    assert g(P, P, 8, 128, _cfg(), P_ODD, None) == E["ALIGN"]
    # empty weights are a no-op that succeeds without touching memory
    assert f(P, P, 0, 128, _cfg(), P, P, P, None) == E["OK"]
    assert g(P, P, 8, 0, _cfg(), P, None) == E["OK"]
    h = L.awq_quantize_pack_checked
    assert h(P, P, None, 8, 128, _cfg(), P, P, P, None, None) == E["NULL"]   # no status word
    assert h(None, P, None, 8, 128, _cfg(), P, P, P, P, None) == E["NULL"]
    assert h(P, P, None, 8, 128, _cfg(4, 48), P, P, P, P, None) == E["CONFIG"]
    assert h(P, P, None, 8, 96, _cfg(4, 64), P, P, P, P, None) == E["SHAPE"]
    assert h(P, P, None, 8, 128, _cfg(), P, P, P, ctypes.c_void_p(0x10002), None) == E["ALIGN"]
    assert h(P, P, ctypes.c_void_p(0x10002), 8, 128, _cfg(), P, P, P, P, None) == E["ALIGN"]


def test_loss_form_choice():
    q = awq.awq_loss_form
    # few tokens: the direct product; as many tokens as channels or more: the G form
    assert q(512, 512, 256, 20) == awq.AWQ_LOSS_DIRECT
    assert q(4096, 4096, 1024, 20) == awq.AWQ_LOSS_DIRECT
    assert q(4096, 4096, 4096, 20) == awq.AWQ_LOSS_GRAM
    assert q(28672, 8192, 65536, 20) == awq.AWQ_LOSS_GRAM
    assert q(4096, 11008, 16384, 20) == awq.AWQ_LOSS_GRAM
    assert q(4096, 40960, 32768, 20) == awq.AWQ_LOSS_DIRECT   # G beyond 32768 channels
    assert q(0, 4096, 4096, 20) == awq.AWQ_LOSS_DIRECT
    for bad in [(-1, 64, 64, 20), (64, 64, 0, 20), (64, 64, 64, 0), (64, 64, 64, 65),
                (1, 1 << 23, 16, 20)]:
        assert q(*bad) == -1
    # in_features beyond 2^22: the search rejects the shape
    assert awq.awq_workspace_bytes(1, 1 << 23, 16, awq.qconfig(4, 128, 1), 20, 0) == 0
    # the choice agrees with the workspace: the G form holds X^T, G' (fp16) and at least one
    # fp32 partial of G's upper block triangle (136 tiles of 256 x 256) besides dW
    cfg = awq.qconfig(4, 128, 1)
    direct = awq.awq_workspace_bytes(4096, 4096, 1024, cfg, 20, 20)
    gram = awq.awq_workspace_bytes(4096, 4096, 4096, cfg, 20, 20)
    assert gram - direct >= 4096 * 4096 * 2 * 2 + 136 * 256 * 256 * 4


def test_profile_hook_set_and_clear(L):
    assert L.awq_set_profile_events(None, None, None, None, None, None) == E["OK"]
    ev = (ctypes.c_void_p * 8)()
    assert L.awq_set_profile_pass_events(ev, 2) == E["OK"]
    assert L.awq_set_profile_pass_events(None, 0) == E["OK"]   # clears it
    assert L.awq_set_profile_pass_events(None, 1) == E["NULL"]
    assert L.awq_set_profile_pass_events(ev, -1) == E["SHAPE"]
    big = (ctypes.c_void_p * (4 * 65))()
    assert L.awq_set_profile_pass_events(big, 65) == E["SHAPE"]
    with pytest.raises(ValueError):
        awq.awq_set_profile_pass_events([None] * 5)
    awq.awq_set_profile_pass_events([])


# The grid points a pass when the library chooses (alpha_batch <= 0), on the shapes the
# policy was measured on (20 grid points, 4-bit, g = 128, zero point): (M, K, N) -> points
# a pass.  Batched where all of these hold: dW of 20 points above 192 MiB, at least 4
# points within it, in_features >= 2048 (G form) or n_tokens >= 2048 (direct form), and
# the pass's loss blocks filling at least 9/10 of their last round on 256 compute units.
DEFAULT_BATCH = {
    (4096, 4096, 4096): 6,      # G form, 128 blocks a point: 768 = 3 rounds
    (4096, 4096, 2048): 6,      # direct form, 128 blocks a point
    (3072, 3072, 3072): 10,     # 72 blocks a point: 720 of 768
    (4096, 3072, 3072): 8,      # 96 a point: 768
    (2048, 8192, 8192): 6,
    (8192, 2048, 2048): 6,
    (4608, 4096, 4096): 5,      # 144 a point: 720 of 768 (4 points: 576 of 768, not taken)
    (6144, 2048, 2048): 8,
    (4096, 5120, 5120): 20,     # 4 points: 640 of 768 blocks
    (5120, 5120, 5120): 20,     # only 3 points fit
    (11008, 4096, 16384): 20,   # only 2 fit
    (11008, 1024, 1024): 20,    # in_features below 2048
    (4096, 4096, 1024): 20,     # direct form with fewer than 2048 tokens
    (4096, 4096, 1536): 20,
    (2048, 2048, 2048): 20,     # all 20 points fit in 192 MiB
    (28672, 8192, 65536): 20,
}


@pytest.mark.parametrize("shape", sorted(DEFAULT_BATCH))
def test_default_batch(shape):
    M, K, N = shape
    cfg = awq.qconfig(4, 128, 1)
    b = DEFAULT_BATCH[shape]
    assert awq.awq_workspace_bytes(M, K, N, cfg, 20, 0) == awq.awq_workspace_bytes(M, K, N, cfg, 20, b)
    if b < 20:
        assert awq.awq_workspace_bytes(M, K, N, cfg, 20, 0) < awq.awq_workspace_bytes(M, K, N, cfg, 20, b + 1)


def test_stats_ex_validation(L):
    f = L.awq_act_stats_ex
    q = awq.awq_act_stats_ex_workspace_bytes
    ws = q(64, 256, awq.AWQ_STAT_EMA_MEAN, 16)
    assert ws > 0 and ws % 256 == 0
    assert q(64, 256, 4, 0) == 0 and q(64, 256, -1, 0) == 0
    assert q(64, 256, awq.AWQ_STAT_EMA_MEAN, 0) == 0
    # the RMS ratio keeps two sums per split, so it needs more scratch than the mean
    assert q(4096, 4096, awq.AWQ_STAT_RMS_RATIO, 0) > q(4096, 4096, awq.AWQ_STAT_MEAN_ABS, 0)
    assert q(4096, 4096, awq.AWQ_STAT_MEAN_ABS, 0) == awq.awq_act_stats_workspace_bytes(4096, 4096)
    assert f(P, 64, 256, 4, 0, 0.9, P, P, 1 << 30, None) == E["CONFIG"]
    assert f(P, 64, 256, awq.AWQ_STAT_EMA_MEAN, 0, 0.9, P, P, 1 << 30, None) == E["SHAPE"]
    assert f(P, 64, 256, awq.AWQ_STAT_EMA_MEAN, 16, 1.0, P, P, 1 << 30, None) == E["CONFIG"]
    assert f(P, 64, 256, awq.AWQ_STAT_EMA_MEAN, 16, -0.1, P, P, 1 << 30, None) == E["CONFIG"]
    assert f(P, 64, 256, awq.AWQ_STAT_EMA_MEAN, 16, float("nan"), P, P, 1 << 30, None) == E["CONFIG"]
    assert f(P, 64, 256, awq.AWQ_STAT_EMA_MEAN, 16, 0.9, P, P, ws - 1, None) == E["WORKSPACE"]
    assert f(P, 64, 256, awq.AWQ_STAT_MAX_ABS, 0, 0.0, None, P, 1 << 30, None) == E["NULL"]
    assert f(P_ODD, 64, 256, awq.AWQ_STAT_MAX_ABS, 0, 0.0, P, P, 1 << 30, None) == E["ALIGN"]


def test_table_threshold_hadamard_validation(L):
    t = L.awq_search_scale_table
    need = awq.awq_workspace_bytes(256, 256, 64, awq.qconfig(), 3, 1)

    def tab(W=P, X=P, S=P, n=3, M=256, K=256, N=64, cfg=None, ws_bytes=1 << 40, s=P, ws=P):
        return t(W, X, S, n, M, K, N, cfg if cfg is not None else _cfg(), s, P, P, P, ws,
                 ws_bytes, None)

    assert tab(S=None) == E["NULL"]
    assert tab(ws=None) == E["WORKSPACE"]
    assert tab(n=0) == E["ALPHA"] and tab(n=65) == E["ALPHA"]
    assert tab(cfg=_cfg(4, 96)) == E["CONFIG"]
    assert tab(K=200) == E["SHAPE"]
    assert tab(ws_bytes=need - 1) == E["WORKSPACE"]
    assert tab(S=ctypes.c_void_p(0x10008)) == E["ALIGN"]   # the table needs 16 bytes
    th = L.awq_threshold_scales
    assert th(None, 16, 70.0, 2.0, P, None) == E["NULL"]
    assert th(P, 0, 70.0, 2.0, P, None) == E["SHAPE"]
    assert th(P, 32769, 70.0, 2.0, P, None) == E["SHAPE"]
    assert th(P, 16, 100.5, 2.0, P, None) == E["CONFIG"]
    assert th(P, 16, float("nan"), 2.0, P, None) == E["CONFIG"]
    assert th(P, 16, 70.0, 0.0, P, None) == E["CONFIG"]
    assert th(P, 16, 70.0, float("inf"), P, None) == E["CONFIG"]
    assert th(ctypes.c_void_p(0x10002), 16, 70.0, 2.0, P, None) == E["ALIGN"]
    h = L.awq_hadamard_rotate
    assert h(None, 4, 128, 64, P, None) == E["NULL"]
    assert h(P, 4, 128, 3, P, None) == E["CONFIG"]
    assert h(P, 4, 128, 1024, P, None) == E["CONFIG"]
    assert h(P, 4, 96, 64, P, None) == E["SHAPE"]          # block does not divide K
    assert h(P, 4, 4, 4, P, None) == E["SHAPE"]            # K not a multiple of 8
    assert h(P, -1, 128, 64, P, None) == E["SHAPE"]
    assert h(P, 1 << 20, 1 << 12, 64, P, None) == E["SHAPE"]
    assert h(P_ODD, 4, 128, 64, P, None) == E["ALIGN"]
    assert h(P, 0, 128, 64, P, None) == E["OK"]            # empty: nothing to do


def test_w4a16_validation(L):
    f = L.awq_w4a16_matmul

    def call(x=P, s=None, T=2, c=P, sc=P, z=P, M=64, K=256, cfg=None, y=P, ws=None,
             ws_bytes=0):
        return f(x, s, T, c, sc, z, M, K, cfg if cfg is not None else _cfg(), y, ws, ws_bytes,
                 None)

    assert call(x=None) == E["NULL"] and call(c=None) == E["NULL"] and call(y=None) == E["NULL"]
    assert call(cfg=_cfg(4, 48)) == E["CONFIG"]
    assert call(K=200) == E["SHAPE"]                   # not a multiple of the group
    assert call(K=32768 + 128) == E["SHAPE"]           # beyond the GEMV's channel limit
    assert call(T=-1) == E["SHAPE"]
    assert call(x=P_ODD) == E["ALIGN"]
    assert call(c=ctypes.c_void_p(0x10008)) == E["ALIGN"]
    assert call(s=ctypes.c_void_p(0x10004)) == E["ALIGN"]
    assert call(y=ctypes.c_void_p(0x10001)) == E["ALIGN"]
    assert call(T=0) == E["OK"] and call(M=0) == E["OK"]
    # the fold workspace: 2 T K bytes rounded to 256, none below two tokens
    need = awq.awq_w4a16_workspace_bytes(3, 256)
    assert need == 1536 and awq.awq_w4a16_workspace_bytes(1, 256) == 0
    assert awq.awq_w4a16_workspace_bytes(2, 32768 + 32) == 0
    assert call(s=P, T=3, ws=P, ws_bytes=need - 1, M=0) == E["WORKSPACE"]
    assert call(s=P, T=3, ws=ctypes.c_void_p(0x10008), ws_bytes=need) == E["ALIGN"]
    assert call(s=P, T=3, ws=P, ws_bytes=need, M=0) == E["OK"]
    assert call(s=None, T=3, ws=P, ws_bytes=1, M=0) == E["OK"]    # no s: the workspace is unused
    assert call(s=P, T=1, ws=P, ws_bytes=1, M=0) == E["OK"]       # one token: never folded


def test_clip_validation(L):
    f = L.awq_clip_search
    need = awq.awq_clip_workspace_bytes(64, 256, 100, awq.qconfig())
    assert need > 0 and need % 256 == 0

    def call(W=P, X=P, s=P, M=64, K=256, N=100, cfg=None, ratios=(1.0, 0.9, 0.8), n=None,
             clip=P, best=None, errors=None, ws=P, ws_bytes=1 << 40):
        rl = (ctypes.c_float * max(1, len(ratios)))(*ratios)
        return f(W, X, s, M, K, N, cfg if cfg is not None else _cfg(), rl,
                 len(ratios) if n is None else n, clip, best, errors, ws, ws_bytes, None)

    assert call(W=None) == E["NULL"] and call(clip=None) == E["NULL"]
    assert call(ws=None) == E["WORKSPACE"] and call(ws_bytes=need - 1) == E["WORKSPACE"]
    assert call(ratios=(1.0, 0.0)) == E["ALPHA"] and call(ratios=(1.5,)) == E["ALPHA"]
    assert call(ratios=(float("nan"),)) == E["ALPHA"]
    assert call(ratios=(), n=0) == E["ALPHA"] and call(ratios=tuple([0.5] * 65)) == E["ALPHA"]
    assert call(cfg=_cfg(4, 48)) == E["CONFIG"] and call(K=200) == E["SHAPE"]
    assert call(N=0) == E["SHAPE"]
    assert call(X=P_ODD) == E["ALIGN"] and call(ws=ctypes.c_void_p(0x10010)) == E["ALIGN"]
    assert call(M=0) == E["OK"]
    g = L.awq_quantize_pack_clipped
    assert g(P, P, None, 8, 128, _cfg(), P, P, P, None) == E["NULL"]
    assert g(P, P, ctypes.c_void_p(0x10002), 8, 128, _cfg(), P, P, P, None) == E["ALIGN"]
    assert g(P, P, P, 0, 128, _cfg(), P, P, P, None) == E["OK"]


def test_probe_validation(L):
    """The measurement probes check their arguments on the host like the other calls."""
    for probe in (L.awq_probe_mfma, L.awq_probe_lds):
        assert probe(4, 4, None, None) == E["NULL"]
        assert probe(0, 4, P, None) == E["SHAPE"]
        assert probe(4, 0, P, None) == E["SHAPE"]
        assert probe((1 << 16) + 1, 4, P, None) == E["SHAPE"]
        assert probe(4, (1 << 20) + 1, P, None) == E["SHAPE"]
        assert probe(1 << 16, 1 << 13, P, None) == E["SHAPE"]      # product above 2^28
        assert probe(4, 4, ctypes.c_void_p(0x10004), None) == E["ALIGN"]
    for probe in (L.awq_probe_read, L.awq_probe_write):
        assert probe(None, 1024, None) == E["NULL"]
        assert probe(P, 0, None) == E["SHAPE"]
        assert probe(P, 1000, None) == E["SHAPE"]          # not a multiple of 16
        assert probe(ctypes.c_void_p(0x10008), 1024, None) == E["ALIGN"]
    c = L.awq_probe_copy
    assert c(None, P, 1024, None) == E["NULL"] and c(P, None, 1024, None) == E["NULL"]
    assert c(P, P, 8, None) == E["SHAPE"]
    assert c(P, ctypes.c_void_p(0x10008), 1024, None) == E["ALIGN"]
    assert L.awq_probe_wall_clock_khz(0, None) == E["NULL"]
