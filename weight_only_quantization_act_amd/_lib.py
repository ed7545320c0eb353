"""ctypes binding of libawq_act.so: argument marshalling only.

Every step of the path runs in the library's HIP kernels; this module checks tensor
dtypes, devices and contiguity, hands raw device pointers and the current HIP stream to
the C ABI, and turns non-zero status codes into exceptions.  There is no fallback: if
the library is missing, every call raises.
"""
from __future__ import annotations

import contextlib
import ctypes
import functools
import os
from typing import Optional, Sequence

import torch  # imported first so that the library binds to torch's HIP runtime

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libawq_act.so")

AWQ_OK = 0
AWQ_E_HIP = 7
AWQ_W_NONFINITE = 8
AWQ_E_ALIGN = 9
AWQ_W_SCALE_OVERFLOW = 10
AWQ_MAX_ALPHA = 64


class AwqError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_str(status)}")


class awq_qconfig(ctypes.Structure):
    _fields_ = [("w_bit", ctypes.c_int32), ("group_size", ctypes.c_int32),
                ("zero_point", ctypes.c_int32)]


_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_sz = ctypes.c_size_t
_cfgp = ctypes.POINTER(awq_qconfig)

_SIGNATURES = {
    "awq_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "awq_act_stats_workspace_bytes": (_sz, [_i64, _i64]),
    "awq_act_stats": (ctypes.c_int, [_vp, _i64, _i64, _vp, _vp, _sz, _vp]),
    "awq_act_stats_noalloc": (ctypes.c_int, [_vp, _i64, _i64, _vp, _vp]),
    "awq_workspace_bytes": (_sz, [_i64, _i64, _i64, _cfgp, _i32, _i32]),
    "awq_loss_form": (ctypes.c_int, [_i64, _i64, _i64, _i32]),
    "awq_search_scales": (ctypes.c_int, [_vp, _vp, _vp, _i64, _i64, _i64, _cfgp, _vp, _i32,
                                         _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "awq_fake_quant_delta": (ctypes.c_int, [_vp, _vp, _i64, _i64, _cfgp, _vp, _vp]),
    "awq_quantize_pack": (ctypes.c_int, [_vp, _vp, _i64, _i64, _cfgp, _vp, _vp, _vp, _vp]),
    "awq_set_profile_events": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp]),
    "awq_set_profile_pass_events": (ctypes.c_int, [ctypes.POINTER(_vp), _i32]),
    "awq_set_stats_profile_events": (ctypes.c_int, [_vp, _vp]),
    "awq_act_stats_ex_workspace_bytes": (_sz, [_i64, _i64, _i32, _i64]),
    "awq_act_stats_ex": (ctypes.c_int, [_vp, _i64, _i64, _i32, _i64, ctypes.c_double, _vp, _vp,
                                        _sz, _vp]),
    "awq_search_scale_table": (ctypes.c_int, [_vp, _vp, _vp, _i32, _i64, _i64, _i64, _cfgp, _vp,
                                              _vp, _vp, _vp, _vp, _sz, _vp]),
    "awq_threshold_scales": (ctypes.c_int, [_vp, _i64, ctypes.c_double, ctypes.c_float, _vp,
                                            _vp]),
    "awq_hadamard_rotate": (ctypes.c_int, [_vp, _i64, _i64, _i32, _vp, _vp]),
    "awq_w4a16_matmul": (ctypes.c_int, [_vp, _vp, _i64, _vp, _vp, _vp, _i64, _i64, _cfgp, _vp,
                                        _vp, _sz, _vp]),
    "awq_w4a16_workspace_bytes": (_sz, [_i64, _i64]),
    "awq_clip_workspace_bytes": (_sz, [_i64, _i64, _i64, _cfgp]),
    "awq_clip_search": (ctypes.c_int, [_vp, _vp, _vp, _i64, _i64, _i64, _cfgp, _vp, _i32, _vp,
                                       _vp, _vp, _vp, _sz, _vp]),
    "awq_quantize_pack_clipped": (ctypes.c_int, [_vp, _vp, _vp, _i64, _i64, _cfgp, _vp, _vp, _vp,
                                                 _vp]),
    "awq_quantize_pack_checked": (ctypes.c_int, [_vp, _vp, _vp, _i64, _i64, _cfgp, _vp, _vp, _vp,
                                                 _vp, _vp]),
    "awq_probe_mfma": (ctypes.c_int, [_i32, _i32, _vp, _vp]),
    "awq_probe_lds": (ctypes.c_int, [_i32, _i32, _vp, _vp]),
    "awq_probe_read": (ctypes.c_int, [_vp, _i64, _vp]),
    "awq_probe_write": (ctypes.c_int, [_vp, _i64, _vp]),
    "awq_probe_copy": (ctypes.c_int, [_vp, _vp, _i64, _vp]),
    "awq_probe_wall_clock_khz": (ctypes.c_int, [_i32, ctypes.POINTER(_i32)]),
}

AWQ_STAT_MEAN_ABS, AWQ_STAT_MAX_ABS, AWQ_STAT_RMS_RATIO, AWQ_STAT_EMA_MEAN = 0, 1, 2, 3

_LIB: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """Load libawq_act.so (built in-tree by weight_only_quantization_act_amd.build)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m weight_only_quantization_act_amd.build` (no fallback exists)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = L
    return _LIB


def status_str(status: int) -> str:
    return lib().awq_status_str(int(status)).decode()


def _check(status: int, where: str):
    if status != AWQ_OK:
        raise AwqError(status, where)


def qconfig(w_bit: int = 4, group_size: int = 128, zero_point: int = 1) -> awq_qconfig:
    return awq_qconfig(int(w_bit), int(group_size), int(zero_point))


def _stream_ptr(stream=None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def _on_stream(fn):
    """Run the wrapper with `stream` (when given) as torch's current stream, so that the
    outputs and temporary workspaces it allocates belong to the stream the kernels are
    enqueued on: the caching allocator then never hands a block that those kernels may
    still use to work on another stream."""
    @functools.wraps(fn)
    def wrapper(*args, stream=None, **kwargs):
        ctx = torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()
        with ctx:
            return fn(*args, stream=stream, **kwargs)
    return wrapper


def _dev(t: torch.Tensor, dtype: torch.dtype, name: str, shape=None) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device (HIP) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    return t


def _ptr(t: torch.Tensor) -> int:
    return int(t.data_ptr())


def _buf(nbytes: int, device) -> torch.Tensor:
    # at least 256 bytes so that a zero-size request still yields a valid device pointer
    return torch.empty(max(256, int(nbytes)), dtype=torch.uint8, device=device)


# ---------------------------------------------------------------------------------------
def awq_act_stats_workspace_bytes(n_tokens: int, in_features: int) -> int:
    return int(lib().awq_act_stats_workspace_bytes(n_tokens, in_features))


def awq_act_stats_ex_workspace_bytes(n_tokens: int, in_features: int, statistic: int,
                                     batch_tokens: int = 0) -> int:
    return int(lib().awq_act_stats_ex_workspace_bytes(n_tokens, in_features, statistic,
                                                      batch_tokens))


@_on_stream
def awq_act_stats(X: torch.Tensor, out: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """a_i = mean over tokens of |X[t, i]| for X fp16 [N, K]  ->  fp32 [K] (device)."""
    _dev(X, torch.float16, "X")
    if X.dim() != 2:
        raise ValueError("X must be 2-D [n_tokens, in_features]")
    N, K = X.shape
    a = out if out is not None else torch.empty(max(K, 1), dtype=torch.float32, device=X.device)[:K]
    need = awq_act_stats_workspace_bytes(N, K)
    ws = workspace if workspace is not None else _buf(need, X.device)
    st = lib().awq_act_stats(_ptr(X), N, K, _ptr(a) if K else _ptr(ws), _ptr(ws),
                             ws.numel() * ws.element_size(), _stream_ptr(stream))
    _check(st, "awq_act_stats")
    return a


AWQ_NOALLOC_SCRATCH_BYTES = 8 << 20


@_on_stream
def awq_act_stats_noalloc(X: torch.Tensor, out: torch.Tensor, stream=None) -> torch.Tensor:
    """awq_act_stats with the library's static device scratch instead of a workspace (for
    callers that cannot allocate: the output is the caller's, nothing is allocated here).
    Calls that overlap on one GPU race on that scratch."""
    _dev(X, torch.float16, "X")
    if X.dim() != 2:
        raise ValueError("X must be 2-D [n_tokens, in_features]")
    N, K = X.shape
    _dev(out, torch.float32, "out")
    if out.numel() < max(K, 1):
        raise ValueError("out must hold in_features floats")
    st = lib().awq_act_stats_noalloc(_ptr(X) if X.numel() else _ptr(out), N, K, _ptr(out),
                                     _stream_ptr(stream))
    _check(st, "awq_act_stats_noalloc")
    return out[:K]


def awq_workspace_bytes(out_features: int, in_features: int, n_tokens: int, cfg: awq_qconfig,
                        n_alpha: int, alpha_batch: int = 0) -> int:
    return int(lib().awq_workspace_bytes(out_features, in_features, n_tokens,
                                         ctypes.byref(cfg), n_alpha, alpha_batch))


AWQ_LOSS_DIRECT, AWQ_LOSS_GRAM = 0, 1


def awq_loss_form(out_features: int, in_features: int, n_tokens: int, n_alpha: int) -> int:
    """AWQ_LOSS_DIRECT or AWQ_LOSS_GRAM: the form awq_search_scales takes for these sizes."""
    return int(lib().awq_loss_form(out_features, in_features, n_tokens, n_alpha))


@_on_stream
def awq_search_scales(W: torch.Tensor, X: torch.Tensor, a: torch.Tensor,
                      alphas: Sequence[float], cfg: awq_qconfig,
                      workspace: Optional[torch.Tensor] = None, alpha_batch: int = 0,
                      stream=None):
    """Grid search over alpha.  Returns device tensors (s [K] fp32, losses [n_alpha] fp64,
    best [1] int32, status [1] int32); nothing is synchronised.  Without a workspace one
    is allocated for `alpha_batch` grid points a pass (0: the library's choice, sized for
    the last-level cache); with one, its size sets the points a pass."""
    _dev(W, torch.float16, "W")
    _dev(X, torch.float16, "X")
    M, K = W.shape
    N = X.shape[0]
    if X.dim() != 2 or X.shape[1] != K:
        raise ValueError("X must be [n_tokens, in_features] with W's in_features")
    _dev(a, torch.float32, "a", (K,))
    al = (ctypes.c_float * max(1, len(alphas)))(*[float(v) for v in alphas])
    n_alpha = len(alphas)
    dev = W.device
    s = torch.empty(max(K, 1), dtype=torch.float32, device=dev)
    losses = torch.empty(max(n_alpha, 1), dtype=torch.float64, device=dev)
    best = torch.empty(1, dtype=torch.int32, device=dev)
    status = torch.empty(1, dtype=torch.int32, device=dev)
    if workspace is None:
        workspace = _buf(awq_workspace_bytes(M, K, N, cfg, n_alpha, alpha_batch), dev)
    a_ptr = _ptr(a) if K else _ptr(s)
    st = lib().awq_search_scales(_ptr(W) if W.numel() else _ptr(workspace),
                                 _ptr(X) if X.numel() else _ptr(workspace), a_ptr, M, K, N,
                                 ctypes.byref(cfg), al, n_alpha, _ptr(s), _ptr(losses),
                                 _ptr(best), _ptr(status), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(),
                                 _stream_ptr(stream))
    _check(st, "awq_search_scales")
    return {"s": s[:K], "losses": losses[:n_alpha], "best": best, "status": status}


@_on_stream
def awq_fake_quant_delta(W: torch.Tensor, s: torch.Tensor, cfg: awq_qconfig,
                         stream=None) -> torch.Tensor:
    """fp16 W - Q(W diag(s)) diag(s)^-1 for one scale vector."""
    _dev(W, torch.float16, "W")
    M, K = W.shape
    _dev(s, torch.float32, "s", (K,))
    dW = torch.empty_like(W)
    if W.numel() == 0:
        return dW
    st = lib().awq_fake_quant_delta(_ptr(W), _ptr(s), M, K, ctypes.byref(cfg), _ptr(dW),
                                    _stream_ptr(stream))
    _check(st, "awq_fake_quant_delta")
    return dW


@_on_stream
def awq_quantize_pack(W: torch.Tensor, s: torch.Tensor, cfg: awq_qconfig, stream=None):
    """Packed codes uint8 [M, K/2], fp16 scales [M, K/g], fp16 zeros [M, K/g]."""
    _dev(W, torch.float16, "W")
    M, K = W.shape
    _dev(s, torch.float32, "s", (K,))
    g = cfg.group_size
    codes = torch.empty((M, K // 2), dtype=torch.uint8, device=W.device)
    scales = torch.empty((M, K // g if g else 0), dtype=torch.float16, device=W.device)
    zeros = torch.empty_like(scales)
    if W.numel() == 0:
        return codes, scales, zeros
    st = lib().awq_quantize_pack(_ptr(W), _ptr(s), M, K, ctypes.byref(cfg), _ptr(codes),
                                 _ptr(scales), _ptr(zeros), _stream_ptr(stream))
    _check(st, "awq_quantize_pack")
    return codes, scales, zeros


@_on_stream
def awq_quantize_pack_checked(W: torch.Tensor, s: torch.Tensor, cfg: awq_qconfig,
                              clip: Optional[torch.Tensor] = None, stream=None):
    """awq_quantize_pack (or its clipped form) with the device status word: returns codes,
    scales, zeros and status int32 [1] (AWQ_OK, or AWQ_W_SCALE_OVERFLOW when a stored
    fp16 step is not finite)."""
    _dev(W, torch.float16, "W")
    M, K = W.shape
    _dev(s, torch.float32, "s", (K,))
    g = cfg.group_size
    dev = W.device
    if clip is not None:
        _dev(clip, torch.float32, "clip", (M, K // g))
    codes = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((M, K // g), dtype=torch.float16, device=dev)
    zeros = torch.empty_like(scales)
    status = torch.empty(1, dtype=torch.int32, device=dev)
    if W.numel() == 0:  # nothing to pack; the call still writes the status word
        dummy = _ptr(_buf(256, dev))
        ptrs = (dummy, dummy, None, dummy, dummy, dummy)
    else:
        ptrs = (_ptr(W), _ptr(s), _ptr(clip) if clip is not None else None, _ptr(codes),
                _ptr(scales), _ptr(zeros))
    pw, ps, pcl, pc, psc, pz = ptrs
    st = lib().awq_quantize_pack_checked(pw, ps, pcl, M, K, ctypes.byref(cfg), pc, psc, pz,
                                         _ptr(status), _stream_ptr(stream))
    _check(st, "awq_quantize_pack_checked")
    return codes, scales, zeros, status


def awq_set_profile_events(gemm_start=None, gemm_stop=None, fq_start=None, fq_stop=None,
                           gram_start=None, gram_stop=None):
    """Arm the one-shot per-thread event hook of the next awq_search_scales call.
    Arguments are hipEvent_t handles (int), or objects exposing one as `.handle`."""
    def h(e):
        if e is None:
            return None
        return int(e) if isinstance(e, int) else int(e.handle)
    _check(lib().awq_set_profile_events(h(gemm_start), h(gemm_stop), h(fq_start), h(fq_stop),
                                        h(gram_start), h(gram_stop)),
           "awq_set_profile_events")


def awq_set_profile_pass_events(events) -> None:
    """Arm the one-shot per-thread per-pass hook of the next search: `events` is a list of
    4 n_pass hipEvent_t handles (int, None, or objects with `.handle`), for pass p [4p],
    [4p + 1] around its fake quantisation and [4p + 2], [4p + 3] around its loss product.
    An empty list clears the hook."""
    hs = [None if e is None else (int(e) if isinstance(e, int) else int(e.handle))
          for e in events]
    if len(hs) % 4:
        raise ValueError("awq_set_profile_pass_events: 4 events per pass")
    arr = (_vp * max(1, len(hs)))(*hs)
    _check(lib().awq_set_profile_pass_events(arr, len(hs) // 4), "awq_set_profile_pass_events")


def awq_set_stats_profile_events(pass_start=None, pass_stop=None):
    """Arm the one-shot per-thread event hook of the next statistics call (events around
    its streaming pass over X).  Arguments as for awq_set_profile_events."""
    def h(e):
        if e is None:
            return None
        return int(e) if isinstance(e, int) else int(e.handle)
    _check(lib().awq_set_stats_profile_events(h(pass_start), h(pass_stop)),
           "awq_set_stats_profile_events")


@_on_stream
def awq_probe_mfma(blocks: int, iters: int, stream=None) -> torch.Tensor:
    """Enqueue the matrix-core probe; returns its per-block clock ticks (device int64
    [blocks][2]: shader clock, 100 MHz real time)."""
    clocks = torch.zeros((int(blocks), 2), dtype=torch.int64, device="cuda")
    _check(lib().awq_probe_mfma(int(blocks), int(iters), _ptr(clocks), _stream_ptr(stream)),
           "awq_probe_mfma")
    return clocks


@_on_stream
def awq_probe_lds(blocks: int, iters: int, stream=None) -> torch.Tensor:
    """Enqueue the LDS-read probe; per-block clock ticks as for awq_probe_mfma."""
    clocks = torch.zeros((int(blocks), 2), dtype=torch.int64, device="cuda")
    _check(lib().awq_probe_lds(int(blocks), int(iters), _ptr(clocks), _stream_ptr(stream)),
           "awq_probe_lds")
    return clocks


def awq_probe_read(src: torch.Tensor, stream=None):
    """Enqueue one streaming read of the whole (contiguous, device) tensor."""
    if not (isinstance(src, torch.Tensor) and src.is_cuda and src.is_contiguous()):
        raise ValueError("src must be a contiguous device tensor")
    _check(lib().awq_probe_read(_ptr(src), src.numel() * src.element_size(), _stream_ptr(stream)),
           "awq_probe_read")


def awq_probe_write(dst: torch.Tensor, stream=None):
    """Enqueue one streaming write over the whole (contiguous, device) tensor."""
    if not (isinstance(dst, torch.Tensor) and dst.is_cuda and dst.is_contiguous()):
        raise ValueError("dst must be a contiguous device tensor")
    _check(lib().awq_probe_write(_ptr(dst), dst.numel() * dst.element_size(),
                                 _stream_ptr(stream)), "awq_probe_write")


def awq_probe_copy(src: torch.Tensor, dst: torch.Tensor, stream=None):
    """Enqueue one streaming copy of src into dst (contiguous device tensors, same size)."""
    for t in (src, dst):
        if not (isinstance(t, torch.Tensor) and t.is_cuda and t.is_contiguous()):
            raise ValueError("src and dst must be contiguous device tensors")
    nb = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nb:
        raise ValueError("src and dst differ in size")
    _check(lib().awq_probe_copy(_ptr(src), _ptr(dst), nb, _stream_ptr(stream)), "awq_probe_copy")


def awq_probe_wall_clock_khz(device: int = 0) -> int:
    """Frequency of the device's real-time counter in kHz."""
    v = ctypes.c_int32(0)
    _check(lib().awq_probe_wall_clock_khz(int(device), ctypes.byref(v)), "awq_probe_wall_clock_khz")
    return int(v.value)


@_on_stream
def quantize_layer(W: torch.Tensor, X: torch.Tensor, alphas: Sequence[float],
                   cfg: awq_qconfig, search_workspace: Optional[torch.Tensor] = None,
                   stats_workspace: Optional[torch.Tensor] = None, stream=None):
    """The whole per-layer path: statistics -> alpha search -> pack (all on device).
    The result holds the search's status word ("status": AWQ_OK or AWQ_W_NONFINITE) and
    the pack's ("pack_status": AWQ_OK or AWQ_W_SCALE_OVERFLOW)."""
    a = awq_act_stats(X, workspace=stats_workspace, stream=stream)
    res = awq_search_scales(W, X, a, alphas, cfg, workspace=search_workspace, stream=stream)
    codes, scales, zeros, pst = awq_quantize_pack_checked(W, res["s"], cfg, stream=stream)
    res.update({"a": a, "codes": codes, "scales": scales, "zeros": zeros, "pack_status": pst})
    return res


@_on_stream
def awq_act_stats_ex(X: torch.Tensor, statistic: int, batch_tokens: int = 0, momentum: float = 0.9,
                     stream=None) -> torch.Tensor:
    """Per-channel statistic of X fp16 [N, K] (see AWQ_STAT_*) -> fp32 [K]."""
    _dev(X, torch.float16, "X")
    N, K = X.shape
    a = torch.empty(max(K, 1), dtype=torch.float32, device=X.device)
    need = awq_act_stats_ex_workspace_bytes(N, K, statistic, batch_tokens)
    ws = _buf(need, X.device)
    st = lib().awq_act_stats_ex(_ptr(X), N, K, statistic, batch_tokens, float(momentum), _ptr(a),
                                _ptr(ws), ws.numel(), _stream_ptr(stream))
    _check(st, "awq_act_stats_ex")
    return a[:K]


@_on_stream
def awq_search_scale_table(W: torch.Tensor, X: torch.Tensor, s_table: torch.Tensor,
                           cfg: awq_qconfig, workspace: Optional[torch.Tensor] = None,
                           stream=None):
    """The search over explicit candidate scales s_table fp32 [n_cand, K]."""
    _dev(W, torch.float16, "W")
    _dev(X, torch.float16, "X")
    M, K = W.shape
    N = X.shape[0]
    _dev(s_table, torch.float32, "s_table")
    n = s_table.shape[0]
    if X.dim() != 2 or X.shape[1] != K:
        raise ValueError("X must be [n_tokens, in_features] with W's in_features")
    if s_table.dim() != 2 or s_table.shape[1] != K:
        raise ValueError("s_table must be [n_cand, in_features]")
    dev = W.device
    s = torch.empty(max(K, 1), dtype=torch.float32, device=dev)
    losses = torch.empty(max(n, 1), dtype=torch.float64, device=dev)
    best = torch.empty(1, dtype=torch.int32, device=dev)
    status = torch.empty(1, dtype=torch.int32, device=dev)
    if workspace is None:
        workspace = _buf(awq_workspace_bytes(M, K, N, cfg, n, 0), dev)
    st = lib().awq_search_scale_table(_ptr(W) if W.numel() else _ptr(workspace), _ptr(X),
                                      _ptr(s_table) if s_table.numel() else _ptr(s), n, M, K, N,
                                      ctypes.byref(cfg), _ptr(s), _ptr(losses), _ptr(best),
                                      _ptr(status), _ptr(workspace), workspace.numel(),
                                      _stream_ptr(stream))
    _check(st, "awq_search_scale_table")
    return {"s": s[:K], "losses": losses[:n], "best": best, "status": status}


@_on_stream
def awq_threshold_scales(a: torch.Tensor, percentile: float, factor: float,
                         stream=None) -> torch.Tensor:
    """s_i = factor where a_i exceeds the percentile threshold, else 1."""
    _dev(a, torch.float32, "a")
    K = a.shape[0]
    s = torch.empty_like(a)
    st = lib().awq_threshold_scales(_ptr(a), K, float(percentile), float(factor), _ptr(s),
                                    _stream_ptr(stream))
    _check(st, "awq_threshold_scales")
    return s


@_on_stream
def awq_hadamard_rotate(A: torch.Tensor, block: int, out: Optional[torch.Tensor] = None,
                        stream=None) -> torch.Tensor:
    """Rows of A fp16 [R, K] times blockwise H_block / sqrt(block)."""
    _dev(A, torch.float16, "A")
    R, K = A.shape
    out = torch.empty_like(A) if out is None else _dev(out, torch.float16, "out", (R, K))
    if A.numel() == 0:
        return out
    st = lib().awq_hadamard_rotate(_ptr(A), R, K, int(block), _ptr(out), _stream_ptr(stream))
    _check(st, "awq_hadamard_rotate")
    return out


def awq_w4a16_workspace_bytes(n_tokens: int, in_features: int) -> int:
    return int(lib().awq_w4a16_workspace_bytes(n_tokens, in_features))


@_on_stream
def awq_w4a16_matmul(x: torch.Tensor, codes: torch.Tensor, scales: torch.Tensor,
                     zeros: torch.Tensor, cfg: awq_qconfig, s: Optional[torch.Tensor] = None,
                     out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                     stream=None) -> torch.Tensor:
    """y [T, M] fp16 = x~ [T, K] times the dequantised packed weights (x~ = x / s if s).

    With s given and two or more tokens a workspace for the fold of x / s is allocated
    unless one is passed; an empty workspace keeps the vector kernel."""
    _dev(x, torch.float16, "x")
    if x.dim() != 2:
        raise ValueError("x must be 2-D [n_tokens, in_features]")
    T, K = x.shape
    M = codes.shape[0]
    _dev(codes, torch.uint8, "codes", (M, K // 2))
    _dev(scales, torch.float16, "scales", (M, K // cfg.group_size))
    _dev(zeros, torch.float16, "zeros", (M, K // cfg.group_size))
    if s is not None:
        _dev(s, torch.float32, "s", (K,))
    y = out if out is not None else torch.empty((T, M), dtype=torch.float16, device=x.device)
    _dev(y, torch.float16, "out", (T, M))
    if T == 0 or M == 0:
        return y
    dummy = _buf(256, x.device) if (K == 0) else None
    px = _ptr(x) if K else _ptr(dummy)
    pc = _ptr(codes) if K else _ptr(dummy)
    ps = _ptr(scales) if K else _ptr(dummy)
    pz = _ptr(zeros) if K else _ptr(dummy)
    if workspace is None and s is not None:
        need = awq_w4a16_workspace_bytes(T, K)
        workspace = _buf(need, x.device) if need else None
    pw, nw = None, 0
    if workspace is not None and workspace.numel() > 0:
        _dev(workspace, torch.uint8, "workspace")
        pw, nw = _ptr(workspace), workspace.numel()
    st = lib().awq_w4a16_matmul(px, _ptr(s) if (s is not None and K) else None, T, pc, ps, pz,
                                M, K, ctypes.byref(cfg), _ptr(y), pw, nw, _stream_ptr(stream))
    _check(st, "awq_w4a16_matmul")
    return y


def awq_clip_workspace_bytes(out_features: int, in_features: int, n_tokens: int,
                             cfg: awq_qconfig) -> int:
    return int(lib().awq_clip_workspace_bytes(out_features, in_features, n_tokens,
                                              ctypes.byref(cfg)))


@_on_stream
def awq_clip_search(W: torch.Tensor, X: torch.Tensor, s: torch.Tensor, ratios: Sequence[float],
                    cfg: awq_qconfig, want_errors: bool = False,
                    workspace: Optional[torch.Tensor] = None, stream=None):
    """Per (row, group) clip ratio after the scale search.  Returns device tensors
    clip [M, K/g] fp32, best [M, K/g] int32 and (if asked) errors [n, M, K/g] fp32."""
    _dev(W, torch.float16, "W")
    _dev(X, torch.float16, "X")
    M, K = W.shape
    N = X.shape[0]
    if X.dim() != 2 or X.shape[1] != K:
        raise ValueError("X must be [n_tokens, in_features] with W's in_features")
    _dev(s, torch.float32, "s", (K,))
    n = len(ratios)
    rl = (ctypes.c_float * max(1, n))(*[float(v) for v in ratios])
    ng = K // cfg.group_size
    dev = W.device
    clip = torch.empty((M, ng), dtype=torch.float32, device=dev)
    best = torch.empty((M, ng), dtype=torch.int32, device=dev)
    errors = torch.empty((n, M, ng), dtype=torch.float32, device=dev) if want_errors else None
    if workspace is None:
        workspace = _buf(awq_clip_workspace_bytes(M, K, N, cfg), dev)
    if M == 0 or K == 0:
        return {"clip": clip, "best": best, "errors": errors}
    st = lib().awq_clip_search(_ptr(W), _ptr(X), _ptr(s), M, K, N, ctypes.byref(cfg), rl, n,
                               _ptr(clip), _ptr(best), _ptr(errors) if want_errors else None,
                               _ptr(workspace), workspace.numel(), _stream_ptr(stream))
    _check(st, "awq_clip_search")
    return {"clip": clip, "best": best, "errors": errors}


@_on_stream
def awq_quantize_pack_clipped(W: torch.Tensor, s: torch.Tensor, clip: torch.Tensor,
                              cfg: awq_qconfig, stream=None):
    """awq_quantize_pack with per-(row, group) range ratios clip [M, K/g] fp32."""
    _dev(W, torch.float16, "W")
    M, K = W.shape
    _dev(s, torch.float32, "s", (K,))
    _dev(clip, torch.float32, "clip", (M, K // cfg.group_size))
    dev = W.device
    codes = torch.empty((M, K // 2), dtype=torch.uint8, device=dev)
    scales = torch.empty((M, K // cfg.group_size), dtype=torch.float16, device=dev)
    zeros = torch.empty((M, K // cfg.group_size), dtype=torch.float16, device=dev)
    if M == 0 or K == 0:
        return codes, scales, zeros
    st = lib().awq_quantize_pack_clipped(_ptr(W), _ptr(s), _ptr(clip), M, K, ctypes.byref(cfg),
                                         _ptr(codes), _ptr(scales), _ptr(zeros),
                                         _stream_ptr(stream))
    _check(st, "awq_quantize_pack_clipped")
    return codes, scales, zeros
