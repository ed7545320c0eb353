"""The allocation-free statistics entry point (awq_act_stats_noalloc), through the C ABI,
against awq_act_stats on the same inputs: bit for bit, on two calls in a row (the second
on a smaller input, so that it runs over what the first left in the static array), and its
host-side rejection of shapes whose partials do not fit that array."""
import ctypes
import os

import numpy as np
import pytest
import torch

import weight_only_quantization_act_amd as awq
from synth import CONFIGS, make_layer, small_spec
from tests.gpu_util import dev, host, requires_gpu, say

SCRATCH = awq.AWQ_NOALLOC_SCRATCH_BYTES


def _fn():
    return awq.lib().awq_act_stats_noalloc


def test_noalloc_host_checks():
    """Checks that run before any HIP call: NULL pointers, invalid sizes, and partials that
    would need more than the static array (2^21 channels, 512 tokens: 16 MiB)."""
    f = _fn()
    P = ctypes.c_void_p(0x10000)
    assert f(None, 64, 64, P, None) == 1                        # AWQ_E_NULL
    assert f(P, 0, 64, P, None) == 2                            # AWQ_E_SHAPE
    assert awq.awq_act_stats_workspace_bytes(512, 1 << 21) > SCRATCH
    assert f(P, 512, 1 << 21, P, None) == 5                     # AWQ_E_WORKSPACE
    assert f(ctypes.c_void_p(0x10002), 64, 64, P, None) == 9    # AWQ_E_ALIGN
    # every shape of the workloads fits
    for N, K in [(256, 512), (4096, 4096), (16384, 11008), (65536, 8192), (32768, 5120)]:
        assert awq.awq_act_stats_workspace_bytes(N, K) <= SCRATCH
    header = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                          "include", "awq_act.h")
    assert "#define AWQ_NOALLOC_SCRATCH_BYTES (8u << 20)" in open(header).read()
    assert SCRATCH == 8 << 20


def _noalloc(X: torch.Tensor) -> torch.Tensor:
    N, K = X.shape
    a = torch.full((max(K, 1),), float("nan"), dtype=torch.float32, device=X.device)
    st = _fn()(X.data_ptr(), N, K, a.data_ptr(),
               torch.cuda.current_stream().cuda_stream)
    assert st == 0, awq.status_str(st)
    return a[:K]


@pytest.mark.gpu
@requires_gpu
def test_noalloc_matches_workspace_entry_twice():
    """A large input, then a smaller and ragged one (channels not a multiple of 8, so the
    scalar-load path): each equal to awq_act_stats bit for bit."""
    big = make_layer(CONFIGS["c2"][0]).X
    small = make_layer(small_spec("na", 8, 1001, 300, x_dist="t4", outlier_count=10)).X
    for name, X in (("4096x4096", big), ("300x1001", small)):
        say(f"noalloc stats {name}")
        Xd = dev(X)
        got = _noalloc(Xd)
        want = awq.awq_act_stats(Xd)
        torch.cuda.synchronize()
        assert np.array_equal(host(got).view(np.uint32), host(want).view(np.uint32)), name


@pytest.mark.gpu
@requires_gpu
def test_noalloc_empty_channels_and_one_token():
    Xd = torch.empty((5, 0), dtype=torch.float16, device="cuda")
    a = torch.empty(1, dtype=torch.float32, device="cuda")
    assert _fn()(Xd.data_ptr() or a.data_ptr(), 5, 0, a.data_ptr(), None) == 0
    X1 = dev(make_layer(small_spec("n1", 8, 256, 1)).X)
    got = _noalloc(X1)
    torch.cuda.synchronize()
    assert np.array_equal(host(got).view(np.uint32), host(awq.awq_act_stats(X1)).view(np.uint32))
