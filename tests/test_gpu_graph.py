"""The whole per-layer path captured in a HIP graph and replayed.

The library enqueues only kernel launches on the caller's stream (no allocation, copy,
memset or synchronisation inside a call; the alpha grid travels in kernel arguments), so a
layer can be captured once and replayed, which removes the launch overhead that dominates
small layers.  Each replay is compared bit for bit with the eager result, with eager work
and synchronisations of the program between the replays.
"""
import numpy as np
import pytest
import torch

import weight_only_quantization_act_amd as awq
from synth import CONFIGS, alpha_grid, make_layer, small_spec
from tests.gpu_util import dev, host, requires_gpu, say

pytestmark = [pytest.mark.gpu, requires_gpu]

KEYS = ("a", "losses", "best", "s", "codes", "scales", "zeros")


def _snapshot(res):
    return {k: host(res[k]).copy() for k in KEYS}


def _same(x, y):
    return np.array_equal(np.ascontiguousarray(x).view(np.uint8),
                          np.ascontiguousarray(y).view(np.uint8))


@pytest.mark.parametrize("case", ["c1", "gram"])
def test_layer_graph_replays_match_eager(case):
    if case == "c1":
        spec = CONFIGS["c1"][0]
    else:  # a shape that takes the G form of the loss
        spec = small_spec("g", 300, 256, 3000, w_bit=4, group_size=128, zero_point=1, seed=5)
    L = make_layer(spec)
    M, K, N = spec.out_features, spec.in_features, spec.n_tokens
    cfg = awq.qconfig(spec.w_bit, spec.group_size, spec.zero_point)
    alphas = alpha_grid(20)
    say(f"graph {case}: {M}x{K}x{N}, form {awq.awq_loss_form(M, K, N, 20)}")
    Wd, Xd = dev(L.W), dev(L.X)
    ws_s = torch.empty(awq.awq_workspace_bytes(M, K, N, cfg, 20, 0), dtype=torch.uint8,
                       device="cuda")
    ws_a = torch.empty(awq.awq_act_stats_workspace_bytes(N, K), dtype=torch.uint8, device="cuda")

    def layer():
        return awq.quantize_layer(Wd, Xd, alphas, cfg, search_workspace=ws_s, stats_workspace=ws_a)

    eager = _snapshot(layer())
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            layer()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = layer()

    # other eager work of the program between replays: a different layer through the same
    # entry points (its own buffers)
    L2 = make_layer(small_spec("o", 64, K, 200, seed=9))
    W2, X2 = dev(L2.W), dev(L2.X)
    for rep in range(4):
        g.replay()
        torch.cuda.synchronize()
        got = _snapshot(out)
        for k in KEYS:
            assert _same(got[k], eager[k]), (case, rep, k)
        awq.quantize_layer(W2, X2, alphas, cfg)
        torch.cuda.synchronize()
    del g
