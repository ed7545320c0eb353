"""The measurement probes run through the C ABI and return sane clocks (they compute nothing
the path uses; these checks guard the figures the benchmark derives from them)."""
import pytest
import torch

import weight_only_quantization_act_amd as awq

pytestmark = pytest.mark.gpu


def test_mfma_and_lds_probe_clocks():
    for probe in (awq.awq_probe_mfma, awq.awq_probe_lds):
        clocks = probe(8, 64)
        torch.cuda.synchronize()
        t = clocks.cpu()
        assert t.shape == (8, 2)
        assert bool((t[:, 0] > 0).all()) and bool((t[:, 1] > 0).all())
        # shader clock against the real-time counter: a plausible GPU clock
        wall_ghz = awq.awq_probe_wall_clock_khz(0) * 1e-6
        assert 0.001 < wall_ghz < 1.0, wall_ghz
        ghz = (t[:, 0].double() / t[:, 1].double() * wall_ghz).median().item()
        assert 0.3 < ghz < 3.5, ghz


def test_stream_probes_write_read_copy():
    buf = torch.zeros(1 << 20, dtype=torch.uint8, device="cuda")
    awq.awq_probe_write(buf)
    awq.awq_probe_read(buf)
    torch.cuda.synchronize()
    # the write probe stores fp16 ones everywhere
    assert bool((buf.view(torch.float16) == 1.0).all())
    # the copy probe moves every byte, including a ragged tail past the last full batch
    src = torch.randint(0, 256, ((1 << 20) + 48,), dtype=torch.uint8, device="cuda")
    dst = torch.zeros_like(src)
    awq.awq_probe_copy(src, dst)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)
