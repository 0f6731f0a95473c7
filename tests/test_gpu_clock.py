"""pca_clock_stamp on the GPU: two stamps around about 50 ms of attention
launches see every XCD of the chip, and each XCD's average shader clock lies
between the chip's lowest and highest DPM clocks (0.5 - 2.4 GHz, a margin
either way for counter granularity)."""
import pytest
import torch

import prefill_causal_attention_amd as pca
import workloads

from _gpu_helpers import dev, require_gpu, say

pytestmark = pytest.mark.gpu


def test_clock_stamp_gives_every_xcd_a_plausible_clock():
    require_gpu()
    w = workloads.custom(31, [4096], 32, 8, 128)
    buf, qo, ko, vo = workloads.qkv_inputs(w)
    d = dev(buf)
    o = torch.empty((4096, 4096), dtype=torch.bfloat16, device="cuda")
    a = torch.zeros(pca.CLOCK_STAMP_WORDS, dtype=torch.int64, device="cuda")
    b = torch.zeros_like(a)
    say("clock_stamp around 400 attention launches (s=4096, GQA 32/8)")
    pca.clock_stamp(a)
    for _ in range(400):
        pca.prefill_attention(d[:, :4096], d[:, ko:ko + 1024], d[:, vo:vo + 1024], o, 32, 8, 128)
    pca.clock_stamp(b)
    torch.cuda.synchronize()
    per_xcd = pca.shader_clock_mhz(a.cpu().numpy(), b.cpu().numpy())
    say(f"shader clock per XCD (MHz): {per_xcd}")
    assert sorted(per_xcd) == list(range(8)), per_xcd
    assert all(400.0 < f < 2600.0 for f in per_xcd.values()), per_xcd
