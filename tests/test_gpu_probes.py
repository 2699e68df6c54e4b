"""GPU checks of the measured-ceiling probes (moe_probe_stream_copy,
moe_probe_stream_read, moe_probe_mfma) through the C ABI: the copy is
byte-exact on sizes that end inside a block, the read covers every word
exactly once (the XOR of its per-wave outputs is the XOR of the input's
words), and the MFMA loop runs and writes one finite value per wave."""
import numpy as np
import pytest
import torch

import mixture_experts_ffn_top_amd as m
from tests.gpu_util import say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096 * 16 + 48, (1 << 24) + 16 * 1023])
def test_stream_copy_is_exact(nbytes):
    say(f"stream copy {nbytes} bytes")
    g = torch.Generator().manual_seed(nbytes)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, generator=g).cuda()
    dst = torch.zeros(nbytes + 64, dtype=torch.uint8, device="cuda")
    m.probe_stream_copy(src, dst[:nbytes])
    torch.cuda.synchronize()
    assert torch.equal(dst[:nbytes].cpu(), src.cpu())
    assert int(dst[nbytes:].count_nonzero()) == 0   # nothing written past the end


@pytest.mark.parametrize("nbytes,out_len", [(16, 4), (32768 + 48, 64), ((1 << 24) + 16 * 1023, 16384),
                                            ((1 << 24) + 16 * 1023, 8)])
def test_stream_read_covers_every_word_once(nbytes, out_len):
    say(f"stream read {nbytes} bytes, {out_len} outputs")
    g = torch.Generator().manual_seed(nbytes + out_len)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, generator=g)
    want = int(np.bitwise_xor.reduce(src.numpy().view(np.uint32)))
    out = torch.zeros(out_len + 8, dtype=torch.int32, device="cuda")
    m.probe_stream_read(src.cuda(), out[:out_len])
    torch.cuda.synchronize()
    got = int(np.bitwise_xor.reduce(out[:out_len].cpu().numpy().view(np.uint32)))
    assert got == want
    assert int(out[out_len:].count_nonzero()) == 0   # nothing written past out_len


@pytest.mark.parametrize("kind", [0, 1])
def test_mfma_probe_runs(kind):
    say(f"mfma probe kind {kind}")
    wg = 3
    out = torch.full((wg * 8,), float("nan"), dtype=torch.float32, device="cuda")
    flops = m.probe_mfma(kind, wg, 5, out)
    torch.cuda.synchronize()
    assert flops == wg * 8 * 5 * 8 * (32768 if kind == 0 else 131072)
    assert bool(torch.isfinite(out).all())
