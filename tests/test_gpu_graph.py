"""The whole layer captured in a HIP graph and replayed (torch.cuda.graph on
ROCm records hipGraph nodes).  The library's calls allocate nothing, set no
memory with hipMemset and never synchronise, so a forward pass can be
captured once and replayed; the tests replay it several times with eager work
on other inputs in between and compare every replay bit for bit with the
eager result of the captured input (the kernels are deterministic)."""
import pytest
import torch

import synth
from tests.gpu_util import say

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def moe():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import mixture_experts_ffn_top_amd as m
    m.lib()
    return m


@pytest.mark.parametrize("cid,changes", [
    (1, {}),                                                     # softmax gate, bf16
    (2, {"T": 512}),                                             # Mixtral dims, split-K down tail round
    (3, {"T": 512}),                                             # sink router, shared experts
    (4, {"T": 300}),                                             # interleaved swigluoai with biases
    (5, {"T": 256, "E": 16, "H": 1024, "D": 512}),               # fp8 block-scaled
    (6, {"T": 256, "E": 16, "H": 1024, "D": 512}),               # MXFP4 x MXFP8
    (7, {"T": 64, "E": 16, "H": 1024, "D": 512}),                # MXFP4 weights x bf16 activations (W4A16)
    (8, {}),                                                     # single-launch FFN (decode)
    (9, {"T": 64, "E": 16, "H": 1024, "D": 512}),                # single-launch FFN, MXFP4 x MXFP8
    (10, {"T": 64, "E": 16, "H": 1024, "D": 512}),               # single-launch FFN, MXFP4 x bf16
    # one expert-parallel rank's share, row buffers sized to the rows it receives
    (2, {"T": 512, "expert_slice": (2, 3)}),
    # shared experts on their own stream, forked after the per-token quantise (fp8, W4A8)
    (5, {"T": 256, "E": 8, "k": 3, "s": 1, "n_shared": 1, "H": 512, "D": 256, "shared_dim": 384}),
    (6, {"T": 256, "E": 8, "k": 2, "s": 2, "n_shared": 2, "H": 512, "D": 256, "shared_dim": 384}),
])
def test_layer_replays_in_a_graph(moe, cid, changes):
    changes = dict(changes)
    sl = changes.pop("expert_slice", None)
    cfg = synth.scaled(synth.get_config(cid), **changes)
    say(f"[graph] cfg={cid} {changes} slice={sl}")
    inp = synth.make_inputs(cfg, DEV)
    x = inp["x"]
    x_other = (inp["x"].float() * -0.5 + 0.25).to(inp["x"].dtype)
    if sl is None:
        layer = moe.MoELayer(cfg, inp)
    else:
        layer = moe.MoELayer(cfg, inp, expert_slice=sl, max_rows=0)
        layer.reserve_rows(max(layer.local_rows(x), layer.local_rows(x_other)))
    want = layer.forward(x)["y"].clone()
    other = layer.forward(x_other)["y"].clone()
    torch.cuda.synchronize()
    assert not torch.equal(want, other)

    # warm up on a side stream, then capture one forward pass of x
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            layer.forward(x)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        y_static = layer.forward(x)["y"]
    torch.cuda.synchronize()

    for rep in range(3):
        # eager work on the other input writes the same output buffer
        got_other = layer.forward(x_other)["y"].clone()
        torch.cuda.synchronize()
        assert torch.equal(got_other, other), f"eager pass {rep} differs"
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(y_static, want), f"replay {rep} differs from the eager result"
    graph.reset()
