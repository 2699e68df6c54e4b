"""bench.py's algorithmic work per layer step, against per-config figures
worked out by hand from the workloads' tensor shapes: the FLOP of the grouped
FFN (6 R H D, R = T k), the bytes of the softmax router (x and W_gate read
once, indices and weights written) and of the combine (O read once, the slot
rows and weights read, y written in bf16)."""
import pytest

import bench
import synth


@pytest.mark.parametrize("cid,ffn_flop", [(1, 1.007e8), (2, 2.886e12), (3, 4.639e11), (4, 8.154e11),
                                           (5, 1.1545e13)])
def test_ffn_flops(cid, ffn_flop):
    w = bench.algorithmic_work(synth.get_config(cid))
    assert w["gate_up_flops"] + w["down_flops"] == pytest.approx(ffn_flop, rel=1e-3)
    assert w["gate_up_flops"] == 2 * w["down_flops"]


@pytest.mark.parametrize("cid,mb", [(1, 0.0379), (2, 33.7), (4, 23.9)])
def test_softmax_router_bytes(cid, mb):
    assert bench.algorithmic_work(synth.get_config(cid))["route_bytes"] / 1e6 == pytest.approx(mb, rel=2e-3)


@pytest.mark.parametrize("cid,mb", [(2, 167.8), (4, 212.5), (5, 2115.0)])
def test_combine_bytes(cid, mb):
    assert bench.algorithmic_work(synth.get_config(cid))["combine_bytes"] / 1e6 == pytest.approx(mb, rel=1e-3)


def test_combine_bytes_with_shared_experts():
    # the sink config's routed rows (436.6 MB) plus each token's
    # two shared-expert rows of fp32 and their two sink weights
    cfg = synth.get_config(3)
    extra = cfg.n_shared * cfg.T * (4 * cfg.H + 4)
    assert (bench.algorithmic_work(cfg)["combine_bytes"] - extra) / 1e6 == pytest.approx(436.6, rel=1e-3)
