"""bench.py's algorithmic work per layer step, against per-config figures
worked out by hand from the workloads' tensor shapes: the FLOP of the grouped
FFN (6 R H D, R = T k), the bytes of the softmax router (x and W_gate read
once, indices and weights written) and of the combine (O read once, the slot
rows and weights read, y written in bf16)."""
import os

import pytest

import bench
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


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


def test_single_launch_ffn_bytes():
    # Mixtral decode (T=64, top-2: 128 rows), all 8 experts with rows: per
    # expert 2*14336*4096 + 4096*14336 bf16 weights = 352,321,536 bytes; x rows
    # 128*4096*2, A written and read 2*128*14336*2, O 128*4096*4 (fp32)
    cfg = synth.get_config(8)
    assert bench.fused_ffn_bytes(cfg, 8) == 8 * 352_321_536 + 1_048_576 + 7_340_032 + 2_097_152
    # MXFP4 decode (T=256, top-8: 2048 rows), 142 experts with rows: per
    # expert 44,040,192 E2M1 codes at half a byte plus one scale byte per 32:
    # 23,396,352 bytes; x rows 2048*7168 codes + scales = 15,138,816; A
    # 2*2048*2048 codes + scales = 8,650,752; O 2048*7168*2 (bf16)
    cfg = synth.get_config(9)
    assert bench.fused_ffn_bytes(cfg, 142) == 142 * 23_396_352 + 15_138_816 + 8_650_752 + 29_360_128
    # the same experts with bf16 rows (W4A16): x 2048*7168*2, A 2*2048*2048*2, O fp32 2048*7168*4
    cfg = synth.get_config(10)
    assert bench.fused_ffn_bytes(cfg, 142) == 142 * 23_396_352 + 29_360_128 + 16_777_216 + 58_720_256


def test_algorithmic_work_with_local_rows():
    """An expert-parallel share: the GEMM flops and the combine's O bytes
    follow the rows the local experts received; the bucketing still reads
    every slot."""
    import synth
    cfg = synth.scaled(synth.get_config(2), T=32768)
    full = bench.algorithmic_work(cfg)
    part = bench.algorithmic_work(cfg, rows=8318)
    assert part["gate_up_flops"] == 4.0 * 8318 * 4096 * 14336
    assert part["down_flops"] == 2.0 * 8318 * 14336 * 4096
    assert part["build_indices_bytes"] == full["build_indices_bytes"]
    assert full["combine_bytes"] - part["combine_bytes"] == 4 * (32768 * 2 - 8318) * 4096


@pytest.mark.parametrize("argv", [["--cfg", "2", "--ep-share", "3"], ["--cfg", "3", "--ep-share", "8"],
                                  ["--cfg", "8", "--ep-share", "2"], ["--gpus", "2"]])
def test_bench_refuses_unsupported_runs(argv):
    """Runs the bench cannot make exit with status 2 and a message, before any GPU use."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv], capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 2, r.stderr
    assert "bench.py" in r.stderr
