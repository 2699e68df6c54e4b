"""Throughput of the MoE FFN forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--cfg 2] [--no-cpu-baseline]

One step is the whole layer on one batch: moe_route -> moe_build_indices ->
moe_grouped_ffn (gate_up GEMM + fused activation, down GEMM) -> moe_combine,
on seeded synthetic inputs already resident in HBM.  The default workload is
the Mixtral-shape layer: T=4096 tokens, hidden 4096, 8 experts, top-2 softmax
gate, moe_dim 14336, concatenated gate_up, SiLU, bf16 operands with fp32
accumulation.

Prints one JSON line: whole-layer tokens/s, the roofline of the dominant
kernel (the grouped gate_up GEMM, timed with HIP events recorded around its
launch on the stream it runs on), and the CPU oracle timed on a bounded
sample of the same workload.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE layer tokens/s + achieved TFLOPS (% MFMA peak), Mixtral shape, T=4096"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gate_up_gemm_mixtral_traffic.json")


class HipEvents:
    """Raw hipEvent_t handles through libamdhip64 (timing on any stream)."""

    def __init__(self, n: int):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.ev = (ctypes.c_void_p * n)()
        for i in range(n):
            h = ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(h)) == 0
            self.ev[i] = h
        self.n = n

    def record(self, i: int, stream: int):
        assert self.hip.hipEventRecord(ctypes.c_void_p(self.ev[i]), ctypes.c_void_p(stream)) == 0

    def triple(self, i: int):
        arr = (ctypes.c_void_p * 3)(self.ev[i], self.ev[i + 1], self.ev[i + 2])
        return arr

    def span(self, i: int, n: int):
        return (ctypes.c_void_p * n)(*[self.ev[i + j] for j in range(n)])

    def elapsed_ms(self, a: int, b: int) -> float:
        ms = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(self.ev[a]),
                                            ctypes.c_void_p(self.ev[b])) == 0
        return float(ms.value)

    def close(self):
        for i in range(self.n):
            self.hip.hipEventDestroy(ctypes.c_void_p(self.ev[i]))


def algorithmic_work(cfg) -> dict:
    """Algorithmic work of one layer step: the flops of the two grouped GEMMs
    and the HBM bytes of the bandwidth kernels (each tensor read or written
    once), the figures the roofline fractions are computed from."""
    T, H, D, E, k = cfg.T, cfg.H, cfg.D, cfg.E, cfg.k
    R = T * k
    if cfg.router == "softmax":   # reads x and W_gate, writes indices and weights
        route_bytes = 2 * T * H + 2 * H * E + 8 * T * k
    else:                         # reads the logits and the bias, writes indices and weights (and sink weights)
        route_bytes = 4 * T * (E + cfg.s) + 4 * E + 8 * T * k + 4 * T * cfg.s
    # build_indices: the CSR (histogram, scan, scatter: 20 bytes per routed row)
    # plus, for the fp8 and W4A8 layers, the quantisation of x (each token
    # once: bf16 read, codes and scales written; the GEMM gathers the rows)
    idx_bytes = 20 * R + 4 * (E + 1)
    if cfg.operand_dtype == "fp8":
        idx_bytes += 2 * T * H + T * H + 4 * T * (H // 128)
    elif cfg.operand_dtype == "mxfp4":
        idx_bytes += 2 * T * H + T * H + T * (H // 32)
    o_bytes = 4 if cfg.operand_dtype in ("bf16", "mxfp4_a16") else 2   # expert rows O: fp32 or bf16
    n_sh = getattr(cfg, "n_shared", 0)
    # combine: read every routed row of O (and each token's shared-expert rows),
    # the slot rows and weights (and the sink weights), write y in bf16
    comb_bytes = o_bytes * (R + n_sh * T) * H + 8 * R + 4 * n_sh * T + 2 * T * H
    return {"gate_up_flops": 4.0 * R * H * D, "down_flops": 2.0 * R * D * H, "route_bytes": route_bytes,
            "build_indices_bytes": idx_bytes, "combine_bytes": comb_bytes}


def measure_ceilings(moe, torch) -> dict:
    """Practical ceilings on this chip, measured with the library's probes
    right after the timed steps (same clocks): an MFMA loop on every CU for
    bf16 and fp8, and a 1 GiB streaming copy (bytes read + bytes written).
    The best of five launches each."""
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev).cuda_stream
    ev = HipEvents(2)
    wg = 1024
    out = torch.empty(wg * 8, dtype=torch.float32, device=dev)

    def best_rate(launch):
        launch()
        torch.cuda.synchronize()
        best = 0.0
        for _ in range(5):
            ev.record(0, stream)
            work = launch()
            ev.record(1, stream)
            torch.cuda.synchronize()
            best = max(best, work / (ev.elapsed_ms(0, 1) * 1e-3))
        return best

    res = {}
    for kind, name, iters in ((0, "bf16", 4000), (1, "fp8", 2000)):
        res[f"mfma_{name}_tflops"] = round(best_rate(lambda: moe.probe_mfma(kind, wg, iters, out)) / 1e12, 1)
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)

    def copy():
        moe.probe_stream_copy(src, dst)
        return 2 * n

    res["stream_copy_gbs"] = round(best_rate(copy) / 1e9, 1)
    ev.close()
    del src, dst
    return res


def _with_measured(roof: dict, ceil: dict, dtype_key: str) -> dict:
    """Adds the measured ceiling of the roofline's bound and the fraction of it."""
    mp = ceil["stream_copy_gbs"] if roof["bound"] == "hbm" else ceil[dtype_key]
    roof["measured_peak"] = mp
    roof["frac_of_measured"] = round(roof["achieved"] / mp, 4)
    return roof


def _src_hash() -> str:
    """Hash of the sources that make the bf16 GEMM kernels."""
    h = hashlib.sha256()
    for f in ("ffn_bf16.hip", "common.h", "kernels.h"):
        h.update(open(os.path.join(ROOT, "mixture_experts_ffn_top_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def _traffic():
    """HBM bytes per gate_up launch from the committed rocprofv3 counter
    summary, or None when it is missing or the kernel source changed since."""
    try:
        d = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if d.get("kernel_source_sha256_16") != _src_hash():
        return None
    return d.get("bytes_per_launch")


PROFILE_CMDS = """# commands (repo root as $REPO, run from /tmp with TMPDIR=/tmp):
#   rocprofv3 --kernel-trace --stats -f csv -d $REPO/gpurun_out/prof/trace -o bench -- \\
#       python3 $REPO/bench.py --no-cpu-baseline > $REPO/gpurun_out/prof/trace.log
#   rocprofv3 --pmc FETCH_SIZE --kernel-include-regex 'grouped_gemm|router|csr|combine|permute' -f csv \\
#       -d $REPO/gpurun_out/prof/FETCH_SIZE -o bench -- python3 $REPO/bench.py --steps 3 --warmup 1 --no-cpu-baseline
#   (the same with WRITE_SIZE into .../WRITE_SIZE)
#   rocprofv3 --pmc FETCH_SIZE -f csv -d $REPO/gpurun_out/prof/copy_FETCH_SIZE -o copy -- \\
#       python3 $REPO/bench.py --copy-calibration        (and WRITE_SIZE into .../copy_WRITE_SIZE)
#   python3 bench.py --summarize-profile gpurun_out/prof    (writes the files under profiles/)"""

# the MX workloads' kernel traces, summarised by the same --summarize-profile call
EXTRA_TRACES = [
    ("trace3", 3, "sink_router_shared_experts_layer_kernel_stats.txt",
     "sigmoid-sink router layer with two shared experts: T=8192 tokens, hidden 2048, 128 experts, top-6 + 2 sink "
     "lanes, moe_dim 768, SiLU, bf16"),
    ("trace4", 4, "gptoss_shape_layer_kernel_stats.txt",
     "gpt-oss-shape layer: T=4096 tokens, hidden 2880, 32 experts, top-4 softmax gate, moe_dim 2880, interleaved "
     "gate_up, swigluoai (alpha 1.702, limit 7), biases, bf16"),
    ("trace5", 5, "fp8_block_scaled_layer_kernel_stats.txt",
     "fp8 block-scaled layer: T=16384 tokens, hidden 7168, 256 experts, top-8 sigmoid router, moe_dim 2048, "
     "SiLU, e4m3 operands with 128-wide fp32 block scales"),
    ("trace6", 6, "mxfp4_w4a8_layer_kernel_stats.txt",
     "MXFP4 x MXFP8 (W4A8) layer: T=16384 tokens, hidden 7168, 256 experts, top-8 sigmoid router, "
     "moe_dim 2048, SiLU"),
    ("trace7", 7, "mxfp4_w4a16_decode_kernel_stats.txt",
     "MXFP4 W4A16 layer on a decode-sized batch: T=256 tokens, hidden 7168, 256 experts, top-8 sigmoid "
     "router, moe_dim 2048, SiLU"),
    ("trace8", 8, "mixtral_decode_fused_ffn_kernel_stats.txt",
     "Mixtral decode batch through the single-launch FFN: T=64 tokens, hidden 4096, 8 experts, top-2 softmax "
     "router, moe_dim 14336, SiLU"),
]


def _short(name: str) -> str:
    name = name.strip('"').replace("(anonymous namespace)::", "")
    return name.split("(")[0].replace("void ", "")


def summarize_profile(d: str):
    """Turn the rocprofv3 outputs of PROFILE_CMDS into the committed summaries."""
    import csv
    prof = os.path.join(ROOT, "profiles")
    # kernel statistics of the bench run
    rows = list(csv.DictReader(open(os.path.join(d, "trace", "bench_kernel_stats.csv"))))
    mine = [r for r in rows if "moe::" in r["Name"]]
    line = None
    for ln in open(os.path.join(d, "trace.log")):
        if ln.startswith('{"metric"'):
            line = json.loads(ln)
    bd = line["breakdown_ms"] if line else {}
    out = ["# rocprofv3 kernel statistics: Mixtral-shape MoE FFN layer (bench.py default workload)",
           "# workload: T=4096 tokens, hidden 4096, 8 experts, top-2 softmax gate, moe_dim 14336,",
           "#           concatenated gate_up, SiLU, bf16 operands, fp32 accumulate",
           PROFILE_CMDS,
           f"# calls = warmup + timed steps of bench.py.  Durations in microseconds; only this library's",
           "# kernels are listed (the torch kernels that generate the synthetic inputs are omitted).",
           f"# bench.py's own HIP-event timing in the same run: gate_up {bd.get('gate_up', 0) * 1e3:.1f} us, "
           f"down {bd.get('down', 0) * 1e3:.1f} us per launch.", "",
           f"{'kernel':58s}{'calls':>7s}{'avg_us':>10s}{'min_us':>10s}{'max_us':>10s}"]
    for r in sorted(mine, key=lambda r: -float(r["TotalDurationNs"])):
        out.append(f"{_short(r['Name']):58s}{int(r['Calls']):7d}{float(r['AverageNs']) / 1e3:10.1f}"
                   f"{float(r['MinNs']) / 1e3:10.1f}{float(r['MaxNs']) / 1e3:10.1f}")
    out += ["", "# gate_up = grouped_gemm_bf16_kernel<0,...> (SiLU, concatenated, gathered x, bf16 out)",
            "# down    = grouped_gemm_bf16_kernel<1,...> (fp32 out)",
            "# mfma_probe_* and stream_copy_kernel are the measured-ceiling probes bench.py runs once after",
            "# the timed steps (6 launches each), not part of the layer"]
    open(os.path.join(prof, "mixtral_layer_kernel_stats.txt"), "w").write("\n".join(out) + "\n")

    for sub, cid, name, title in EXTRA_TRACES:
        stats = os.path.join(d, sub, "bench_kernel_stats.csv")
        if not os.path.exists(stats):
            continue
        rows = [r for r in csv.DictReader(open(stats)) if "moe::" in r["Name"]]
        bd = {}
        for ln in open(os.path.join(d, sub + ".log")):
            if ln.startswith('{"metric"'):
                bd = json.loads(ln)["breakdown_ms"]
        out = [f"# rocprofv3 kernel statistics: {title}",
               "# command (repo root as $REPO, run from /tmp with TMPDIR=/tmp):",
               f"#   rocprofv3 --kernel-trace --stats -f csv -d $REPO/gpurun_out/prof/{sub} -o bench -- \\",
               f"#       python3 $REPO/bench.py --cfg {cid} --steps 10 --warmup 3 --no-cpu-baseline "
               f"> $REPO/gpurun_out/prof/{sub}.log",
               "#   python3 bench.py --summarize-profile gpurun_out/prof",
               "# calls = warmup + timed steps.  Durations in microseconds; only this library's kernels.",
               f"# bench.py's own HIP-event timing in the same run: gate_up {bd.get('gate_up', 0) * 1e3:.1f} us, "
               f"down {bd.get('down', 0) * 1e3:.1f} us per launch.", "",
               f"{'kernel':58s}{'calls':>7s}{'avg_us':>10s}{'min_us':>10s}{'max_us':>10s}"]
        for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
            out.append(f"{_short(r['Name']):58s}{int(r['Calls']):7d}{float(r['AverageNs']) / 1e3:10.1f}"
                       f"{float(r['MinNs']) / 1e3:10.1f}{float(r['MaxNs']) / 1e3:10.1f}")
        open(os.path.join(prof, name), "w").write("\n".join(out) + "\n")

    # HBM traffic from FETCH_SIZE / WRITE_SIZE, calibrated on a plain copy of known size
    def counters(path):
        per = {}
        for r in csv.DictReader(open(path)):
            per.setdefault(_short(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
        return per
    n_copy = 1 << 30
    cf = counters(os.path.join(d, "copy_FETCH_SIZE", "copy_counter_collection.csv"))
    cw = counters(os.path.join(d, "copy_WRITE_SIZE", "copy_counter_collection.csv"))
    copy_f = [v for k, vs in cf.items() if "copyBuffer" in k for v in vs]
    copy_w = [v for k, vs in cw.items() if "copyBuffer" in k for v in vs]
    f_factor = n_copy / (sum(copy_f) / len(copy_f) * 1024)
    w_factor = n_copy / (sum(copy_w) / len(copy_w) * 1024)
    fe = counters(os.path.join(d, "FETCH_SIZE", "bench_counter_collection.csv"))
    wr = counters(os.path.join(d, "WRITE_SIZE", "bench_counter_collection.csv"))
    out = ["# HBM traffic per launch from rocprofv3 counters: Mixtral-shape MoE FFN layer (bench.py workload)",
           PROFILE_CMDS,
           f"# calibration, a plain 1 GiB device copy: FETCH_SIZE {sum(copy_f) / len(copy_f):.0f} KiB -> read factor "
           f"{f_factor:.3f}; WRITE_SIZE {sum(copy_w) / len(copy_w):.0f} KiB -> write factor {w_factor:.3f}",
           "# bytes = counter KiB x 1024 x factor, averaged over the launches of each kernel.", "",
           f"{'kernel':58s}{'read_MB':>10s}{'write_MB':>10s}{'total_MB':>10s}"]
    gu = None
    for k in fe:
        rd = sum(fe[k]) / len(fe[k]) * 1024 * f_factor
        wb = sum(wr.get(k, [0.0])) / max(len(wr.get(k, [])), 1) * 1024 * w_factor
        out.append(f"{k:58s}{rd / 1e6:10.1f}{wb / 1e6:10.1f}{(rd + wb) / 1e6:10.1f}")
        if k.startswith("moe::grouped_gemm_bf16_kernel<0"):
            gu = (rd, wb)
    out += ["", "# algorithmic bytes per launch for comparison: gate_up reads the 8 experts' gate_up weights",
            "# (1879.0 MB) and the rows of the 4096 tokens (33.6 MB, each read once) and writes A (235.0 MB);",
            "# down reads the down weights (939.5 MB) and A (235.0 MB) and writes O fp32 (134.2 MB).",
            "# Traffic above that is weight tiles fetched again by m-blocks that missed each other in L2,",
            "# and activation rows re-read from the Infinity Cache."]
    open(os.path.join(prof, "mixtral_layer_hbm_traffic.txt"), "w").write("\n".join(out) + "\n")
    if gu:
        json.dump({"kernel": "grouped gate_up GEMM (bf16, SiLU, concatenated, gathered x)",
                   "workload": "Mixtral-shape layer, T=4096", "bytes_per_launch": round(gu[0] + gu[1]),
                   "read_bytes": round(gu[0]), "write_bytes": round(gu[1]),
                   "fetch_factor": round(f_factor, 4), "write_factor": round(w_factor, 4),
                   "kernel_source_sha256_16": _src_hash(), "source": "profiles/mixtral_layer_hbm_traffic.txt"},
                  open(TRAFFIC_FILE, "w"), indent=1)
    print(f"[bench] wrote the profile summaries under {prof}", file=sys.stderr)


def cpu_baseline(cfg, inp, n_tokens: int):
    """The oracle as it stands, on a sample of the workload's tokens."""
    import numpy as np
    import synth
    from oracle import moe_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = len(os.sched_getaffinity(0))
    hin = synth.to_host(inp)
    rng = np.random.default_rng(0)
    tokens = np.arange(cfg.T) if n_tokens >= cfg.T else np.sort(rng.choice(cfg.T, n_tokens, replace=False))
    t0 = time.perf_counter()
    r = O.route(hin, cfg)
    y = O.layer(hin, cfg, indices=r["indices"], weights=r["weights"], tokens=tokens)
    dt = time.perf_counter() - t0
    assert np.all(np.isfinite(y))
    return {"value": round(n_tokens / dt, 3), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": (f"the whole workload ({cfg.T} tokens)" if n_tokens >= cfg.T else
                       f"{n_tokens} of {cfg.T} tokens (seeded), all experts they route to, routing of all "
                       f"{cfg.T} tokens") + f"; {dt:.1f} s on the host, float64 numpy"}


def bench_backward(args, cfg, inp, moe, torch):
    """Time the backward of the routed experts: combine backward, the grouped
    FFN backward (its 8 phase events) and the gather of dx, on resident inputs
    and the routing of one forward pass."""
    import synth
    dev = torch.device("cuda:0")
    layer = moe.MoELayer(cfg, inp)
    layer.forward(inp["x"])
    dy = synth.make_grad_output(cfg, dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    K, W = args.steps, args.warmup
    NE = 10  # 0 start, 1..8 the FFN backward's events, 9 end
    ev = HipEvents(NE * (K + W))

    def step(i):
        b = NE * i
        ev.record(b, stream)
        layer.backward(dy, timing_events=ev.span(b + 1, 8))
        ev.record(b + 9, stream)

    print(f"[bench] backward: warmup {W}", file=sys.stderr, flush=True)
    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    print(f"[bench] backward: timing {K} steps", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    for i in range(W, W + K):
        step(i)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1000.0 / K

    def mean_ms(a, b):
        return sum(ev.elapsed_ms(NE * i + a, NE * i + b) for i in range(W, W + K)) / K

    names = ["combine_backward", "dA", "gate_up_recompute", "dX", "transposes", "dW_down", "dW_gate_up",
             "bias_grads", "dx_gather"]
    t = {n: mean_ms(j, j + 1) for j, n in enumerate(names)}
    ev.close()
    ceil = measure_ceilings(moe, torch)
    R = cfg.T * cfg.k
    rhd = 2.0 * R * cfg.H * cfg.D
    flops = {"dA": rhd, "gate_up_recompute": 2 * rhd, "dX": 2 * rhd, "dW_down": rhd, "dW_gate_up": 2 * rhd}
    peak = PEAK_BF16_TFLOPS
    dom = max(flops, key=lambda n: t[n])
    tf = {n: flops[n] / (t[n] * 1e-3) / 1e12 for n in flops}
    total_tf = sum(flops.values()) / (sum(t[n] for n in flops) * 1e-3) / 1e12
    line = {
        "metric": "MoE layer backward tokens/s + achieved TFLOPS (% MFMA peak)",
        "value": round(cfg.T / (ms_step * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{cfg.name} MoE FFN backward (routed experts): T={cfg.T} hidden={cfg.H} "
                               f"experts={cfg.E} top-{cfg.k} moe_dim={cfg.D} {cfg.gate_up_format} {cfg.activation}",
                   "tokens": cfg.T, "hidden_dim": cfg.H, "num_experts": cfg.E, "top_k": cfg.k, "moe_dim": cfg.D,
                   "parallelism": "none (1 GPU)"},
        "roofline": _with_measured({"bound": "mfma", "achieved": round(tf[dom], 2), "peak": peak, "unit": "TFLOP/s",
                                    "frac": round(tf[dom] / peak, 4), "traffic": None, "kernel": dom,
                                    "flops_per_launch": flops[dom], "avg_launch_ms": round(t[dom], 4)},
                                   ceil, "mfma_bf16_tflops"),
        "gemm_tflops": {n: round(v, 1) for n, v in tf.items()},
        "gemms_mfma_frac": round(total_tf / peak, 4),
        "gemms_frac_of_measured": round(total_tf / ceil["mfma_bf16_tflops"], 4),
        "measured_ceilings": ceil,
        "breakdown_ms": {n: round(v, 4) for n, v in t.items()},
    }
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cfg", type=int, default=2)
    ap.add_argument("--cpu-sample", type=int, default=4096,
                    help="tokens the oracle baseline runs (capped at the workload's T)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward pass of the routed experts (bf16 workloads) instead of the forward")
    ap.add_argument("--scale-tokens", type=int, default=1, metavar="N",
                    help="secondary data point: run the workload with N times its tokens, where the small "
                         "bandwidth kernels leave the launch-latency regime (the config-size line is the reported one)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 3 times (HBM counter calibration)")
    ap.add_argument("--summarize-profile", metavar="DIR",
                    help="only write the profiles/ summaries from the rocprofv3 outputs in DIR (no GPU)")
    args = ap.parse_args()
    if args.summarize_profile:
        summarize_profile(args.summarize_profile)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus})", file=sys.stderr)
        sys.exit(2)

    import torch
    import mixture_experts_ffn_top_amd as moe
    import synth

    if args.copy_calibration:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read_per_launch": n, "bytes_written_per_launch": n,
                          "launches": 3}), flush=True)
        return

    cfg = synth.get_config(args.cfg)
    if args.scale_tokens > 1:
        cfg = synth.scaled(cfg, T=cfg.T * args.scale_tokens)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    print(f"[bench] generating workload cfg {cfg.cfg_id} ({cfg.name})", file=sys.stderr, flush=True)
    inp = synth.make_inputs(cfg, dev)
    if args.backward:
        if cfg.operand_dtype != "bf16" or getattr(cfg, "n_shared", 0):
            print("bench.py --backward: the backward is built for bf16 layers without shared experts",
                  file=sys.stderr)
            sys.exit(2)
        bench_backward(args, cfg, inp, moe, torch)
        return
    layer = moe.MoELayer(cfg, inp)
    stream = torch.cuda.current_stream(dev).cuda_stream
    K, W = args.steps, args.warmup
    # per step: 0 start, 1 after route, 2 after indices, 3..5 ffn (gate_up start, mid, end),
    # 6 after combine, 7..9 the shared experts' ffn (if any)
    NE = 10
    ev = HipEvents(NE * (K + W))
    has_shared = getattr(cfg, "n_shared", 0) > 0

    def step(i):
        base = NE * i
        slots = {1: base + 1, 2: base + 2, 3: base + 6}
        ev.record(base + 0, stream)
        layer.forward(inp["x"], mark=lambda j: ev.record(slots[j], stream), ffn_events=ev.triple(base + 3),
                      shared_events=ev.triple(base + 7) if has_shared else None)

    print(f"[bench] warmup {W}", file=sys.stderr, flush=True)
    for i in range(W):
        step(i)
    torch.cuda.synchronize()
    print(f"[bench] timing {K} steps", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    for i in range(W, W + K):
        step(i)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    ms_step = dt * 1000.0 / K

    def mean_ms(a, b):
        return sum(ev.elapsed_ms(NE * i + a, NE * i + b) for i in range(W, W + K)) / K

    t_route, t_idx = mean_ms(0, 1), mean_ms(1, 2)
    t_gu, t_dn = mean_ms(3, 4), mean_ms(4, 5)
    t_shared = mean_ms(7, 9) if has_shared else 0.0
    t_comb = (mean_ms(9, 6) if has_shared else mean_ms(5, 6))
    t_layer_dev = mean_ms(0, 6)
    ev.close()
    print("[bench] measured ceilings (MFMA loop, streaming copy)", file=sys.stderr, flush=True)
    ceil = measure_ceilings(moe, torch)

    R = cfg.T * cfg.k
    work = algorithmic_work(cfg)
    gu_flops, dn_flops = work["gate_up_flops"], work["down_flops"]
    route_bytes, idx_bytes, comb_bytes = work["route_bytes"], work["build_indices_bytes"], work["combine_bytes"]
    # fp8 and the MXFP4 x MXFP8 product (which runs at the fp8 MFMA rate) take the fp8 peak
    peak = PEAK_BF16_TFLOPS if cfg.operand_dtype in ("bf16", "mxfp4_a16") else PEAK_FP8_TFLOPS
    gu_tf = gu_flops / (t_gu * 1e-3) / 1e12
    ffn_tf = (gu_flops + dn_flops) / ((t_gu + t_dn) * 1e-3) / 1e12
    roof = {"bound": "mfma", "achieved": round(gu_tf, 2), "peak": peak, "unit": "TFLOP/s",
            "frac": round(gu_tf / peak, 4), "traffic": _traffic() if cfg.cfg_id == 2 else None,
            "kernel": "grouped gate_up GEMM + fused activation",
            "flops_per_launch": gu_flops, "avg_launch_ms": round(t_gu, 4)}
    if cfg.operand_dtype == "mxfp4_a16":
        # a decode-sized batch: the gate_up GEMM is bound by streaming the
        # 4-bit weights (and E8M0 scales) of every expert that has a row,
        # plus the gathered bf16 rows in and the bf16 A out
        off = layer.last_offsets.cpu()
        used = int(((off[1:] - off[:-1]) > 0).sum())
        gu_bytes = used * (2 * cfg.D * cfg.H // 2 + 2 * cfg.D * cfg.H // 32) + R * cfg.H * 2 + R * cfg.D * 2
        gbs = gu_bytes / (t_gu * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None,
                "kernel": "grouped gate_up GEMM + fused activation (MXFP4 weights, bf16 activations)",
                "bytes_per_launch": gu_bytes, "experts_with_rows": used, "avg_launch_ms": round(t_gu, 4)}
    if getattr(cfg, "fused", False):
        # the FFN is one launch (gate_up and down together) on a decode-sized
        # batch: bound by streaming the bf16 weights of the experts that have
        # rows, plus x rows in, A out and back in, O out
        off = layer.last_offsets.cpu()
        used = int(((off[1:] - off[:-1]) > 0).sum())
        ffn_bytes = (used * (2 * cfg.D * cfg.H + cfg.H * cfg.D) * 2 + R * cfg.H * 2 + 2 * R * cfg.D * 2
                     + R * cfg.H * 4)
        t_ffn = t_gu + t_dn
        gbs = ffn_bytes / (t_ffn * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None,
                "kernel": "single-launch expert FFN (gate_up + activation + down, bf16)",
                "bytes_per_launch": ffn_bytes, "experts_with_rows": used, "avg_launch_ms": round(t_ffn, 4)}
    mfma_key = "mfma_bf16_tflops" if peak == PEAK_BF16_TFLOPS else "mfma_fp8_tflops"
    roof = _with_measured(roof, ceil, mfma_key)
    hbm = {"route": route_bytes / (t_route * 1e-3) / 1e9, "build_indices": idx_bytes / (t_idx * 1e-3) / 1e9,
           "combine": comb_bytes / (t_comb * 1e-3) / 1e9}
    line = {
        "metric": METRIC, "value": round(cfg.T / (ms_step * 1e-3), 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": K, "warmup": W, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": {"bf16": "bf16", "fp8": "fp8", "mxfp4": "mxfp4_w4a8", "mxfp4_a16": "mxfp4_w4a16"}[cfg.operand_dtype],
        "data": "synthetic",
        "config": {"workload": ("" if args.scale_tokens == 1 else f"[secondary: {args.scale_tokens}x tokens] ")
                               + f"{cfg.name} MoE FFN forward: T={cfg.T} hidden={cfg.H} experts={cfg.E} "
                               f"top-{cfg.k} {cfg.router} router moe_dim={cfg.D} {cfg.gate_up_format} "
                               f"{cfg.activation}", "tokens": cfg.T, "hidden_dim": cfg.H,
                   "num_experts": cfg.E, "top_k": cfg.k, "moe_dim": cfg.D, "parallelism": "none (1 GPU)"},
        "roofline": roof,
        "ffn_tflops": round(ffn_tf, 2), "ffn_mfma_frac": round(ffn_tf / peak, 4),
        "ffn_frac_of_measured": round(ffn_tf / ceil[mfma_key], 4),
        "breakdown_ms": {"route": round(t_route, 4), "build_indices": round(t_idx, 4),
                         "gate_up": round(t_gu, 4), "down": round(t_dn, 4),
                         **({"shared_experts_ffn": round(t_shared, 4)} if has_shared else {}),
                         "combine": round(t_comb, 4), "layer_device": round(t_layer_dev, 4)},
        "hbm_gbs": {n: round(v, 1) for n, v in hbm.items()},
        "hbm_frac": {n: round(v / PEAK_HBM_GBS, 4) for n, v in hbm.items()},
        "hbm_frac_of_measured": {n: round(v / ceil["stream_copy_gbs"], 4) for n, v in hbm.items()},
        "measured_ceilings": ceil,
        "weight_layout": "out_in (transposed stacked weights, laid out once at load)",
    }
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle on a token sample)", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(cfg, inp, min(args.cpu_sample, cfg.T))
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
