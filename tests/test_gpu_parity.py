"""GPU parity: every step of the HIP path against the CPU oracle, through the C ABI.

Bars: indices, CSR offsets, permutations and fp8 codes bit-exact; router
weights within 1e-5 relative; bf16 layer output within 2e-2 x RMS and fp8
within 6e-2 x RMS of the oracle's float64 output.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import moe_oracle as O
from tests.gpu_util import assert_rel, bf16_floor, host, rel_rms_err, sample_tokens, say

pytestmark = pytest.mark.gpu

DEV = "cuda"
W_RTOL = 1e-5
BF16_TOL = 2e-2
FP8_TOL = 6e-2


@pytest.fixture(scope="module")
def moe():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import mixture_experts_ffn_top_amd as m
    m.lib()
    return m


def _gen(cfg):
    say(f"[gen] cfg={cfg.cfg_id}:{cfg.name} T={cfg.T} H={cfg.H} E={cfg.E} k={cfg.k} D={cfg.D}")
    return synth.make_inputs(cfg, DEV)


# ---------------------------------------------------------------- routers

@pytest.mark.parametrize("cid,T,extra", [
    (1, 64, {}), (2, 4096, {}), (4, 4096, {}), (1, 1, {}), (4, 77, {}),
    # 33..64 and 65..128 experts (4 and 8 MFMA expert tiles), hidden sizes
    # below one 256-column chunk and with a ragged last chunk
    (1, 45, dict(E=64, k=6, H=1000)), (1, 33, dict(E=100, k=4, H=264)),
    (1, 16, dict(E=128, k=8, H=8)), (1, 300, dict(E=40, k=3, H=776)),
])
def test_softmax_router_x_form(moe, cid, T, extra):
    cfg = synth.scaled(synth.get_config(cid), T=T, **extra)
    inp = _gen(cfg)
    say(f"[route softmax x] cfg={cid} T={T} {extra}")
    idx, w, _, lo = moe.route(router="softmax", k=cfg.k, E=cfg.E, x=inp["x"], w_gate=inp["w_gate"],
                              return_logits=True)
    torch.cuda.synchronize()
    ref_logits = O.gate_logits(host(inp["x"]), host(inp["w_gate"]))
    err, rms = rel_rms_err(host(lo), ref_logits)
    say(f"  logits max err / rms = {err:.2e}")
    assert err <= 2e-5
    # selection and weights on the GPU's own float32 logits
    ridx, rw = O.route_softmax_topk(host(lo), cfg.k)
    assert np.array_equal(host(idx), ridx)
    assert_rel(host(w), rw, W_RTOL, "softmax weights")


@pytest.mark.parametrize("renorm,scale", [(True, 1.0), (False, 2.5)])
def test_softmax_router_logits_form_and_ties(moe, renorm, scale):
    rng = np.random.default_rng(1)
    T, E, k = 300, 40, 5
    z = rng.choice(np.array([-1.0, 0.0, 0.25, 3.0], np.float32), size=(T, E))   # many exact ties
    z[:100] = rng.standard_normal((100, E)).astype(np.float32)
    zt = torch.from_numpy(z).to(DEV)
    gs = torch.tensor([0.5], device=DEV)
    idx, w, _, _ = moe.route(router="softmax", k=k, E=E, logits=zt, route_scale=scale,
                             global_scale=gs, renormalize=renorm)
    ridx, rw = O.route_softmax_topk(z, k, scale, 0.5, renormalize=renorm)
    assert np.array_equal(host(idx), ridx)
    assert_rel(host(w), rw, W_RTOL, "softmax weights")


@pytest.mark.parametrize("cid,T", [(3, 8192), (5, 16384), (3, 1), (3, 333)])
def test_sigmoid_sink_router(moe, cid, T):
    cfg = synth.scaled(synth.get_config(cid), T=T)
    g = torch.Generator(device=DEV)
    g.manual_seed(100 + cid)
    logits = (torch.randn((T, cfg.E + cfg.s), generator=g, device=DEV) * cfg.logit_std).contiguous()
    bias = (torch.rand((cfg.E,), generator=g, device=DEV) * 0.2 - 0.1)
    gs = torch.tensor([cfg.global_scale], device=DEV)
    say(f"[route sigmoid] cfg={cid} T={T}")
    idx, w, sw, _ = moe.route(router="sigmoid", k=cfg.k, E=cfg.E, s=cfg.s, logits=logits,
                              expert_bias=bias, route_scale=cfg.route_scale, global_scale=gs)
    ridx, rw, rsw = O.route_sigmoid_sink(host(logits), cfg.E, cfg.k, cfg.s, host(bias),
                                         cfg.route_scale, cfg.global_scale)
    assert np.array_equal(host(idx), ridx)
    assert_rel(host(w), rw, W_RTOL, "expert weights")
    if cfg.s:
        assert_rel(host(sw), rsw, W_RTOL, "sink weights")


def test_sigmoid_router_extremes(moe):
    """Underflowing and saturated sigmoids, exact ties, a bias that forces
    selection, and a logits row wider than E+s."""
    E, k, s = 64, 6, 2
    rows = [np.full(E + s + 3, -300.0), np.full(E + s + 3, 50.0), np.zeros(E + s + 3)]
    r = np.linspace(-250, -100, E + s + 3)
    rows.append(r)
    z = np.stack(rows).astype(np.float32)
    bias = np.zeros(E, np.float32)
    bias[17] = 5.0
    zt = torch.from_numpy(z).to(DEV)
    full = moe.route(router="sigmoid", k=k, E=E, s=s, logits=zt, expert_bias=torch.from_numpy(bias).to(DEV),
                     route_scale=2.5)
    ridx, rw, rsw = O.route_sigmoid_sink(z, E, k, s, bias, 2.5, 1.0)
    assert np.array_equal(host(full[0]), ridx)
    assert np.all(np.isfinite(host(full[1]))) and np.all(np.isfinite(host(full[2])))
    assert_rel(host(full[1]), rw, W_RTOL, "expert weights")
    assert_rel(host(full[2]), rsw, W_RTOL, "sink weights")


# ---------------------------------------------------------------- CSR and permute

def _routing(T, E, k, seed, mode="random"):
    rng = np.random.default_rng(seed)
    if mode == "random":
        idx = np.stack([rng.permutation(E)[:k] for _ in range(T)])
    elif mode == "one_expert":
        idx = np.zeros((T, k), np.int64)
        idx[:, 1:] = np.arange(1, k)[None, :]
    elif mode == "half_empty":
        idx = np.stack([rng.permutation(E // 2)[:k] * 2 for _ in range(T)])
    return idx.astype(np.int32), rng.random((T, k)).astype(np.float32)


@pytest.mark.parametrize("T,E,k,start,L,mode,masked", [
    (8192, 128, 6, 0, 128, "random", False),
    (16384, 256, 8, 0, 256, "random", True),
    (16384, 256, 8, 32, 32, "random", False),
    (4096, 8, 2, 0, 8, "one_expert", False),
    (1000, 64, 4, 0, 64, "half_empty", True),
    (1, 8, 2, 0, 8, "random", False),
    (5000, 1024, 3, 0, 1024, "random", False),
])
def test_build_indices(moe, T, E, k, start, L, mode, masked):
    idx, w = _routing(T, E, k, 7 + T, mode)
    mask = (np.random.default_rng(3).random(T) > 0.25).astype(np.uint8) if masked else None
    say(f"[csr] T={T} E={E} k={k} start={start} L={L} mode={mode} masked={masked}")
    out = moe.build_indices(torch.from_numpy(idx).to(DEV), L, expert_start=start,
                            weights=torch.from_numpy(w).to(DEV),
                            token_mask=torch.from_numpy(mask).to(DEV) if mask is not None else None)
    ref = O.build_indices(idx, L, start, mask, w)
    off = host(out["offsets"])
    assert np.array_equal(off, ref["offsets"])
    n = int(off[-1])
    assert np.array_equal(host(out["sorted_token"])[:n], ref["sorted_token"])
    assert np.array_equal(host(out["row_of_slot"])[:T * k], ref["row_of_slot"])
    assert np.array_equal(host(out["sorted_weight"])[:n], ref["sorted_weight"].astype(np.float32))


@pytest.mark.parametrize("fp8", [False, True, "tokens"])
def test_permute(moe, fp8):
    T, E, k, H = 3000, 16, 3, 7168 if fp8 else 2880
    idx, _ = _routing(T, E, k, 11)
    g = torch.Generator(device=DEV)
    g.manual_seed(5)
    x = (torch.randn((T, H), generator=g, device=DEV) * 3).to(torch.bfloat16)
    x[5, :128] = 0                       # an all-zero group
    say(f"[permute] fp8={fp8} T={T} H={H}")
    mode = {False: "bf16", True: "fp8", "tokens": "fp8_tokens"}[fp8]
    out = moe.build_indices(torch.from_numpy(idx).to(DEV), E, x=x, xperm_dtype=mode)
    ref = O.build_indices(idx, E)
    n = int(host(out["offsets"])[-1])
    xh = host(x)
    if mode == "bf16":
        assert np.array_equal(host(out["x_perm"])[:n], O.permute_rows(xh, ref["sorted_token"]))
    elif mode == "fp8_tokens":
        codes, sc = O.quantize_rows_block128(xh)
        assert np.array_equal(host(out["x_perm"])[:T], codes)
        assert np.array_equal(host(out["x_perm_scale"])[:T], sc)
    else:
        codes, sc = O.quantize_rows_block128(xh)
        assert np.array_equal(host(out["x_perm"])[:n], codes[ref["sorted_token"]])
        assert np.array_equal(host(out["x_perm_scale"])[:n], sc[ref["sorted_token"]])


# ---------------------------------------------------------------- grouped FFN + whole layer

def _run_layer(moe, cfg, inp, *, gather=True, token_mask=None):
    layer = moe.MoELayer(cfg, inp, gather=gather)
    res = layer.forward(inp["x"], token_mask=token_mask)
    torch.cuda.synchronize()
    return layer, res


def _check_layer(cfg, inp, res, tokens, tol, token_mask=None):
    hin = synth.to_host(inp)
    idx = host(res["indices"])
    w = host(res["weights"]).astype(np.float64)
    sw = host(res["sink_weights"]).astype(np.float64) if res.get("sink_weights") is not None else None
    y_ref = O.layer(hin, cfg, indices=idx, weights=w, tokens=tokens, token_mask=token_mask, sink_weights=sw)
    y = host(res["y"])[tokens]
    err, rms = rel_rms_err(y, y_ref)
    say(f"  y max err / rms = {err:.3e} (bf16 floor {bf16_floor(y_ref):.3e}, rms {rms:.3e})")
    assert np.all(np.isfinite(y))
    assert err <= tol
    return err


def _check_routing(cfg, inp, res):
    hin = synth.to_host(inp, keys=["logits", "expert_bias"])
    if cfg.router == "sigmoid_sink":
        ridx, rw, rsw = O.route_sigmoid_sink(hin["logits"], cfg.E, cfg.k, cfg.s, hin["expert_bias"],
                                             cfg.route_scale, cfg.global_scale)
        assert np.array_equal(host(res["indices"]), ridx)
        assert_rel(host(res["weights"]), rw, W_RTOL, "expert weights")
        if cfg.s:
            assert_rel(host(res["sink_weights"]), rsw, W_RTOL, "sink weights")


@pytest.mark.parametrize("cid,changes,nsample", [
    (1, {}, 64),
    (3, {"T": 1024}, 1024),
    (4, {"T": 512}, 512),
    (2, {"T": 256, "H": 1024, "D": 2048}, 256),
    (1, {"T": 100, "H": 1000, "D": 200}, 100),       # K not a multiple of the 64-wide k tile
    (4, {"T": 90, "H": 296, "D": 72, "E": 3, "k": 2}, 90),   # ragged N and K in both GEMMs
])
def test_layer_small(moe, cid, changes, nsample):
    cfg = synth.scaled(synth.get_config(cid), **changes)
    inp = _gen(cfg)
    for gather in (True, False):
        say(f"[layer] cfg={cid} {changes} gather={gather}")
        _, res = _run_layer(moe, cfg, inp, gather=gather)
        _check_routing(cfg, inp, res)
        _check_layer(cfg, inp, res, sample_tokens(cfg.T, nsample), BF16_TOL)


@pytest.mark.parametrize("cid,nsample", [(2, 96), (3, 384), (4, 256)])
def test_layer_full_size(moe, cid, nsample):
    cfg = synth.get_config(cid)
    inp = _gen(cfg)
    say(f"[layer full] cfg={cid}")
    _, res = _run_layer(moe, cfg, inp)
    _check_routing(cfg, inp, res)
    _check_layer(cfg, inp, res, sample_tokens(cfg.T, nsample, seed=cid), BF16_TOL)


@pytest.mark.parametrize("act,alpha,limit,fmt,bias", [
    ("silu", 0.0, 7.0, "concatenated", False),
    ("gelu_tanh", 0.0, 0.0, "concatenated", True),
    ("swigluoai", 1.702, 7.0, "interleaved", True),
    ("swigluoai", 1.702, 7.0, "concatenated", False),
    ("silu", 0.0, 0.0, "interleaved", True),
])
def test_activation_variants_clamp_stress(moe, act, alpha, limit, fmt, bias):
    """x scaled x8 so that |gate|, |up| reach well past limit = 7."""
    cfg = synth.scaled(synth.get_config(4), T=300, H=512, D=384, E=6, k=2, activation=act, alpha=alpha,
                       limit=limit, gate_up_format=fmt, has_bias=bias, x_std=8.0, w_std=0.05)
    inp = _gen(cfg)
    say(f"[variant] {act} alpha={alpha} limit={limit} {fmt} bias={bias}")
    _, res = _run_layer(moe, cfg, inp)
    _check_layer(cfg, inp, res, np.arange(cfg.T), BF16_TOL)


def test_expert_scales_and_local_slice(moe):
    cfg = synth.scaled(synth.get_config(3), T=700, E=24, k=4, s=4, H=512, D=256, n_shared=0)
    inp = _gen(cfg)
    hin = synth.to_host(inp)
    idx, w, _, _ = moe.route(router="sigmoid", k=cfg.k, E=cfg.E, s=cfg.s, logits=inp["logits"],
                             expert_bias=inp["expert_bias"], route_scale=cfg.route_scale)
    start, L = 5, 11
    ew = moe.ExpertWeights.from_stacked(inp["w_gate_up"][start:start + L].contiguous(),
                                        inp["w_down"][start:start + L].contiguous())
    g = torch.Generator(device=DEV)
    g.manual_seed(9)
    sgu_all = torch.rand((cfg.E,), generator=g, device=DEV) + 0.5
    sd_all = torch.rand((cfg.E,), generator=g, device=DEV) + 0.5
    mask = (torch.rand((cfg.T,), generator=g, device=DEV) > 0.3).to(torch.uint8)
    ind = moe.build_indices(idx, L, expert_start=start, weights=w, token_mask=mask)
    O_ = moe.grouped_ffn(ind["offsets"], cfg.T * cfg.k, ew, x=inp["x"], sorted_token=ind["sorted_token"],
                         gate_up_expert_scales=sgu_all[start:start + L].contiguous(),
                         down_expert_scales=sd_all[start:start + L].contiguous())
    y = moe.combine(O_, ind["row_of_slot"], cfg.T, cfg.k, weights=w, token_mask=mask)
    torch.cuda.synchronize()
    y_ref = O.layer(hin, cfg, indices=host(idx), weights=host(w).astype(np.float64),
                    token_mask=host(mask), expert_start=start, num_local=L,
                    gate_up_expert_scales=host(sgu_all), down_expert_scales=host(sd_all))
    valid = host(mask) != 0
    # the output RMS is taken over the valid tokens: masked rows are zero by definition
    err, _ = rel_rms_err(host(y)[valid], y_ref[valid])
    say(f"  slice+scales y err/rms = {err:.3e} (bf16 floor {bf16_floor(y_ref[valid]):.3e})")
    assert err <= BF16_TOL
    assert np.all(host(y)[~valid] == 0)


@pytest.mark.parametrize("mode", ["one_expert", "half_empty", "k_eq_E", "single_expert"])
def test_layer_routing_edge_cases(moe, mode):
    base = synth.scaled(synth.get_config(1), T=200, H=256, D=256)
    if mode == "k_eq_E":
        cfg = synth.scaled(base, E=4, k=4)
    elif mode == "single_expert":
        cfg = synth.scaled(base, E=1, k=1)
    else:
        cfg = synth.scaled(base, E=8, k=2)
    inp = _gen(cfg)
    T, E, k = cfg.T, cfg.E, cfg.k
    if mode in ("one_expert", "half_empty"):
        idx, w = _routing(T, E, k, 1, mode)
    else:
        idx = np.tile(np.arange(k, dtype=np.int32), (T, 1))
        w = np.random.default_rng(2).random((T, k)).astype(np.float32)
    it, wt = torch.from_numpy(idx).to(DEV), torch.from_numpy(w).to(DEV)
    ew = moe.ExpertWeights.from_stacked(inp["w_gate_up"], inp["w_down"])
    ind = moe.build_indices(it, E, weights=wt)
    O_ = moe.grouped_ffn(ind["offsets"], T * k, ew, x=inp["x"], sorted_token=ind["sorted_token"])
    y = moe.combine(O_, ind["row_of_slot"], T, k, weights=wt)
    torch.cuda.synchronize()
    y_ref = O.layer(synth.to_host(inp), cfg, indices=idx, weights=w.astype(np.float64))
    err, _ = rel_rms_err(host(y), y_ref)
    say(f"[edge] {mode}: y err/rms = {err:.3e}")
    assert err <= BF16_TOL


def test_grouped_ffn_rows_and_determinism(moe):
    """Expert rows O against the oracle's per-expert MLP, and two runs
    bit-identical (no atomics on floating point anywhere)."""
    cfg = synth.scaled(synth.get_config(4), T=600, H=640, D=448, E=5, k=2)
    inp = _gen(cfg)
    layer, r1 = _run_layer(moe, cfg, inp)
    O1 = r1["O"].clone()
    y1 = r1["y"].clone()
    r2 = layer.forward(inp["x"])
    torch.cuda.synchronize()
    assert torch.equal(O1, r2["O"]) and torch.equal(y1, r2["y"])
    hin = synth.to_host(inp)
    ind = r1["index"]
    off = host(ind["offsets"])
    st = host(ind["sorted_token"])
    Oh = host(O1)
    for e in range(cfg.E):
        rows = np.arange(off[e], off[e + 1])
        if rows.size == 0:
            continue
        ref = O.expert_mlp(hin["x"][st[rows]], hin["w_gate_up"][e], hin["w_down"][e], fmt=cfg.gate_up_format,
                           activation=cfg.activation, alpha=cfg.alpha, limit=cfg.limit,
                           b_gate_up=hin["b_gate_up"][e], b_down=hin["b_down"][e])
        err, _ = rel_rms_err(Oh[rows], ref)
        assert err <= 1e-2, f"expert {e}: O err/rms {err:.3e}"


@pytest.mark.parametrize("D", [4096, 4040])
def test_down_split_k_tail_round(moe, D):
    """A down GEMM whose tiles fill less than half of one round is split
    along K (D = 4040 also gives the last part a ragged k stage): the expert
    rows match the oracle's per-expert MLP, two runs are bit-identical, every
    partial slot the split needs was written and the arrival counters are
    back at zero afterwards."""
    cfg = synth.scaled(synth.get_config(2), T=256, H=512, D=D, E=4, k=2)
    inp = _gen(cfg)
    R = cfg.T * cfg.k
    layer = moe.MoELayer(cfg, inp)
    act_bytes = (R * D * 2 + 255) // 256 * 256
    counters = layer.act_ws[act_bytes:act_bytes + 256 * 4].view(torch.int32)
    partial = layer.act_ws[act_bytes + 256 * 4:].view(torch.float32)
    partial.fill_(float("nan"))
    r1 = layer.forward(inp["x"])
    torch.cuda.synchronize()
    # the split the kernel derives from the tile count and the CU count
    G = torch.cuda.get_device_properties(0).multi_processor_count
    off = host(r1["index"]["offsets"])
    tiles = sum((int(off[e + 1] - off[e]) + 255) // 256 for e in range(cfg.E)) * ((cfg.H + 255) // 256)
    slots = min(256, R // 16)
    rem = tiles % G
    S = min(4, G // rem, slots // rem, ((D + 63) // 64) // 4) if 0 < rem and 2 * rem <= G else 1
    say(f"[split] D={D} tiles={tiles} G={G} S={S}")
    assert S >= 2, "the case is meant to exercise the split"
    assert torch.all(counters == 0)
    written = partial[: rem * S * 256 * 256].view(rem * S, -1)
    assert not torch.isnan(written).any(dim=1).any(), "a split part left its partial slot unwritten"
    O1 = r1["O"].clone()
    r2 = layer.forward(inp["x"])
    torch.cuda.synchronize()
    assert torch.equal(O1, r2["O"])
    hin = synth.to_host(inp)
    st = host(r1["index"]["sorted_token"])
    Oh = host(O1)
    for e in range(cfg.E):
        rows = np.arange(off[e], off[e + 1])
        if rows.size == 0:
            continue
        ref = O.expert_mlp(hin["x"][st[rows]], hin["w_gate_up"][e], hin["w_down"][e], fmt=cfg.gate_up_format,
                           activation=cfg.activation, alpha=cfg.alpha, limit=cfg.limit)
        err, _ = rel_rms_err(Oh[rows], ref)
        say(f"  expert {e}: O err/rms {err:.3e}")
        assert err <= 1e-2, f"expert {e}: O err/rms {err:.3e}"


def test_shared_indices(moe):
    for T, n in [(1, 1), (77, 2), (8192, 2), (300, 5)]:
        off, st = moe.shared_indices(T, n, torch.device(DEV))
        torch.cuda.synchronize()
        assert np.array_equal(host(off), np.arange(n + 1) * T)
        assert np.array_equal(host(st)[: n * T], np.tile(np.arange(T), n))


@pytest.mark.parametrize("cid,changes,nsample", [
    (1, {"T": 256, "n_shared": 1, "shared_dim": 256}, 256),                   # always-on, weight 1
    (1, {"T": 200, "n_shared": 3, "shared_dim": 136}, 200),                   # several, ragged dims
    (4, {"T": 300, "H": 512, "D": 384, "E": 6, "k": 2, "n_shared": 2, "shared_dim": 256}, 300),  # bias, interleaved
    (3, {"T": 700, "E": 32, "D": 256, "shared_dim": 512}, 700),               # sink-gated, two lanes
])
def test_layer_with_shared_experts(moe, cid, changes, nsample):
    cfg = synth.scaled(synth.get_config(cid), **changes)
    inp = _gen(cfg)
    say(f"[shared] cfg={cid} {changes}")
    _, res = _run_layer(moe, cfg, inp)
    _check_routing(cfg, inp, res)
    _check_layer(cfg, inp, res, sample_tokens(cfg.T, nsample), BF16_TOL)
    # masked tokens give zero rows, shared experts included
    mask = torch.ones(cfg.T, dtype=torch.uint8, device=DEV)
    mask[::7] = 0
    _, res_m = _run_layer(moe, cfg, inp, token_mask=mask)
    ym = host(res_m["y"])
    assert np.all(ym[host(mask) == 0] == 0)
    _check_layer(cfg, inp, res_m, sample_tokens(cfg.T, nsample), BF16_TOL, token_mask=host(mask))


def test_abi_errors_on_gpu_path(moe):
    """Invalid arguments are refused before any launch, also from the binding."""
    x = torch.zeros((4, 24), dtype=torch.bfloat16, device=DEV)
    wg = torch.zeros((8, 24), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(moe.MoEError):
        moe.route(router="softmax", k=9, E=8, x=x, w_gate=wg)
    with pytest.raises(moe.MoEError):
        moe.route(router="sigmoid", k=3, E=8, s=0, logits=torch.zeros((4, 8), device=DEV))


# ---------------------------------------------------------------- fp8 block-scaled path

def _check_fp8_act(cfg, inp, res, layer):
    """The re-quantised activation against the oracle's re-quantisation of its
    own activation.  The two activations differ by float32 rounding, so a code
    may land one e4m3 step away where a value sits near a rounding boundary;
    the dequantised values must agree to within one step of the row scale."""
    hin = synth.to_host(inp)
    ind = res["index"]
    off = host(ind["offsets"])
    st = host(ind["sorted_token"])
    R, D = layer.R, cfg.D
    n = int(off[-1])
    ws = host(layer.act_ws)
    codes_gpu = ws[: R * D].reshape(R, D)[:n]
    so = ((R * D + 255) // 256) * 256
    scale_gpu = ws[so: so + R * (D // 128) * 4].view(np.float32).reshape(R, D // 128)[:n]
    xq = O.layer_inputs_x(hin, "fp8")
    same = total = 0
    worst = 0.0
    for e in range(cfg.E):
        rows = np.arange(off[e], off[e + 1])
        if rows.size == 0:
            continue
        wgu = O.dequant_weight_block128(hin["w_gate_up"][e], hin["w_gate_up_scale"][e])
        h = xq[st[rows]] @ wgu
        a = O.gated_activation(h[:, :D], h[:, D:], cfg.activation, cfg.alpha, cfg.limit).astype(np.float32)
        codes_ref, sc_ref = O.quantize_rows_block128(a)
        cg = codes_gpu[rows]
        same += int(np.sum(cg == codes_ref))
        total += cg.size
        deq_g = O.dequant_rows_block128(cg, scale_gpu[rows])
        deq_r = O.dequant_rows_block128(codes_ref, sc_ref)
        # one e4m3 step at the value in the normal range; in the subnormal
        # range (|q| < 2^-6, absolute steps of 2^-9) values this close to zero
        # move by a few steps for float32-level differences of the activation,
        # so there the bound is the smallest normal 2^-6 -- all in units of the
        # (oracle) row scale
        step = np.maximum(np.abs(O.e4m3_decode(codes_ref)) * 2.0 ** -3, 2.0 ** -6) * np.repeat(sc_ref, 128, axis=1)
        ratio = np.abs(deq_g - deq_r) / step
        worst = max(worst, float(ratio.max()))
    frac = same / max(total, 1)
    say(f"  fp8 activation codes identical: {frac:.5f}; worst |gpu - oracle| = {worst:.3f} e4m3 steps")
    # each side rounds to the nearest code (half a step each) and the two
    # activations differ at float32 level: two steps bound the sum
    assert frac >= 0.99
    assert worst <= 2.0


@pytest.mark.parametrize("changes,nsample,gather", [
    ({"T": 512, "E": 8, "H": 512, "D": 256}, 512, True),
    ({"T": 512, "E": 8, "H": 512, "D": 256}, 512, False),
    ({"T": 2048, "E": 16, "k": 4}, 256, True),              # full hidden / moe dims of the fp8 layer
])
def test_fp8_layer_small(moe, changes, nsample, gather):
    cfg = synth.scaled(synth.get_config(5), **changes)
    inp = _gen(cfg)
    say(f"[fp8 layer] {changes} gather={gather}")
    layer, res = _run_layer(moe, cfg, inp, gather=gather)
    _check_routing(cfg, inp, res)
    _check_fp8_act(cfg, inp, res, layer)
    _check_layer(cfg, inp, res, sample_tokens(cfg.T, nsample, seed=3), FP8_TOL)


def test_fp8_zero_scales(moe):
    """Zero block scales (with nonzero codes under them) contribute nothing,
    also in the first k block of a tile, and all-zero tokens (scale 1, zero
    codes) pass through: the GEMMs keep their accumulator units across them."""
    cfg = synth.scaled(synth.get_config(5), T=512, E=8, H=512, D=256)
    inp = _gen(cfg)
    gus, ds = inp["w_gate_up_scale"], inp["w_down_scale"]   # [E, H/128, 2D/128], [E, D/128, H/128]
    gus[0, 0, :] = 0.0          # expert 0: the first k block of every gate_up column block
    gus[1, 2, 0] = 0.0          # expert 1: one gate block in the middle of K
    gus[2, :, 3] = 0.0          # expert 2: a whole up column block
    ds[3, 1, :] = 0.0           # expert 3: a down k block
    ds[4, :, 2] = 0.0           # expert 4: a whole down column block
    inp["x"][5:9] = 0.0         # whole tokens at zero
    inp["x"][20, 128:256] = 0.0  # one zero 128-group of a token
    say("[fp8 zero scales]")
    layer, res = _run_layer(moe, cfg, inp)
    _check_fp8_act(cfg, inp, res, layer)
    _check_layer(cfg, inp, res, np.arange(cfg.T), FP8_TOL)


def test_fp8_layer_full_size(moe):
    cfg = synth.get_config(5)
    inp = _gen(cfg)
    say("[fp8 layer full] T=16384 H=7168 E=256 k=8 D=2048")
    _, res = _run_layer(moe, cfg, inp)
    _check_routing(cfg, inp, res)
    _check_layer(cfg, inp, res, sample_tokens(cfg.T, 12, seed=5), FP8_TOL)


# ---------------------------------------------------------------- MX: MXFP4 weights x MXFP8 activations

@pytest.mark.parametrize("mode", ["mxfp8_tokens", "mxfp8"])
def test_mx_permute(moe, mode):
    """MXFP8 quantisation of the activations: codes and E8M0 scale bytes
    bit-exact, including an all-zero block, bf16 subnormals and a block
    whose largest value saturates."""
    T, E, k, H = 3000, 16, 3, 7168
    idx, _ = _routing(T, E, k, 12)
    g = torch.Generator(device=DEV)
    g.manual_seed(6)
    x = (torch.randn((T, H), generator=g, device=DEV) * 3).to(torch.bfloat16)
    x[5, :32] = 0
    x[7, 32:64] = (torch.randn(32, generator=g, device=DEV) * 1e-39).to(torch.bfloat16)
    x[9, 64:96] = (torch.randn(32, generator=g, device=DEV) * 1e30).to(torch.bfloat16)
    x[11, 96:128] = 511.0                 # scales into 511 > 448: saturates
    say(f"[mx permute] {mode} T={T} H={H}")
    out = moe.build_indices(torch.from_numpy(idx).to(DEV), E, x=x, xperm_dtype=mode)
    ref = O.build_indices(idx, E)
    n = int(host(out["offsets"])[-1])
    codes, sc = O.mxfp8_quantize_rows(host(x))
    if mode == "mxfp8_tokens":
        assert np.array_equal(host(out["x_perm"])[:T], codes)
        assert np.array_equal(host(out["x_perm_scale"])[:T], sc)
    else:
        assert np.array_equal(host(out["x_perm"])[:n], codes[ref["sorted_token"]])
        assert np.array_equal(host(out["x_perm_scale"])[:n], sc[ref["sorted_token"]])


def _check_mx_act(cfg, inp, res, layer):
    """The MXFP8 re-quantised activation against the oracle's re-quantisation
    of its own activation.  A value near a rounding boundary (or a block max
    near a power of two, which moves the shared exponent) may land one step
    away; dequantised, the two must agree within two steps of the coarser of
    the two encodings."""
    hin = synth.to_host(inp)
    ind = res["index"]
    off = host(ind["offsets"])
    st = host(ind["sorted_token"])
    R, D = layer.R, cfg.D
    n = int(off[-1])
    ws = host(layer.act_ws)
    codes_gpu = ws[: R * D].reshape(R, D)[:n]
    so = ((R * D + 255) // 256) * 256
    scale_gpu = ws[so: so + R * (D // 32)].reshape(R, D // 32)[:n]
    xq = O.layer_inputs_x(hin, "mxfp4")
    same = total = 0
    worst = 0.0
    for e in range(cfg.E):
        rows = np.arange(off[e], off[e + 1])
        if rows.size == 0:
            continue
        wgu = O.mx_dequant_fp4(hin["w_gate_up"][e], hin["w_gate_up_scale"][e]).T
        h = xq[st[rows]] @ wgu
        if cfg.has_bias:
            h = h + hin["b_gate_up"][e].astype(np.float64)[None, :]
        gg, uu = O.split_gate_up(h, cfg.gate_up_format)
        a = O.gated_activation(gg, uu, cfg.activation, cfg.alpha, cfg.limit).astype(np.float32)
        codes_ref, sc_ref = O.mxfp8_quantize_rows(a)
        cg = codes_gpu[rows]
        same += int(np.sum(cg == codes_ref))
        total += cg.size
        deq_g = O.mx_dequant_fp8(cg, scale_gpu[rows])
        deq_r = O.mx_dequant_fp8(codes_ref, sc_ref)

        def step(c, s):   # one e4m3 step at the value (2^-6 of the scale in the subnormal range)
            return np.maximum(np.abs(O.e4m3_decode(c)) * 2.0 ** -3, 2.0 ** -6) * np.repeat(O.e8m0_decode(s), 32, axis=1)
        ratio = np.abs(deq_g - deq_r) / np.maximum(step(codes_ref, sc_ref), step(cg, scale_gpu[rows]))
        worst = max(worst, float(ratio.max()))
    frac = same / max(total, 1)
    say(f"  MXFP8 activation codes identical: {frac:.5f}; worst |gpu - oracle| = {worst:.3f} e4m3 steps")
    assert frac >= 0.99
    assert worst <= 2.0


@pytest.mark.parametrize("changes,nsample,gather", [
    ({"T": 512, "E": 8, "H": 512, "D": 256}, 512, True),
    ({"T": 512, "E": 8, "H": 512, "D": 256}, 512, False),
    ({"T": 300, "E": 5, "k": 2, "H": 128, "D": 128}, 300, True),      # one k stage in each GEMM
    ({"T": 777, "E": 6, "k": 4, "H": 384, "D": 640, "activation": "swigluoai", "alpha": 1.702, "limit": 7.0,
      "gate_up_format": "interleaved", "has_bias": True}, 777, True),
    ({"T": 400, "E": 4, "k": 2, "H": 256, "D": 384, "activation": "gelu_tanh", "has_bias": True}, 400, False),
    ({"T": 2048, "E": 16, "k": 4}, 256, True),                # full hidden / moe dims of the layer
])
def test_mx_layer_small(moe, changes, nsample, gather):
    cfg = synth.scaled(synth.get_config(6), **changes)
    inp = _gen(cfg)
    say(f"[mx layer] {changes} gather={gather}")
    layer, res = _run_layer(moe, cfg, inp, gather=gather)
    _check_routing(cfg, inp, res)
    _check_mx_act(cfg, inp, res, layer)
    _check_layer(cfg, inp, res, sample_tokens(cfg.T, nsample, seed=4), FP8_TOL)


def test_mx_layer_full_size(moe):
    cfg = synth.get_config(6)
    inp = _gen(cfg)
    say("[mx layer full] T=16384 H=7168 E=256 k=8 D=2048 MXFP4 W4A8")
    _, res = _run_layer(moe, cfg, inp)
    _check_routing(cfg, inp, res)
    _check_layer(cfg, inp, res, sample_tokens(cfg.T, 12, seed=6), FP8_TOL)


@pytest.mark.parametrize("changes,nsample,gather", [
    ({"T": 512, "E": 8, "H": 512, "D": 256}, 512, True),
    ({"T": 300, "E": 5, "k": 2, "H": 384, "D": 128}, 300, False),   # one k stage in the down GEMM
    ({"T": 777, "E": 6, "k": 4, "H": 384, "D": 640, "activation": "swigluoai", "alpha": 1.702, "limit": 7.0,
      "gate_up_format": "interleaved", "has_bias": True}, 777, True),
    ({"T": 64, "E": 32, "k": 4, "H": 1024, "D": 512, "activation": "gelu_tanh", "has_bias": True}, 64, True),
    # at most 32 rows per expert on average: the 32-row tile with the 6-stage pipeline
    ({"T": 40, "E": 16, "k": 2, "H": 256, "D": 384, "activation": "swigluoai", "alpha": 1.702, "limit": 7.0,
      "gate_up_format": "interleaved", "has_bias": True}, 40, False),
])
def test_mx_w4a16_layer_small(moe, changes, nsample, gather):
    cfg = synth.scaled(synth.get_config(7), **changes)
    inp = _gen(cfg)
    say(f"[mx w4a16 layer] {changes} gather={gather}")
    _, res = _run_layer(moe, cfg, inp, gather=gather)
    _check_routing(cfg, inp, res)
    _check_layer(cfg, inp, res, sample_tokens(cfg.T, nsample, seed=7), BF16_TOL)


def test_mx_w4a16_layer_full_size(moe):
    cfg = synth.get_config(7)
    inp = _gen(cfg)
    say("[mx w4a16 layer full] T=256 H=7168 E=256 k=8 D=2048 MXFP4 W4A16")
    _, res = _run_layer(moe, cfg, inp)
    _check_routing(cfg, inp, res)
    _check_layer(cfg, inp, res, sample_tokens(cfg.T, 8, seed=8), BF16_TOL)



# ---------------------------------------------------------------- single-launch L1 + L2 (bf16)

@pytest.mark.parametrize("changes", [
    {"T": 64, "E": 8, "k": 2, "H": 512, "D": 256},
    {"T": 37, "E": 8, "k": 2, "H": 256, "D": 384, "activation": "swigluoai", "alpha": 1.702, "limit": 7.0,
     "gate_up_format": "interleaved", "has_bias": True},
    {"T": 200, "E": 5, "k": 3, "H": 320, "D": 128, "activation": "gelu_tanh", "has_bias": True},
    {"T": 9, "E": 64, "k": 6, "H": 1024, "D": 512},          # most experts empty, single rows
    {"T": 50, "E": 4, "k": 2, "H": 320, "D": 1664, "has_bias": True},  # down split in 3 uneven parts, N tail
    {"T": 33, "E": 3, "k": 1, "H": 128, "D": 1152, "activation": "swigluoai", "alpha": 1.702, "limit": 7.0},  # 5 parts
])
def test_fused_ffn_layer(moe, changes):
    """The single-launch FFN against the oracle, twice in a row on the same
    workspace (the second call reuses the control words the first left at
    zero), with no timed-out wait, and against the two-launch FFN."""
    cfg = synth.scaled(synth.get_config(8), **changes)
    inp = _gen(cfg)
    say(f"[fused] {changes}")
    layer = moe.MoELayer(cfg, inp)
    assert layer.fused
    for call in range(2):
        res = layer.forward(inp["x"])
        torch.cuda.synchronize()
        _check_layer(cfg, inp, res, np.arange(cfg.T), BF16_TOL)
        assert moe.fused_error_word(layer.act_ws) == 0, f"call {call}: a wait timed out"
    ind = res["index"]
    n = int(host(ind["offsets"])[-1])
    o_fused = host(res["O"])[:n].astype(np.float64)
    o_two = moe.grouped_ffn(ind["offsets"], layer.R, layer.w, x=inp["x"], sorted_token=ind["sorted_token"],
                            activation=cfg.activation, alpha=cfg.alpha, limit=cfg.limit,
                            gate_up_format=cfg.gate_up_format)
    torch.cuda.synchronize()
    err, _ = rel_rms_err(o_fused, host(o_two)[:n].astype(np.float64))
    say(f"  fused vs two-launch O: max err / rms = {err:.2e}")
    assert err <= BF16_TOL


def test_fused_ffn_permuted_rows(moe):
    """The single-launch FFN on permuted rows (x_perm) instead of the gather."""
    cfg = synth.scaled(synth.get_config(8), T=48, E=6, k=2, H=256, D=1024, has_bias=True)
    inp = _gen(cfg)
    say("[fused x_perm] T=48 E=6 k=2 H=256 D=1024 (down split in 2 parts)")
    layer = moe.MoELayer(cfg, inp, gather=False)
    assert layer.fused
    res = layer.forward(inp["x"])
    torch.cuda.synchronize()
    _check_layer(cfg, inp, res, np.arange(cfg.T), BF16_TOL)
    assert moe.fused_error_word(layer.act_ws) == 0


def test_fused_ffn_then_smaller_batch(moe):
    """Two calls in a row, the second with fewer tokens and a different
    routing: the first call's arrival counters must not leak into the second."""
    big = synth.scaled(synth.get_config(8), T=128, H=512, D=256)
    small = synth.scaled(big, T=17)
    inp_b, inp_s = _gen(big), synth.make_inputs(small, DEV, salt=3)
    say("[fused] T=128 then T=17 on one workspace")
    lb = moe.MoELayer(big, inp_b)
    ls = moe.MoELayer(small, inp_s)
    ls.act_ws = lb.act_ws        # one workspace, sized for the larger call
    rb = lb.forward(inp_b["x"])
    rs = ls.forward(inp_s["x"])
    torch.cuda.synchronize()
    _check_layer(big, inp_b, rb, np.arange(big.T), BF16_TOL)
    _check_layer(small, inp_s, rs, np.arange(small.T), BF16_TOL)
    assert moe.fused_error_word(lb.act_ws) == 0


def test_fused_ffn_big_small_big(moe):
    """One workspace sized for 4096 rows, called with 4096, then 34, then
    4096 rows again: a smaller call must not disturb the control words a
    larger call needs (the arrival counters sit at the end of the buffer,
    A and the split partials in front of them)."""
    big = synth.scaled(synth.get_config(8), T=2048, H=256, D=1024)
    small = synth.scaled(big, T=17)
    inp_b, inp_s = _gen(big), synth.make_inputs(small, DEV, salt=5)
    say("[fused] T=2048, T=17, T=2048 on one workspace (down split in 2 parts)")
    lb = moe.MoELayer(big, inp_b)
    ls = moe.MoELayer(small, inp_s)
    ls.act_ws = lb.act_ws
    for name, layer, cfg, inp in (("big", lb, big, inp_b), ("small", ls, small, inp_s), ("big again", lb, big, inp_b)):
        res = layer.forward(inp["x"])
        torch.cuda.synchronize()
        say(f"  {name}")
        _check_layer(cfg, inp, res, np.arange(cfg.T), BF16_TOL)
        assert moe.fused_error_word(lb.act_ws) == 0, name


def test_fused_ffn_full_size(moe):
    cfg = synth.get_config(8)
    inp = _gen(cfg)
    say("[fused full] Mixtral decode T=64 H=4096 E=8 k=2 D=14336, one launch")
    layer, res = _run_layer(moe, cfg, inp)
    _check_routing(cfg, inp, res)
    _check_layer(cfg, inp, res, sample_tokens(cfg.T, 16, seed=9), BF16_TOL)
    assert moe.fused_error_word(layer.act_ws) == 0
