"""GPU parity of the backward pass (moe_combine_backward, moe_grouped_ffn_backward,
moe_transpose_bf16) against the backward oracle, through the C ABI.

Each step gets the GPU's own inputs (routing, bucketing, O, dO), so that a
difference belongs to that step.  Bars:
  * dO: each element within one bf16 step of the oracle's bf16(w * dy)
    (the GPU rounds the float32 product);
  * the router-weight gradient dw: max error <= 1e-5 x rms (float32 dots);
  * dX, dx, dW_gu, dW_d, db_gu, db_d: max error <= 2e-2 x rms, the bar of the
    bf16 forward (the backward stores dA, the recomputed A and dH in bf16 as
    the forward stores A);
  * experts with no rows: exactly zero weight and bias gradients;
  * two runs bit-identical; the transpose bit-exact.
"""
import numpy as np
import pytest
import torch

import synth
from oracle import moe_backward as B
from oracle import moe_oracle as O
from tests.gpu_util import host, rel_rms_err, sample_tokens, say

pytestmark = pytest.mark.gpu

DEV = "cuda"
BF16_TOL = 2e-2
DW_TOL = 1e-5


@pytest.fixture(scope="module")
def moe():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import mixture_experts_ffn_top_amd as m
    m.lib()
    return m


def _check(name, got, want, tol=BF16_TOL):
    err, rms = rel_rms_err(got, want)
    say(f"  {name}: max err / rms = {err:.2e} (rms {rms:.3e})")
    assert err <= tol, f"{name}: {err:.3e} > {tol:.1e}"


def _check_dO(got, want):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert np.all(np.abs(got - want) <= np.abs(want) * 2.0 ** -7), "dO: more than one bf16 step off"
    same = float(np.mean(got == want))
    say(f"  dO: {same * 100:.3f} % identical to the oracle's")
    assert same >= 0.99


def _backward_case(moe, cfg, *, gather=True, mask=None, salt=0):
    inp = synth.make_inputs(cfg, DEV, salt=salt)
    say(f"[bwd] T={cfg.T} H={cfg.H} E={cfg.E} k={cfg.k} D={cfg.D} {cfg.activation} {cfg.gate_up_format} "
        f"bias={cfg.has_bias} gather={gather} mask={mask is not None}")
    layer = moe.MoELayer(cfg, inp, gather=gather)
    mask_t = None if mask is None else torch.from_numpy(mask).to(DEV)
    res = layer.forward(inp["x"], token_mask=mask_t)
    dy = synth.make_grad_output(cfg, DEV, salt=salt)
    g = layer.backward(dy)
    torch.cuda.synchronize()
    return inp, res, dy, g, layer


def _oracle_ffn(cfg, inp, res, dO_rows):
    """The oracle's expert backward on the GPU's bucketing and dO."""
    ind = res["index"]
    off = host(ind["offsets"]).astype(np.int64)
    st = host(ind["sorted_token"]).astype(np.int64)
    x = host(inp["x"]).astype(np.float64)
    wgu = host(inp["w_gate_up"]).astype(np.float64)
    wd = host(inp["w_down"]).astype(np.float64)
    bgu = host(inp["b_gate_up"]).astype(np.float64) if cfg.has_bias else None
    L, R = cfg.E, int(off[-1])
    out = {"dX": np.zeros((R, cfg.H)), "dW_gu": np.zeros((L, cfg.H, 2 * cfg.D)), "dW_d": np.zeros((L, cfg.D, cfg.H)),
           "db_gu": np.zeros((L, 2 * cfg.D)), "db_d": np.zeros((L, cfg.H))}
    for e in range(L):
        p0, p1 = int(off[e]), int(off[e + 1])
        if p1 == p0:
            continue
        r = B.expert_backward(x[st[p0:p1]], dO_rows[p0:p1], wgu[e], wd[e], fmt=cfg.gate_up_format,
                              activation=cfg.activation, alpha=cfg.alpha, limit=cfg.limit,
                              b_gate_up=None if bgu is None else bgu[e])
        out["dX"][p0:p1] = r["dX"]
        for kk in ("dW_gu", "dW_d", "db_gu", "db_d"):
            out[kk][e] = r[kk]
    return out, off


def _compare_all(cfg, inp, res, dy, g, mask=None):
    T, k, H = cfg.T, cfg.k, cfg.H
    ind = res["index"]
    rs = host(ind["row_of_slot"]).astype(np.int64).reshape(T, k)
    off = host(ind["offsets"]).astype(np.int64)
    R = int(off[-1])
    O_gpu = host(res["O"])[:R]
    dO_ref, dw_ref = B.combine_backward(host(dy), O_gpu, rs, R, host(res["weights"]), mask)
    dO_gpu = host(g["dO"])[:R].astype(np.float64)
    _check_dO(dO_gpu, dO_ref)
    _check("dw", host(g["dw"]), dw_ref, DW_TOL)
    ref, off = _oracle_ffn(cfg, inp, res, dO_gpu)
    _check("d_x_perm", host(g["d_x_perm"])[:R], ref["dX"])
    dx_ref = np.zeros((T, H))
    for j in range(k):
        ok = rs[:, j] >= 0
        dx_ref[ok] += ref["dX"][rs[ok, j]]
    _check("dx", host(g["dx"]), dx_ref)
    _check("d_w_gate_up", host(g["d_w_gate_up"]), ref["dW_gu"].transpose(0, 2, 1))
    _check("d_w_down", host(g["d_w_down"]), ref["dW_d"].transpose(0, 2, 1))
    if cfg.has_bias:
        _check("d_b_gate_up", host(g["d_b_gate_up"]), ref["db_gu"])
        _check("d_b_down", host(g["d_b_down"]), ref["db_d"])
    empty = np.nonzero(off[1:] == off[:-1])[0]
    for e in empty:
        assert np.all(host(g["d_w_gate_up"][e]) == 0) and np.all(host(g["d_w_down"][e]) == 0), f"expert {e}"
        if cfg.has_bias:
            assert np.all(host(g["d_b_gate_up"][e]) == 0) and np.all(host(g["d_b_down"][e]) == 0)
    if mask is not None:
        assert np.all(host(g["dx"])[mask == 0] == 0)
    return empty


@pytest.mark.parametrize("changes", [
    {},                                                          # the tiny workload: T=64 H=256 E=8 top-2 D=512
    {"T": 50, "E": 4, "k": 2, "H": 192, "D": 320, "activation": "swigluoai", "alpha": 1.702, "limit": 7.0,
     "gate_up_format": "interleaved", "has_bias": True},
    {"T": 33, "E": 5, "k": 3, "H": 128, "D": 256, "activation": "gelu_tanh", "has_bias": True},
    {"T": 300, "E": 3, "k": 2, "H": 320, "D": 128},              # several 256-row blocks, ragged M and N tails
    {"T": 8, "E": 16, "k": 2, "H": 64, "D": 64},                 # most experts empty
    {"T": 1, "E": 4, "k": 1, "H": 64, "D": 128, "activation": "silu", "limit": 7.0},
    {"T": 20, "E": 3, "k": 3, "H": 64, "D": 64},                  # k = E: every expert gets every token
    {"T": 40, "E": 1, "k": 1, "H": 128, "D": 128, "has_bias": True},  # one expert
])
def test_backward_small(moe, changes):
    cfg = synth.scaled(synth.get_config(1), **changes)
    inp, res, dy, g, _ = _backward_case(moe, cfg)
    _compare_all(cfg, inp, res, dy, g)


def test_backward_masked_permuted_and_clamped(moe):
    """x_perm (permuted rows) instead of the gather, masked tokens, and x
    scaled up so that the swigluoai clamps block part of the gradient."""
    cfg = synth.scaled(synth.get_config(4), T=96, H=192, E=6, k=3, D=192, x_std=8.0)
    mask = np.ones(cfg.T, np.uint8)
    mask[::7] = 0
    inp, res, dy, g, _ = _backward_case(moe, cfg, gather=False, mask=mask)
    _compare_all(cfg, inp, res, dy, g, mask)


def test_backward_expert_scales(moe):
    """Per-leg expert scales, through moe_grouped_ffn_backward directly."""
    cfg = synth.scaled(synth.get_config(1), T=40, E=4, k=2, H=128, D=192, has_bias=True)
    inp = synth.make_inputs(cfg, DEV)
    say("[bwd scales] T=40 E=4 k=2 H=128 D=192")
    idx, w, _, _ = moe.route(router="softmax", k=cfg.k, E=cfg.E, x=inp["x"], w_gate=inp["w_gate"])
    ind = moe.build_indices(idx, cfg.E, weights=w)
    R = cfg.T * cfg.k
    wts = moe.ExpertWeights.from_stacked(inp["w_gate_up"], inp["w_down"], b_gate_up=inp["b_gate_up"],
                                         b_down=inp["b_down"])
    gen = torch.Generator(device=DEV).manual_seed(5)
    dO = torch.randn((R, cfg.H), generator=gen, device=DEV).to(torch.bfloat16)
    sgu = torch.tensor([1.0, 0.5, 2.0, 0.75], device=DEV)
    sd = torch.tensor([0.25, 1.5, 1.0, 3.0], device=DEV)
    g = moe.grouped_ffn_backward(ind["offsets"], R, wts, dO, x=inp["x"], sorted_token=ind["sorted_token"],
                                 gate_up_expert_scales=sgu, down_expert_scales=sd)
    torch.cuda.synchronize()
    off = host(ind["offsets"]).astype(np.int64)
    st = host(ind["sorted_token"]).astype(np.int64)
    x = host(inp["x"]).astype(np.float64)
    wgu, wd = host(inp["w_gate_up"]).astype(np.float64), host(inp["w_down"]).astype(np.float64)
    bgu = host(inp["b_gate_up"]).astype(np.float64)
    dOh = host(dO).astype(np.float64)
    for e in range(cfg.E):
        p0, p1 = int(off[e]), int(off[e + 1])
        if p1 == p0:
            continue
        r = B.expert_backward(x[st[p0:p1]], dOh[p0:p1], wgu[e], wd[e], b_gate_up=bgu[e],
                              gate_up_scale=float(host(sgu)[e]), down_scale=float(host(sd)[e]))
        _check(f"e{e} d_x_perm", host(g["d_x_perm"])[p0:p1], r["dX"])
        _check(f"e{e} d_w_gate_up", host(g["d_w_gate_up"][e]), r["dW_gu"].T)
        _check(f"e{e} d_w_down", host(g["d_w_down"][e]), r["dW_d"].T)
        _check(f"e{e} d_b_gate_up", host(g["d_b_gate_up"][e]), r["db_gu"])
        _check(f"e{e} d_b_down", host(g["d_b_down"][e]), r["db_d"])


def test_backward_deterministic(moe):
    cfg = synth.scaled(synth.get_config(1), T=200, E=4, k=2, H=256, D=256, has_bias=True)
    inp, res, dy, g1, layer = _backward_case(moe, cfg)
    snap = {kk: v.clone() for kk, v in g1.items() if v is not None}
    g2 = layer.backward(dy)
    torch.cuda.synchronize()
    for kk, v in snap.items():
        assert torch.equal(v, g2[kk]), kk


def test_transpose_bf16(moe):
    gen = torch.Generator(device=DEV).manual_seed(3)
    src = torch.randn((3, 128, 192), generator=gen, device=DEV).to(torch.bfloat16)
    say("[transpose] [3, 128, 192]")
    dst = moe.transpose_bf16(src)
    back = moe.transpose_bf16(dst)
    torch.cuda.synchronize()
    assert torch.equal(dst, src.transpose(1, 2).contiguous())
    assert torch.equal(back, src)


def test_backward_full_size_sampled(moe):
    """The Mixtral-shape layer (T=4096, H=4096, E=8, top-2, D=14336): dO and dw
    in full, dx and dX for sampled tokens, and for two experts the weight
    gradients of sampled intermediate columns."""
    cfg = synth.get_config(2)
    inp, res, dy, g, _ = _backward_case(moe, cfg)
    T, k, H, D = cfg.T, cfg.k, cfg.H, cfg.D
    ind = res["index"]
    rs = host(ind["row_of_slot"]).astype(np.int64).reshape(T, k)
    off = host(ind["offsets"]).astype(np.int64)
    st = host(ind["sorted_token"]).astype(np.int64)
    R = int(off[-1])
    dO_ref, dw_ref = B.combine_backward(host(dy), host(res["O"])[:R], rs, R, host(res["weights"]))
    dO = host(g["dO"])[:R].astype(np.float64)
    _check_dO(dO, dO_ref)
    _check("dw", host(g["dw"]), dw_ref, DW_TOL)
    x = host(inp["x"]).astype(np.float64)
    toks = sample_tokens(T, 6, seed=11)
    need = sorted({int(np.searchsorted(off, rs[t, j], side="right") - 1) for t in toks for j in range(k)})
    dX_ref = {}
    for e in need:
        wgu = host(inp["w_gate_up"][e]).astype(np.float64)
        wd = host(inp["w_down"][e]).astype(np.float64)
        rows = [int(rs[t, j]) for t in toks for j in range(k) if off[e] <= rs[t, j] < off[e + 1]]
        r = B.expert_backward(x[st[rows]], dO[rows], wgu, wd)
        for i, p in enumerate(rows):
            dX_ref[p] = r["dX"][i]
        del wgu, wd
    rows = sorted(dX_ref)
    _check("d_x_perm (sampled rows)", host(g["d_x_perm"])[rows], np.stack([dX_ref[p] for p in rows]))
    dx_ref = np.stack([sum(dX_ref[int(rs[t, j])] for j in range(k)) for t in toks])
    _check("dx (sampled tokens)", host(g["dx"])[toks], dx_ref)
    cols = np.array([0, 1, 777, 8191, D - 1])
    for e in (0, cfg.E - 1):
        p0, p1 = int(off[e]), int(off[e + 1])
        say(f"  expert {e}: {p1 - p0} rows, columns {cols.tolist()}")
        gi, ui = cols, D + cols   # concatenated gate_up
        wmini = torch.cat([inp["w_gate_up"][e][:, gi], inp["w_gate_up"][e][:, ui]], dim=1)
        c = B.expert_backward_cols(x[st[p0:p1]], dO[p0:p1], host(wmini).astype(np.float64),
                                   host(inp["w_down"][e][cols]).astype(np.float64), np.arange(cols.size))
        dwgu = host(g["d_w_gate_up"][e])
        _check("  d_w_gate_up gate rows", dwgu[gi], c["dW_gu_gate"])
        _check("  d_w_gate_up up rows", dwgu[ui], c["dW_gu_up"])
        _check("  d_w_down columns", host(g["d_w_down"][e])[:, cols].T, c["dW_d_rows"])
