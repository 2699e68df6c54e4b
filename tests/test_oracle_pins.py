"""Pins of the CPU oracle to facts outside itself (CPU only).

Each test checks one oracle function against something the pages or the
mathematics fix independently of the oracle's own code: hand-derived worked
examples (tests/golden), closed forms evaluated with mpmath, brute force in
plain Python, invariants, and special cases that reduce to a library routine
(torch's CPU casts and activation functions).
"""
import json
import math
import os

import mpmath
import numpy as np
import pytest
import torch

from oracle import moe_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")
mpmath.mp.dps = 50


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _expr(s):
    return {"0": 0.0, "1": 1.0, "-1": -1.0, "-2": -2.0, "-3": -3.0, "-5": -5.0,
            "ln3": math.log(3.0), "-ln3": -math.log(3.0)}[s]


# ---------------------------------------------------------------- formats

def test_bf16_round_matches_torch_cast():
    rng = np.random.default_rng(1)
    vals = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(10.0) ** rng.integers(-30, 30, 20000).astype(np.float32),
        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.4e38, -3.4e38, 1e-40, np.inf, -np.inf], np.float32),
    ]).astype(np.float32)
    ours = O.bf16_round(vals)
    ref = torch.from_numpy(vals).to(torch.bfloat16).float().numpy()
    assert np.array_equal(ours.view(np.uint32), ref.view(np.uint32))
    assert np.isnan(O.bf16_round(np.array([np.nan], np.float32)))[0]


def test_e4m3_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = O.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    both_nan = np.isnan(ours) & np.isnan(ref)
    assert np.array_equal(ours[~both_nan], ref[~both_nan])
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    assert np.sum(np.isnan(ours)) == 2   # 0x7F and 0xFF


def test_e4m3_encode_roundtrip_midpoints_and_torch():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = O.e4m3_decode(codes).astype(np.float32)
    enc = O.e4m3_encode(vals)
    # -0.0 encodes as 0x80 (sign kept), everything else round-trips exactly
    assert np.array_equal(enc, codes)
    # midpoints between neighbours and +-1 float32 ulp around them, inside +-448
    pos = np.sort(np.unique(np.abs(vals)))
    mids = ((pos[1:] + pos[:-1]) / 2).astype(np.float32)
    probe = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9))])
    probe = np.concatenate([probe, -probe]).astype(np.float32)
    ref = torch.from_numpy(probe).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.e4m3_encode(probe), ref)
    # random values; torch's cast does not saturate, so clamp first for it
    rng = np.random.default_rng(2)
    r = (rng.standard_normal(50000) * 10.0 ** rng.uniform(-4, 3, 50000)).astype(np.float32)
    rc = np.clip(r, -448, 448).astype(np.float32)
    ref = torch.from_numpy(rc).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.e4m3_encode(r), ref)


def test_e4m3_golden_values():
    g = _load("e4m3_values.json")
    vals = np.array([c[0] for c in g["cases"]], np.float32)
    want = np.array([c[1] for c in g["cases"]], np.uint8)
    assert np.array_equal(O.e4m3_encode(vals), want)


def test_block128_quantisation_bounds():
    rng = np.random.default_rng(3)
    a = (rng.standard_normal((7, 384)) * rng.uniform(0.01, 30, (7, 1))).astype(np.float32)
    a[3, 128:256] = 0.0                       # an all-zero group
    codes, s = O.quantize_rows_block128(a)
    assert s.dtype == np.float32 and s.shape == (7, 3)
    assert s[3, 1] == 1.0 and np.all(codes[3, 128:256] == 0)
    deq = O.dequant_rows_block128(codes, s)
    g = a.reshape(7, 3, 128)
    # the amax element of every non-zero group maps to +-448 exactly
    for r in range(7):
        for b in range(3):
            if np.abs(g[r, b]).max() == 0:
                continue
            j = int(np.argmax(np.abs(g[r, b])))
            assert O.e4m3_decode(codes[r, b * 128 + j:b * 128 + j + 1])[0] == math.copysign(448.0, g[r, b, j])
    # relative error <= 2^-4 in the normal range, <= half a subnormal step below it
    scale = np.repeat(s, 128, axis=1).astype(np.float64)
    err = np.abs(deq - a)
    normal = np.abs(a) >= scale * 2.0 ** -6
    assert np.all(err[normal] <= 2.0 ** -4 * np.abs(a[normal]) * (1 + 1e-6))
    assert np.all(err[~normal] <= scale[~normal] * 2.0 ** -10 * (1 + 1e-6))


def test_dequant_weight_block_layout_matches_torch():
    rng = np.random.default_rng(4)
    codes = rng.integers(0, 256, (256, 384), dtype=np.uint8)
    codes[codes == 0x7F] = 0
    codes[codes == 0xFF] = 0
    sc = rng.uniform(0.5, 2.0, (2, 3)).astype(np.float32)
    ours = O.dequant_weight_block128(codes, sc)
    v = torch.from_numpy(codes).view(torch.float8_e4m3fn).double()
    big = torch.from_numpy(np.kron(sc.astype(np.float64), np.ones((128, 128))))
    assert np.array_equal(ours, (v * big).numpy())


# ---------------------------------------------------------------- activations

def _mp_sig(x):
    return 1 / (1 + mpmath.e ** (-x))


@pytest.mark.parametrize("g,u", [(0.0, 1.0), (1.0, 2.0), (-3.0, 0.5), (7.5, -9.0), (-20.0, 3.0), (40.0, 1.0)])
def test_activation_closed_forms(g, u):
    G, U = mpmath.mpf(g), mpmath.mpf(u)
    silu = G * _mp_sig(G) * U
    assert O.gated_activation(np.array([g]), np.array([u]), "silu")[0] == pytest.approx(float(silu), rel=1e-14, abs=1e-300)
    # clamped silu, limit 7: gate <= 7, up in [-7, 7]
    Gc, Uc = min(G, 7), max(min(U, 7), -7)
    cs = Gc * _mp_sig(Gc) * Uc
    assert O.gated_activation(np.array([g]), np.array([u]), "silu", limit=7.0)[0] == pytest.approx(float(cs), rel=1e-14, abs=1e-300)
    # swigluoai with the pages' canonical constants alpha = 1.702, limit = 7.0
    oai = Gc * _mp_sig(mpmath.mpf("1.702") * Gc) * (Uc + 1)
    assert O.gated_activation(np.array([g]), np.array([u]), "swigluoai", alpha=1.702, limit=7.0)[0] == pytest.approx(float(oai), rel=1e-14, abs=1e-300)
    # gelu_tanh with the printed constants
    gel = mpmath.mpf("0.5") * G * (1 + mpmath.tanh(mpmath.mpf("0.7978845608028654") * (G + mpmath.mpf("0.044715") * G ** 3))) * U
    assert O.gated_activation(np.array([g]), np.array([u]), "gelu_tanh")[0] == pytest.approx(float(gel), rel=1e-13, abs=1e-300)


def test_activations_match_torch_library():
    rng = np.random.default_rng(5)
    g = rng.standard_normal(5000) * 6
    u = rng.standard_normal(5000) * 6
    tg, tu = torch.from_numpy(g), torch.from_numpy(u)
    silu = (torch.nn.functional.silu(tg) * tu).numpy()
    assert np.allclose(O.gated_activation(g, u, "silu"), silu, rtol=1e-13, atol=1e-15)
    gelu = (torch.nn.functional.gelu(tg, approximate="tanh") * tu).numpy()
    assert np.allclose(O.gated_activation(g, u, "gelu_tanh"), gelu, rtol=1e-12, atol=1e-12)
    # swigluoai with alpha = 1 and no clamp is silu(g) * (u + 1)
    assert np.allclose(O.gated_activation(g, u, "swigluoai", alpha=1.0, limit=0.0),
                       (torch.nn.functional.silu(tg) * (tu + 1)).numpy(), rtol=1e-13, atol=1e-15)
    # clamps hit exactly +-limit
    a = O.gated_activation(np.array([100.0]), np.array([-100.0]), "silu", limit=7.0)[0]
    assert a == pytest.approx(7.0 / (1 + math.exp(-7.0)) * -7.0, rel=1e-15)
    assert O.gated_activation(np.array([0.0]), np.array([5.0]), "gelu_tanh")[0] == 0.0
    assert O.gated_activation(np.array([0.0]), np.array([5.0]), "silu")[0] == 0.0


# ---------------------------------------------------------------- routers

def test_sink_router_golden():
    g = _load("sink_router_worked.json")
    logits = np.array([[_expr(v) for v in row] for row in g["logits_exprs"]], np.float32)
    E, k, s = g["E"], g["k"], g["s"]
    for t, bias in enumerate([g["expert_bias"], g["expert_bias_token1"]]):
        idx, w, sw = O.route_sigmoid_sink(logits[t:t + 1], E, k, s, np.array(bias, np.float32),
                                          g["route_scale"], g["global_scale"])
        assert idx[0].tolist() == g["expected_indices"][t]
        assert np.allclose(w[0], g["expected_expert_weights"][t], rtol=g["weight_rtol"])
        assert np.allclose(sw[0], g["expected_sink_weights"][t], rtol=g["weight_rtol"])


def test_softmax_router_golden():
    g = _load("softmax_router_worked.json")
    logits = np.array([[_expr(v) for v in row] for row in g["logits_exprs"]], np.float32)
    idx, w = O.route_softmax_topk(logits, g["k"])
    assert idx.tolist() == g["expected_indices"]
    assert np.allclose(w, g["expected_weights"], rtol=g["weight_rtol"])


def _py_topk(keys, k):
    """Brute force: Python's own sort, largest key first, then lower index."""
    return sorted(range(len(keys)), key=lambda i: (-float(keys[i]), i))[:k]


def test_sink_router_identity_and_selection_brute_force():
    rng = np.random.default_rng(6)
    E, k, s = 10, 3, 1
    z = (rng.standard_normal((200, E + s)) * 2).astype(np.float32)
    b = rng.uniform(-0.1, 0.1, E).astype(np.float32)
    idx, w, sw = O.route_sigmoid_sink(z, E, k, s, b, 2.5, 1.5)
    key = O.sigmoid_f32(z[:, :E]) + b
    for t in range(z.shape[0]):
        assert idx[t].tolist() == _py_topk(key[t], k)
        lanes = [mpmath.mpf(float(z[t, i])) for i in idx[t]] + [mpmath.mpf(float(z[t, E + j])) for j in range(s)]
        sig = [_mp_sig(v) for v in lanes]
        tot = mpmath.fsum(sig)
        want = [float(v / tot * mpmath.mpf(2.5) * mpmath.mpf(1.5)) for v in sig]
        got = list(w[t]) + list(sw[t])
        assert np.allclose(got, want, rtol=1e-13)


def test_sigmoid_key_is_the_correctly_rounded_steps():
    rng = np.random.default_rng(7)
    z = (rng.standard_normal(3000) * 8).astype(np.float32)
    got = O.sigmoid_f32(z)
    for zi, gi in zip(z[:500], got[:500]):
        e = np.float32(float(mpmath.e ** (-mpmath.mpf(float(zi)))))
        want = np.float32(1.0) / (np.float32(1.0) + e)
        assert gi == want
    # monotone non-decreasing in z
    o = np.argsort(z)
    assert np.all(np.diff(got[o]) >= 0)


def test_sink_router_underflow_saturation_and_bias():
    E, k, s = 4, 2, 2
    # all lanes far below the sigmoid's float32 underflow: log-sigmoid(z) -> z, weights -> softmax(z)
    z = np.array([[-300.0, -200.0, -250.0, -400.0, -210.0, -220.0]], np.float32)
    idx, w, sw = O.route_sigmoid_sink(z, E, k, s, None, 1.0, 1.0)
    assert idx[0].tolist() == [0, 1]          # all keys are 0.0: ties to the lower index
    lanes = [-300.0, -200.0, -210.0, -220.0]
    m = max(lanes)
    ex = [math.exp(v - m) for v in lanes]
    want = [v / math.fsum(ex) for v in ex]
    got = list(w[0]) + list(sw[0])
    assert np.all(np.isfinite(got))
    assert np.allclose(got, want, rtol=1e-12)
    # saturation: every lane sigmoid -> 1, every weight = scale / (k + s)
    z = np.full((1, 6), 40.0, np.float32)
    idx, w, sw = O.route_sigmoid_sink(z, E, k, s, None, 2.5, 2.0)
    assert np.allclose(list(w[0]) + list(sw[0]), [5.0 / 4] * 4, rtol=1e-15)
    # zero bias: selection is the top-k of the raw logits (sigmoid is monotone)
    rng = np.random.default_rng(8)
    z = (rng.standard_normal((100, E + s)) * 3).astype(np.float32)
    idx, _, _ = O.route_sigmoid_sink(z, E, k, s, None)
    for t in range(100):
        assert idx[t].tolist() == _py_topk(z[t, :E], k)
    # a huge bias forces selection but the weight still uses the raw logit
    b = np.array([0, 0, 0, 100.0], np.float32)
    z = np.array([[3.0, 2.0, 1.0, -9.0, 0.0, 0.0]], np.float32)
    idx, w, sw = O.route_sigmoid_sink(z, E, k, s, b)
    assert idx[0].tolist() == [3, 0]
    sig = [1 / (1 + math.exp(9.0)), 1 / (1 + math.exp(-3.0)), 0.5, 0.5]
    assert np.allclose(list(w[0]) + list(sw[0]), [v / sum(sig) for v in sig], rtol=1e-12)
    # linear in route_scale * global_scale
    _, w1, s1 = O.route_sigmoid_sink(z, E, k, s, b, 1.0, 1.0)
    _, w2, s2 = O.route_sigmoid_sink(z, E, k, s, b, 3.0, 0.5)
    assert np.allclose(w2, 1.5 * w1, rtol=1e-15) and np.allclose(s2, 1.5 * s1, rtol=1e-15)


def test_softmax_router_identities():
    rng = np.random.default_rng(9)
    E, k = 8, 3
    z = (rng.standard_normal((300, E)) * 1.5).astype(np.float32)
    idx, w = O.route_softmax_topk(z, k, 2.0, 0.5)
    idx_full, w_full = O.route_softmax_topk(z, k, renormalize=False)
    for t in range(z.shape[0]):
        assert idx[t].tolist() == _py_topk(z[t], k)
        # full softmax, then restrict to the top-k and renormalise (mpmath)
        ex = [mpmath.e ** mpmath.mpf(float(v)) for v in z[t]]
        tot = mpmath.fsum(ex)
        p = [v / tot for v in ex]
        sel = [p[i] for i in idx[t]]
        ssum = mpmath.fsum(sel)
        assert np.allclose(w[t], [float(v / ssum) for v in sel], rtol=1e-13)
        assert np.allclose(w_full[t], [float(v) for v in sel], rtol=1e-13)
    # k = E renormalised is the full softmax; k = 1 gives weight = scale
    _, wE = O.route_softmax_topk(z, E)
    _, wf = O.route_softmax_topk(z, E, renormalize=False)
    assert np.allclose(wE, wf, rtol=1e-13)
    _, w1 = O.route_softmax_topk(z, 1, 2.0, 0.5)
    assert np.allclose(w1, 1.0, rtol=1e-15)


def test_gate_logits_brute_force():
    rng = np.random.default_rng(10)
    x = O.bf16_round(rng.standard_normal((5, 24)))
    wg = O.bf16_round(rng.standard_normal((3, 24)) * 0.02)
    got = O.gate_logits(x, wg)
    for t in range(5):
        for e in range(3):
            assert got[t, e] == pytest.approx(math.fsum(float(x[t, h]) * float(wg[e, h]) for h in range(24)), rel=1e-14, abs=1e-18)


# ---------------------------------------------------------------- bucketing

def _py_csr(idx, num_local, start, mask):
    T, k = len(idx), len(idx[0])
    lists = [[] for _ in range(num_local)]
    for t in range(T):
        if mask is not None and not mask[t]:
            continue
        for j in range(k):
            e = int(idx[t][j]) - start
            if 0 <= e < num_local:
                lists[e].append(t * k + j)
    return lists


@pytest.mark.parametrize("start,num_local,use_mask", [(0, 16, False), (4, 8, True), (0, 16, True), (15, 1, False)])
def test_build_indices_brute_force_and_invariants(start, num_local, use_mask):
    rng = np.random.default_rng(11 + start)
    T, k, E = 97, 3, 16
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    idx[5] = [0, 1, 2]                 # a few fixed rows
    mask = rng.random(T) > 0.2 if use_mask else None
    w = rng.random((T, k))
    r = O.build_indices(idx, num_local, start, mask, w)
    lists = _py_csr(idx.tolist(), num_local, start, mask)
    off = r["offsets"]
    assert off[0] == 0 and np.all(np.diff(off) >= 0)
    assert [int(off[e + 1] - off[e]) for e in range(num_local)] == [len(v) for v in lists]
    flat = [s for v in lists for s in v]
    assert r["sorted_slot"].tolist() == flat
    assert r["sorted_token"].tolist() == [s // k for s in flat]
    ros = r["row_of_slot"]
    assert np.sum(ros >= 0) == len(flat) == off[-1]
    for p, s in enumerate(flat):
        assert ros[s] == p
        assert r["sorted_weight"][p] == w.reshape(-1)[s]
    for e in range(num_local):
        for p in range(off[e], off[e + 1]):
            assert idx.reshape(-1)[flat[p]] == e + start


def test_permute_combine_roundtrip():
    rng = np.random.default_rng(12)
    T, E, H = 50, 6, 32
    x = O.bf16_round(rng.standard_normal((T, H)))
    idx = rng.integers(0, E, (T, 1)).astype(np.int32)
    r = O.build_indices(idx, E)
    xp = O.permute_rows(x, r["sorted_token"])
    y = O.combine(xp, r["row_of_slot"].reshape(T, 1), np.ones((T, 1)))
    assert np.array_equal(y, x.astype(np.float64))
    mask = np.arange(T) % 3 != 0
    y = O.combine(xp, r["row_of_slot"].reshape(T, 1), None, mask)
    assert np.array_equal(y[mask], x[mask]) and np.all(y[~mask] == 0)


# ---------------------------------------------------------------- expert MLP / layer

class _Cfg:
    def __init__(self, **kw):
        self.__dict__.update(dict(router="softmax", s=0, gate_up_format="concatenated", has_bias=False,
                                  activation="silu", alpha=0.0, limit=0.0, operand_dtype="bf16",
                                  route_scale=1.0, global_scale=1.0))
        self.__dict__.update(kw)


def test_single_expert_is_dense_mlp_brute_force():
    rng = np.random.default_rng(13)
    T, H, D = 4, 6, 3
    x = O.bf16_round(rng.standard_normal((T, H)))
    wgu = O.bf16_round(rng.standard_normal((1, H, 2 * D)) * 0.3)
    wd = O.bf16_round(rng.standard_normal((1, D, H)) * 0.3)
    cfg = _Cfg(T=T, H=H, E=1, k=1, D=D)
    y = O.layer({"x": x, "w_gate_up": wgu, "w_down": wd}, cfg,
                indices=np.zeros((T, 1), np.int32), weights=np.ones((T, 1)))
    for t in range(T):
        a = []
        for d in range(D):
            g = math.fsum(float(x[t, h]) * float(wgu[0, h, d]) for h in range(H))
            u = math.fsum(float(x[t, h]) * float(wgu[0, h, D + d]) for h in range(H))
            a.append(float(O.bf16_round(np.array([g / (1 + math.exp(-g)) * u]))[0]))
        for hh in range(H):
            want = math.fsum(a[d] * float(wd[0, d, hh]) for d in range(D))
            assert y[t, hh] == pytest.approx(want, rel=1e-12, abs=1e-15)


@pytest.mark.parametrize("fmt,act,bias", [("concatenated", "silu", False), ("interleaved", "swigluoai", True),
                                          ("concatenated", "gelu_tanh", True)])
def test_layer_equals_dense_all_experts(fmt, act, bias):
    rng = np.random.default_rng(14)
    T, H, D, E, k = 12, 16, 8, 5, 2
    x = O.bf16_round(rng.standard_normal((T, H)))
    inp = {"x": x, "w_gate_up": O.bf16_round(rng.standard_normal((E, H, 2 * D)) * 0.3),
           "w_down": O.bf16_round(rng.standard_normal((E, D, H)) * 0.3),
           "b_gate_up": O.bf16_round(rng.standard_normal((E, 2 * D)) * 0.1),
           "b_down": O.bf16_round(rng.standard_normal((E, H)) * 0.1)}
    cfg = _Cfg(T=T, H=H, E=E, k=k, D=D, gate_up_format=fmt, activation=act, has_bias=bias,
               alpha=1.702 if act == "swigluoai" else 0.0, limit=7.0 if act == "swigluoai" else 0.0)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    w = rng.random((T, k))
    y = O.layer(inp, cfg, indices=idx, weights=w)
    # dense: every expert on every token, weighted by a sparse [T, E] matrix
    dense = np.zeros((T, E))
    for t in range(T):
        for j in range(k):
            dense[t, idx[t, j]] += w[t, j]
    yd = np.zeros((T, H))
    for e in range(E):
        o = O.expert_mlp(x, inp["w_gate_up"][e], inp["w_down"][e], fmt=fmt, activation=act,
                         alpha=cfg.alpha, limit=cfg.limit,
                         b_gate_up=inp["b_gate_up"][e] if bias else None,
                         b_down=inp["b_down"][e] if bias else None)
        yd += dense[:, e:e + 1] * o
    assert np.allclose(y, yd, rtol=1e-12, atol=1e-14)


def test_interleaved_is_a_column_permutation_of_concatenated():
    rng = np.random.default_rng(15)
    H, D = 16, 8
    x = O.bf16_round(rng.standard_normal((9, H)))
    w_il = O.bf16_round(rng.standard_normal((H, 2 * D)) * 0.3)
    b_il = O.bf16_round(rng.standard_normal(2 * D) * 0.1)
    wd = O.bf16_round(rng.standard_normal((D, H)) * 0.3)
    w_cat = np.concatenate([w_il[:, 0::2], w_il[:, 1::2]], axis=1)
    b_cat = np.concatenate([b_il[0::2], b_il[1::2]])
    a = O.expert_mlp(x, w_il, wd, fmt="interleaved", activation="swigluoai", alpha=1.702, limit=7.0, b_gate_up=b_il)
    b = O.expert_mlp(x, w_cat, wd, fmt="concatenated", activation="swigluoai", alpha=1.702, limit=7.0, b_gate_up=b_cat)
    assert np.allclose(a, b, rtol=1e-13, atol=1e-15)


def test_router_weight_placement_invariance():
    """Weighting the expert output at the combine equals weighting the
    activation before the down projection, with the down bias weighted too
    (the _apply_bias note that the down bias is multiplied by the routing probs)."""
    rng = np.random.default_rng(16)
    H, D = 16, 8
    x = rng.standard_normal((7, H))
    wgu = rng.standard_normal((H, 2 * D)) * 0.3
    wd = rng.standard_normal((D, H)) * 0.3
    bd = rng.standard_normal(H) * 0.1
    p = rng.random(7)
    o = O.expert_mlp(x, wgu, wd, b_down=bd, act_format="none")
    h = x @ wgu
    a = O.gated_activation(h[:, :D], h[:, D:], "silu") * p[:, None]
    alt = a @ wd + p[:, None] * bd[None, :]
    assert np.allclose(p[:, None] * o, alt, rtol=1e-12, atol=1e-14)


def test_expert_scales_are_linear_before_bias():
    rng = np.random.default_rng(17)
    H, D = 16, 8
    x = rng.standard_normal((5, H))
    wgu = rng.standard_normal((H, 2 * D)) * 0.3
    wd = rng.standard_normal((D, H)) * 0.3
    bgu = rng.standard_normal(2 * D) * 0.1
    bd = rng.standard_normal(H) * 0.1
    a = O.expert_mlp(x, wgu, wd, b_gate_up=bgu, b_down=bd, gate_up_scale=4.0, down_scale=0.5, act_format="none")
    b = O.expert_mlp(x, wgu * 4.0, wd * 0.5, b_gate_up=bgu, b_down=bd, act_format="none")
    assert np.allclose(a, b, rtol=1e-13, atol=1e-15)


def test_fp8_layer_uses_dequantised_operands():
    """The fp8 layer equals the plain MLP on dequantised weights and on the
    per-token 1x128 dequantised activations, with A requantised per row."""
    rng = np.random.default_rng(18)
    T, H, D, E, k = 6, 256, 128, 3, 2
    x = O.bf16_round(rng.standard_normal((T, H)))
    wq = rng.integers(0, 0x7E, (E, H, 2 * D), dtype=np.uint8) | (rng.integers(0, 2, (E, H, 2 * D), dtype=np.uint8) << 7)
    wdq = rng.integers(0, 0x60, (E, D, H), dtype=np.uint8) | (rng.integers(0, 2, (E, D, H), dtype=np.uint8) << 7)
    ws = rng.uniform(1e-4, 3e-4, (E, 2, 2)).astype(np.float32)
    wds = rng.uniform(1e-4, 3e-4, (E, 1, 2)).astype(np.float32)
    inp = {"x": x, "w_gate_up": wq, "w_gate_up_scale": ws, "w_down": wdq, "w_down_scale": wds}
    cfg = _Cfg(T=T, H=H, E=E, k=k, D=D, operand_dtype="fp8")
    idx = np.array([[0, 1], [2, 0], [1, 2], [0, 2], [1, 0], [2, 1]], np.int32)
    w = rng.random((T, k))
    y = O.layer(inp, cfg, indices=idx, weights=w)
    tx = torch.from_numpy(x)
    xq = []
    for t in range(T):
        row = []
        for b in range(H // 128):
            g = tx[t, b * 128:(b + 1) * 128]
            s = torch.tensor(float(np.float32(g.abs().max().item()) / np.float32(448.0)), dtype=torch.float32)
            q = (g / s).clamp(-448, 448).to(torch.float8_e4m3fn).double() * s.double()
            row.append(q)
        xq.append(torch.cat(row))
    xq = torch.stack(xq).numpy()
    for t in range(T):
        acc = np.zeros(H)
        for j in range(k):
            e = idx[t, j]
            wgu = torch.from_numpy(wq[e]).view(torch.float8_e4m3fn).double().numpy() * np.kron(ws[e], np.ones((128, 128)))
            wdd = torch.from_numpy(wdq[e]).view(torch.float8_e4m3fn).double().numpy() * np.kron(wds[e], np.ones((128, 128)))
            h = xq[t:t + 1] @ wgu
            a = O.gated_activation(h[:, :D], h[:, D:], "silu").astype(np.float32)
            codes, s = O.quantize_rows_block128(a)
            acc += w[t, j] * (O.dequant_rows_block128(codes, s) @ wdd)[0]
        assert np.allclose(y[t], acc, rtol=1e-12, atol=1e-12)


def test_tokens_subset_and_mask_and_local_slice():
    rng = np.random.default_rng(19)
    T, H, D, E, k = 20, 16, 8, 6, 2
    inp = {"x": O.bf16_round(rng.standard_normal((T, H))),
           "w_gate_up": O.bf16_round(rng.standard_normal((E, H, 2 * D)) * 0.3),
           "w_down": O.bf16_round(rng.standard_normal((E, D, H)) * 0.3)}
    cfg = _Cfg(T=T, H=H, E=E, k=k, D=D)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    w = rng.random((T, k))
    full = O.layer(inp, cfg, indices=idx, weights=w)
    sub = O.layer(inp, cfg, indices=idx, weights=w, tokens=np.array([3, 7, 11]))
    assert np.allclose(sub, full[[3, 7, 11]], rtol=1e-14, atol=1e-16)
    mask = np.arange(T) % 4 != 1
    ym = O.layer(inp, cfg, indices=idx, weights=w, token_mask=mask)
    assert np.all(ym[~mask] == 0) and np.allclose(ym[mask], full[mask], rtol=1e-14, atol=1e-16)
    # two expert-parallel slices add up to the whole layer
    a = O.layer(inp, cfg, indices=idx, weights=w, expert_start=0, num_local=2)
    b = O.layer(inp, cfg, indices=idx, weights=w, expert_start=2, num_local=4)
    assert np.allclose(a + b, full, rtol=1e-12, atol=1e-14)


def test_small_configs_run_end_to_end():
    import synth
    for cid in (1, 3, 4, 6, 7):
        cfg = synth.scaled(synth.get_config(cid), T=16)
        inp = synth.to_host(synth.make_inputs(synth.scaled(cfg, H=min(cfg.H, 256), D=min(cfg.D, 256), E=min(cfg.E, 16)), "cpu"))
        c2 = synth.scaled(cfg, H=min(cfg.H, 256), D=min(cfg.D, 256), E=min(cfg.E, 16))
        r = O.route(inp, c2)
        y = O.layer(inp, c2, indices=r["indices"], weights=r["weights"])
        assert y.shape == (16, c2.H) and np.all(np.isfinite(y))
        if c2.router == "sigmoid_sink":
            tot = r["weights"].sum(1) + r["sink_weights"].sum(1)
            assert np.allclose(tot, c2.route_scale * c2.global_scale, rtol=1e-12)
        else:
            assert np.allclose(r["weights"].sum(1), 1.0, rtol=1e-12)


def test_topk_ties_in_wide_rows_brute_force():
    """Many exactly equal keys in rows wider than numpy's small-sort cutoff:
    the selection must still put equal keys in ascending index order."""
    rng = np.random.default_rng(20)
    E, k = 96, 8
    z = rng.choice(np.array([-1.0, 0.0, 0.5, 2.0], np.float32), size=(60, E))
    idx, _ = O.route_softmax_topk(z, k)
    idx2, _, _ = O.route_sigmoid_sink(z, E, k, 0)
    for t in range(60):
        assert idx[t].tolist() == _py_topk(z[t], k)
        assert idx2[t].tolist() == _py_topk(O.sigmoid_f32(z[t]), k)


def test_combine_brute_force():
    rng = np.random.default_rng(21)
    T, k, H, R = 9, 3, 5, 20
    O_rows = rng.standard_normal((R, H))
    rs = rng.integers(-1, R, (T, k))
    w = rng.random((T, k))
    mask = np.arange(T) != 4
    y = O.combine(O_rows, rs, w, mask)
    for t in range(T):
        for h in range(H):
            want = 0.0 if not mask[t] else math.fsum(w[t, j] * O_rows[rs[t, j], h] for j in range(k) if rs[t, j] >= 0)
            assert y[t, h] == pytest.approx(want, rel=1e-14, abs=1e-15)


@pytest.mark.parametrize("fmt,act", [("concatenated", "silu"), ("interleaved", "swigluoai"), ("concatenated", "gelu_tanh")])
def test_expert_mlp_bias_scales_brute_force(fmt, act):
    """Plain-Python expert MLP with bias, expert scales, either gate_up
    layout and each activation, against expert_mlp."""
    rng = np.random.default_rng(22)
    n, H, D = 3, 5, 4
    x = rng.standard_normal((n, H))
    wgu = rng.standard_normal((H, 2 * D)) * 0.5
    wd = rng.standard_normal((D, H)) * 0.5
    bgu = rng.standard_normal(2 * D) * 0.3
    bd = rng.standard_normal(H) * 0.3
    sgu, sd = 1.5, 0.75
    alpha, limit = (1.702, 7.0) if act == "swigluoai" else (0.0, 0.0)
    got = O.expert_mlp(x, wgu, wd, fmt=fmt, activation=act, alpha=alpha, limit=limit,
                       b_gate_up=bgu, b_down=bd, gate_up_scale=sgu, down_scale=sd, act_format="none")
    for r in range(n):
        h = [sgu * math.fsum(x[r, i] * wgu[i, c] for i in range(H)) + bgu[c] for c in range(2 * D)]
        a = []
        for d in range(D):
            gi, ui = (d, D + d) if fmt == "concatenated" else (2 * d, 2 * d + 1)
            g, u = h[gi], h[ui]
            if act == "silu":
                a.append(g / (1 + math.exp(-g)) * u)
            elif act == "swigluoai":
                g, u = min(g, limit), max(min(u, limit), -limit)
                a.append(g / (1 + math.exp(-alpha * g)) * (u + 1))
            else:
                a.append(0.5 * g * (1 + math.tanh(0.7978845608028654 * (g + 0.044715 * g ** 3))) * u)
        for c in range(H):
            want = sd * math.fsum(a[d] * wd[d, c] for d in range(D)) + bd[c]
            assert got[r, c] == pytest.approx(want, rel=1e-12, abs=1e-14)


def _mlp_brute(xr, wgu, wd):
    """silu gated MLP of one row in Python loops; A rounded to bf16 as stored."""
    H, D2 = wgu.shape
    D = D2 // 2
    a = []
    for d in range(D):
        g = math.fsum(float(xr[h]) * float(wgu[h, d]) for h in range(H))
        u = math.fsum(float(xr[h]) * float(wgu[h, D + d]) for h in range(H))
        a.append(float(O.bf16_round(np.array([g / (1 + math.exp(-g)) * u]))[0]))
    return [math.fsum(a[d] * float(wd[d, hh]) for d in range(D)) for hh in range(wd.shape[1])]


@pytest.mark.parametrize("router", ["sigmoid_sink", "softmax"])
def test_shared_experts_brute_force(router):
    """Shared experts add sum_i sw[t,i] * MLP_i(x[t]) to the routed output:
    sw = the sink-lane weights for the sigmoid router (sink_gate_router_kernel
    page: sink lanes are gated shared experts), 1 for the softmax router's
    always-on shared experts (StackedMoE page: has_shared_experts).  Checked
    against Python loops, and masked tokens stay zero rows."""
    rng = np.random.default_rng(31)
    T, H, D, E, k, S, Ds = 5, 6, 3, 3, 1, 2, 4
    x = O.bf16_round(rng.standard_normal((T, H)))
    inp = {"x": x, "w_gate_up": O.bf16_round(rng.standard_normal((E, H, 2 * D)) * 0.3),
           "w_down": O.bf16_round(rng.standard_normal((E, D, H)) * 0.3),
           "w_gate_up_shared": O.bf16_round(rng.standard_normal((S, H, 2 * Ds)) * 0.3),
           "w_down_shared": O.bf16_round(rng.standard_normal((S, Ds, H)) * 0.3)}
    if router == "sigmoid_sink":
        inp["logits"] = rng.standard_normal((T, E + S)).astype(np.float32) * 2
        inp["expert_bias"] = np.zeros(E, np.float32)
        cfg = _Cfg(T=T, H=H, E=E, k=k, D=D, router=router, s=S, n_shared=S, shared_dim=Ds, route_scale=2.5)
        r = O.route(inp, cfg)
        sw = r["sink_weights"]
    else:
        inp["w_gate"] = O.bf16_round(rng.standard_normal((E, H)))
        cfg = _Cfg(T=T, H=H, E=E, k=k, D=D, n_shared=S, shared_dim=Ds)
        r = O.route(inp, cfg)
        sw = np.ones((T, S))
    y = O.layer(inp, cfg, indices=r["indices"], weights=r["weights"], sink_weights=r["sink_weights"])
    routed = O.layer(inp, _Cfg(**{**cfg.__dict__, "n_shared": 0}), indices=r["indices"], weights=r["weights"])
    for t in range(T):
        want = [0.0] * H
        for i in range(S):
            o = _mlp_brute(x[t], inp["w_gate_up_shared"][i], inp["w_down_shared"][i])
            want = [want[h] + sw[t, i] * o[h] for h in range(H)]
        assert np.allclose(y[t] - routed[t], want, rtol=1e-11, atol=1e-13)
    mask = np.array([1, 0, 1, 1, 0], np.uint8)
    ym = O.layer(inp, cfg, indices=r["indices"], weights=r["weights"], sink_weights=r["sink_weights"],
                 token_mask=mask)
    assert np.all(ym[mask == 0] == 0.0) and np.allclose(ym[mask == 1], y[mask == 1], rtol=0, atol=0)


# ---------------------------------------------------------------- MX formats
# The pages name MXFP4 / MXFP8 (StackedMoE page: mxfp8_activations); the
# element and scale formats are those of the OCP Microscaling v1.0 spec.

def test_e8m0_decode_matches_torch():
    s = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(s).view(torch.float8_e8m0fnu).double().numpy()
    ours = O.e8m0_decode(s)
    assert np.isnan(ours[255]) and np.isnan(ref[255])
    assert np.array_equal(ours[:255], ref[:255])


def test_e2m1_values_match_torch_e4m3_after_rebias():
    """An E2M1 code (s, e, m) is the e4m3fn code with the exponent re-biased
    from 1 to 7 and the mantissa bit widened to 3 bits; its one subnormal
    (0.5) is the e4m3 normal 2^-1.  Decoded by torch's e4m3 cast."""
    for c in range(16):
        s, e, m = c >> 3, (c >> 1) & 3, c & 1
        if e > 0:
            code = (s << 7) | ((e - 1 + 7) << 3) | (m << 2)
        else:
            code = (s << 7) | ((6 << 3) if m else 0)
        ref = torch.tensor([code], dtype=torch.uint8).view(torch.float8_e4m3fn).double().item()
        got = float(O.e2m1_decode(np.array([c]))[0])
        assert got == ref and math.copysign(1.0, got) == math.copysign(1.0, ref), (c, got, ref)


def test_fp4_packing_is_low_nibble_first():
    codes = np.arange(16, dtype=np.uint8)
    packed = np.array([[0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE]], np.uint8)
    assert np.array_equal(O.unpack_fp4(packed)[0], codes)


def _brute_e4m3(v):
    """Nearest finite e4m3fn value (torch decode of every code), ties to the
    even code, saturating at +-448."""
    allc = np.arange(256)
    vals = torch.from_numpy(allc.astype(np.uint8)).view(torch.float8_e4m3fn).double().numpy()
    fin = [c for c in allc if not np.isnan(vals[c])]
    if abs(v) >= 448.0:
        return 0x7E | (0x80 if v < 0 else 0)
    best = None
    for c in fin:
        d = abs(vals[c] - v)
        key = (d, c & 1)
        if best is None or key < best[0]:
            best = (key, c)
    c = best[1]
    if vals[c] == 0.0:
        return 0x80 if math.copysign(1.0, v) < 0 else 0x00
    return c


def test_mxfp8_quantisation_brute_force():
    rng = np.random.default_rng(31)
    rows = [rng.standard_normal(64) * 10.0 ** rng.integers(-6, 6),
            np.zeros(64), np.r_[np.zeros(31), [-3e-38], rng.standard_normal(32) * 1e30],
            np.r_[np.full(32, 448.0), np.full(32, -511.9)], np.r_[np.full(32, 1.0), np.full(32, 0.75)],
            rng.standard_normal(64) * 1e-40]
    a = O.bf16_round(np.stack(rows))
    codes, scales = O.mxfp8_quantize_rows(a)
    for r in range(a.shape[0]):
        for b in range(2):
            blk = a[r, 32 * b:32 * b + 32].astype(np.float64)
            amax = np.abs(blk).max()
            if amax == 0:
                X = 0
            else:
                X = -127
                while amax * 2.0 ** -X >= 512.0:       # smallest X (>= -127) with amax * 2^-X < 512
                    X += 1
            assert scales[r, b] == X + 127, (r, b, scales[r, b], X)
            for j in range(32):
                want = _brute_e4m3(blk[j] * 2.0 ** -X)
                assert codes[r, 32 * b + j] == want, (r, b, j, blk[j], codes[r, 32 * b + j], want)


def test_mx_dequant_fp4_brute_force():
    rng = np.random.default_rng(32)
    packed = rng.integers(0, 256, (3, 32), dtype=np.uint8)      # 3 rows, K = 64
    scales = rng.integers(110, 140, (3, 2), dtype=np.uint8)
    got = O.mx_dequant_fp4(packed, scales)
    sv = torch.from_numpy(scales).view(torch.float8_e8m0fnu).double().numpy()
    for n in range(3):
        for k in range(64):
            nib = (int(packed[n, k // 2]) >> (4 * (k % 2))) & 15
            assert got[n, k] == float(O.e2m1_decode(np.array([nib]))[0]) * sv[n, k // 32]


def test_mxfp4_layer_uses_dequantised_operands():
    """The MXFP4 (W4A8) layer equals the plain MLP on dequantised MXFP4
    weights (rows along the reduction dimension) and per-token MXFP8
    activations, with A requantised to MXFP8 per row."""
    rng = np.random.default_rng(33)
    T, H, D, E, k = 5, 64, 32, 3, 2
    x = O.bf16_round(rng.standard_normal((T, H)))
    wgu = rng.integers(0, 256, (E, 2 * D, H // 2), dtype=np.uint8)
    wgus = rng.integers(118, 123, (E, 2 * D, H // 32), dtype=np.uint8)
    wd = rng.integers(0, 256, (E, H, D // 2), dtype=np.uint8)
    wds = rng.integers(118, 123, (E, H, D // 32), dtype=np.uint8)
    inp = {"x": x, "w_gate_up": wgu, "w_gate_up_scale": wgus, "w_down": wd, "w_down_scale": wds}
    cfg = _Cfg(T=T, H=H, E=E, k=k, D=D, operand_dtype="mxfp4")
    idx = np.array([[0, 1], [2, 0], [1, 2], [0, 2], [1, 0]], np.int32)
    w = rng.random((T, k))
    y = O.layer(inp, cfg, indices=idx, weights=w)

    def deq(p, s):   # element by element, scales through torch
        sv = torch.from_numpy(np.ascontiguousarray(s)).view(torch.float8_e8m0fnu).double().numpy()
        out = np.zeros((p.shape[0], 2 * p.shape[1]))
        for n in range(p.shape[0]):
            for kk in range(out.shape[1]):
                nib = (int(p[n, kk // 2]) >> (4 * (kk % 2))) & 15
                out[n, kk] = O.e2m1_decode(np.array([nib]))[0] * sv[n, kk // 32]
        return out
    xc, xs = O.mxfp8_quantize_rows(x)
    xq = O.e4m3_decode(xc) * np.repeat(torch.from_numpy(xs).view(torch.float8_e8m0fnu).double().numpy(), 32, axis=1)
    for t in range(T):
        acc = np.zeros(H)
        for j in range(k):
            e = idx[t, j]
            h = xq[t:t + 1] @ deq(wgu[e], wgus[e]).T
            a = O.gated_activation(h[:, :D], h[:, D:], "silu").astype(np.float32)
            ac, asc = O.mxfp8_quantize_rows(a)
            aq = O.e4m3_decode(ac) * np.repeat(torch.from_numpy(asc).view(torch.float8_e8m0fnu).double().numpy(), 32, axis=1)
            acc += w[t, j] * (aq @ deq(wd[e], wds[e]).T)[0]
        assert np.allclose(y[t], acc, rtol=1e-12, atol=1e-12)


def test_mxfp4_w4a16_layer_uses_bf16_activations():
    """W4A16: the same MXFP4 weights times the bf16 activations, A stored as
    bf16 -- the plain MLP on element-wise dequantised weights."""
    rng = np.random.default_rng(34)
    T, H, D, E, k = 4, 64, 32, 2, 2
    x = O.bf16_round(rng.standard_normal((T, H)))
    wgu = rng.integers(0, 256, (E, 2 * D, H // 2), dtype=np.uint8)
    wgus = rng.integers(118, 123, (E, 2 * D, H // 32), dtype=np.uint8)
    wd = rng.integers(0, 256, (E, H, D // 2), dtype=np.uint8)
    wds = rng.integers(118, 123, (E, H, D // 32), dtype=np.uint8)
    inp = {"x": x, "w_gate_up": wgu, "w_gate_up_scale": wgus, "w_down": wd, "w_down_scale": wds}
    cfg = _Cfg(T=T, H=H, E=E, k=k, D=D, operand_dtype="mxfp4_a16")
    idx = np.array([[0, 1], [1, 0], [0, 1], [1, 0]], np.int32)
    w = rng.random((T, k))
    y = O.layer(inp, cfg, indices=idx, weights=w)
    for t in range(T):
        acc = np.zeros(H)
        for j in range(k):
            e = idx[t, j]
            wg = np.array([[float(O.e2m1_decode(np.array([(int(wgu[e, n, kk // 2]) >> (4 * (kk % 2))) & 15]))[0])
                            * 2.0 ** (int(wgus[e, n, kk // 32]) - 127) for kk in range(H)] for n in range(2 * D)])
            wdd = np.array([[float(O.e2m1_decode(np.array([(int(wd[e, n, kk // 2]) >> (4 * (kk % 2))) & 15]))[0])
                             * 2.0 ** (int(wds[e, n, kk // 32]) - 127) for kk in range(D)] for n in range(H)])
            h = x[t:t + 1].astype(np.float64) @ wg.T
            a = O.bf16_round(O.gated_activation(h[:, :D], h[:, D:], "silu")).astype(np.float64)
            acc += w[t, j] * (a @ wdd.T)[0]
        assert np.allclose(y[t], acc, rtol=1e-12, atol=1e-12)
