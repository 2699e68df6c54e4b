"""Pins of the backward oracle (oracle/moe_backward.py), all on the CPU.

Every gradient is checked against central finite differences of the forward
oracle (itself pinned in test_oracle_pins.py) with intermediates unrounded,
so a dropped term, a wrong sign, a transposed operand or a mixed-up gate/up
column fails here.  The bias-gradient reduction is checked against plain
Python loops, and the sampled-column form against the full one.
"""
import itertools

import numpy as np
import pytest

from oracle import moe_backward as B
from oracle import moe_oracle as O

ACTS = [("silu", 0.0, 0.0), ("silu", 0.0, 0.6), ("swigluoai", 1.702, 0.6), ("swigluoai", 1.702, 0.0),
        ("gelu_tanh", 0.0, 0.0)]
FMTS = ["concatenated", "interleaved"]


def _fd(f, a, idx, eps=1e-6):
    a0 = a[idx]
    a[idx] = a0 + eps
    fp = f()
    a[idx] = a0 - eps
    fm = f()
    a[idx] = a0
    return (fp - fm) / (2 * eps)


def _away_from_clamps(rng, shape, scale, limit):
    """Random values none of which sits within 1e-3 of +-limit (a clamp's kink)."""
    v = rng.normal(0, scale, shape)
    if limit > 0:
        bad = np.abs(np.abs(v) - limit) < 1e-3
        v[bad] += 0.01
    return v


@pytest.mark.parametrize("kind,alpha,limit", ACTS)
def test_activation_grad_matches_finite_differences(kind, alpha, limit):
    rng = np.random.default_rng(1)
    g = _away_from_clamps(rng, 400, 2.0, limit)
    u = _away_from_clamps(rng, 400, 2.0, limit)
    dg, du = B.gated_activation_grad(g, u, kind, alpha, limit)
    eps = 1e-6
    fg = (O.gated_activation(g + eps, u, kind, alpha, limit) - O.gated_activation(g - eps, u, kind, alpha, limit)) / (2 * eps)
    fu = (O.gated_activation(g, u + eps, kind, alpha, limit) - O.gated_activation(g, u - eps, kind, alpha, limit)) / (2 * eps)
    np.testing.assert_allclose(dg, fg, rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(du, fu, rtol=1e-6, atol=1e-8)
    if limit > 0:
        # beyond the clamps the gradient is exactly zero
        assert np.all(dg[g > limit] == 0.0)
        assert np.all(du[np.abs(u) > limit] == 0.0)
        assert np.any(g > limit) and np.any(np.abs(u) > limit)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("kind,alpha,limit", ACTS)
def test_expert_backward_matches_finite_differences(fmt, kind, alpha, limit):
    rng = np.random.default_rng(2)
    n, H, D = 3, 5, 4
    x = rng.normal(0, 1, (n, H))
    wgu = rng.normal(0, 0.5, (H, 2 * D))
    wd = rng.normal(0, 0.5, (D, H))
    bgu = rng.normal(0, 0.3, 2 * D)
    bd = rng.normal(0, 0.3, H)
    sgu, sd = 1.3, 0.7
    dO = rng.normal(0, 1, (n, H))

    def loss():
        o = O.expert_mlp(x, wgu, wd, fmt=fmt, activation=kind, alpha=alpha, limit=limit, b_gate_up=bgu,
                         b_down=bd, gate_up_scale=sgu, down_scale=sd, act_format="none")
        return float(np.sum(o * dO))

    # keep every pre-activation off the clamp kinks
    h = sgu * x @ wgu + bgu
    if limit > 0:
        assert np.min(np.abs(np.abs(h) - limit)) > 1e-4
    r = B.expert_backward(x, dO, wgu, wd, fmt=fmt, activation=kind, alpha=alpha, limit=limit, b_gate_up=bgu,
                          gate_up_scale=sgu, down_scale=sd, round_bf16=False)
    for name, arr in (("dX", x), ("dW_gu", wgu), ("dW_d", wd), ("db_gu", bgu), ("db_d", bd)):
        for idx in itertools.product(*[range(s) for s in arr.shape]):
            fd = _fd(loss, arr, idx)
            assert abs(r[name][idx] - fd) <= 1e-6 * (1 + abs(fd)), (name, idx, r[name][idx], fd)


def _tiny_routing(rng, T, E, k, mask=None):
    logits = rng.normal(0, 1, (T, E)).astype(np.float32)
    idx, w = O.route_softmax_topk(logits, k)
    ind = O.build_indices(idx, E, token_mask=mask, expert_weights=w)
    ind["row_of_slot"] = ind["row_of_slot"].reshape(T, k)
    return idx, w, ind


@pytest.mark.parametrize("fmt", FMTS)
def test_layer_backward_matches_finite_differences(fmt):
    """Gradients of L = sum(y * dy) with respect to x, the routing weights and
    every expert parameter, routing held fixed, through the router-weighted
    combine and the per-expert bucketing (one masked token)."""
    rng = np.random.default_rng(3)
    T, E, k, H, D = 6, 3, 2, 4, 3
    mask = np.ones(T, np.uint8)
    mask[4] = 0
    idx, w, ind = _tiny_routing(rng, T, E, k, mask)
    w = np.asarray(w, np.float64).copy()
    x = rng.normal(0, 1, (T, H))
    wgu = rng.normal(0, 0.5, (E, H, 2 * D))
    wd = rng.normal(0, 0.5, (E, D, H))
    bgu = rng.normal(0, 0.3, (E, 2 * D))
    sgu = np.array([1.0, 0.8, 1.2])
    sd = np.array([0.9, 1.1, 1.0])
    dy = rng.normal(0, 1, (T, H))
    st, off, rs = ind["sorted_token"], ind["offsets"], ind["row_of_slot"]
    kw = dict(fmt=fmt, activation="swigluoai", alpha=1.702, limit=0.0)

    def forward_rows():
        o = np.zeros((int(off[-1]), H))
        for e in range(E):
            p0, p1 = int(off[e]), int(off[e + 1])
            if p1 > p0:
                o[p0:p1] = O.expert_mlp(x[st[p0:p1]], wgu[e], wd[e], b_gate_up=bgu[e], gate_up_scale=sgu[e],
                                        down_scale=sd[e], act_format="none", **kw)
        return o

    def loss():
        y = O.combine(forward_rows(), rs, w, mask)
        return float(np.sum(y * dy))

    r = B.layer_backward(x, dy, st, off, rs, w, wgu, wd, expert_out=forward_rows(), token_mask=mask,
                         b_gate_up=bgu, gate_up_scales=sgu, down_scales=sd, round_bf16=False, **kw)
    for name, arr in (("dx", x), ("dw", w), ("dW_gu", wgu), ("dW_d", wd), ("db_gu", bgu)):
        for idx_ in itertools.product(*[range(s) for s in arr.shape]):
            fd = _fd(loss, arr, idx_)
            assert abs(r[name][idx_] - fd) <= 1e-6 * (1 + abs(fd)), (name, idx_, r[name][idx_], fd)
    # the masked token and its slots carry no gradient
    assert np.all(r["dx"][4] == 0) and np.all(r["dw"][4] == 0)


def test_segment_sums_against_loops():
    rng = np.random.default_rng(4)
    rows = rng.normal(0, 1, (23, 5))
    off = [0, 0, 7, 7, 19, 23]
    want = [[sum(rows[p][c] for p in range(off[e], off[e + 1])) for c in range(5)] for e in range(5)]
    np.testing.assert_allclose(B.segment_sums(rows, off), np.array(want), rtol=1e-14, atol=1e-14)


def test_combine_backward_against_loops():
    rng = np.random.default_rng(5)
    T, E, k, H = 7, 4, 2, 3
    mask = np.ones(T, np.uint8)
    mask[2] = 0
    idx, w, ind = _tiny_routing(rng, T, E, k, mask)
    R = int(ind["offsets"][-1])
    dy = rng.normal(0, 1, (T, H))
    Oe = rng.normal(0, 1, (R, H))
    dO, dw = B.combine_backward(dy, Oe, ind["row_of_slot"], R, w, mask, round_bf16=False)
    rs = ind["row_of_slot"]
    for t in range(T):
        for j in range(k):
            p = rs[t][j]
            if p < 0:
                assert dw[t][j] == 0
                continue
            for h in range(H):
                assert abs(dO[p][h] - w[t][j] * dy[t][h]) < 1e-15
            assert abs(dw[t][j] - sum(dy[t][h] * Oe[p][h] for h in range(H))) < 1e-12
    assert np.all(rs[2] == -1)


@pytest.mark.parametrize("fmt", FMTS)
def test_sampled_columns_match_full(fmt):
    rng = np.random.default_rng(6)
    n, H, D = 9, 6, 5
    x = O.bf16_round(rng.normal(0, 1, (n, H))).astype(np.float64)
    wgu = O.bf16_round(rng.normal(0, 0.3, (H, 2 * D))).astype(np.float64)
    wd = O.bf16_round(rng.normal(0, 0.3, (D, H))).astype(np.float64)
    bgu = rng.normal(0, 0.1, 2 * D)
    dO = O.bf16_round(rng.normal(0, 1, (n, H))).astype(np.float64)
    kw = dict(fmt=fmt, activation="silu", limit=0.5, b_gate_up=bgu, gate_up_scale=1.1, down_scale=0.9)
    full = B.expert_backward(x, dO, wgu, wd, **kw)
    cols = [0, 3, 4]
    c = B.expert_backward_cols(x, dO, wgu, wd, cols, **kw)
    np.testing.assert_array_equal(c["dH_gate"], full["dH"][:, c["gate_idx"]])
    np.testing.assert_array_equal(c["dH_up"], full["dH"][:, c["up_idx"]])
    np.testing.assert_allclose(c["dW_gu_gate"], full["dW_gu"][:, c["gate_idx"]].T, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(c["dW_gu_up"], full["dW_gu"][:, c["up_idx"]].T, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(c["dW_d_rows"], full["dW_d"][cols], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(c["db_gu_gate"], full["db_gu"][c["gate_idx"]], rtol=1e-13, atol=1e-13)


def test_rounded_intermediates_are_bf16():
    rng = np.random.default_rng(7)
    n, H, D = 4, 8, 6
    r = B.expert_backward(rng.normal(0, 1, (n, H)), O.bf16_round(rng.normal(0, 1, (n, H))),
                          rng.normal(0, 0.3, (H, 2 * D)), rng.normal(0, 0.3, (D, H)))
    for name in ("A", "dA", "dH"):
        v = r[name]
        np.testing.assert_array_equal(O.bf16_round(v).astype(np.float64), v)
