"""Plain, slow CPU oracle of the MoE FFN backward pass (routed experts, bf16).

TEST INFRASTRUCTURE.  Only the tests may import this module.  It shares no
code with the HIP library and imports nothing from it.

What it computes.  The forward pass of moe_oracle (StackedMoE page weight
shapes, GatedActivation page activations, the down bias inside the router
weighting of _apply_bias on the nemo_automodel experts page, the per-leg
expert scales of the mega_ffn page) is

    h_p = s_gu[e] * (x_t . W_gu[e]) + b_gu[e]       (p: a routed row of token t, expert e)
    a_p = act(split(h_p))                            stored in bf16
    o_p = s_d[e] * (a_p . W_d[e]) + b_d[e]
    y_t = sum_j w[t, j] * o_{p(t, j)}

Given dy = dL/dy its gradients follow by the chain rule:

    dO_p      = w[t, j] * dy_t                      (stored in bf16)
    dw[t, j]  = <dy_t, o_p>                          (the router-weight gradient)
    dA_p      = s_d * dO_p . W_d[e]^T                (stored in bf16)
    dH_p      = [dA_p * d act / d gate, dA_p * d act / d up]   (dL/dh, stored in bf16,
                                                      in W_gu's column order)
    dX_p      = s_gu * dH_p . W_gu[e]^T
    dx_t      = sum_j dX_{p(t, j)}
    dW_gu[e]  = s_gu * sum_p x_t^T dH_p,   db_gu[e] = sum_p dH_p
    dW_d[e]   = s_d  * sum_p a_p^T dO_p,   db_d[e]  = sum_p dO_p

The bias gradients are the per-expert segmented sums of the nemo_automodel
experts page (_DeterministicBiasRepeatInterleave.backward, the deterministic
bias-gradient reduction): one sum per expert over its contiguous rows.

Precision: float64; the intermediates the layer stores (dO, the recomputed
A, dA, dH) are rounded to bf16 at the same points, unless round_bf16=False
(used by the finite-difference pins, which differentiate the unrounded
forward).  The expert scales are constants here: no gradient is taken for
them.
"""
from __future__ import annotations

import numpy as np

from oracle.moe_oracle import (GELU_TANH_A, GELU_TANH_C, _sigmoid64, bf16_round, gated_activation,
                               split_gate_up)


def _bf(a, on):
    return bf16_round(a).astype(np.float64) if on else np.asarray(a, np.float64)


def gated_activation_grad(gate, up, kind, alpha=0.0, limit=0.0):
    """Partial derivatives (d act / d gate, d act / d up) of the GatedActivation
    page's activations, with respect to the unclamped gate and up.

    The clamps (silu and swigluoai with limit > 0: gate = min(gate, limit),
    up = clamp(up, -limit, limit)) pass the gradient where the input lies
    inside the closed range, and block it outside, as a clamp's derivative."""
    g0 = np.asarray(gate, np.float64)
    u0 = np.asarray(up, np.float64)
    mg = np.ones_like(g0)
    mu = np.ones_like(u0)
    g, u = g0, u0
    if kind in ("silu", "swigluoai") and limit > 0:
        g = np.minimum(g0, limit)
        u = np.clip(u0, -limit, limit)
        mg = (g0 <= limit).astype(np.float64)
        mu = ((u0 >= -limit) & (u0 <= limit)).astype(np.float64)
    if kind == "silu":
        s = _sigmoid64(g)
        dg = s * (1.0 + g * (1.0 - s)) * u
        du = g * s
    elif kind == "swigluoai":
        s = _sigmoid64(alpha * g)
        dg = (s + alpha * g * s * (1.0 - s)) * (u + 1.0)
        du = g * s
    elif kind == "gelu_tanh":
        t = np.tanh(GELU_TANH_C * (g + GELU_TANH_A * g ** 3))
        gelu = 0.5 * g * (1.0 + t)
        dgelu = 0.5 * (1.0 + t) + 0.5 * g * (1.0 - t * t) * GELU_TANH_C * (1.0 + 3.0 * GELU_TANH_A * g * g)
        dg = dgelu * u
        du = gelu
    else:
        raise ValueError(f"unknown activation {kind!r}")
    return dg * mg, du * mu


def merge_gate_up(dg, du, fmt):
    """Inverse of split_gate_up: place the gate and up columns in W_gu's
    column order (concatenated [gate | up], or interleaved even/odd)."""
    dg = np.asarray(dg, np.float64)
    du = np.asarray(du, np.float64)
    out = np.empty(dg.shape[:-1] + (2 * dg.shape[-1],), np.float64)
    if fmt == "concatenated":
        out[..., : dg.shape[-1]] = dg
        out[..., dg.shape[-1]:] = du
    elif fmt == "interleaved":
        out[..., 0::2] = dg
        out[..., 1::2] = du
    else:
        raise ValueError(fmt)
    return out


def combine_backward(dy, expert_out, row_of_slot, n_rows, expert_weights=None, token_mask=None,
                     round_bf16=True):
    """Backward of the router-weighted combine:
    dO[row_of_slot[t, j]] = w[t, j] * dy[t] (bf16), and dw[t, j] = <dy[t], O[row]>
    (float64).  Rows of dropped slots and masked tokens get nothing; weights
    None means weight 1 (then dw is None)."""
    dy = np.asarray(dy, np.float64)
    rs = np.asarray(row_of_slot, np.int64)
    T, k = rs.shape
    O = np.asarray(expert_out, np.float64)
    valid = np.ones(T, bool) if token_mask is None else np.asarray(token_mask).astype(bool)
    dO = np.zeros((n_rows, dy.shape[1]), np.float64)
    dw = None if expert_weights is None else np.zeros((T, k), np.float64)
    for j in range(k):
        r = rs[:, j]
        ok = (r >= 0) & valid
        w = np.ones(T) if expert_weights is None else np.asarray(expert_weights, np.float64)[:, j]
        dO[r[ok]] = w[ok, None] * dy[ok]
        if dw is not None:
            dw[ok, j] = np.einsum("th,th->t", dy[ok], O[r[ok]])
    return _bf(dO, round_bf16), dw


def expert_backward(x_rows, dO_rows, w_gate_up, w_down, *, fmt="concatenated", activation="silu",
                    alpha=0.0, limit=0.0, b_gate_up=None, gate_up_scale=1.0, down_scale=1.0,
                    round_bf16=True):
    """One expert's backward on a block of its rows (float64).

    x_rows [n, H] and dO_rows [n, H] are the rows' inputs and output
    gradients; W_gate_up is [H, 2D] and W_down [D, H] (StackedMoE shapes).
    Returns A, dA, dH (per row), dX [n, H], dW_gu [H, 2D], dW_d [D, H],
    db_gu [2D], db_d [H].  The weight and bias gradients are sums over the
    rows given; the per-row results do not depend on the other rows."""
    x = np.asarray(x_rows, np.float64)
    dO = np.asarray(dO_rows, np.float64)
    wgu = np.asarray(w_gate_up, np.float64)
    wd = np.asarray(w_down, np.float64)
    h = float(gate_up_scale) * (x @ wgu)
    if b_gate_up is not None:
        h = h + np.asarray(b_gate_up, np.float64)[None, :]
    g, u = split_gate_up(h, fmt)
    a = _bf(gated_activation(g, u, activation, alpha, limit), round_bf16)
    dA = _bf(float(down_scale) * (dO @ wd.T), round_bf16)
    dg, du = gated_activation_grad(g, u, activation, alpha, limit)
    dH = _bf(merge_gate_up(dg * dA, du * dA, fmt), round_bf16)
    return {
        "A": a, "dA": dA, "dH": dH,
        "dX": float(gate_up_scale) * (dH @ wgu.T),
        "dW_gu": float(gate_up_scale) * (x.T @ dH),
        "dW_d": float(down_scale) * (a.T @ dO),
        "db_gu": dH.sum(axis=0),
        "db_d": dO.sum(axis=0),
    }


def expert_backward_cols(x_rows, dO_rows, w_gate_up, w_down, cols, *, fmt="concatenated",
                         activation="silu", alpha=0.0, limit=0.0, b_gate_up=None, gate_up_scale=1.0,
                         down_scale=1.0, round_bf16=True):
    """expert_backward restricted to the outputs `cols` of the D intermediate
    columns, for sampled checks at full size: for each c in cols, the gate
    and up rows of dW_gu^T (dW_gu[:, gate(c)], dW_gu[:, up(c)], as [len, H]),
    the row dW_d[c, :], db_gu at gate(c) and up(c), and dA, dH at those
    columns.  Each needs only columns c of A and dA, and columns gate(c),
    up(c) of h."""
    x = np.asarray(x_rows, np.float64)
    dO = np.asarray(dO_rows, np.float64)
    wgu = np.asarray(w_gate_up, np.float64)
    wd = np.asarray(w_down, np.float64)
    cols = np.asarray(cols, np.int64)
    D = wd.shape[0]
    gi = cols if fmt == "concatenated" else 2 * cols
    ui = D + cols if fmt == "concatenated" else 2 * cols + 1
    hg = float(gate_up_scale) * (x @ wgu[:, gi])
    hu = float(gate_up_scale) * (x @ wgu[:, ui])
    if b_gate_up is not None:
        b = np.asarray(b_gate_up, np.float64)
        hg = hg + b[gi][None, :]
        hu = hu + b[ui][None, :]
    a = _bf(gated_activation(hg, hu, activation, alpha, limit), round_bf16)
    dA = _bf(float(down_scale) * (dO @ wd[cols].T), round_bf16)
    dg, du = gated_activation_grad(hg, hu, activation, alpha, limit)
    dHg = _bf(dg * dA, round_bf16)
    dHu = _bf(du * dA, round_bf16)
    return {
        "gate_idx": gi, "up_idx": ui, "A": a, "dA": dA, "dH_gate": dHg, "dH_up": dHu,
        "dW_gu_gate": float(gate_up_scale) * (dHg.T @ x),
        "dW_gu_up": float(gate_up_scale) * (dHu.T @ x),
        "dW_d_rows": float(down_scale) * (a.T @ dO),
        "db_gu_gate": dHg.sum(axis=0), "db_gu_up": dHu.sum(axis=0),
    }


def segment_sums(rows, offsets):
    """Per-segment column sums: out[e] = sum of rows[offsets[e]:offsets[e+1]]
    (float64), the shape of the bias-gradient reduction."""
    rows = np.asarray(rows, np.float64)
    off = np.asarray(offsets, np.int64)
    out = np.zeros((off.size - 1, rows.shape[1]), np.float64)
    for e in range(off.size - 1):
        out[e] = rows[off[e]:off[e + 1]].sum(axis=0)
    return out


def layer_backward(x, dy, sorted_token, offsets, row_of_slot, expert_weights, w_gate_up, w_down, *,
                   expert_out=None, token_mask=None, fmt="concatenated", activation="silu", alpha=0.0,
                   limit=0.0, b_gate_up=None, gate_up_scales=None, down_scales=None, round_bf16=True):
    """The whole routed-expert backward on a bucketing (sorted_token, offsets,
    row_of_slot as moe_oracle.build_indices returns them).  x [T, H] and dy
    [T, H]; w_gate_up [L, H, 2D], w_down [L, D, H] (stacked shapes);
    expert_out O [R, H] is the forward's expert output rows (needed for the
    router-weight gradient; None skips it).  Returns dx [T, H], dO, dH, dX
    per row, dW_gu [L, H, 2D], dW_d [L, D, H], db_gu [L, 2D], db_d [L, H],
    dw [T, k]."""
    x = np.asarray(x, np.float64)
    off = np.asarray(offsets, np.int64)
    st = np.asarray(sorted_token, np.int64)
    L = off.size - 1
    R = int(off[-1])
    H = x.shape[1]
    D = np.asarray(w_down).shape[1]
    O = np.zeros((R, H)) if expert_out is None else expert_out
    dO, dw = combine_backward(dy, O, row_of_slot, R, expert_weights, token_mask, round_bf16)
    if expert_out is None:
        dw = None
    dX = np.zeros((R, H))
    dH = np.zeros((R, 2 * D))
    dW_gu = np.zeros((L, H, 2 * D))
    dW_d = np.zeros((L, D, H))
    db_gu = np.zeros((L, 2 * D))
    db_d = np.zeros((L, H))
    for e in range(L):
        p0, p1 = int(off[e]), int(off[e + 1])
        if p1 == p0:
            continue
        r = expert_backward(x[st[p0:p1]], dO[p0:p1], w_gate_up[e], w_down[e], fmt=fmt, activation=activation,
                            alpha=alpha, limit=limit,
                            b_gate_up=None if b_gate_up is None else b_gate_up[e],
                            gate_up_scale=1.0 if gate_up_scales is None else gate_up_scales[e],
                            down_scale=1.0 if down_scales is None else down_scales[e], round_bf16=round_bf16)
        dX[p0:p1] = r["dX"]
        dH[p0:p1] = r["dH"]
        dW_gu[e], dW_d[e], db_gu[e], db_d[e] = r["dW_gu"], r["dW_d"], r["db_gu"], r["db_d"]
    # dx[t] = sum over the token's kept slots of its rows of dX (weight 1)
    rs = np.asarray(row_of_slot, np.int64)
    dx = np.zeros((x.shape[0], H))
    for j in range(rs.shape[1]):
        ok = rs[:, j] >= 0
        dx[ok] += dX[rs[ok, j]]
    return {"dx": dx, "dO": dO, "dH": dH, "dX": dX, "dW_gu": dW_gu, "dW_d": dW_d, "db_gu": db_gu,
            "db_d": db_d, "dw": dw}
