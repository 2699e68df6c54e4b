"""Plain, slow CPU oracle of the MoE FFN forward pass.

TEST INFRASTRUCTURE.  Only the tests, the smoke check of the entry module and
the cpu_baseline leg of the benchmark may import this module.  It shares no
code with the HIP library and imports nothing from it; the product path never
calls it.

What it computes (sources are the five pages this project follows, cited by
page title and section):

* routers -- the softmax top-k gate named by the StackedMoE page (gate_cls /
  MoEGate, router_dtype) and the fused sigmoid + selection-bias router of the
  sink_gate_router_kernel page (its description and its Args list);
* the per-expert bucketing the sink_gate_router_kernel page assigns to
  moe_create_indices, with the outputs listed for _permute_tokens_for_grouped_mm
  on the nemo_automodel.components.moe.experts page;
* the expert MLP: the stacked weights of the StackedMoE page ("Weight tensor
  shapes"), the gated activations of the GatedActivation page
  (fused_activation, alpha, limit), the per-expert biases of _apply_bias and
  the per-leg expert scales of the mega_ffn page;
* the router-weighted combine.

Precision.  Floating point is float64, except where a floating-point value
decides an integer: the router's selection key and the fp8 codes are computed
in float32, the precision the pages fix for scores (scores_type) and for the
activation ("in fp32"), with every float32 step correctly rounded so that the
decision is reproducible.  Stored intermediates are rounded the way the layer
stores them (bf16, e4m3 with 1x128 scales, or MXFP8 for the MXFP4 layer)
before they are used again.

Parity of the whole layer has no worked example on the pages; each part is
pinned separately by the CPU tests (closed forms, identities, brute force,
library special cases).
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
GELU_TANH_C = 0.7978845608028654   # GatedActivation page, "gelu_tanh"
GELU_TANH_A = 0.044715             # GatedActivation page, "gelu_tanh"


# --------------------------------------------------------------------------
# Number formats
# --------------------------------------------------------------------------

def bf16_round(a) -> np.ndarray:
    """Round to bfloat16 (round to nearest even) and return the values as float32.

    Values are first rounded to float32 (the accumulator precision the pages
    name), then to bf16.  NaN stays NaN; overflow rounds to inf as IEEE does.
    """
    a32 = np.ascontiguousarray(np.asarray(a, dtype=np.float64).astype(np.float32))
    u = a32.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) & np.uint64(0xFFFF0000)).astype(np.uint32)
    out = r.view(np.float32).copy()
    out[np.isnan(a32)] = np.nan
    return out


def e4m3_encode(a) -> np.ndarray:
    """float32 values -> OCP float8 e4m3fn codes (uint8), round to nearest even.

    Magnitudes above 448 (the largest finite e4m3fn value) saturate to 448;
    e4m3fn has no infinity.  Subnormals have step 2^-9.  NaN -> 0x7F | sign.
    """
    x = np.asarray(a, dtype=np.float32).astype(np.float64)
    sign = np.signbit(x).astype(np.uint8) << np.uint8(7)
    nan = np.isnan(x)
    ax = np.minimum(np.abs(np.where(nan, 0.0, x)), E4M3_MAX)
    _, e = np.frexp(ax)                       # ax = m * 2^e, m in [0.5, 1)
    ue = np.maximum(e - 1, -6)                # unbiased exponent, clamped to the subnormal one
    step = np.ldexp(1.0, ue - 3)              # 3 mantissa bits
    q = np.rint(ax / step)                    # exact scaling, ties to even
    carry = q >= 16
    ue = np.where(carry, ue + 1, ue)
    q = np.where(carry, 8, q)
    normal = q >= 8
    expf = np.where(normal, ue + 7, 0)
    mant = np.where(normal, q - 8, q)
    code = (expf.astype(np.uint8) << np.uint8(3)) | mant.astype(np.uint8)
    code = np.where(ax == 0, np.uint8(0), code).astype(np.uint8)
    code = code | sign
    code = np.where(nan, np.uint8(0x7F) | sign, code).astype(np.uint8)
    return code


def _e4m3_value(c) -> np.ndarray:
    c = np.asarray(c, dtype=np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    f = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(f == 0, m * 2.0 ** -9, (8 + m) * np.ldexp(1.0, f - 10))
    val = np.where((f == 15) & (m == 7), np.nan, val)
    return s * val


# value of every one of the 256 codes, from the format definition above
_E4M3_TABLE = _e4m3_value(np.arange(256))


def e4m3_decode(codes) -> np.ndarray:
    """OCP float8 e4m3fn codes (uint8) -> float64 values: sign, 4 exponent bits
    (bias 7), 3 mantissa bits; exponent field 0 is subnormal (m * 2^-9);
    0x7F / 0xFF are NaN.  Looked up in the 256-entry table of those values."""
    return _E4M3_TABLE[np.asarray(codes, dtype=np.uint8)]


def quantize_rows_block128(a):
    """Per-row, per-128-column e4m3 quantisation with an fp32 scale per group.

    Group scale s = amax/448 in float32 (s = 1 when amax = 0); each element is
    divided by s in float32 and encoded.  Returns (codes uint8 [N, C],
    scales float32 [N, C/128]).  This is the "per-token 1x128" activation
    quantisation of the FP8 block-scaled layer (StackedMoE page, quant_config
    with block scaling).
    """
    a32 = np.asarray(a, dtype=np.float32)
    n, c = a32.shape
    assert c % 128 == 0
    g = a32.reshape(n, c // 128, 128)
    amax = np.abs(g).max(axis=2)
    s = (amax / np.float32(E4M3_MAX)).astype(np.float32)
    s = np.where(amax == 0, np.float32(1.0), s).astype(np.float32)
    q = (g / s[:, :, None]).astype(np.float32)
    codes = e4m3_encode(q).reshape(n, c)
    return codes, s


def dequant_rows_block128(codes, scales) -> np.ndarray:
    n, c = codes.shape
    v = e4m3_decode(codes).reshape(n, c // 128, 128)
    return (v * np.asarray(scales, np.float64)[:, :, None]).reshape(n, c)


def dequant_weight_block128(codes, scales) -> np.ndarray:
    """[K, N] e4m3 codes with [K/128, N/128] fp32 block scales -> float64 [K, N]."""
    k, n = codes.shape
    v = e4m3_decode(codes).reshape(k // 128, 128, n // 128, 128)
    return (v * np.asarray(scales, np.float64)[:, None, :, None]).reshape(k, n)


# --------------------------------------------------------------------------
# MX block formats (StackedMoE page: optional MXFP4 weights, run W4A8 with
# MXFP8 activations).  The pages name the formats only; their definition is
# the OCP Microscaling (MX) v1.0 specification: 32 consecutive elements along
# the reduction dimension share one E8M0 scale (an 8-bit power-of-two
# exponent, bias 127, 0xFF = NaN); MXFP4 elements are E2M1 (1 sign, 2
# exponent bits with bias 1, 1 mantissa bit, no inf/NaN), MXFP8 elements
# are E4M3 (the OCP e4m3fn format above).
# --------------------------------------------------------------------------

MX_BLOCK = 32
E4M3_EMAX = 8            # largest e4m3 normal: 1.75 * 2^8


def e8m0_decode(s) -> np.ndarray:
    """E8M0 scale bytes -> float64 2^(s - 127); 255 is NaN."""
    s = np.asarray(s, np.int64)
    v = np.ldexp(1.0, s - 127)
    return np.where(s == 255, np.nan, v)


def _e2m1_value(c) -> np.ndarray:
    c = np.asarray(c, np.int64)
    sign = np.where(c & 8, -1.0, 1.0)
    e = (c >> 1) & 3
    m = c & 1
    mag = np.where(e == 0, 0.5 * m, (1.0 + 0.5 * m) * np.ldexp(1.0, e - 1))
    return sign * mag


_E2M1_TABLE = _e2m1_value(np.arange(16))


def e2m1_decode(codes) -> np.ndarray:
    """E2M1 codes (0..15) -> float64: exponent field 0 is subnormal (m * 0.5),
    otherwise (1 + m/2) * 2^(e-1); bit 3 is the sign."""
    return _E2M1_TABLE[np.asarray(codes, np.int64) & 15]


def unpack_fp4(packed) -> np.ndarray:
    """uint8 [..., K/2] -> E2M1 codes [..., K]: element 2i is the low nibble
    of byte i, element 2i+1 the high nibble."""
    p = np.asarray(packed, np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), np.uint8)
    out[..., 0::2] = p & 15
    out[..., 1::2] = p >> 4
    return out


def mx_dequant_fp4(packed, scales) -> np.ndarray:
    """MXFP4 rows: packed codes [N, K/2] and E8M0 scales [N, K/32] -> float64 [N, K]."""
    v = e2m1_decode(unpack_fp4(packed))
    n, k = v.shape
    return (v.reshape(n, k // MX_BLOCK, MX_BLOCK) * e8m0_decode(scales)[:, :, None]).reshape(n, k)


def mxfp8_quantize_rows(a):
    """Per-row MXFP8 quantisation along the columns (blocks of 32).

    For each block: amax = max |v| (float32); a block with amax = 0 gets the
    unit scale (E8M0 127); otherwise the shared exponent is
    X = floor(log2(amax)) - 8 (8 = emax of E4M3), kept >= -127, so that the
    block's largest magnitude scales into [256, 512).  Elements are encoded
    as e4m3(v * 2^-X) with round to nearest even, saturating at 448 (the
    scaling by a power of two is exact in float32).  Returns (codes uint8
    [N, C], E8M0 scales uint8 [N, C/32]).
    """
    a32 = np.asarray(a, dtype=np.float32)
    n, c = a32.shape
    assert c % MX_BLOCK == 0
    g = a32.reshape(n, c // MX_BLOCK, MX_BLOCK)
    amax = np.abs(g).max(axis=2)
    _, ex = np.frexp(amax.astype(np.float64))       # amax = f * 2^ex, f in [0.5, 1)
    X = np.maximum(ex.astype(np.int64) - 1 - E4M3_EMAX, -127)
    X = np.where(amax == 0, 0, X)
    q = (g * np.ldexp(np.float32(1.0), -X)[:, :, None].astype(np.float32)).astype(np.float32)
    codes = e4m3_encode(q).reshape(n, c)
    return codes, (X + 127).astype(np.uint8)


def mx_dequant_fp8(codes, scales) -> np.ndarray:
    n, c = codes.shape
    v = e4m3_decode(codes).reshape(n, c // MX_BLOCK, MX_BLOCK)
    return (v * e8m0_decode(scales)[:, :, None]).reshape(n, c)


# --------------------------------------------------------------------------
# Routers
# --------------------------------------------------------------------------

def sigmoid_f32(z) -> np.ndarray:
    """The float32 sigmoid used for the router's selection key.

    sigma(z) = 1 / (1 + exp(-z)) with exp(-z) rounded once to float32 from a
    float64 evaluation, then a float32 add and a float32 division, each
    correctly rounded.  Fixing the evaluation makes the selection key (and so
    the selected indices) reproducible bit for bit.
    """
    z = np.asarray(z, dtype=np.float32)
    with np.errstate(over="ignore"):
        e = np.exp(-z.astype(np.float64)).astype(np.float32)
        return (np.float32(1.0) / (np.float32(1.0) + e)).astype(np.float32)


def _log_sigmoid64(v) -> np.ndarray:
    v = np.asarray(v, dtype=np.float64)
    return np.minimum(v, 0.0) - np.log1p(np.exp(-np.abs(v)))


def _topk_desc_stable(keys, k) -> np.ndarray:
    """Indices of the k largest keys per row, largest first; equal keys keep
    ascending index order (ties go to the lower expert index)."""
    return np.argsort(-keys, axis=1, kind="stable")[:, :k].astype(np.int32)


def gate_logits(x, w_gate) -> np.ndarray:
    """Softmax-gate logits z = x . W_gate^T (float64).

    x [T, H] and W_gate [E, H] hold bf16 values; the gate is a linear layer in
    the (out_features, in_features) convention of the StackedMoE page's
    transposed-weight properties.
    """
    return np.asarray(x, np.float64) @ np.asarray(w_gate, np.float64).T


def route_softmax_topk(logits, k, route_scale=1.0, global_scale=1.0, renormalize=True):
    """Softmax top-k gate (the StackedMoE page's gate_cls / MoEGate).

    Selection: the k largest float32 logits, largest first, ties to the lower
    index.  Weights (renormalize): softmax over the k selected logits, which
    equals the full softmax restricted to the selected experts and
    renormalised.  Without renormalize: the full-softmax probability of each
    selected expert.  Every weight is multiplied by route_scale*global_scale.
    Returns (indices int32 [T,k], weights float64 [T,k]).
    """
    z = np.asarray(logits, dtype=np.float32)
    idx = _topk_desc_stable(z, k)
    z64 = z.astype(np.float64)
    if renormalize:
        zs = np.take_along_axis(z64, idx, axis=1)
        p = np.exp(zs - zs.max(axis=1, keepdims=True))
        w = p / p.sum(axis=1, keepdims=True)
    else:
        p = np.exp(z64 - z64.max(axis=1, keepdims=True))
        p = p / p.sum(axis=1, keepdims=True)
        w = np.take_along_axis(p, idx, axis=1)
    return idx, w * (float(np.float32(route_scale)) * float(np.float32(global_scale)))


def route_sigmoid_sink(logits, E, k, s, expert_bias=None, route_scale=1.0, global_scale=1.0):
    """Fused sigmoid + selection-bias top-k router with sink lanes
    (sink_gate_router_kernel page).

    1. key_i = sigmoid(z_i) + bias_i for the E routed experts (float32); the
       bias takes part in selection only.
    2. Select the k largest keys, largest first, ties to the lower index.
    3. Softmax over log-sigmoid of [selected raw logits | the s sink logits
       (columns E..E+s-1)]; in exact arithmetic this is
       sigmoid(z_i) / sum_j sigmoid(z_j), and the log-space form stays finite
       where the sigmoids underflow.
    4. Multiply every weight by route_scale*global_scale.
    Returns (indices int32 [T,k], expert weights float64 [T,k],
    sink weights float64 [T,s]).
    """
    z = np.asarray(logits, dtype=np.float32)
    T = z.shape[0]
    b = np.zeros(E, np.float32) if expert_bias is None else np.asarray(expert_bias, np.float32)
    key = (sigmoid_f32(z[:, :E]) + b[None, :]).astype(np.float32)
    idx = _topk_desc_stable(key, k)
    sel = np.take_along_axis(z[:, :E], idx, axis=1)
    lanes = np.concatenate([sel, z[:, E:E + s]], axis=1).astype(np.float64)
    ls = _log_sigmoid64(lanes)
    p = np.exp(ls - ls.max(axis=1, keepdims=True))
    w = p / p.sum(axis=1, keepdims=True)
    w = w * (float(np.float32(route_scale)) * float(np.float32(global_scale)))
    return idx, w[:, :k], w[:, k:k + s].reshape(T, s)


# --------------------------------------------------------------------------
# Bucketing (moe_create_indices / _permute_tokens_for_grouped_mm)
# --------------------------------------------------------------------------

def build_indices(expert_indices, num_local, expert_start=0, token_mask=None, expert_weights=None):
    """Per-expert CSR of the token->expert assignments.

    Assignment (t, j) has flat slot t*k + j.  It is kept when its expert lies
    in [expert_start, expert_start + num_local) and the token is valid
    (token_mask); the rest are dropped (an expert-parallel rank's local slice,
    n_local_experts / experts_start_idx of _permute_tokens_for_grouped_mm).
    Kept slots are ordered by local expert, and by flat slot within one
    expert.  Returns a dict with
      offsets      int32 [num_local+1]  exclusive prefix of per-expert counts
      sorted_token int32 [n_kept]       token of each CSR row
      sorted_slot  int64 [n_kept]       flat slot of each CSR row
      row_of_slot  int32 [T*k]          CSR row of each slot, -1 if dropped
      sorted_weight float64 [n_kept]    routing weight of each CSR row (if given)
    """
    idx = np.asarray(expert_indices, dtype=np.int64)
    T, k = idx.shape
    flat_e = idx.reshape(-1) - int(expert_start)
    keep = (flat_e >= 0) & (flat_e < num_local)
    if token_mask is not None:
        keep &= np.repeat(np.asarray(token_mask).astype(bool), k)
    slots = np.nonzero(keep)[0]
    counts = np.bincount(flat_e[slots], minlength=num_local)[:num_local]
    offsets = np.zeros(num_local + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    order = np.argsort(flat_e[slots], kind="stable")
    perm = slots[order]
    row_of_slot = np.full(T * k, -1, dtype=np.int64)
    row_of_slot[perm] = np.arange(perm.size)
    res = {
        "offsets": offsets.astype(np.int32),
        "sorted_token": (perm // k).astype(np.int32),
        "sorted_slot": perm,
        "row_of_slot": row_of_slot.astype(np.int32),
    }
    if expert_weights is not None:
        res["sorted_weight"] = np.asarray(expert_weights, np.float64).reshape(-1)[perm]
    return res


def permute_rows(x, sorted_token) -> np.ndarray:
    """x_perm[p] = x[sorted_token[p]]."""
    return np.asarray(x)[np.asarray(sorted_token, dtype=np.int64)]


# --------------------------------------------------------------------------
# Expert MLP
# --------------------------------------------------------------------------

def _sigmoid64(v):
    v = np.asarray(v, dtype=np.float64)
    e = np.exp(-np.abs(v))
    return np.where(v >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def gated_activation(gate, up, kind, alpha=0.0, limit=0.0) -> np.ndarray:
    """GatedActivation page, fused_activation:

    silu      silu(gate) * up; a non-zero limit first takes gate = min(gate, limit)
              and up = clamp(up, -limit, limit)
    swigluoai g * sigmoid(alpha*g) * (u + 1), g = min(gate, limit),
              u = clamp(up, -limit, limit); limit = 0 means no clamp
    gelu_tanh gelu(gate) * up, gelu(x) = 0.5 x (1 + tanh(0.7978845608028654
              (x + 0.044715 x^3)))
    """
    g = np.asarray(gate, dtype=np.float64)
    u = np.asarray(up, dtype=np.float64)
    if kind in ("silu", "swigluoai") and limit > 0:
        g = np.minimum(g, limit)
        u = np.clip(u, -limit, limit)
    if kind == "silu":
        return g * _sigmoid64(g) * u
    if kind == "swigluoai":
        return g * _sigmoid64(alpha * g) * (u + 1.0)
    if kind == "gelu_tanh":
        return 0.5 * g * (1.0 + np.tanh(GELU_TANH_C * (g + GELU_TANH_A * g ** 3))) * u
    raise ValueError(f"unknown activation {kind!r}")


def split_gate_up(h, fmt):
    """[.., 2D] gate_up projection -> (gate, up): concatenated [gate | up], or
    interleaved gate = even columns, up = odd columns (StackedMoE page
    gate_up_format; the x[..., ::2] / x[..., 1::2] layout named for
    quick_geglu_deepep)."""
    d2 = h.shape[-1]
    if fmt == "concatenated":
        return h[..., : d2 // 2], h[..., d2 // 2:]
    if fmt == "interleaved":
        return h[..., 0::2], h[..., 1::2]
    raise ValueError(fmt)


def expert_mlp(x_rows, w_gate_up, w_down, *, fmt="concatenated", activation="silu",
               alpha=0.0, limit=0.0, b_gate_up=None, b_down=None,
               gate_up_scale=1.0, down_scale=1.0, act_format="bf16") -> np.ndarray:
    """One expert on a block of rows, float64.

    h = gate_up_scale * (x . W_gate_up) + b_gate_up
    A = activation(split(h)), stored as the layer stores it (bf16, or e4m3
        with per-row 1x128 scales when act_format == "fp8")
    O = down_scale * (A . W_down) + b_down
    W_gate_up is [H, 2D] and W_down is [D, H] (StackedMoE page shapes, one
    expert); the scales are the per-leg expert scales of the mega_ffn page,
    applied to the product before the bias.
    """
    x64 = np.asarray(x_rows, np.float64)
    h = float(gate_up_scale) * (x64 @ np.asarray(w_gate_up, np.float64))
    if b_gate_up is not None:
        h = h + np.asarray(b_gate_up, np.float64)[None, :]
    g, u = split_gate_up(h, fmt)
    a = gated_activation(g, u, activation, alpha, limit)
    if act_format == "bf16":
        a = bf16_round(a).astype(np.float64)
    elif act_format == "fp8":
        codes, sc = quantize_rows_block128(a.astype(np.float32))
        a = dequant_rows_block128(codes, sc)
    elif act_format == "mxfp8":
        codes, sc = mxfp8_quantize_rows(a.astype(np.float32))
        a = mx_dequant_fp8(codes, sc)
    elif act_format != "none":
        raise ValueError(act_format)
    o = float(down_scale) * (a @ np.asarray(w_down, np.float64))
    if b_down is not None:
        o = o + np.asarray(b_down, np.float64)[None, :]
    return o


def combine(expert_out, row_of_slot, expert_weights=None, token_mask=None) -> np.ndarray:
    """y[t] = sum over kept slots j of w[t, j] * O[row_of_slot[t, j]] (float64);
    masked tokens give zero rows.  Weights None means weight 1."""
    rs = np.asarray(row_of_slot, np.int64)
    T, k = rs.shape
    O = np.asarray(expert_out, np.float64)
    y = np.zeros((T, O.shape[1]), np.float64)
    for j in range(k):
        r = rs[:, j]
        ok = r >= 0
        w = np.ones(T) if expert_weights is None else np.asarray(expert_weights, np.float64)[:, j]
        y[ok] += w[ok, None] * O[r[ok]]
    if token_mask is not None:
        y[~np.asarray(token_mask).astype(bool)] = 0.0
    return y


# --------------------------------------------------------------------------
# Whole layer
# --------------------------------------------------------------------------

def _expert_weights_f64(inp, e, operand, suffix=""):
    """One expert's weights as float64 in the StackedMoE page's shapes,
    W_gate_up [H, 2D] and W_down [D, H].  MXFP4 weights arrive as rows along
    the reduction dimension (the MX blocks run along it): gate_up codes
    [2D, H/2] with scales [2D, H/32], down codes [H, D/2] with [H, D/32]."""
    if operand in ("mxfp4", "mxfp4_a16"):
        wgu = mx_dequant_fp4(inp["w_gate_up" + suffix][e], inp["w_gate_up" + suffix + "_scale"][e]).T
        wd = mx_dequant_fp4(inp["w_down" + suffix][e], inp["w_down" + suffix + "_scale"][e]).T
        return wgu, wd
    if operand == "fp8":
        wgu = dequant_weight_block128(inp["w_gate_up" + suffix][e], inp["w_gate_up" + suffix + "_scale"][e])
        wd = dequant_weight_block128(inp["w_down" + suffix][e], inp["w_down" + suffix + "_scale"][e])
    else:
        wgu = np.asarray(inp["w_gate_up" + suffix][e], np.float64)
        wd = np.asarray(inp["w_down" + suffix][e], np.float64)
    return wgu, wd


# how the layer stores the intermediate A, per operand type
_ACT_FORMAT = {"bf16": "bf16", "fp8": "fp8", "mxfp4": "mxfp8", "mxfp4_a16": "bf16"}


def shared_weights(cfg, sink_weights, T):
    """Per-token weight of each shared expert: the sink lanes' routing
    weights for the sigmoid router (sink_gate_router_kernel page: the sink
    lanes are gated shared experts), 1 for the softmax router's always-on
    shared experts (StackedMoE page: has_shared_experts)."""
    if cfg.router == "sigmoid_sink":
        assert cfg.n_shared == cfg.s, "the sink lanes gate the shared experts one to one"
        return np.asarray(sink_weights, np.float64).reshape(T, cfg.n_shared)
    return np.ones((T, cfg.n_shared), np.float64)


def layer_inputs_x(inp, operand):
    """The token activations as the expert GEMMs consume them (float64):
    bf16 values, or for fp8 the dequantised per-token 1x128 e4m3 codes."""
    x = np.asarray(inp["x"], np.float32)
    if operand == "fp8":
        codes, sc = quantize_rows_block128(x)
        return dequant_rows_block128(codes, sc)
    if operand == "mxfp4":
        codes, sc = mxfp8_quantize_rows(x)
        return mx_dequant_fp8(codes, sc)
    return x.astype(np.float64)


def route(inp, cfg, logits=None):
    """Route every token as the configuration says; returns dict with
    indices, weights, sink_weights and the logits used."""
    if cfg.router == "softmax":
        if logits is None:
            logits = gate_logits(inp["x"], inp["w_gate"]).astype(np.float32)
        idx, w = route_softmax_topk(logits, cfg.k, cfg.route_scale, cfg.global_scale)
        return {"logits": logits, "indices": idx, "weights": w,
                "sink_weights": np.zeros((idx.shape[0], 0))}
    logits = inp["logits"] if logits is None else logits
    idx, w, sw = route_sigmoid_sink(logits, cfg.E, cfg.k, cfg.s, inp.get("expert_bias"),
                                    cfg.route_scale, cfg.global_scale)
    return {"logits": logits, "indices": idx, "weights": w, "sink_weights": sw}


def layer(inp, cfg, *, indices=None, weights=None, tokens=None, token_mask=None,
          expert_start=0, num_local=None, gate_up_expert_scales=None,
          down_expert_scales=None, sink_weights=None):
    """MoE FFN forward for the tokens in `tokens` (all by default), float64.

    y[t] = sum_j w[t,j] * MLP_{e(t,j)}(x[t]) over the slots whose expert is
    local and whose token is valid, plus, when the configuration has shared
    experts, sum_i sw[t,i] * MLP_shared_i(x[t]) with the weights of
    `shared_weights` (the shared experts are the same gated MLP with
    moe_dim = shared_dim).  Routing is computed by `route` unless
    indices/weights (and sink_weights) are passed in, to share a routing
    under test.  The experts are visited one at a time: gather the tokens
    that chose it, run its MLP, scatter-add the weighted rows -- the
    per-expert loop of GroupedExperts._forward_loop on the nemo_automodel
    experts page.
    """
    if indices is None or weights is None:
        r = route(inp, cfg)
        indices, weights = r["indices"], r["weights"]
        if sink_weights is None:
            sink_weights = r["sink_weights"]
    indices = np.asarray(indices, np.int64)
    weights = np.asarray(weights, np.float64)
    T = indices.shape[0]
    tokens = np.arange(T) if tokens is None else np.asarray(tokens, np.int64)
    num_local = cfg.E if num_local is None else num_local
    operand = cfg.operand_dtype
    xs = layer_inputs_x({"x": np.asarray(inp["x"])[tokens]}, operand)
    idx_s = indices[tokens] - expert_start
    w_s = weights[tokens]
    valid = np.ones(tokens.size, bool) if token_mask is None else np.asarray(token_mask).astype(bool)[tokens]
    y = np.zeros((tokens.size, cfg.H), np.float64)
    for e in range(num_local):
        sel_t, sel_j = np.nonzero((idx_s == e) & valid[:, None])
        if sel_t.size == 0:
            continue
        wgu, wd = _expert_weights_f64(inp, e + expert_start, operand)
        bgu = inp["b_gate_up"][e + expert_start] if cfg.has_bias else None
        bd = inp["b_down"][e + expert_start] if cfg.has_bias else None
        sgu = 1.0 if gate_up_expert_scales is None else gate_up_expert_scales[e + expert_start]
        sd = 1.0 if down_expert_scales is None else down_expert_scales[e + expert_start]
        o = expert_mlp(xs[sel_t], wgu, wd, fmt=cfg.gate_up_format, activation=cfg.activation,
                       alpha=cfg.alpha, limit=cfg.limit, b_gate_up=bgu, b_down=bd,
                       gate_up_scale=sgu, down_scale=sd, act_format=_ACT_FORMAT[operand])
        np.add.at(y, sel_t, w_s[sel_t, sel_j][:, None] * o)
    if getattr(cfg, "n_shared", 0):
        if cfg.router == "sigmoid_sink" and sink_weights is None:
            sink_weights = route(inp, cfg)["sink_weights"]
        sw = shared_weights(cfg, sink_weights, T)[tokens]
        for i in range(cfg.n_shared):
            wgu, wd = _expert_weights_f64(inp, i, operand, "_shared")
            bgu = inp["b_gate_up_shared"][i] if cfg.has_bias else None
            bd = inp["b_down_shared"][i] if cfg.has_bias else None
            o = expert_mlp(xs, wgu, wd, fmt=cfg.gate_up_format, activation=cfg.activation,
                           alpha=cfg.alpha, limit=cfg.limit, b_gate_up=bgu, b_down=bd,
                           act_format=_ACT_FORMAT[operand])
            y += np.where(valid[:, None], sw[:, i:i + 1] * o, 0.0)
    return y
