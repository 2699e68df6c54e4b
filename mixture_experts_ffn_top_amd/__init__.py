"""MI355X (gfx950) MoE FFN forward pass: thin Python binding of libmoe_mi355x.so.

The four steps of the layer run in the HIP library, called through its C ABI
(include/moe_mi355x.h) with ctypes.  This module only checks tensor dtypes,
shapes and devices, allocates outputs with torch (device memory) and passes
raw pointers plus torch's current stream.  There is no fallback: the first
call raises ImportError when the library has not been built.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_mi355x.so")

MOE_OK, MOE_ERR_INVALID_ARGUMENT, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE_TOO_SMALL, MOE_ERR_HIP = range(5)
ROUTER_SOFTMAX_TOPK, ROUTER_SIGMOID_SINK = 0, 1
ACT = {"silu": 0, "swigluoai": 1, "gelu_tanh": 2}
FMT = {"concatenated": 0, "interleaved": 1}
DTYPE_BF16, DTYPE_FP8_E4M3_BLOCK128, DTYPE_FP32, DTYPE_FP8_E4M3_TOKENS = 0, 1, 2, 3
DTYPE_MXFP4_W4A8, DTYPE_MXFP8, DTYPE_MXFP8_TOKENS, DTYPE_MXFP4_W4A16 = 4, 5, 6, 7
XPERM = {"bf16": DTYPE_BF16, "fp8": DTYPE_FP8_E4M3_BLOCK128, "fp8_tokens": DTYPE_FP8_E4M3_TOKENS,
         "mxfp8": DTYPE_MXFP8, "mxfp8_tokens": DTYPE_MXFP8_TOKENS}
OPERAND = {"bf16": DTYPE_BF16, "fp8": DTYPE_FP8_E4M3_BLOCK128, "mxfp4": DTYPE_MXFP4_W4A8,
           "mxfp4_a16": DTYPE_MXFP4_W4A16}
WEIGHT_IN_OUT, WEIGHT_OUT_IN = 0, 1

_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_f32 = ctypes.c_float


class RouteArgs(ctypes.Structure):
    _fields_ = [("router_kind", _i32), ("num_tokens", _i32), ("n_routed_experts", _i32),
                ("n_experts_per_tok", _i32), ("n_shared_experts", _i32), ("hidden_dim", _i32),
                ("x", _vp), ("w_gate", _vp), ("logits", _vp), ("logits_ld", _i64),
                ("logits_out", _vp), ("expert_bias", _vp), ("global_scale", _vp),
                ("route_scale", _f32), ("renormalize", _i32), ("expert_indices", _vp),
                ("expert_weights", _vp), ("sink_weights", _vp), ("router_dtype", _i32)]


class IndexArgs(ctypes.Structure):
    _fields_ = [("num_tokens", _i32), ("n_experts_per_tok", _i32), ("experts_start_idx", _i32),
                ("n_local_experts", _i32), ("expert_indices", _vp), ("expert_weights", _vp),
                ("token_mask", _vp), ("expert_offsets", _vp), ("sorted_token", _vp),
                ("row_of_slot", _vp), ("sorted_weight", _vp), ("x", _vp), ("hidden_dim", _i32),
                ("xperm_dtype", _i32), ("x_perm", _vp), ("x_perm_scale", _vp),
                ("workspace", _vp), ("workspace_bytes", _i64)]


class FfnArgs(ctypes.Structure):
    _fields_ = [("max_rows", _i32), ("hidden_dim", _i32), ("moe_dim", _i32),
                ("n_local_experts", _i32), ("expert_offsets", _vp), ("operand_dtype", _i32),
                ("x_perm", _vp), ("x_perm_scale", _vp), ("x", _vp), ("sorted_token", _vp),
                ("w_gate_up", _vp), ("w_gate_up_layout", _i32), ("w_gate_up_scale", _vp),
                ("b_gate_up", _vp), ("gate_up_format", _i32), ("w_down", _vp),
                ("w_down_layout", _i32), ("w_down_scale", _vp), ("b_down", _vp),
                ("activation", _i32), ("alpha", _f32), ("limit", _f32),
                ("gate_up_expert_scales", _vp), ("down_expert_scales", _vp),
                ("act_workspace", _vp), ("act_workspace_bytes", _i64), ("out_dtype", _i32),
                ("expert_out", _vp), ("timing_events", _vp), ("num_tokens", _i32)]


class CombineArgs(ctypes.Structure):
    _fields_ = [("num_tokens", _i32), ("n_experts_per_tok", _i32), ("hidden_dim", _i32),
                ("expert_out", _vp), ("out_dtype", _i32), ("row_of_slot", _vp),
                ("expert_weights", _vp), ("token_mask", _vp), ("y", _vp), ("n_shared", _i32),
                ("shared_out", _vp), ("shared_weights", _vp)]


class CombineBwdArgs(ctypes.Structure):
    _fields_ = [("num_tokens", _i32), ("n_experts_per_tok", _i32), ("hidden_dim", _i32), ("dy", _vp),
                ("expert_out", _vp), ("out_dtype", _i32), ("row_of_slot", _vp), ("expert_weights", _vp),
                ("token_mask", _vp), ("d_expert_out", _vp), ("d_expert_weights", _vp)]


class FfnBwdArgs(ctypes.Structure):
    _fields_ = [("max_rows", _i32), ("hidden_dim", _i32), ("moe_dim", _i32), ("n_local_experts", _i32),
                ("expert_offsets", _vp), ("x", _vp), ("sorted_token", _vp), ("x_perm", _vp),
                ("w_gate_up", _vp), ("w_gate_up_stacked", _vp), ("w_down_stacked", _vp), ("b_gate_up", _vp),
                ("gate_up_format", _i32), ("activation", _i32), ("alpha", _f32), ("limit", _f32),
                ("gate_up_expert_scales", _vp), ("down_expert_scales", _vp), ("d_expert_out", _vp),
                ("d_x_perm", _vp), ("d_w_gate_up", _vp), ("d_w_down", _vp), ("d_b_gate_up", _vp),
                ("d_b_down", _vp), ("workspace", _vp), ("workspace_bytes", _i64), ("timing_events", _vp)]


ENTRY_POINTS = ("moe_route", "moe_build_indices", "moe_build_indices_noalloc", "moe_grouped_ffn", "moe_grouped_ffn_fused", "moe_combine",
                "moe_shared_indices", "moe_build_indices_workspace_bytes", "moe_ffn_workspace_bytes",
                "moe_ffn_fused_workspace_bytes", "moe_combine_backward", "moe_grouped_ffn_backward",
                "moe_ffn_backward_workspace_bytes", "moe_transpose_bf16", "moe_probe_mfma",
                "moe_probe_stream_copy", "moe_probe_stream_read", "moe_status_string", "moe_last_error_message", "moe_abi_version")


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m mixture_experts_ffn_top_amd.build`")
    lib = ctypes.CDLL(path)
    for name, argt in (("moe_route", RouteArgs), ("moe_build_indices", IndexArgs),
                       ("moe_build_indices_noalloc", IndexArgs),
                       ("moe_grouped_ffn", FfnArgs), ("moe_grouped_ffn_fused", FfnArgs),
                       ("moe_combine", CombineArgs), ("moe_combine_backward", CombineBwdArgs),
                       ("moe_grouped_ffn_backward", FfnBwdArgs)):
        f = getattr(lib, name)
        f.argtypes = [ctypes.POINTER(argt), _vp]
        f.restype = _i32
    lib.moe_build_indices_workspace_bytes.argtypes = [_i32, _i32, _i32]
    lib.moe_build_indices_workspace_bytes.restype = _i64
    lib.moe_ffn_workspace_bytes.argtypes = [_i32, _i32, _i32]
    lib.moe_ffn_workspace_bytes.restype = _i64
    lib.moe_ffn_fused_workspace_bytes.argtypes = [_i32, _i32, _i32, _i32]
    lib.moe_ffn_fused_workspace_bytes.restype = _i64
    lib.moe_ffn_backward_workspace_bytes.argtypes = [_i32, _i32, _i32, _i32]
    lib.moe_ffn_backward_workspace_bytes.restype = _i64
    lib.moe_transpose_bf16.argtypes = [_vp, _vp, _i32, _i32, _i32, _vp]
    lib.moe_transpose_bf16.restype = _i32
    lib.moe_probe_mfma.argtypes = [_i32, _i32, _i32, _vp, _vp]
    lib.moe_probe_mfma.restype = _i32
    lib.moe_probe_stream_copy.argtypes = [_vp, _vp, _i64, _vp]
    lib.moe_probe_stream_copy.restype = _i32
    lib.moe_probe_stream_read.argtypes = [_vp, _i64, _vp, _i32, _vp]
    lib.moe_probe_stream_read.restype = _i32
    lib.moe_status_string.argtypes = [_i32]
    lib.moe_status_string.restype = ctypes.c_char_p
    lib.moe_last_error_message.argtypes = []
    lib.moe_last_error_message.restype = ctypes.c_char_p
    lib.moe_abi_version.argtypes = []
    lib.moe_abi_version.restype = _i32
    lib.moe_shared_indices.argtypes = [_i32, _i32, _vp, _vp, _vp]
    lib.moe_shared_indices.restype = _i32
    return lib


_LIB = None


def lib() -> ctypes.CDLL:
    """The loaded HIP library (loaded on first use; raises if it is not built)."""
    global _LIB
    if _LIB is None:
        _LIB = load_library()
    return _LIB


class MoEError(ValueError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{lib().moe_status_string(status).decode()}: {msg}")
        self.status = status


def _check(status: int) -> None:
    if status != MOE_OK:
        raise MoEError(status, lib().moe_last_error_message().decode())


def _ptr(t) -> int | None:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream(device=None) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _dt(t, dtype, name):
    if t is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype} (got {t.dtype})")


# ------------------------------------------------------------------ the four calls

def route(*, router: str, k: int, E: int, s: int = 0, x=None, w_gate=None, logits=None,
          expert_bias=None, route_scale: float = 1.0, global_scale=None, renormalize: bool = True,
          return_logits: bool = False):
    """moe_route.  Returns (indices int32 [T,k], weights fp32 [T,k],
    sink_weights fp32 [T,s] or None, logits fp32 [T,E] or None)."""
    src = logits if logits is not None else x
    T = src.shape[0]
    dev = src.device
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    sw = torch.empty((T, s), dtype=torch.float32, device=dev) if s > 0 else None
    lo = torch.empty((T, E), dtype=torch.float32, device=dev) if (return_logits and logits is None) else None
    _dt(x, torch.bfloat16, "x")
    # the gate in bf16, or float32 (router_dtype float32)
    w32 = w_gate is not None and w_gate.dtype == torch.float32
    if not w32:
        _dt(w_gate, torch.bfloat16, "w_gate")
    _dt(logits, torch.float32, "logits")
    _dt(expert_bias, torch.float32, "expert_bias")
    _dt(global_scale, torch.float32, "global_scale")
    a = RouteArgs(router_kind=ROUTER_SOFTMAX_TOPK if router == "softmax" else ROUTER_SIGMOID_SINK,
                  num_tokens=T, n_routed_experts=E, n_experts_per_tok=k, n_shared_experts=s,
                  hidden_dim=x.shape[1] if x is not None else 0,
                  x=_ptr(x), w_gate=_ptr(w_gate), logits=_ptr(logits),
                  logits_ld=logits.stride(0) if logits is not None else 0,
                  logits_out=_ptr(lo), expert_bias=_ptr(expert_bias), global_scale=_ptr(global_scale),
                  route_scale=route_scale, renormalize=int(renormalize),
                  expert_indices=_ptr(idx), expert_weights=_ptr(w), sink_weights=_ptr(sw),
                  router_dtype=DTYPE_FP32 if w32 else DTYPE_BF16)
    _check(lib().moe_route(ctypes.byref(a), _stream(dev)))
    return idx, w, sw, lo


def build_indices(indices, n_local: int, *, expert_start: int = 0, weights=None, token_mask=None,
                  x=None, xperm_dtype: str = "bf16", noalloc: bool = False, out: dict | None = None):
    """moe_build_indices (noalloc=True: moe_build_indices_noalloc, whose
    scratch is the library's static array).  Returns a dict of device
    tensors: offsets, sorted_token, row_of_slot, sorted_weight (if weights),
    x_perm / x_perm_scale (if x); `out` may pass those output buffers in."""
    T, k = indices.shape
    dev = indices.device
    _dt(indices, torch.int32, "indices")
    _dt(weights, torch.float32, "weights")
    _dt(token_mask, torch.uint8, "token_mask")
    R = T * k
    given = out or {}
    out = {"offsets": given.get("offsets", torch.empty(n_local + 1, dtype=torch.int32, device=dev)),
           "sorted_token": given.get("sorted_token", torch.empty(max(R, 1), dtype=torch.int32, device=dev)),
           "row_of_slot": given.get("row_of_slot", torch.empty(max(R, 1), dtype=torch.int32, device=dev))}
    if weights is not None:
        out["sorted_weight"] = given.get("sorted_weight", torch.empty(max(R, 1), dtype=torch.float32, device=dev))
    H = 0
    if xperm_dtype not in XPERM:
        raise ValueError(f"xperm_dtype must be one of {sorted(XPERM)}")
    quant = xperm_dtype != "bf16"
    mx = xperm_dtype.startswith("mx")
    rows = T if xperm_dtype.endswith("_tokens") else R
    if x is not None:
        _dt(x, torch.bfloat16, "x")
        H = x.shape[1]
        out["x_perm"] = given.get("x_perm", torch.empty((max(rows, 1), H), dtype=torch.uint8 if quant else
                                                        torch.bfloat16, device=dev))
        if mx:
            out["x_perm_scale"] = given.get("x_perm_scale", torch.empty((max(rows, 1), H // 32), dtype=torch.uint8,
                                                                        device=dev))
        elif quant:
            out["x_perm_scale"] = given.get("x_perm_scale", torch.empty((max(rows, 1), H // 128),
                                                                        dtype=torch.float32, device=dev))
    if noalloc:
        ws = None
    else:
        wsb = lib().moe_build_indices_workspace_bytes(T, k, n_local)
        ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=dev)
    a = IndexArgs(num_tokens=T, n_experts_per_tok=k, experts_start_idx=expert_start,
                  n_local_experts=n_local, expert_indices=_ptr(indices), expert_weights=_ptr(weights),
                  token_mask=_ptr(token_mask), expert_offsets=_ptr(out["offsets"]),
                  sorted_token=_ptr(out["sorted_token"]), row_of_slot=_ptr(out["row_of_slot"]),
                  sorted_weight=_ptr(out.get("sorted_weight")), x=_ptr(x), hidden_dim=H,
                  xperm_dtype=XPERM[xperm_dtype],
                  x_perm=_ptr(out.get("x_perm")), x_perm_scale=_ptr(out.get("x_perm_scale")),
                  workspace=_ptr(ws), workspace_bytes=ws.numel() if ws is not None else 0)
    _check((lib().moe_build_indices_noalloc if noalloc else lib().moe_build_indices)(ctypes.byref(a), _stream(dev)))
    return out


def ffn_workspace(max_rows: int, D: int, operand: str, device, *, fused: bool = False, L: int = 0,
                  H: int = 0) -> torch.Tensor:
    """The act_workspace of moe_grouped_ffn, or (fused) of moe_grouped_ffn_fused,
    allocated zero-filled as the single-launch form needs its control words."""
    if fused:
        n = lib().moe_ffn_fused_workspace_bytes(max_rows, H, D, L)
        return torch.zeros(max(n, 256), dtype=torch.uint8, device=device)
    n = lib().moe_ffn_workspace_bytes(max_rows, D, OPERAND[operand])
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def fused_error_word(act_workspace: torch.Tensor) -> int:
    """The error word of a moe_grouped_ffn_fused workspace (reads the device)."""
    return int(act_workspace[8:12].view(torch.int32).item())


def grouped_ffn(offsets, max_rows: int, weights: "ExpertWeights", *, x_perm=None, x_perm_scale=None,
                x=None, sorted_token=None, activation="silu", alpha=0.0, limit=0.0,
                gate_up_format="concatenated", gate_up_expert_scales=None, down_expert_scales=None,
                out_dtype=torch.float32, act_workspace=None, out=None, timing_events=None, fused=False):
    """moe_grouped_ffn (or, fused=True, moe_grouped_ffn_fused: both GEMMs in
    one launch, for bf16 or MXFP4 x MXFP8 operands).  Returns O [max_rows, H]
    (rows past offsets[-1] unwritten).

    timing_events: optional ctypes array of 3 hipEvent_t handles, recorded
    before the gate_up GEMM, between the GEMMs and after the down GEMM."""
    dev = offsets.device
    L, H, D = weights.L, weights.H, weights.D
    if act_workspace is None:
        act_workspace = ffn_workspace(max_rows, D, weights.operand, dev, fused=fused, L=L, H=H)
    if out is None:
        out = torch.empty((max(max_rows, 1), H), dtype=out_dtype, device=dev)
    _dt(offsets, torch.int32, "offsets")
    a = FfnArgs(max_rows=max_rows, hidden_dim=H, moe_dim=D, n_local_experts=L,
                expert_offsets=_ptr(offsets),
                operand_dtype=OPERAND[weights.operand],
                x_perm=_ptr(x_perm), x_perm_scale=_ptr(x_perm_scale), x=_ptr(x),
                sorted_token=_ptr(sorted_token),
                w_gate_up=_ptr(weights.w_gate_up), w_gate_up_layout=weights.layout,
                w_gate_up_scale=_ptr(weights.w_gate_up_scale), b_gate_up=_ptr(weights.b_gate_up),
                gate_up_format=FMT[gate_up_format], w_down=_ptr(weights.w_down),
                w_down_layout=weights.down_layout, w_down_scale=_ptr(weights.w_down_scale),
                b_down=_ptr(weights.b_down), activation=ACT[activation], alpha=alpha, limit=limit,
                gate_up_expert_scales=_ptr(gate_up_expert_scales),
                down_expert_scales=_ptr(down_expert_scales),
                act_workspace=_ptr(act_workspace), act_workspace_bytes=act_workspace.numel(),
                out_dtype=DTYPE_BF16 if out_dtype == torch.bfloat16 else DTYPE_FP32,
                expert_out=_ptr(out),
                timing_events=ctypes.addressof(timing_events) if timing_events is not None else None,
                num_tokens=x.shape[0] if x is not None else 0)
    _check((lib().moe_grouped_ffn_fused if fused else lib().moe_grouped_ffn)(ctypes.byref(a), _stream(dev)))
    return out


def combine(expert_out, row_of_slot, T: int, k: int, *, weights=None, token_mask=None, out=None,
            shared_out=None, shared_weights=None, n_shared: int = 0):
    """moe_combine.  Returns y bf16 [T, H].  shared_out [n_shared*T, H] (rows
    of the shared experts, bucketed by moe_shared_indices) is added with
    shared_weights [T, n_shared] (the sink weights), or weight 1 if None."""
    H = expert_out.shape[1]
    dev = expert_out.device
    y = out if out is not None else torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    _dt(shared_weights, torch.float32, "shared_weights")
    if shared_out is not None and shared_out.dtype != expert_out.dtype:
        raise ValueError("shared_out must have the dtype of expert_out")
    a = CombineArgs(num_tokens=T, n_experts_per_tok=k, hidden_dim=H, expert_out=_ptr(expert_out),
                    out_dtype=DTYPE_BF16 if expert_out.dtype == torch.bfloat16 else DTYPE_FP32,
                    row_of_slot=_ptr(row_of_slot), expert_weights=_ptr(weights),
                    token_mask=_ptr(token_mask), y=_ptr(y), n_shared=n_shared,
                    shared_out=_ptr(shared_out), shared_weights=_ptr(shared_weights))
    _check(lib().moe_combine(ctypes.byref(a), _stream(dev)))
    return y


def combine_backward(dy, row_of_slot, n_rows: int, k: int, *, expert_out=None, weights=None, token_mask=None,
                     out=None, weight_grad=True):
    """moe_combine_backward.  Returns (dO bf16 [n_rows, H], dw fp32 [T, k] or
    None): dO[row_of_slot[t, j]] = w[t, j] dy[t] and dw[t, j] = <dy[t], O[row]>
    (weight_grad needs expert_out)."""
    _dt(dy, torch.bfloat16, "dy")
    T, H = dy.shape
    dev = dy.device
    dO = out if out is not None else torch.empty((max(n_rows, 1), H), dtype=torch.bfloat16, device=dev)
    dw = torch.empty((T, k), dtype=torch.float32, device=dev) if weight_grad else None
    o_dt = DTYPE_BF16 if expert_out is not None and expert_out.dtype == torch.bfloat16 else DTYPE_FP32
    a = CombineBwdArgs(num_tokens=T, n_experts_per_tok=k, hidden_dim=H, dy=_ptr(dy), expert_out=_ptr(expert_out),
                       out_dtype=o_dt, row_of_slot=_ptr(row_of_slot), expert_weights=_ptr(weights),
                       token_mask=_ptr(token_mask), d_expert_out=_ptr(dO), d_expert_weights=_ptr(dw))
    _check(lib().moe_combine_backward(ctypes.byref(a), _stream(dev)))
    return dO, dw


def ffn_backward_workspace(max_rows: int, H: int, D: int, L: int, device) -> torch.Tensor:
    """The workspace of moe_grouped_ffn_backward (no initial contents needed)."""
    n = lib().moe_ffn_backward_workspace_bytes(max_rows, H, D, L)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def grouped_ffn_backward(offsets, max_rows: int, weights: "ExpertWeights", d_expert_out, *, x=None,
                         sorted_token=None, x_perm=None, activation="silu", alpha=0.0, limit=0.0,
                         gate_up_format="concatenated", gate_up_expert_scales=None, down_expert_scales=None,
                         workspace=None, grads=None, bias_grads=None, timing_events=None):
    """moe_grouped_ffn_backward (bf16).  Returns a dict: d_x_perm fp32
    [max_rows, H], d_w_gate_up fp32 [L, 2D, H], d_w_down fp32 [L, H, D], and
    d_b_gate_up [L, 2D] / d_b_down [L, H] when bias_grads (default: when the
    weights have biases).  `grads` may hold preallocated outputs."""
    if weights.operand != "bf16":
        raise ValueError("the backward runs on bf16 weights")
    w_gu_oi, w_gu_st, w_d_st = weights.backward_views()
    dev = offsets.device
    L, H, D = weights.L, weights.H, weights.D
    if bias_grads is None:
        bias_grads = weights.b_gate_up is not None
    g = dict(grads or {})
    g.setdefault("d_x_perm", torch.empty((max(max_rows, 1), H), dtype=torch.float32, device=dev))
    g.setdefault("d_w_gate_up", torch.empty((L, 2 * D, H), dtype=torch.float32, device=dev))
    g.setdefault("d_w_down", torch.empty((L, H, D), dtype=torch.float32, device=dev))
    if bias_grads:
        g.setdefault("d_b_gate_up", torch.empty((L, 2 * D), dtype=torch.float32, device=dev))
        g.setdefault("d_b_down", torch.empty((L, H), dtype=torch.float32, device=dev))
    if workspace is None:
        workspace = ffn_backward_workspace(max_rows, H, D, L, dev)
    _dt(offsets, torch.int32, "offsets")
    _dt(d_expert_out, torch.bfloat16, "d_expert_out")
    a = FfnBwdArgs(max_rows=max_rows, hidden_dim=H, moe_dim=D, n_local_experts=L, expert_offsets=_ptr(offsets),
                   x=_ptr(x), sorted_token=_ptr(sorted_token), x_perm=_ptr(x_perm),
                   w_gate_up=_ptr(w_gu_oi), w_gate_up_stacked=_ptr(w_gu_st),
                   w_down_stacked=_ptr(w_d_st), b_gate_up=_ptr(weights.b_gate_up),
                   gate_up_format=FMT[gate_up_format], activation=ACT[activation], alpha=alpha,
                   limit=limit, gate_up_expert_scales=_ptr(gate_up_expert_scales),
                   down_expert_scales=_ptr(down_expert_scales), d_expert_out=_ptr(d_expert_out),
                   d_x_perm=_ptr(g["d_x_perm"]), d_w_gate_up=_ptr(g["d_w_gate_up"]), d_w_down=_ptr(g["d_w_down"]),
                   d_b_gate_up=_ptr(g.get("d_b_gate_up")), d_b_down=_ptr(g.get("d_b_down")),
                   workspace=_ptr(workspace), workspace_bytes=workspace.numel(),
                   timing_events=ctypes.cast(timing_events, ctypes.c_void_p) if timing_events is not None else None)
    _check(lib().moe_grouped_ffn_backward(ctypes.byref(a), _stream(dev)))
    return g


def transpose_bf16(src, out=None):
    """moe_transpose_bf16: [B, R, C] -> [B, C, R] (bf16, R and C multiples of 64)."""
    _dt(src, torch.bfloat16, "src")
    B, R, C = src.shape
    dst = out if out is not None else torch.empty((B, C, R), dtype=torch.bfloat16, device=src.device)
    _check(lib().moe_transpose_bf16(_ptr(src), _ptr(dst), B, R, C, _stream(src.device)))
    return dst


def probe_mfma(kind: int, workgroups: int, iters: int, out):
    """moe_probe_mfma: the MFMA-loop ceiling probe (kind 0 bf16, 1 fp8).
    out: fp32 device tensor of workgroups * 8 elements.  Returns the flops the
    launch performs."""
    _dt(out, torch.float32, "out")
    if out.numel() < workgroups * 8:
        raise ValueError("probe_mfma: out needs workgroups * 8 elements")
    _check(lib().moe_probe_mfma(kind, workgroups, iters, _ptr(out), _stream(out.device)))
    return workgroups * 8 * iters * 8 * (32768 if kind == 0 else 131072)


def probe_stream_copy(src, dst):
    """moe_probe_stream_copy: dst <- src (same byte size, a multiple of 16)."""
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("probe_stream_copy: src and dst must have the same size in bytes")
    _check(lib().moe_probe_stream_copy(_ptr(src), _ptr(dst), nbytes, _stream(src.device)))
    return dst


def probe_stream_read(src, out):
    """moe_probe_stream_read: reads src (a multiple of 16 bytes); out (int32,
    at least 4 entries) receives one XOR of the 32-bit words read per wave."""
    nbytes = src.numel() * src.element_size()
    _check(lib().moe_probe_stream_read(_ptr(src), nbytes, _ptr(out), out.numel(), _stream(src.device)))
    return out


def shared_indices(T: int, n_shared: int, device):
    """moe_shared_indices.  Returns (offsets int32 [n_shared+1], sorted_token
    int32 [n_shared*T]): the buckets of the shared experts, every token in each."""
    off = torch.empty(n_shared + 1, dtype=torch.int32, device=device)
    st = torch.empty(max(n_shared * T, 1), dtype=torch.int32, device=device)
    _check(lib().moe_shared_indices(T, n_shared, _ptr(off), _ptr(st), _stream(device)))
    return off, st


# ------------------------------------------------------------------ weights and the whole layer

@dataclass
class ExpertWeights:
    """Stacked expert weights as the library consumes them.

    layout WEIGHT_IN_OUT: the StackedMoE page's stacked shapes themselves,
    w_gate_up [L, H, 2D] and w_down [L, D, H] (bf16 reads them directly).
    layout WEIGHT_OUT_IN: their transposed views, w_gate_up [L, 2D, H] and
    w_down [L, H, D] (every operand type).  down_layout, when given, sets
    the down GEMM's layout apart from the gate_up GEMM's.
    operand "mxfp4" (W4A8) / "mxfp4_a16" (W4A16): packed E2M1 w_gate_up
    [L, 2D, H/2], w_down [L, H, D/2] with E8M0 scales [L, 2D, H/32] /
    [L, H, D/32] (rows along K, OUT_IN).
    """
    w_gate_up: torch.Tensor
    w_down: torch.Tensor
    L: int
    H: int
    D: int
    operand: str = "bf16"
    layout: int = WEIGHT_OUT_IN
    w_gate_up_scale: torch.Tensor | None = None
    w_down_scale: torch.Tensor | None = None
    b_gate_up: torch.Tensor | None = None
    b_down: torch.Tensor | None = None
    down_layout: int | None = None
    # views the backward reads, made on first use: the gate_up weights in
    # OUT_IN [L, 2D, H] and both weights in the stacked [L, H, 2D] / [L, D, H]
    _bwd: dict | None = None

    def __post_init__(self):
        if self.down_layout is None:
            self.down_layout = self.layout

    @staticmethod
    def from_stacked(w_gate_up, w_down, *, b_gate_up=None, b_down=None, w_gate_up_scale=None,
                     w_down_scale=None, operand="bf16", layout=WEIGHT_OUT_IN):
        """Take stacked [L, H, 2D] / [L, D, H] weights.  IN_OUT keeps them as
        they are; OUT_IN lays them out once, at load time, as their transposed
        views (one copy: the stacked tensors are not kept).  MXFP4 weights
        already come as rows along K ([L, 2D, H/2] / [L, H, D/2]) and are kept."""
        if operand in ("mxfp4", "mxfp4_a16"):
            if layout != WEIGHT_OUT_IN:
                raise ValueError("MXFP4 weights are rows along the reduction dimension (OUT_IN)")
            for t, name in ((w_gate_up, "w_gate_up"), (w_down, "w_down"), (w_gate_up_scale, "w_gate_up_scale"),
                            (w_down_scale, "w_down_scale")):
                _dt(t, torch.uint8, name)
            L, D2, Hh = w_gate_up.shape
            return ExpertWeights(w_gate_up.contiguous(), w_down.contiguous(), L, 2 * Hh, D2 // 2, operand,
                                 layout, w_gate_up_scale.contiguous(), w_down_scale.contiguous(),
                                 b_gate_up, b_down)
        if layout == WEIGHT_IN_OUT and operand != "bf16":
            raise ValueError("only bf16 weights are read in the stacked (IN_OUT) layout")
        L, H, D2 = w_gate_up.shape
        D = D2 // 2
        if layout == WEIGHT_OUT_IN:
            w_gate_up = w_gate_up.transpose(1, 2).contiguous()
            w_down = w_down.transpose(1, 2).contiguous()
            if w_gate_up_scale is not None:
                w_gate_up_scale = w_gate_up_scale.transpose(1, 2).contiguous()
                w_down_scale = w_down_scale.transpose(1, 2).contiguous()
        else:
            w_gate_up, w_down = w_gate_up.contiguous(), w_down.contiguous()
        return ExpertWeights(w_gate_up, w_down, L, H, D, operand, layout, w_gate_up_scale,
                             w_down_scale, b_gate_up, b_down)

    def backward_views(self):
        """(w_gate_up OUT_IN [L, 2D, H], w_gate_up stacked [L, H, 2D], w_down
        stacked [L, D, H]): the weights as the backward reads them, the missing
        ones transposed on the device on the first call and kept."""
        if self.operand != "bf16":
            raise ValueError("the backward runs on bf16 weights")
        if self._bwd is None:
            def tr(t):   # [L, R, C] -> [L, C, R]
                if t.shape[1] % 64 == 0 and t.shape[2] % 64 == 0:
                    return transpose_bf16(t)
                return t.transpose(1, 2).contiguous()
            gu_io = self.layout == WEIGHT_IN_OUT
            d_io = self.down_layout == WEIGHT_IN_OUT
            gu_oi = tr(self.w_gate_up) if gu_io else self.w_gate_up
            gu_st = self.w_gate_up if gu_io else tr(self.w_gate_up)
            d_st = self.w_down if d_io else tr(self.w_down)
            self._bwd = {"w_gate_up": gu_oi, "w_gate_up_stacked": gu_st, "w_down_stacked": d_st}
        b = self._bwd
        return b["w_gate_up"], b["w_gate_up_stacked"], b["w_down_stacked"]


class MoELayer:
    """The whole forward pass over pre-allocated buffers: route ->
    build_indices -> grouped_ffn -> combine, all on torch's current stream.

    expert_slice=(start, n) keeps only the routed experts [start, start + n):
    one expert-parallel rank's share (moe.experts page, GroupedExperts:
    experts_start_idx / n_local_experts).  Its weights are those experts'
    slices of the stacked tensors, assignments to other experts are dropped
    by the bucketing, and the combine sums the local slots only (in an
    expert-parallel layer the other ranks' slots arrive by the exchange
    that one GPU leaves out).  max_rows bounds the rows the local experts
    receive (default T*k, every slot); a smaller bound, such as the row count
    an expert-parallel rank learns from its exchange, sizes the row buffers
    and the GEMM grids, and every call must stay within it."""

    def __init__(self, cfg, inputs: dict, *, layout=WEIGHT_OUT_IN, gather=True, fused=None, expert_slice=None,
                 max_rows=None, overlap_shared=True):
        self.cfg = cfg
        dev = inputs["x"].device
        self.device = dev
        self.gather = gather
        # the single-launch FFN (bf16 or MXFP4 x MXFP8): on when the configuration asks for it
        self.fused = getattr(cfg, "fused", False) if fused is None else fused
        e0, L = expert_slice if expert_slice is not None else (0, cfg.E)
        if not (0 <= e0 and L >= 1 and e0 + L <= cfg.E):
            raise ValueError(f"expert_slice {expert_slice} is not a slice of the {cfg.E} routed experts")
        if expert_slice is not None and getattr(cfg, "n_shared", 0):
            raise ValueError("expert_slice covers the routed experts of layers without shared experts")
        self.expert_start, self.n_local = e0, L

        def local(t):
            return t if t is None or (e0, L) == (0, cfg.E) else t[e0:e0 + L]
        self.w = ExpertWeights.from_stacked(
            local(inputs["w_gate_up"]), local(inputs["w_down"]), b_gate_up=local(inputs.get("b_gate_up")),
            b_down=local(inputs.get("b_down")), w_gate_up_scale=local(inputs.get("w_gate_up_scale")),
            w_down_scale=local(inputs.get("w_down_scale")), operand=cfg.operand_dtype, layout=layout)
        self.w_gate = inputs.get("w_gate")
        self.logits = inputs.get("logits")
        self.expert_bias = inputs.get("expert_bias")
        self.global_scale = torch.tensor([cfg.global_scale], dtype=torch.float32, device=dev)
        T, k = cfg.T, cfg.k
        self.out_dtype = torch.float32 if cfg.operand_dtype in ("bf16", "mxfp4_a16") else torch.bfloat16
        self.reserve_rows(T * k if max_rows is None else max_rows)
        self.y = torch.empty((T, cfg.H), dtype=torch.bfloat16, device=dev)
        # shared experts: their own weights and buckets (every token in each)
        self.n_shared = getattr(cfg, "n_shared", 0)
        if self.n_shared:
            if cfg.router == "sigmoid_sink" and self.n_shared != cfg.s:
                raise ValueError("the sink lanes gate the shared experts one to one: n_shared must equal s")
            if cfg.operand_dtype == "fp8" and not gather:
                raise ValueError("fp8 shared experts read the per-token codes: use gather=True")
            self.w_shared = ExpertWeights.from_stacked(
                inputs["w_gate_up_shared"], inputs["w_down_shared"], b_gate_up=inputs.get("b_gate_up_shared"),
                b_down=inputs.get("b_down_shared"), w_gate_up_scale=inputs.get("w_gate_up_shared_scale"),
                w_down_scale=inputs.get("w_down_shared_scale"), operand=cfg.operand_dtype, layout=layout)
            Rs = self.n_shared * T
            self.R_shared = Rs
            self.shared_offsets, self.shared_token = shared_indices(T, self.n_shared, dev)
            self.act_ws_shared = ffn_workspace(Rs, cfg.shared_dim, cfg.operand_dtype, dev)
            self.O_shared = torch.empty((max(Rs, 1), cfg.H), dtype=self.out_dtype, device=dev)
            # the shared experts' FFN depends on x alone (and, for the fp8 and
            # MXFP8 operands, on its per-token codes), not on the routing: it
            # runs on a second stream (default priority) beside the routing,
            # the bucketing and the routed FFN, so that its tiles fill the
            # CUs the routed GEMMs leave idle in their last rounds
            self.side = torch.cuda.Stream(device=dev) if overlap_shared and dev.type == "cuda" else None

    def reserve_rows(self, max_rows: int):
        """(Re)size the row buffers (activation workspace, expert rows O) and
        the bound the GEMM grids are sized for to max_rows rows."""
        c = self.cfg
        R = int(max_rows)
        if not 0 <= R <= c.T * c.k:
            raise ValueError(f"max_rows must be in [0, T*k = {c.T * c.k}] (got {max_rows})")
        self.R = R
        self.act_ws = ffn_workspace(R, c.D, c.operand_dtype, self.device, fused=self.fused, L=self.n_local, H=c.H)
        self.O = torch.empty((max(R, 1), c.H), dtype=self.out_dtype, device=self.device)

    def _route(self, x):
        c = self.cfg
        if c.router == "softmax":
            return route(router="softmax", k=c.k, E=c.E, x=x, w_gate=self.w_gate,
                         route_scale=c.route_scale, global_scale=self.global_scale)
        return route(router="sigmoid", k=c.k, E=c.E, s=c.s, logits=self.logits,
                     expert_bias=self.expert_bias, route_scale=c.route_scale, global_scale=self.global_scale)

    def local_rows(self, x, token_mask=None) -> int:
        """Rows the local experts receive for x: the routing and bucketing
        alone, then a synchronising read of the count (set-up, not the step)."""
        idx, w, _, _ = self._route(x)
        ind = build_indices(idx, self.n_local, expert_start=self.expert_start, weights=w, token_mask=token_mask)
        return int(ind["offsets"][-1].item())

    def forward(self, x, token_mask=None, mark=None, ffn_events=None, shared_events=None):
        """One layer pass.  mark(i), if given, is called on the host after
        each of the routing (i=1) and bucketing (i=2) calls, just before the
        combine (i=4, once the shared experts' stream has joined) and after
        it (i=3); ffn_events are hipEvent_t handles recorded inside the
        grouped FFN call (before gate_up, between the GEMMs, after down), and
        shared_events the same for the shared experts' FFN call (on their
        stream)."""
        c = self.cfg
        fp8 = c.operand_dtype in ("fp8", "mxfp4")
        side = self.side if self.n_shared else None
        main = torch.cuda.current_stream(self.device) if side is not None else None
        O_sh = None
        if side is not None and not fp8:
            side.wait_stream(main)
            with torch.cuda.stream(side):
                O_sh = self._shared_ffn(x, None, shared_events)
        idx, w, sw, _ = self._route(x)
        if mark:
            mark(1)
        if fp8:
            # the fp8 / MXFP8 operand: every token quantised once; gathered by
            # the GEMM (gather=True) or quantised per permuted row here
            q = "fp8" if c.operand_dtype == "fp8" else "mxfp8"
            ind = build_indices(idx, self.n_local, expert_start=self.expert_start, weights=w,
                                token_mask=token_mask, x=x, xperm_dtype=q + "_tokens" if self.gather else q)
            xg = ind.pop("x_perm") if self.gather else None
        else:
            ind = build_indices(idx, self.n_local, expert_start=self.expert_start, weights=w,
                                token_mask=token_mask, x=None if self.gather else x)
            xg = x if self.gather else None
        self.last_offsets = ind["offsets"]
        if mark:
            mark(2)
        if side is not None and fp8:
            side.wait_stream(main)
            with torch.cuda.stream(side):
                O_sh = self._shared_ffn(xg, ind.get("x_perm_scale"), shared_events)
        O = grouped_ffn(ind["offsets"], self.R, self.w, x_perm=ind.get("x_perm"),
                        x_perm_scale=ind.get("x_perm_scale"), x=xg,
                        sorted_token=ind["sorted_token"] if self.gather else None,
                        activation=c.activation, alpha=c.alpha, limit=c.limit,
                        gate_up_format=c.gate_up_format, out_dtype=self.out_dtype,
                        act_workspace=self.act_ws, out=self.O, timing_events=ffn_events, fused=self.fused)
        if side is not None:
            main.wait_stream(side)
        elif self.n_shared:
            O_sh = self._shared_ffn(xg if fp8 else x, ind.get("x_perm_scale") if fp8 else None, shared_events)
        if mark:
            mark(4)
        y = combine(O, ind["row_of_slot"], c.T, c.k, weights=w, token_mask=token_mask, out=self.y,
                    shared_out=O_sh, shared_weights=sw if c.router == "sigmoid_sink" else None,
                    n_shared=self.n_shared)
        if mark:
            mark(3)
        self.last = {"x": x, "weights": w, "index": ind, "O": O, "token_mask": token_mask, "x_gather": xg,
                     "indices": idx, "O_shared": O_sh, "sink_weights": sw}
        return {"y": y, "indices": idx, "weights": w, "sink_weights": sw, "index": ind, "O": O,
                "O_shared": O_sh}

    def _shared_ffn(self, xs, xs_scale, timing_events):
        """The shared experts' FFN on every token (their buckets hold all T
        tokens), on the current stream."""
        c = self.cfg
        return grouped_ffn(self.shared_offsets, self.R_shared, self.w_shared, x_perm_scale=xs_scale, x=xs,
                           sorted_token=self.shared_token, activation=c.activation, alpha=c.alpha,
                           limit=c.limit, gate_up_format=c.gate_up_format, out_dtype=self.out_dtype,
                           act_workspace=self.act_ws_shared, out=self.O_shared, timing_events=timing_events)

    def stage_calls(self):
        """The routing, bucketing and combine calls of the last forward, each
        as a zero-argument callable on the same inputs and output buffers
        (to time a bandwidth kernel alone, e.g. from a cold cache)."""
        c = self.cfg
        f = self.last
        x, w, ind, tm = f["x"], f["weights"], f["index"], f["token_mask"]
        if c.router == "softmax":
            def rt():
                return route(router="softmax", k=c.k, E=c.E, x=x, w_gate=self.w_gate, route_scale=c.route_scale,
                             global_scale=self.global_scale)
        else:
            def rt():
                return route(router="sigmoid", k=c.k, E=c.E, s=c.s, logits=self.logits,
                             expert_bias=self.expert_bias, route_scale=c.route_scale,
                             global_scale=self.global_scale)
        idx = f["indices"]
        if c.operand_dtype in ("fp8", "mxfp4"):
            q = "fp8" if c.operand_dtype == "fp8" else "mxfp8"

            def bi():
                return build_indices(idx, self.n_local, expert_start=self.expert_start, weights=w,
                                     token_mask=tm, x=x, xperm_dtype=q + "_tokens" if self.gather else q)
        else:
            def bi():
                return build_indices(idx, self.n_local, expert_start=self.expert_start, weights=w,
                                     token_mask=tm, x=None if self.gather else x)

        def cb():
            return combine(f["O"], ind["row_of_slot"], c.T, c.k, weights=w, token_mask=tm, out=self.y,
                           shared_out=f["O_shared"], shared_weights=f["sink_weights"] if c.router == "sigmoid_sink"
                           else None, n_shared=self.n_shared)
        return {"route": rt, "build_indices": bi, "combine": cb}

    def backward(self, dy, *, workspace=None, timing_events=None, weight_grad=True):
        """Backward of the routed experts of the last forward (bf16 layers,
        routing held fixed): returns dx bf16 [T, H], the router-weight
        gradient dw [T, k], dO, and the expert weight and bias gradients."""
        c = self.cfg
        if c.operand_dtype != "bf16":
            raise ValueError("the backward is built for bf16 layers")
        if self.n_shared:
            raise ValueError("the backward covers the routed experts only")
        f = self.last
        ind = f["index"]
        dO, dw = combine_backward(dy, ind["row_of_slot"], self.R, c.k, expert_out=f["O"], weights=f["weights"],
                                  token_mask=f["token_mask"], weight_grad=weight_grad)
        if workspace is None:
            if getattr(self, "bwd_ws", None) is None:
                self.bwd_ws = ffn_backward_workspace(self.R, c.H, c.D, self.n_local, self.device)
            workspace = self.bwd_ws
        g = grouped_ffn_backward(ind["offsets"], self.R, self.w, dO, x=f["x_gather"],
                                 sorted_token=ind["sorted_token"] if self.gather else None,
                                 x_perm=ind.get("x_perm"), activation=c.activation, alpha=c.alpha, limit=c.limit,
                                 gate_up_format=c.gate_up_format, workspace=workspace,
                                 timing_events=timing_events)
        dx = combine(g["d_x_perm"], ind["row_of_slot"], c.T, c.k, weights=None, token_mask=f["token_mask"])
        g.update({"dx": dx, "dw": dw, "dO": dO})
        return g


__all__ = ["lib", "route", "build_indices", "grouped_ffn", "combine", "shared_indices", "ExpertWeights", "MoELayer",
           "ffn_workspace", "fused_error_word", "combine_backward", "grouped_ffn_backward", "ffn_backward_workspace",
           "transpose_bf16",
           "MoEError", "load_library", "ENTRY_POINTS", "LIB_PATH"]
