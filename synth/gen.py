"""Seeded tensor generators for the MoE workloads.

Every tensor is drawn with its own torch.Generator, seeded from
(cfg_id, tensor_id, expert, salt), on the device the caller names, in float32,
then stored in the layer's input dtype:

  tensor_id 0 x ~N(0, x_std)              bf16 [T, H]
            1 w_gate ~N(0, w_std)          bf16 [E, H]        (softmax router)
            1 logits ~N(0, logit_std)      fp32 [T, E+s]      (sigmoid router)
            2 expert_bias ~U(-r, r)        fp32 [E]           (sigmoid router)
            3 w_gate_up ~N(0, w_std)       bf16 [E, H, 2D]
            4 w_down ~N(0, w_std)          bf16 [E, D, H]
            5 b_gate_up ~N(0, w_std)       bf16 [E, 2D]       (has_bias)
            6 b_down ~N(0, w_std)          bf16 [E, H]        (has_bias)

For the fp8 workload the weights are handed over already quantised, as the
layer receives them: float8_e4m3fn codes plus one fp32 scale per 128x128
block (amax/448).  That quantisation is data preparation of the weights,
done here with torch's own cast; it is not a step of the layer.

For the MXFP4 workload the weights are drawn directly in their stored form:
rows along the reduction dimension (gate_up [E, 2D, H/2], down [E, H, D/2]),
two E2M1 codes per byte with every code equally likely, and one E8M0 scale
byte per 32 codes, uniform in [118, 121] (tensor ids 11 and 12), which gives
weights of about the bf16 workloads' spread.

The same seed gives the same tensors on a given device type; a CPU run and a
GPU run draw different numbers, which is why parity always copies the GPU's
inputs to the host before calling the oracle.
"""
from __future__ import annotations

import torch

from .configs import MoEConfig

_FP8_MAX = 448.0


def _seed(cfg_id: int, tensor_id: int, expert: int, salt: int) -> int:
    s = 0x9E3779B97F4A7C15
    for v in (cfg_id, tensor_id, expert, salt):
        s = (s * 6364136223846793005 + (v & 0xFFFFFFFF) + 1442695040888963407) & ((1 << 63) - 1)
    return s


def _gen(device, cfg_id, tensor_id, expert, salt) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed(cfg_id, tensor_id, expert, salt))
    return g


def _normal(shape, std, device, cfg_id, tid, expert, salt):
    g = _gen(device, cfg_id, tid, expert, salt)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std


def _quant_fp8_blocks(w: torch.Tensor):
    """[K, N] fp32 -> (uint8 codes [K, N], fp32 scales [K/128, N/128])."""
    K, N = w.shape
    wb = w.reshape(K // 128, 128, N // 128, 128)
    amax = wb.abs().amax(dim=(1, 3))
    scale = torch.where(amax > 0, amax / _FP8_MAX, torch.ones_like(amax))
    q = (wb / scale[:, None, :, None]).clamp(-_FP8_MAX, _FP8_MAX)
    codes = q.reshape(K, N).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, scale.contiguous()


def _mxfp4(rows, K, device, cfg_id, tid, sid, expert, salt):
    """Random MXFP4 rows: packed E2M1 codes [rows, K/2] and E8M0 scales [rows, K/32]."""
    g = _gen(device, cfg_id, tid, expert, salt)
    codes = torch.randint(0, 256, (rows, K // 2), generator=g, device=device, dtype=torch.uint8)
    g = _gen(device, cfg_id, sid, expert, salt)
    scales = torch.randint(118, 122, (rows, K // 32), generator=g, device=device, dtype=torch.uint8)
    return codes, scales


def make_inputs(cfg: MoEConfig, device="cpu", salt: int = 0) -> dict:
    """Draw every input tensor of one workload on `device`."""
    d = torch.device(device)
    c, T, H, E, D = cfg.cfg_id, cfg.T, cfg.H, cfg.E, cfg.D
    out: dict = {"cfg": cfg}
    out["x"] = (_normal((T, H), cfg.x_std, d, c, 0, 0, salt)).to(torch.bfloat16)
    if cfg.router == "softmax":
        wg = _normal((E, H), cfg.w_std, d, c, 1, 0, salt)
        out["w_gate"] = wg if getattr(cfg, "router_dtype", "bf16") == "float32" else wg.to(torch.bfloat16)
    else:
        out["logits"] = _normal((T, E + cfg.s), cfg.logit_std, d, c, 1, 0, salt).contiguous()
        g = _gen(d, c, 2, 0, salt)
        r = cfg.bias_range
        out["expert_bias"] = (torch.rand((E,), generator=g, device=d, dtype=torch.float32) * (2 * r) - r)
    if cfg.operand_dtype == "bf16":
        wgu = torch.empty((E, H, 2 * D), device=d, dtype=torch.bfloat16)
        wd = torch.empty((E, D, H), device=d, dtype=torch.bfloat16)
        for e in range(E):
            wgu[e] = _normal((H, 2 * D), cfg.w_std, d, c, 3, e, salt).to(torch.bfloat16)
            wd[e] = _normal((D, H), cfg.w_std, d, c, 4, e, salt).to(torch.bfloat16)
        out["w_gate_up"], out["w_down"] = wgu, wd
    elif cfg.operand_dtype in ("mxfp4", "mxfp4_a16"):
        assert H % 32 == 0 and D % 32 == 0
        wgu = torch.empty((E, 2 * D, H // 2), device=d, dtype=torch.uint8)
        wgus = torch.empty((E, 2 * D, H // 32), device=d, dtype=torch.uint8)
        wd = torch.empty((E, H, D // 2), device=d, dtype=torch.uint8)
        wds = torch.empty((E, H, D // 32), device=d, dtype=torch.uint8)
        for e in range(E):
            wgu[e], wgus[e] = _mxfp4(2 * D, H, d, c, 3, 11, e, salt)
            wd[e], wds[e] = _mxfp4(H, D, d, c, 4, 12, e, salt)
        out["w_gate_up"], out["w_gate_up_scale"] = wgu, wgus
        out["w_down"], out["w_down_scale"] = wd, wds
    else:
        assert H % 128 == 0 and D % 128 == 0
        wgu = torch.empty((E, H, 2 * D), device=d, dtype=torch.uint8)
        wgus = torch.empty((E, H // 128, 2 * D // 128), device=d, dtype=torch.float32)
        wd = torch.empty((E, D, H), device=d, dtype=torch.uint8)
        wds = torch.empty((E, D // 128, H // 128), device=d, dtype=torch.float32)
        for e in range(E):
            wgu[e], wgus[e] = _quant_fp8_blocks(_normal((H, 2 * D), cfg.w_std, d, c, 3, e, salt))
            wd[e], wds[e] = _quant_fp8_blocks(_normal((D, H), cfg.w_std, d, c, 4, e, salt))
        out["w_gate_up"], out["w_gate_up_scale"] = wgu, wgus
        out["w_down"], out["w_down_scale"] = wd, wds
    if cfg.has_bias:
        out["b_gate_up"] = _normal((E, 2 * D), cfg.w_std, d, c, 5, 0, salt).to(torch.bfloat16)
        out["b_down"] = _normal((E, H), cfg.w_std, d, c, 6, 0, salt).to(torch.bfloat16)
    if cfg.n_shared:
        # shared experts: the same gated MLP with moe_dim = shared_dim, in the
        # layer's operand dtype (tensor ids 7..10, one stream per shared expert;
        # MX scale streams 13 and 14)
        S, Ds = cfg.n_shared, cfg.shared_dim
        if cfg.operand_dtype in ("mxfp4", "mxfp4_a16"):
            assert Ds % 32 == 0
            sgu = torch.empty((S, 2 * Ds, H // 2), device=d, dtype=torch.uint8)
            sgus = torch.empty((S, 2 * Ds, H // 32), device=d, dtype=torch.uint8)
            sd = torch.empty((S, H, Ds // 2), device=d, dtype=torch.uint8)
            sds = torch.empty((S, H, Ds // 32), device=d, dtype=torch.uint8)
            for i in range(S):
                sgu[i], sgus[i] = _mxfp4(2 * Ds, H, d, c, 7, 13, i, salt)
                sd[i], sds[i] = _mxfp4(H, Ds, d, c, 8, 14, i, salt)
            out["w_gate_up_shared"], out["w_gate_up_shared_scale"] = sgu, sgus
            out["w_down_shared"], out["w_down_shared_scale"] = sd, sds
        elif cfg.operand_dtype == "bf16":
            sgu = torch.empty((S, H, 2 * Ds), device=d, dtype=torch.bfloat16)
            sd = torch.empty((S, Ds, H), device=d, dtype=torch.bfloat16)
            for i in range(S):
                sgu[i] = _normal((H, 2 * Ds), cfg.w_std, d, c, 7, i, salt).to(torch.bfloat16)
                sd[i] = _normal((Ds, H), cfg.w_std, d, c, 8, i, salt).to(torch.bfloat16)
            out["w_gate_up_shared"], out["w_down_shared"] = sgu, sd
        else:
            assert Ds % 128 == 0
            sgu = torch.empty((S, H, 2 * Ds), device=d, dtype=torch.uint8)
            sgus = torch.empty((S, H // 128, 2 * Ds // 128), device=d, dtype=torch.float32)
            sd = torch.empty((S, Ds, H), device=d, dtype=torch.uint8)
            sds = torch.empty((S, Ds // 128, H // 128), device=d, dtype=torch.float32)
            for i in range(S):
                sgu[i], sgus[i] = _quant_fp8_blocks(_normal((H, 2 * Ds), cfg.w_std, d, c, 7, i, salt))
                sd[i], sds[i] = _quant_fp8_blocks(_normal((Ds, H), cfg.w_std, d, c, 8, i, salt))
            out["w_gate_up_shared"], out["w_gate_up_shared_scale"] = sgu, sgus
            out["w_down_shared"], out["w_down_shared_scale"] = sd, sds
        if cfg.has_bias:
            out["b_gate_up_shared"] = _normal((S, 2 * Ds), cfg.w_std, d, c, 9, 0, salt).to(torch.bfloat16)
            out["b_down_shared"] = _normal((S, H), cfg.w_std, d, c, 10, 0, salt).to(torch.bfloat16)
    return out


def to_host(inputs: dict, keys=None) -> dict:
    """Copy generated tensors to numpy: bf16 -> exact float32, uint8 stays uint8."""
    res = {}
    for kname, v in inputs.items():
        if keys is not None and kname not in keys:
            continue
        if isinstance(v, torch.Tensor):
            t = v.detach().cpu()
            if t.dtype == torch.bfloat16:
                t = t.float()
            res[kname] = t.numpy()
        else:
            res[kname] = v
    return res


def fp8_codes_to_float_torch(codes: torch.Tensor) -> torch.Tensor:
    """Helper for tests: decode e4m3fn codes with torch's own cast."""
    return codes.view(torch.float8_e4m3fn).float()


__all__ = ["make_inputs", "to_host", "fp8_codes_to_float_torch"]


def make_grad_output(cfg: MoEConfig, device="cpu", salt: int = 0) -> torch.Tensor:
    """The upstream gradient dy = dL/dy of a backward pass: bf16 [T, H], N(0, 1)
    (tensor id 21)."""
    d = torch.device(device)
    return _normal((cfg.T, cfg.H), 1.0, d, cfg.cfg_id, 21, 0, salt).to(torch.bfloat16)
