"""The MoE FFN workloads, as plain data.

Names follow the StackedMoE page (hidden_dim, num_experts,
num_experts_per_token, moe_dim, gate_up_format, has_bias), the
GatedActivation page (fused_activation, alpha, limit) and the
sink_gate_router_kernel page (n_shared_experts, route_scale, global_scale).
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass


@dataclass(frozen=True)
class MoEConfig:
    cfg_id: int
    name: str
    T: int                      # tokens
    H: int                      # hidden_dim
    E: int                      # num_experts (routed)
    k: int                      # num_experts_per_token
    D: int                      # moe_dim
    router: str = "softmax"     # "softmax" | "sigmoid_sink"
    s: int = 0                  # n_shared_experts (sink lanes), sigmoid router only
    n_shared: int = 0           # shared experts with an FFN (sigmoid router: gated by the sink lanes,
                                # so n_shared == s; softmax router: always on, weight 1)
    shared_dim: int = 0         # shared_experts_dim: moe_dim of the shared experts
    gate_up_format: str = "concatenated"   # | "interleaved"
    has_bias: bool = False
    activation: str = "silu"    # "silu" | "swigluoai" | "gelu_tanh"
    alpha: float = 0.0
    limit: float = 0.0
    operand_dtype: str = "bf16"  # "bf16" | "fp8" | "mxfp4" (MXFP4 weights, MXFP8 activations: W4A8)
                                 # | "mxfp4_a16" (MXFP4 weights, bf16 activations: W4A16)
    route_scale: float = 1.0
    global_scale: float = 1.0
    fused: bool = False         # run the FFN as one launch (moe_grouped_ffn_fused)
    logit_std: float = 2.0      # sigmoid router: logits are an input ~N(0, logit_std)
    bias_range: float = 0.1     # sigmoid router: selection bias ~U(-r, r)
    x_std: float = 1.0
    w_std: float = 0.02
    router_dtype: str = "bf16"  # softmax gate: "bf16" or "float32" (StackedMoE router_dtype)

    @property
    def R(self) -> int:
        """Routed rows T*k (the most rows the grouped GEMMs can see)."""
        return self.T * self.k

    @property
    def ffn_flops(self) -> int:
        """Algorithmic FLOPs of both grouped GEMMs: 2*R*H*2D + 2*R*D*H."""
        return 6 * self.R * self.H * self.D


CONFIGS = {
    1: MoEConfig(1, "tiny", T=64, H=256, E=8, k=2, D=512),
    2: MoEConfig(2, "mixtral", T=4096, H=4096, E=8, k=2, D=14336),
    3: MoEConfig(3, "sink", T=8192, H=2048, E=128, k=6, D=768,
                 router="sigmoid_sink", s=2, n_shared=2, shared_dim=768,
                 route_scale=2.5, global_scale=1.0),
    4: MoEConfig(4, "gptoss", T=4096, H=2880, E=32, k=4, D=2880,
                 gate_up_format="interleaved", has_bias=True,
                 activation="swigluoai", alpha=1.702, limit=7.0),
    5: MoEConfig(5, "fp8", T=16384, H=7168, E=256, k=8, D=2048,
                 router="sigmoid_sink", s=0, operand_dtype="fp8",
                 route_scale=1.0, global_scale=1.0),
    # the fp8 layer's shape with MXFP4 experts run W4A8 (StackedMoE page:
    # MXFP4 weights with MXFP8 activations)
    6: MoEConfig(6, "mxfp4", T=16384, H=7168, E=256, k=8, D=2048,
                 router="sigmoid_sink", s=0, operand_dtype="mxfp4",
                 route_scale=1.0, global_scale=1.0),
    # the same experts run W4A16 on a decode-sized batch, where the layer is
    # bound by streaming the 4-bit weights
    7: MoEConfig(7, "mxfp4_a16", T=256, H=7168, E=256, k=8, D=2048,
                 router="sigmoid_sink", s=0, operand_dtype="mxfp4_a16",
                 route_scale=1.0, global_scale=1.0),
    # the Mixtral layer on a decode-sized batch, FFN in one launch
    8: MoEConfig(8, "mixtral_decode", T=64, H=4096, E=8, k=2, D=14336, fused=True),
    # the MXFP4 experts run W4A8 on a decode-sized batch, FFN in one launch
    # (mega_ffn page: the block-scaled single-launch L1 + L2 with MXFP8
    # activations re-quantised between the legs)
    9: MoEConfig(9, "mxfp4_decode", T=256, H=7168, E=256, k=8, D=2048,
                 router="sigmoid_sink", s=0, operand_dtype="mxfp4",
                 route_scale=1.0, global_scale=1.0, fused=True),
    # config 7's batch (MXFP4 experts, bf16 activations) with the FFN in one launch
    10: MoEConfig(10, "mxfp4_a16_decode", T=256, H=7168, E=256, k=8, D=2048,
                  router="sigmoid_sink", s=0, operand_dtype="mxfp4_a16",
                  route_scale=1.0, global_scale=1.0, fused=True),
}


def get_config(i: int) -> MoEConfig:
    return CONFIGS[i]


def scaled(cfg: MoEConfig, **changes) -> MoEConfig:
    """A copy of a workload with some sizes changed (smaller parity cases)."""
    return dataclasses.replace(cfg, **changes)
