"""Seeded synthetic inputs for the MoE FFN forward pass.

This package only draws random tensors with the shapes and distributions of
the five workloads (and smaller variants of them).  It holds none of the
layer's arithmetic: the oracle and the GPU path both receive the tensors it
makes, and neither imports the other.
"""
from .configs import CONFIGS, MoEConfig, get_config, scaled
from .gen import make_grad_output, make_inputs, to_host

__all__ = ["CONFIGS", "MoEConfig", "get_config", "scaled", "make_inputs", "make_grad_output", "to_host"]
