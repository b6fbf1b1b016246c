"""Seeded synthetic inputs for the MoE expert operation of a verification pass.

This package holds no arithmetic of the expert operation itself.  It produces:

* expert weights W_gate, W_up [N][d_ff][d] and W_down [N][d][d_ff], each entry
  sigma * N(0, 1) rounded to fp32 (then to bf16 for bf16 layers), every expert of
  every tensor drawn from its own counter-based stream so it can be regenerated
  alone (see ``csrc/synth.c``);
* token activations x [n][d] ~ N(0, 1), same generator;
* routing traces: per token the ids of its m experts and their fp32 routing
  weights (``routing.py``), and windows of n consecutive tokens copied into a pass.

Both the GPU path's tests and the CPU oracle's tests take their inputs from here.
"""
from .lib import (  # noqa: F401
    mix64, key_of, normal_f64, normal_f32, normal_bf16, bf16_to_f32, f32_to_bf16,
)
from .layers import CONFIGS, LayerSpec, layer_spec, expert_weights, layer_weights, pass_x, router_weights  # noqa: F401,E501
from . import routing  # noqa: F401
