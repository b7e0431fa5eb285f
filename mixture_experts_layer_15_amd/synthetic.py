"""Seeded synthetic inputs for the MoE FFN layer.

This module only draws inputs; it computes no step of the layer.  Both the HIP
path and the fp64 oracle consume the exact bytes it returns, so the choice of
generator affects reproducibility, not parity.

Recipe (one stream per tensor and per expert, so experts can be drawn
independently and large tensors never need a full-size fp32 temporary):

* x ~ N(0, 1)                         shape [T, d]
* W_r ~ N(0, 1/d)                     shape [d, E]      (router, fan_in = d)
* W_gate, W_up ~ N(0, 1/d)            shape [E, d, d_ff] (fan_in = d)
* W_down ~ N(0, 1/d_ff)               shape [E, d_ff, d] (fan_in = d_ff)
* dy ~ N(0, 1)                        shape [T, d]      (upstream gradient of y,
  for the backward)
* router bias: none (zero-initialised gate bias, TorchTitan 1K-GPU article
  section 4.2), except for the skewed-routing case, where b_e is the fp32
  rounding of a * ln p_e with p_e = (e+1)^-s / sum_i i^-s (a Zipf(s) prior
  over experts, expert 0 the most popular) and a the config's zipf_scale.

Normals are fp32 draws from torch's generator on the chosen device, scaled by
fp32(1/sqrt(fan_in)) and rounded to nearest-even into bf16 for bf16 layers.
The CPU generator and the GPU generator produce different streams; small
layers are drawn on the CPU (identical everywhere), large ones on the GPU.
"""
from __future__ import annotations

import math
from typing import Dict, Optional

import torch

from .configs import MoEConfig

_TENSOR_ID = {"x": 0, "w_router": 1, "w_gate": 2, "w_up": 3, "w_down": 4, "dy": 5}


def torch_dtype(cfg: MoEConfig) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[cfg.dtype]


def _gen(device: str, seed: int, tensor: str, part: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((seed * 7919 + _TENSOR_ID[tensor]) * 1_000_003 + part)
    return g


def _normal(shape, std: float, dt: torch.dtype, device: str, seed: int,
            tensor: str, part: int) -> torch.Tensor:
    g = _gen(device, seed, tensor, part)
    v = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        v.mul_(torch.tensor(std, dtype=torch.float32, device=device))
    return v.to(dt)


def zipf_bias(E: int, s: float, scale: float = 1.0) -> torch.Tensor:
    """fp32 of scale * ln p_e for a Zipf(s) prior p over E experts (expert 0
    most popular)."""
    w = [(e + 1) ** (-s) for e in range(E)]
    h = math.fsum(w)
    return torch.tensor([scale * math.log(v / h) for v in w], dtype=torch.float32)


def make_inputs(cfg: MoEConfig, seed: int = 0, device: str = "cpu",
                experts: Optional[int] = None) -> Dict[str, Optional[torch.Tensor]]:
    """Draw every input of the layer.

    Returns a dict with ``x``, ``w_router``, ``bias`` (fp32 or None),
    ``w_gate``, ``w_up`` and ``w_down``, all contiguous, on ``device``.
    ``experts`` (optional) draws only the first few experts' FFN weights,
    for tests that never route elsewhere.
    """
    dt = torch_dtype(cfg)
    T, d, E, F = cfg.T, cfg.d, cfg.E, cfg.d_ff
    nE = E if experts is None else experts
    out: Dict[str, Optional[torch.Tensor]] = {}
    out["x"] = _normal((T, d), 1.0, dt, device, seed, "x", 0)
    out["w_router"] = _normal((d, E), 1.0 / math.sqrt(d), dt, device, seed, "w_router", 0)
    out["bias"] = None if cfg.zipf_bias is None else zipf_bias(E, cfg.zipf_bias,
                                                                  cfg.zipf_scale).to(device)
    for name, shape, fan_in in (("w_gate", (d, F), d), ("w_up", (d, F), d),
                                ("w_down", (F, d), F)):
        w = torch.empty((nE,) + shape, dtype=dt, device=device)
        for e in range(nE):
            w[e] = _normal(shape, 1.0 / math.sqrt(fan_in), dt, device, seed, name, e)
        out[name] = w
    return out


def make_dy(cfg: MoEConfig, seed: int = 0, device: str = "cpu") -> torch.Tensor:
    """Upstream gradient dL/dy [T, d] in the layer's dtype, N(0, 1)."""
    return _normal((cfg.T, cfg.d), 1.0, torch_dtype(cfg), device, seed, "dy", 0)
