"""The five layer configurations this library is measured and tested on.

Plain data only: sizes, temperature, capacity factor as a rational, and the
dtype of activations and weights.  Nothing here computes any step of the layer.

Where each number comes from (page titles as printed on the pages):

* ``tiny`` -- a small fp32 layer that the fp64 oracle finishes in well under a
  second; used for element-by-element parity.
* ``zaya1`` -- hidden size h = 2048 and E = 16 experts per layer from the
  parameter table of "AMD GPU深度学习优化与ZAYA1大模型实践" (section 2), top-1
  routing from the same section, sequence length 4096 (table lower bound),
  expert-FFN shape 2048 x 8192 from "AMD MI300X平台上的MoE模型训练实践" section
  2.1 (GEMM shapes chosen for the expert feed-forward network).
* ``wide`` -- FFN width 8192, 128 experts, capacity factor 1.25, gate
  temperature 0.3, top-2, from the TorchTitan 1K-GPU article, section 2.1.
* ``skewed`` -- a routing stress case: 64 experts, top-2, capacity factor 1.25,
  temperature 0.3, with a Zipf(s = 1.2) log-popularity router bias scaled by
  0.4, so that about 30% of the tokens have expert 0 among their two choices
  (30.3% on the CPU-drawn inputs of seed 0; the unscaled prior, whose mass on
  expert 0 is 29.3%, sends 77% of the tokens there on N(0, 1)-scale logits).
* ``longseq`` -- 65,536 tokens x hidden 6,144 from "Training a 1T-Params MoE on
  EU public infrastructure" (the activation-offload paragraph), as one GPU's
  share with 8 local experts.
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Optional


@dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int               # tokens in the batch
    d: int               # model (hidden) width
    E: int               # experts
    k: int               # experts chosen per token
    d_ff: int            # expert FFN width (GeGLU inner width)
    temperature: float   # router softmax temperature tau (> 0)
    cap_num: int         # capacity factor numerator   (cap_den == 0: no limit)
    cap_den: int         # capacity factor denominator
    renormalize: bool    # gates renormalised over the chosen k experts
    dtype: str           # "f32" or "bf16" for activations and weights
    zipf_bias: Optional[float] = None  # Zipf exponent of the router bias, or None for no bias
    zipf_scale: float = 1.0  # factor on the Zipf log-prior bias
    drop_policy: int = 0  # 0: overflow dropped in token order; 1: choice order (first choices first)
    layout: int = 0       # 0: compact expert-grouped rows; 1: padded to C rows per expert
    # dynamic expert count: threshold > 0 lets each token take k_min .. k
    # experts, the fewest whose softmax mass reaches the threshold
    route_threshold: float = 0.0
    k_min: int = 0

    def scaled(self, **kw) -> "MoEConfig":
        """A copy with some fields replaced (used to make small test cases)."""
        return replace(self, **kw)


CONFIGS = [
    MoEConfig("tiny", T=256, d=64, E=4, k=1, d_ff=128, temperature=1.0,
              cap_num=0, cap_den=0, renormalize=False, dtype="f32"),
    MoEConfig("zaya1", T=4096, d=2048, E=16, k=1, d_ff=8192, temperature=1.0,
              cap_num=0, cap_den=0, renormalize=False, dtype="bf16"),
    MoEConfig("wide", T=16384, d=4096, E=128, k=2, d_ff=8192, temperature=0.3,
              cap_num=5, cap_den=4, renormalize=True, dtype="bf16"),
    MoEConfig("skewed", T=32768, d=2048, E=64, k=2, d_ff=4096, temperature=0.3,
              cap_num=5, cap_den=4, renormalize=True, dtype="bf16", zipf_bias=1.2,
              zipf_scale=0.4),
    MoEConfig("longseq", T=65536, d=6144, E=8, k=2, d_ff=4096, temperature=1.0,
              cap_num=5, cap_den=4, renormalize=True, dtype="bf16"),
]

BY_NAME = {c.name: c for c in CONFIGS}

# Variant of the wide layer with the page's 2-4 experts per token (TorchTitan
# 1K-GPU article, section 2.1): up to 4 experts, at least 2, the fewest whose
# softmax mass reaches 0.6 (on seed-0 inputs 54% of tokens take 2, 20% take
# 3, 26% take 4).  Not one of the five measured layers: it is measured and
# tested beside them.
WIDE_DYNAMIC = BY_NAME["wide"].scaled(name="wide_dynamic", k=4, k_min=2, route_threshold=0.6)


def get(name_or_index) -> MoEConfig:
    if isinstance(name_or_index, int):
        return CONFIGS[name_or_index]
    if name_or_index == WIDE_DYNAMIC.name:
        return WIDE_DYNAMIC
    return BY_NAME[name_or_index]
