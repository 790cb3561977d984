"""Layer shapes and batch recipes of the synthetic workloads.

Each layer is one MoE layer's gate and up projections in spectral form:
E experts, input width din, output width dout, spectral rank r, top-k routing.
The shapes follow public MoE models (Qwen3-30B-A3B, Mixtral-8x7B,
DeepSeek-MoE-16B); all values are random, seeded, and synthetic.
"""
from dataclasses import dataclass, field
from typing import Dict, Optional, Tuple

WIDTH_SET = (0, 1, 2, 3, 4, 6, 8, 16)


@dataclass(frozen=True)
class LayerSpec:
    name: str          # seed family: layers with the same name share factors
    E: int
    din: int
    dout: int
    r: int
    k: int
    decay: float       # a_{e,k} = k^-decay * LogNormal(0, ln_sigma), k from 1
    ln_sigma: float
    bits: object       # "uniform" or {width: percent}
    outlier_frac: float  # fraction of input channels scaled for every token
    outlier_scale: float
    phi_fp16: bool     # Phi values fp16-representable (False: fp32 factors)


@dataclass(frozen=True)
class Workload:
    name: str
    layer: LayerSpec
    T: int
    routing: Tuple     # ("uniform",) or ("zipf", s)


TINY = LayerSpec("tiny", E=4, din=64, dout=96, r=64, k=2, decay=0.5,
                 ln_sigma=0.3, bits="uniform", outlier_frac=0.0,
                 outlier_scale=1.0, phi_fp16=False)

QWEN3_30B_A3B = LayerSpec(
    "qwen3_30b_a3b", E=128, din=2048, dout=768, r=2048, k=8, decay=0.7,
    ln_sigma=0.5, bits={0: 10, 1: 20, 2: 40, 3: 15, 4: 10, 8: 4, 16: 1},
    outlier_frac=0.005, outlier_scale=20.0, phi_fp16=True)

MIXTRAL_8X7B = LayerSpec(
    "mixtral_8x7b", E=8, din=4096, dout=14336, r=4096, k=2, decay=0.7,
    ln_sigma=0.5, bits={0: 5, 1: 10, 2: 40, 3: 25, 4: 15, 8: 5},
    outlier_frac=0.005, outlier_scale=20.0, phi_fp16=True)

DEEPSEEK_MOE_16B = LayerSpec(
    "deepseek_moe_16b", E=64, din=2048, dout=1408, r=2048, k=6, decay=0.7,
    ln_sigma=0.5, bits={1: 5, 2: 25, 3: 35, 4: 25, 6: 5, 8: 4, 16: 1},
    outlier_frac=0.005, outlier_scale=20.0, phi_fp16=True)

# Test-only shape: r = 2048 with most columns at 8 and 16 bits, so that one
# unit of the one-launch kernel holds more K steps and plane words than its
# registers and LDS arena take at once; ragged dout.
HEAVY = LayerSpec("heavy", E=4, din=2048, dout=200, r=2048, k=2, decay=0.5,
                  ln_sigma=0.3, bits={16: 60, 8: 30, 1: 10}, outlier_frac=0.0,
                  outlier_scale=1.0, phi_fp16=True)

# Test-only shape: wide columns (mostly 6- and 8-bit, many fp16) and a ragged
# dout, so that one 64-row slab of one expert holds more plane masks and
# fp16 columns than a work-group stages at once.
WIDE = LayerSpec("wide", E=4, din=3072, dout=4133, r=3072, k=2, decay=0.5,
                 ln_sigma=0.3, bits={4: 10, 6: 30, 8: 50, 16: 10}, outlier_frac=0.0,
                 outlier_scale=1.0, phi_fp16=True)

# Test-only shape beyond the matrix-core kernels' limits (r and din above
# 4096): gate/up runs the projection and the lane-per-row expert kernel.
BEYOND = LayerSpec("beyond", E=2, din=4112, dout=40, r=4112, k=2, decay=0.5,
                   ln_sigma=0.3, bits="uniform", outlier_frac=0.0, outlier_scale=1.0,
                   phi_fp16=True)

LAYERS: Dict[str, LayerSpec] = {l.name: l for l in
                                (TINY, QWEN3_30B_A3B, MIXTRAL_8X7B, DEEPSEEK_MOE_16B, WIDE, HEAVY,
                                 BEYOND)}

WORKLOADS: Dict[str, Workload] = {w.name: w for w in (
    Workload("tiny_t8", TINY, 8, ("uniform",)),
    Workload("beyond_t1", BEYOND, 1, ("uniform",)),
    Workload("beyond_t8", BEYOND, 8, ("uniform",)),
    Workload("tiny_t1", TINY, 1, ("uniform",)),
    Workload("tiny_t4", TINY, 4, ("uniform",)),
    Workload("wide_t2", WIDE, 2, ("uniform",)),
    Workload("wide_t8", WIDE, 8, ("uniform",)),
    Workload("tiny_t64", TINY, 64, ("zipf", 1.1)),
    Workload("qwen3_30b_a3b_t1", QWEN3_30B_A3B, 1, ("uniform",)),
    Workload("qwen3_30b_a3b_t4", QWEN3_30B_A3B, 4, ("uniform",)),
    Workload("heavy_t1", HEAVY, 1, ("uniform",)),
    Workload("qwen3_30b_a3b_t32", QWEN3_30B_A3B, 32, ("zipf", 1.1)),
    Workload("mixtral_8x7b_t1", MIXTRAL_8X7B, 1, ("uniform",)),
    Workload("mixtral_8x7b_t8", MIXTRAL_8X7B, 8, ("uniform",)),
    Workload("deepseek_moe_16b_t512", DEEPSEEK_MOE_16B, 512, ("zipf", 1.0)),
)}


def workload(name: str) -> Workload:
    return WORKLOADS[name]
