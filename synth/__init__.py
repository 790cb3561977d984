"""Seeded synthetic inputs for the spectral MoE gate/up path.

This package only draws random tensors with the shapes and statistics of the
layers being modelled (shared orthogonal bases, spectral magnitudes, unit
direction columns, per-column widths, activations and top-k routing lists).
It holds none of the method's arithmetic: no quantization, packing,
projection or expert products live here.  Both the CPU oracle tests and the
GPU tests/benchmark draw their inputs from it.
"""
from .configs import LAYERS, WORKLOADS, LayerSpec, Workload, workload
from .generate import DownType, Layer, make_layer, make_batch, make_down, make_gates, histogram_bits

__all__ = [
    "LAYERS", "WORKLOADS", "LayerSpec", "Workload", "workload",
    "Layer", "DownType", "make_layer", "make_batch", "make_down", "make_gates", "histogram_bits",
]
