"""CPU oracle for the spectral MoE gate/up path -- TEST INFRASTRUCTURE ONLY.

Only the tests, the package's ``smoke()`` check and the benchmark's CPU
baseline may import anything under ``oracle/``.  The product path (the HIP
library and its Python binding) never calls it and shares no code with it.

Plain, slow, float64 numpy restatement of what BitsMoE computes, written from
the BitsMoE blog note (okazaki-yumemi.github.io, "BitsMoE: Cost-Aware Bit
Allocation In spectral Space for MoE LLM Quantization"), sections
"Methodology / first split" (shared basis and the factored product), "second
split" (magnitude/direction split), "Usage" (the width set) and "execution"
(bit-plane packing):

* ``quantize``  - per-column uniform asymmetric quantizer of unit directions
                  at widths {0,1,2,3,4,6,8,16} (0 omitted, 16 = fp16).
* ``fmt``       - an independent writer/reader of the packed blob format,
                  used to byte-compare the library packer and for round trips.
* ``path``      - z = Phi^T x, y_e = sum_k a_{e,k} z_k p_hat_{e,k},
                  h = SiLU(y_gate) * y_up.
* ``ssd``       - shared-basis spectral decomposition of stacked expert
                  weights (one SVD) and the dense reconstruction.

Every function is pinned by the ``-m "not gpu"`` tests to closed forms,
library routines, brute force or hand-derived values; see the docstrings.
"""
from . import quantize, fmt, path, ssd  # noqa: F401
