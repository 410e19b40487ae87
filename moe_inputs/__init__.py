"""Seeded synthetic inputs for the MoE layer forward.

This module holds shapes and random inputs only: it does none of the
layer's arithmetic (no routing, no softmax, no FFN).  Both the CPU oracle
(`oracle/`) and the GPU path's tests and benchmark draw their inputs from
here, so the two sides see the same bits.

Storage conventions
-------------------
* bf16 tensors are numpy ``uint16`` arrays holding the raw bfloat16 bits
  (round-to-nearest-even from a float32 draw).
* fp32 tensors are numpy ``float32`` arrays.
* Weights use the ``[out, in]`` (nn.Linear) layout, so every GEMM operand
  is contiguous along the contracted dimension.

Recipe (stated again in the design doc)
----------------------------------
Every tensor (and every expert's slice of a per-expert tensor) gets its
own PCG64 stream, ``default_rng([seed, config_tag, tensor_tag, index])``,
so tensors can be drawn in parallel threads and any one of them can be
regenerated alone.  Activations are N(0, 1); weights are N(0, 1/d_in)
with d_in the contracted dimension; bf16 tensors are rounded to nearest
even.  The per-expert router bias that models hot experts is computed,
not drawn: b_e = -s * ln(e + 1) for the local expert index e within a
head, so softmax(b) over one head is exactly the Zipf(s) pmf.  The
selection-only balancing bias of the routing variants, when a workload asks
for one, is 0.001 * n_e with n_e drawn uniformly from [-steps, steps] (stream
tag 11): the state such a bias reaches after some updates of step 0.001.
"""
from .configs import MoEConfig, CONFIGS, SMALL, VARIANTS, SMALL_VARIANTS, config_by_name  # noqa: F401
from .gen import generate, bf16_bits_from_f32, Inputs  # noqa: F401
