"""Plain, slow CPU oracle for one sparse mixture-of-experts FFN layer (forward and backward).

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import, call or execute anything in this package.  It
shares no code with the HIP path (``sparse_mixture_experts_17_amd``) and imports
nothing from it; the HIP path never imports it.

Everything is float64 NumPy.  Inputs arrive already widened exactly from their
stored element type, so the oracle sees the same values the GPU receives.

Modules
  moe_oracle   the layer: router, softmax, top-k, gates, aux statistics,
               capacity dispatch, SwiGLU experts, combine, near-tie report,
               the FP8 (E4M3) and MXFP4 weight decodes, the E4M3 encoder and
               MXFP8 rounding of activations, and the backward pass
               (gradients with the routing held fixed)
  bruteforce   pure-Python evaluation of the dense "every expert, unchosen
               gates zero" form, for tiny inputs
  param_count  parameter and FLOP arithmetic of whole MoE models

Parity status (pins live in tests/test_oracle_*.py):
  every function here is pinned; the only unpinned statement is which of two
  experts a token picks when their probabilities differ by less than 1e-6
  ("near ties"), where any order is accepted and the token is only reported.
"""
from . import moe_oracle, bruteforce, param_count  # noqa: F401
