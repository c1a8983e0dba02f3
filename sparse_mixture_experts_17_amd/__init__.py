"""MI355X (gfx950) sparse mixture-of-experts FFN layer, forward and backward passes.

The layer runs in hand-written HIP kernels behind the C ABI of include/moe.h
(libmoe_mi355x.so, built in-tree by ``build.py``).  This package is its thin
Python binding: ``moe_route``, ``moe_permute``, ``moe_expert_ffn``,
``moe_combine``, ``moe_forward`` (and ``moe_forward_noalloc``, which uses the
library's static scratch) and ``moe_backward`` take torch device tensors and
pass their pointers and the current HIP stream through.
"""
from ._lib import (LIB_PATH, MOE_A_MXFP8, MOE_A_NATIVE, MOE_BF16, MOE_F32, MOE_SCORE_SIGMOID,  # noqa: F401
                   MOE_SCORE_SOFTMAX, MOE_STATIC_SCRATCH_BYTES, MOE_W_FP8_E4M3, MOE_W_MXFP4, MOE_W_NATIVE, MoeError,
                   MoeShape, MoeWScales, lib)
from .moe import (BackwardOutputs, ForwardOutputs, TORCH_DTYPE, alloc_backward, alloc_forward,  # noqa: F401
                  backward, forward, make_shape, moe_backward, moe_backward_workspace_bytes, moe_capacity,
                  moe_combine, moe_expert_ffn, moe_forward, moe_forward_noalloc, moe_mxfp8_quantize, moe_permute,
                  moe_route, moe_status_str, moe_workspace_bytes)
