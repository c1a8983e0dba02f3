"""MI355X (gfx950) sparse mixture-of-experts FFN layer, forward pass.

The layer runs in hand-written HIP kernels behind the C ABI of include/moe.h
(libmoe_mi355x.so, built in-tree by ``build.py``).  This package is its thin
Python binding: ``moe_route``, ``moe_permute``, ``moe_expert_ffn``,
``moe_combine`` and ``moe_forward`` take torch device tensors and pass their
pointers and the current HIP stream through.
"""
from ._lib import (LIB_PATH, MOE_BF16, MOE_F32, MOE_SCORE_SIGMOID, MOE_SCORE_SOFTMAX,  # noqa: F401
                   MOE_W_FP8_E4M3, MOE_W_MXFP4, MOE_W_NATIVE, MoeError, MoeShape, MoeWScales, lib)
from .moe import (ForwardOutputs, TORCH_DTYPE, alloc_forward, forward, make_shape, moe_capacity,  # noqa: F401
                  moe_combine, moe_expert_ffn, moe_forward, moe_permute, moe_route, moe_status_str,
                  moe_workspace_bytes)
