"""moe_forward_noalloc (the entry point that allocates nothing) against moe_forward.

Both run the same kernels, so every output must be bit-identical.  Two calls in a row on the
library's shared static scratch, the second with a smaller input (so stale contents of the
first call lie in the scratch), plus a third large call after it; each checked against
moe_forward with its own workspace."""
import numpy as np
import pytest
import torch

import sparse_mixture_experts_17_amd as moe
import workloads as wl
from workloads.device import upload

import gpu_parity as gp

pytestmark = pytest.mark.gpu

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")

NAMES = ["y", "idx", "gate", "counts", "kept", "f", "P", "aux", "offsets", "row_of"]


def _run_both(w):
    inp = wl.make_inputs(w)
    dev = upload(inp)
    shape, _ = gp.shape_of(w)
    assert moe.moe_workspace_bytes(shape) <= moe.MOE_STATIC_SCRATCH_BYTES
    ref = moe.forward(shape, dev.x, dev.w_r, dev.b_r, dev.w_gate, dev.w_up, dev.w_down, dev.shared,
                      scales=dev.scales, shared_scales=dev.shared_scales)
    out = moe.alloc_forward(shape)
    for t in (out.y, out.gate, out.f, out.P, out.aux):
        t.fill_(float("nan"))
    for t in (out.idx, out.counts, out.kept, out.offsets, out.row_token, out.row_of):
        t.fill_(-9)
    sg, su, sd = dev.shared if dev.shared is not None else (None, None, None)
    moe.moe_forward_noalloc(shape, dev.x, dev.w_r, dev.b_r, dev.w_gate, dev.w_up, dev.w_down, sg, su, sd,
                            dev.scales, dev.shared_scales, out.y, out.idx, out.gate, out.counts, out.kept, out.f,
                            out.P, out.aux, out.offsets, out.row_token, out.row_of)
    torch.cuda.synchronize()
    for n in NAMES:
        a, b = getattr(out, n), getattr(ref, n)
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), n
    R = int(ref.offsets[-1])
    assert torch.equal(out.row_token[:R], ref.row_token[:R])
    return shape


@needs_gpu
def test_noalloc_matches_forward_two_calls_second_smaller():
    big = wl.scaled(wl.get("deepseek_v3"), name="noalloc_big", T=96, d=1024, d_e=512, E=64, k=6, d_e_shared=512,
                    capacity_factor=1.0)
    small = wl.scaled(big, name="noalloc_small", T=9)
    decode = wl.scaled(wl.get("mixtral_decode"), name="noalloc_decode", T=16, d=1024, d_e=2048)
    s_big = _run_both(big)
    s_small = _run_both(small)
    assert moe.moe_workspace_bytes(s_small) < moe.moe_workspace_bytes(s_big)
    _run_both(decode)
    _run_both(wl.scaled(decode, name="noalloc_decode_fp8", weights="fp8_e4m3"))


@needs_gpu
def test_noalloc_rejects_shape_beyond_scratch():
    shape = moe.make_shape(4096, 4096, 14336, 8, 2, dtype=moe.MOE_BF16)
    assert moe.moe_workspace_bytes(shape) > moe.MOE_STATIC_SCRATCH_BYTES
    e = torch.empty(1, device="cuda")
    out = moe.alloc_forward(moe.make_shape(1, 4096, 14336, 8, 2, dtype=moe.MOE_BF16))
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_forward_noalloc(shape, e, e, None, e, e, e, None, None, None, None, None, out.y, out.idx, out.gate,
                                out.counts, out.kept, out.f, out.P, out.aux, None, None, None)
    assert ei.value.status == 4
