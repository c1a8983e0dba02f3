"""moe_forward under HIP graph capture: the layer allocates nothing and records no memset, so
a captured call replays to the eager call's outputs bit for bit.  Every replay is checked, with
eager work and synchronisations between the replays."""
import pytest
import torch

import sparse_mixture_experts_17_amd as moe
import workloads as wl
from workloads.device import upload

import gpu_parity as gp

pytestmark = pytest.mark.gpu

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")

BASE = {w: wl.get(w) for w in wl.WORKLOADS}
CASES = [
    # decode: one-launch routing and dispatch, decode tiles
    wl.scaled(BASE["mixtral_decode"], name="graph_decode", T=16, d=512, d_e=1024, E=8, k=2),
    # several router blocks, capacity drops, stream tiles
    wl.scaled(BASE["switch_capacity"], name="graph_capacity", T=700, d=256, d_e=512, E=16, k=2, capacity_factor=1.0),
    # logits-GEMM router, shared expert
    wl.scaled(BASE["deepseek_v3"], name="graph_many_experts", T=300, d=512, d_e=256, E=256, k=8, d_e_shared=256),
    # MXFP4 decode with the down product in two K chunks
    wl.scaled(BASE["mixtral_decode_mxfp4"], name="graph_mxfp4_ksplit", T=16, d=384, d_e=2048, E=8, k=2),
    # large tiles: the down product scheduled from work counters that a kernel in the graph zeroes
    wl.scaled(BASE["mixtral_prefill"], name="graph_large_tiles", T=2000, d=256, d_e=384, E=8, k=2),
]
FIELDS = ["y", "idx", "gate", "counts", "kept", "f", "P", "aux", "offsets", "row_of"]


def _snapshot(out):
    return {k: getattr(out, k).clone() for k in FIELDS}


@needs_gpu
@pytest.mark.parametrize("w", CASES, ids=[w.name for w in CASES])
def test_forward_graph_replay(w):
    inp = wl.make_inputs(w, 0)
    dev = upload(inp)
    other = upload(wl.make_inputs(w, 1))
    shape, _ = gp.shape_of(w)

    def call(d, out):
        return moe.forward(shape, d.x, d.w_r, d.b_r, d.w_gate, d.w_up, d.w_down, d.shared, out=out,
                           scales=d.scales, shared_scales=d.shared_scales)

    out = moe.alloc_forward(shape)
    call(dev, out)                                     # eager reference (also sets up the kernels)
    torch.cuda.synchronize()
    ref = _snapshot(out)

    side = moe.alloc_forward(shape)
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call(dev, out)                                 # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for t in (out.y, out.gate, out.f, out.P, out.aux):
        t.fill_(float("nan"))
    with torch.cuda.graph(g):
        call(dev, out)
    for r in range(3):
        call(other, side)                              # eager work on other inputs between replays
        torch.cuda.synchronize()
        out.y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for k in FIELDS:
            a, b = getattr(out, k), ref[k]
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"replay {r}: {k} differs"
