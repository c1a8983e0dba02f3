"""What rounding h to bf16 between the two expert products costs, on the CPU.

The bf16 workloads keep activations in bf16 (fp32 accumulation), so h = SiLU(a) * b is rounded
to the nearest bf16 before the down product.  This test recomputes a layer in float64 with
exactly that one rounding added (the routing, gates and dispatch are the oracle's) and measures
max|dy|/rms(y) against the oracle's output.  It is not part of the oracle: it bounds what any
bf16-h kernel can reach on a case, whatever its accumulation order.

* The Switch raw-gate case at capacity factor 1.25 (T = 333, 170 tokens dropped) measures
  2.154e-2 -- above the 2e-2 bound -- which is why its GPU test is an expected failure of that
  bound (the GPU measures the same figure).
* The Switch workload at full size (8,192 tokens, renormalised gates, 5,841 dropped) measures
  1.78e-2: within the bound, with little room.
"""
import numpy as np
import pytest

import workloads as wl
from oracle import moe_oracle as mo


def _bf16(a):
    return wl.bf16_to_f32(wl.f32_to_bf16_bits(np.asarray(a, np.float32))).astype(np.float64)


def emulated_error(w: wl.Workload) -> tuple[float, int]:
    inp = wl.make_inputs(w, 0)
    x, w_r = wl.as_f64(inp.x, w.dtype), wl.as_f64(inp.w_r, w.dtype)
    cap = -1 if w.capacity_factor is None else mo.capacity(w.T, w.k, w.E, w.capacity_factor)
    experts = [tuple(wl.as_f64(m, w.dtype) for m in inp.expert(e)) for e in range(w.E)]
    ref = mo.moe_forward(x, w_r, experts, w.k, cap, inp.b_r, w.renormalize)
    disp = ref.disp
    O = np.zeros((int(disp.offsets[-1]), w.d))
    for e in range(w.E):
        lo, hi = int(disp.offsets[e]), int(disp.offsets[e + 1])
        if hi > lo:
            wg, wu, wd = experts[e]
            X = x[disp.row_token[lo:hi]]
            h = mo.silu(X @ wg.T) * (X @ wu.T)
            O[lo:hi] = _bf16(h) @ wd.T                       # the one added rounding
    y = np.zeros((w.T, w.d))
    for j in range(w.k):
        rows = disp.row_of[:, j]
        keep = rows >= 0
        y[keep] += ref.gate[keep, j:j + 1] * O[rows[keep]]
    return mo.rel_err(y, ref.y), int(disp.dropped.size)


def test_bf16_h_rounding_alone_exceeds_bound_on_switch_raw_p():
    w = wl.scaled(wl.get("switch_capacity"), name="switch_raw_p", T=333, d=256, d_e=256, E=16, k=1,
                  renormalize=False)
    err, dropped = emulated_error(w)
    assert dropped == 170
    assert 2.15e-2 < err < 2.16e-2, err
    assert err > 2e-2


@pytest.mark.timeout(300)
def test_bf16_h_rounding_on_switch_workload_full_size():
    err, dropped = emulated_error(wl.get("switch_capacity"))
    assert dropped == 5841
    assert 1.7e-2 < err < 1.85e-2, err
