"""The MXFP8 activations of the HIP path: the rounding of x (moe_mxfp8_quantize, the kernel the
layer uses) against the oracle's quantiser bit for bit, and the rounding of h seen through an
identity down projection: every code inside the range the oracle says is reachable."""
import numpy as np
import pytest
import torch

import sparse_mixture_experts_17_amd as moe
import workloads as wl
from oracle import moe_oracle as mo

import gpu_parity as gp

pytestmark = pytest.mark.gpu

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")


def _rows():
    """bf16 rows with blocks over a wide range of magnitudes, plus hand-made blocks: all zero,
    saturating maxima (block max mantissa above 1.75), exact E4M3 midpoints (ties), signed
    zeros, values whose scaled form is E4M3-subnormal, and single-element blocks."""
    g = np.random.default_rng(71)
    rows, K = 96, 512
    v = g.standard_normal((rows, K)).astype(np.float32) * np.exp2(g.integers(-30, 30, (rows, K // 32, 1))).repeat(
        32, axis=2).reshape(rows, K).astype(np.float32)
    v[0, :32] = 0.0
    v[1, :32] = g.standard_normal(32) * 0.1
    v[1, 7] = 7.75                                   # max 7.75: scale 2^-6, 496 saturates to 448
    v[2, :32] = 1.0625                               # between 1.0 and 1.125 once the block max is 256
    v[2, 0] = 256.0
    v[2, 1:5] = [1.1875, -1.0625, 3.25, 0.515625]    # more midpoints at several exponents
    v[3, :32] = -0.0
    v[3, 5] = 1.0
    v[4, :32] = 2.0 ** -9 * np.arange(32)           # scaled into E4M3's subnormal range
    v[4, 31] = 100.0
    v[5, :32] = 0.0
    v[5, 17] = -3.0e-20
    return wl.bf16_to_f32(wl.f32_to_bf16_bits(v)), wl.f32_to_bf16_bits(v)


@needs_gpu
def test_mxfp8_quantize_bit_exact():
    vals, bits = _rows()
    rows, K = vals.shape
    x = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    codes = torch.empty((rows, K), dtype=torch.uint8, device="cuda")
    scales = torch.empty((rows, K // 32), dtype=torch.uint8, device="cuda")
    moe.moe_mxfp8_quantize(x, codes, scales)
    torch.cuda.synchronize()
    want_q, want_s = mo.mxfp8_quantize_rows(vals.astype(np.float64))
    got_q, got_s = codes.cpu().numpy(), scales.cpu().numpy()
    assert np.array_equal(got_s, want_s), np.argwhere(got_s != want_s)[:5]
    bad = np.argwhere(got_q != want_q)
    assert bad.size == 0, [(tuple(i), vals[tuple(i)], got_q[tuple(i)], want_q[tuple(i)]) for i in bad[:5]]


@needs_gpu
def test_mxfp8_quantize_rejects_bad_sizes():
    x = torch.zeros((4, 48), dtype=torch.bfloat16, device="cuda")
    c = torch.empty((4, 48), dtype=torch.uint8, device="cuda")
    s = torch.empty((4, 2), dtype=torch.uint8, device="cuda")
    with pytest.raises(moe.MoeError) as ei:
        moe.moe_mxfp8_quantize(x, c, s)
    assert ei.value.status == 2


def _identity_weights(d, weights):
    """W_d = I as stored weights: FP8 (code of 1.0 on the diagonal, row scale 1) or MXFP4 (E2M1 1.0
    in the diagonal's nibble, every block scale 2^0)."""
    if weights == "fp8_e4m3":
        q = np.zeros((d, d), np.uint8)
        np.fill_diagonal(q, 0x38)
        return q, np.ones(d, np.float32)
    q = np.zeros((d, d // 2), np.uint8)
    for n in range(d):
        q[n, n // 2] = 0x2 if n % 2 == 0 else 0x20
    return q, np.full((d // 32, d), 127, np.uint8)


@needs_gpu
@pytest.mark.parametrize("weights", ["fp8_e4m3", "mxfp4"])
@pytest.mark.parametrize("T", [16, 300, 1000])              # decode, stream and large tiles
def test_h_codes_within_reachable_range(weights, T):
    """One dense expert with W_d = I: y is h's MXFP8 value.  Every element must lie in the range
    reachable from the exact h (mxfp8_round_interval with products accurate to MX_EPS); the
    share that differs from the oracle's own rounding is reported (midpoint cases)."""
    d = 512
    w = wl.scaled(wl.get("mixtral_prefill_fp8_mx"), name="hcodes", T=T, d=d, d_e=d, E=1, k=1, weights=weights)
    inp = wl.make_inputs(w)
    (qg, sg), (qu, su), _ = inp.expert_q(0)
    qd, sd = _identity_weights(d, weights)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    x = dev(inp.x.view(np.int16)).view(torch.bfloat16)
    shape, _ = gp.shape_of(w)
    out = moe.forward(shape, x, dev(inp.w_r.view(np.int16)).view(torch.bfloat16), None, dev(qg[None]), dev(qu[None]),
                      dev(qd[None]), scales=(dev(sg[None]), dev(su[None]), dev(sd[None])))
    torch.cuda.synchronize()
    y = out.y.cpu().numpy().astype(np.float64)
    X = mo.mxfp8_round_rows(wl.as_f64(inp.x, "bf16"))
    Wg, Wu = gp.dequant(qg, sg, weights), gp.dequant(qu, su, weights)
    hq, qlo, qhi, _ = mo.swiglu_mx_deviation(X, Wg, Wu, np.eye(d), gp.MX_EPS)
    flips = float(np.mean(y != hq))
    gp.log(f"[h codes {weights} T={T}] differ from the oracle's rounding: {flips:.2e} of {y.size}; "
           f"reachable range wider than one value: {float(np.mean(qhi > qlo)):.2e}")
    bad = np.argwhere((y < qlo) | (y > qhi))
    assert bad.size == 0, [(tuple(i), y[tuple(i)], qlo[tuple(i)], hq[tuple(i)], qhi[tuple(i)]) for i in bad[:5]]
    assert flips < 0.01
