"""The seeded input generator: determinism, laws and bf16 storage."""
import numpy as np
import torch

import workloads as wl


def test_bf16_rounding_matches_torch():
    g = np.random.default_rng(0)
    a = (g.standard_normal(100000) * np.exp(g.uniform(-20, 20, 100000))).astype(np.float32)
    a[:4] = [0.0, -0.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8]      # exact ties round to even
    ours = wl.f32_to_bf16_bits(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = wl.bf16_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(a).to(torch.bfloat16).float().numpy())


def test_deterministic_and_independent_streams():
    w = wl.scaled(wl.get("switch_capacity"), T=32, d=128, d_e=128, E=4)
    a, b = wl.make_inputs(w, seed=0), wl.make_inputs(w, seed=0)
    assert np.array_equal(a.x, b.x) and np.array_equal(a.w_r, b.w_r) and np.array_equal(a.b_r, b.b_r)
    for e in range(w.E):
        for m1, m2 in zip(a.expert(e), b.expert(e)):
            assert np.array_equal(m1, m2)
    # one expert regenerates the same whatever E is
    w2 = wl.scaled(w, E=9)
    assert all(np.array_equal(m1, m2) for m1, m2 in zip(a.expert(2), wl.make_inputs(w2).expert(2)))
    assert not np.array_equal(wl.make_inputs(w, seed=1).x, a.x)
    st = a.experts_stacked(threads=3)
    assert all(np.array_equal(st[i][3], a.expert(3)[i]) for i in range(3))


def test_laws():
    w = wl.scaled(wl.get("mixtral_decode"), T=256, d=1024, d_e=512, E=2)
    inp = wl.make_inputs(w)
    x = wl.as_f64(inp.x, "bf16")
    assert abs(x.mean()) < 0.02 and abs(x.std() - 1) < 0.02
    wg, wu, wd = (wl.as_f64(m, "bf16") for m in inp.expert(0))
    assert abs(wg.std() * np.sqrt(w.d) - 1) < 0.02 and abs(wd.std() * np.sqrt(w.d_e) - 1) < 0.02
    sw = wl.make_inputs(wl.scaled(wl.get("switch_capacity"), T=4, d=128, d_e=128, E=4096))
    assert sw.b_r.dtype == np.float32 and abs(sw.b_r.std() - np.sqrt(1.5)) < 0.05


def test_workload_table():
    names = list(wl.WORKLOADS)
    assert names[:5] == ["tiny_fp32", "switch_capacity", "mixtral_prefill", "mixtral_decode", "deepseek_v3"]
    assert wl.get("deepseek_v3_grouped").scoring == "sigmoid"
    assert wl.get("deepseek_v3").d_e_shared == 2048
    assert wl.get("tiny_fp32").dtype == "f32"
