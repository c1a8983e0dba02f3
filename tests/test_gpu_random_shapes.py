"""Parity over seeded random small shapes: every router path (thread per token, wave per token,
logits GEMM), capacity on and off, grouped sigmoid routing, fp32 / bf16 / FP8 / MXFP4 weights, a
shared expert or none, ragged token counts.  Each case runs the forward protocol (with the
determinism check) and, for native weights, the backward protocol of gpu_parity."""
from __future__ import annotations

import random

import pytest
import torch

import workloads as wl

import gpu_parity as gp

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="no GPU")
pytestmark = pytest.mark.gpu

BASES = {"bf16": "mixtral_prefill", "f32": "tiny_fp32", "fp8": "mixtral_prefill_fp8",
         "mxfp4": "mixtral_prefill_mxfp4", "sigmoid": "deepseek_v3_grouped"}


def random_case(rng: random.Random, i: int) -> wl.Workload:
    kind = rng.choice(sorted(BASES))
    E = rng.choice([1, 2, 4, 6, 8, 12, 16, 17, 32, 48, 64, 96, 128, 192, 256, 320, 512])
    kw = dict(name=f"random{i}_{kind}", T=rng.choice([1, 5, 16, 17, 63, 64, 65, 130, 257, 500]),
              d=rng.choice([128, 256, 384, 512]), d_e=rng.choice([128, 256, 384]), E=E,
              k=rng.randint(1, min(E, 8)), d_e_shared=rng.choice([0, 0, 128, 256]),
              capacity_factor=rng.choice([None, None, 1.0, 1.25, 2.0]), renormalize=rng.choice([True, True, False]))
    if kind == "sigmoid":
        n_group = rng.choice([g for g in (1, 2, 4, 8) if E % g == 0])
        topk_group = rng.randint(1, n_group)
        if kw["k"] > topk_group * (E // n_group):
            n_group, topk_group = 1, 1
        kw.update(n_group=n_group, topk_group=topk_group)
    else:
        kw["router_bias_var"] = rng.choice([None, 0.5])
    return wl.scaled(wl.get(BASES[kind]), **kw)


_rng = random.Random(20261203)
CASES = [random_case(_rng, i) for i in range(24)]


@needs_gpu
@pytest.mark.parametrize("w", CASES, ids=[w.name for w in CASES])
def test_random_shape(w):
    seed = int(w.name[len("random"):].split("_")[0])
    gp.run_forward(w, seed=seed, repeat_check=True)
    if w.weights == "native":
        gp.run_backward(w, seed=seed)
