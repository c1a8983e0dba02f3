"""Seeded synthetic inputs for the sparse mixture-of-experts FFN layer.

This module is the one thing the CPU oracle's tests and the HIP path's tests,
smoke check and benchmark share.  It draws the token rows and the router and
expert weights, and stores them in the element type each workload names.  It
holds none of the layer's arithmetic: no routing, no softmax, no capacity rule,
no expert FFN.  The capacity *factor* is carried as a number; turning it into a
per-expert slot count is left to the two sides that are being compared.

Random streams
--------------
NumPy ``Generator(PCG64)`` over ``SeedSequence(seed, spawn_key=...)``, one
independent stream per tensor, so that any expert can be regenerated on its own
(the oracle does this at the large workloads, one expert at a time):

    (0,)        x        [T, d]      N(0, 1)
    (1,)        W_r      [E, d]      N(0, 1/d)
    (2,)        b_r      [E]         N(0, v_b)       (only where a workload has it)
    (3, e, 0)   W_g[e]   [d_e, d]    N(0, 1/d)
    (3, e, 1)   W_u[e]   [d_e, d]    N(0, 1/d)
    (3, e, 2)   W_d[e]   [d, d_e]    N(0, 1/d_e)
    (4, 0..2)   shared expert W_g, W_u, W_d, same laws with its own d_e

The second argument of N(., .) is a variance.  Weights are drawn as float32
standard normals and multiplied by the float32 value of sqrt(variance),
i.e. 1/sqrt(fan_in) for the weights.  Where a
workload is bf16 the float32 value is then rounded to the nearest bf16 (ties to
even) and kept as raw uint16 bit patterns; ``bf16_to_f32`` widens them exactly.
The router bias stays float32 in every workload.
"""
from __future__ import annotations

import concurrent.futures as _cf
import os
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "WORKLOADS", "Workload", "get", "scaled", "f32_to_bf16_bits", "bf16_to_f32",
    "Inputs", "make_inputs",
]


@dataclass(frozen=True)
class Workload:
    """Shape and value recipe of one synthetic layer call."""
    name: str
    T: int                 # tokens
    d: int                 # model width
    d_e: int               # routed expert hidden width
    E: int                 # routed experts
    k: int                 # experts per token
    dtype: str             # "f32" or "bf16": element type of x and every weight
    capacity_factor: float | None = None   # None: no capacity limit
    router_bias_var: float | None = None   # variance of the per-expert logit bias
    d_e_shared: int = 0    # 0: no shared expert
    renormalize: bool = True
    scoring: str = "softmax"   # "softmax", or "sigmoid" (the bias then only steers selection)
    n_group: int = 1           # expert groups for group-limited routing
    topk_group: int = 1        # groups a token may use
    weights: str = "native"    # expert weights: "native" (dtype), "fp8_e4m3" (codes + row scales) or
                               # "mxfp4" (E2M1 codes + E8M0 scales per 32 along the row)
    act: str | None = None     # activations of the expert products: None (dtype) or "mxfp8"
    note: str = ""


WORKLOADS: dict[str, Workload] = {w.name: w for w in [
    Workload("tiny_fp32", T=64, d=512, d_e=1024, E=8, k=2, dtype="f32",
             note="tiny fp32 layer, the toy layer shape of the kevinluzbetak.com page"),
    Workload("switch_capacity", T=8192, d=1024, d_e=4096, E=64, k=1, dtype="bf16",
             capacity_factor=1.25, router_bias_var=1.5,
             note="Switch-style top-1 with capacity factor 1.25; skewed router bias"),
    Workload("mixtral_prefill", T=4096, d=4096, d_e=14336, E=8, k=2, dtype="bf16",
             note="Mixtral 8x7B layer shape, prefill batch"),
    Workload("mixtral_decode", T=16, d=4096, d_e=14336, E=8, k=2, dtype="bf16",
             note="Mixtral 8x7B layer shape, decode batch (weight streaming)"),
    Workload("deepseek_v3", T=4096, d=7168, d_e=2048, E=256, k=8, dtype="bf16",
             d_e_shared=2048,
             note="DeepSeek-V3 fine-grained layer: 256 routed + 1 shared expert"),
    Workload("deepseek_v3_grouped", T=4096, d=7168, d_e=2048, E=256, k=8, dtype="bf16",
             d_e_shared=2048, scoring="sigmoid", n_group=8, topk_group=4, router_bias_var=1e-4,
             note="the DeepSeek-V3 router rule on the same shape: sigmoid affinities, a selection-only "
                  "per-expert bias (std 0.01), each token limited to 4 of 8 expert groups"),
    Workload("mixtral_decode_fp8", T=16, d=4096, d_e=14336, E=8, k=2, dtype="bf16", weights="fp8_e4m3",
             note="Mixtral decode batch with FP8 E4M3 expert weights (one byte each, one fp32 scale per row)"),
    Workload("mixtral_prefill_fp8", T=4096, d=4096, d_e=14336, E=8, k=2, dtype="bf16", weights="fp8_e4m3",
             note="Mixtral prefill batch with FP8 E4M3 expert weights"),
    Workload("deepseek_v3_fp8", T=4096, d=7168, d_e=2048, E=256, k=8, dtype="bf16", d_e_shared=2048,
             weights="fp8_e4m3",
             note="DeepSeek-V3-shaped layer with FP8 E4M3 routed and shared expert weights"),
    Workload("mixtral_decode_mxfp4", T=16, d=4096, d_e=14336, E=8, k=2, dtype="bf16", weights="mxfp4",
             note="Mixtral decode batch with MXFP4 expert weights (4-bit E2M1, E8M0 scale per 32)"),
    Workload("mixtral_prefill_mxfp4", T=4096, d=4096, d_e=14336, E=8, k=2, dtype="bf16", weights="mxfp4",
             note="Mixtral prefill batch with MXFP4 expert weights"),
    Workload("mixtral_prefill_fp8_mx", T=4096, d=4096, d_e=14336, E=8, k=2, dtype="bf16", weights="fp8_e4m3",
             act="mxfp8",
             note="Mixtral prefill batch, FP8 E4M3 weights and MXFP8 activations (scaled FP8 MFMA)"),
    Workload("mixtral_prefill_mxfp4_mx", T=4096, d=4096, d_e=14336, E=8, k=2, dtype="bf16", weights="mxfp4",
             act="mxfp8",
             note="Mixtral prefill batch, MXFP4 weights and MXFP8 activations (scaled FP8 x FP4 MFMA)"),
    Workload("mixtral_decode_fp8_mx", T=16, d=4096, d_e=14336, E=8, k=2, dtype="bf16", weights="fp8_e4m3",
             act="mxfp8", note="Mixtral decode batch, FP8 E4M3 weights and MXFP8 activations"),
    Workload("deepseek_v3_fp8_mx", T=4096, d=7168, d_e=2048, E=256, k=8, dtype="bf16", d_e_shared=2048,
             weights="fp8_e4m3", act="mxfp8",
             note="DeepSeek-V3-shaped layer, FP8 E4M3 weights and MXFP8 activations"),
]}


def get(name: str) -> Workload:
    return WORKLOADS[name]


def scaled(base: Workload, **changes) -> Workload:
    """A copy of a workload with some fields changed (small parity cases)."""
    d = dict(base.__dict__)
    d.update(changes)
    if "name" not in changes:
        d["name"] = base.name + "_" + "_".join(f"{k}{v}" for k, v in changes.items())
    return Workload(**d)


# --------------------------------------------------------------------------- bf16 storage

def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); return uint16 bits.

    Inputs are finite (normal draws), so no NaN handling is needed here.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def quantize_e4m3_rows(w: np.ndarray):
    """FP8 E4M3 storage of a float32 weight matrix, one scale per row.

    Checkpoint preparation, not part of the layer: scale = max|row| / 448 (1 for an
    all-zero row), codes = the row divided by its scale, rounded to the nearest E4M3
    value by torch's float8_e4m3fn conversion.  Returns (codes uint8 [n, k], scale f32 [n]).
    """
    import torch
    t = torch.from_numpy(np.ascontiguousarray(w, dtype=np.float32))
    amax = t.abs().amax(dim=1)
    scale = torch.where(amax > 0, amax / 448.0, torch.ones_like(amax))
    q = (t / scale[:, None]).to(torch.float8_e4m3fn)
    return q.view(torch.uint8).numpy().copy(), scale.numpy().copy()


def quantize_mxfp4_rows(w: np.ndarray, block: int = 32):
    """MXFP4 storage of a float32 weight matrix [n, k] (k a multiple of `block`).

    Checkpoint preparation, not part of the layer, following the OCP MX recipe: each block of
    32 consecutive elements of a row shares the E8M0 scale 2^(floor(log2 amax) - 2) (2 is the
    largest E2M1 exponent); elements divided by it go to the nearest E2M1 magnitude (ties to
    the even code), saturating at 6.  Returns (packed [n, k/2] uint8: element 2j in the low
    nibble of byte j; scales [k/block, n] uint8, block-major).
    """
    w = np.ascontiguousarray(w, dtype=np.float32)
    n, k = w.shape
    wb = w.reshape(n, k // block, block)
    amax = np.abs(wb).max(axis=2)
    with np.errstate(divide="ignore"):
        ex = np.where(amax > 0, np.floor(np.log2(np.maximum(amax, 1e-38))) - 2, -127)
    code = np.clip(ex + 127, 0, 254).astype(np.int64)
    scale = np.exp2(code - 127.0).astype(np.float32)
    x = np.abs(wb) / scale[:, :, None]
    # nearest E2M1 code, ties to the even code: the grid is uniform on [0, 2) (step 0.5,
    # codes 0-4), [2, 4) (step 1, codes 4-6) and [4, 6] (step 2, codes 6-7); rint rounds
    # half to even, which is the even code on every piece
    m = np.where(x < 2.0, np.rint(x * 2.0), np.where(x < 4.0, 4.0 + np.rint(x - 2.0), 6.0 + np.rint((x - 4.0) / 2.0)))
    m = np.minimum(m, 7).astype(np.int64)
    codes = (m | np.where(wb < 0, 8, 0)).astype(np.uint8).reshape(n, k)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return packed, np.ascontiguousarray(code.T.astype(np.uint8))


def quantize_rows(w: np.ndarray, weights: str):
    """(codes, scales) of a float32 matrix in the workload's weight format."""
    return quantize_e4m3_rows(w) if weights == "fp8_e4m3" else quantize_mxfp4_rows(w)


# --------------------------------------------------------------------------- drawing

def _draw(seed: int, key: tuple, shape, var: float, dtype: str) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=key)))
    z = g.standard_normal(shape, dtype=np.float32)
    if var != 1.0:
        z *= np.float32(np.sqrt(var))
    if dtype == "bf16":
        return f32_to_bf16_bits(z)
    return z


@dataclass
class Inputs:
    """Host copies of one workload's inputs (bf16 as uint16 bits, else float32).

    Expert weights are produced on demand by ``expert(e)`` so that a caller can
    stream them (the largest workload holds 22.6 GB of bf16 weights).
    """
    wl: Workload
    seed: int
    x: np.ndarray
    w_r: np.ndarray
    b_r: np.ndarray | None
    _cache: dict = field(default_factory=dict, repr=False)

    def expert(self, e: int):
        """(W_g [d_e,d], W_u [d_e,d], W_d [d,d_e]) of routed expert e."""
        wl = self.wl
        if e in self._cache:
            return self._cache[e]
        return (
            _draw(self.seed, (3, e, 0), (wl.d_e, wl.d), 1.0 / wl.d, wl.dtype),
            _draw(self.seed, (3, e, 1), (wl.d_e, wl.d), 1.0 / wl.d, wl.dtype),
            _draw(self.seed, (3, e, 2), (wl.d, wl.d_e), 1.0 / wl.d_e, wl.dtype),
        )

    def expert_q(self, e: int):
        """Quantised workloads: ((codes, scales) of W_g, of W_u, of W_d) of routed expert e,
        from the same float32 draws as ``expert``."""
        wl = self.wl
        return (
            quantize_rows(_draw(self.seed, (3, e, 0), (wl.d_e, wl.d), 1.0 / wl.d, "f32"), wl.weights),
            quantize_rows(_draw(self.seed, (3, e, 1), (wl.d_e, wl.d), 1.0 / wl.d, "f32"), wl.weights),
            quantize_rows(_draw(self.seed, (3, e, 2), (wl.d, wl.d_e), 1.0 / wl.d_e, "f32"), wl.weights),
        )

    def shared_q(self):
        """Quantised workloads: the shared expert's ((codes, scales) x 3), or None."""
        wl = self.wl
        if wl.d_e_shared <= 0:
            return None
        return (
            quantize_rows(_draw(self.seed, (4, 0), (wl.d_e_shared, wl.d), 1.0 / wl.d, "f32"), wl.weights),
            quantize_rows(_draw(self.seed, (4, 1), (wl.d_e_shared, wl.d), 1.0 / wl.d, "f32"), wl.weights),
            quantize_rows(_draw(self.seed, (4, 2), (wl.d, wl.d_e_shared), 1.0 / wl.d_e_shared, "f32"), wl.weights),
        )

    def shared(self):
        """Shared expert weights, or None."""
        wl = self.wl
        if wl.d_e_shared <= 0:
            return None
        return (
            _draw(self.seed, (4, 0), (wl.d_e_shared, wl.d), 1.0 / wl.d, wl.dtype),
            _draw(self.seed, (4, 1), (wl.d_e_shared, wl.d), 1.0 / wl.d, wl.dtype),
            _draw(self.seed, (4, 2), (wl.d, wl.d_e_shared), 1.0 / wl.d_e_shared, wl.dtype),
        )

    def dy(self) -> np.ndarray:
        """Upstream gradient dL/dy [T, d] for the backward pass: float32 N(0, 1)."""
        return _draw(self.seed, (5,), (self.wl.T, self.wl.d), 1.0, "f32")

    def experts_stacked(self, threads: int | None = None):
        """All routed experts stacked: W_g [E,d_e,d], W_u [E,d_e,d], W_d [E,d,d_e].

        Drawn in parallel threads (NumPy releases the GIL while filling arrays).
        """
        wl = self.wl
        npdt = np.uint16 if wl.dtype == "bf16" else np.float32
        wg = np.empty((wl.E, wl.d_e, wl.d), npdt)
        wu = np.empty((wl.E, wl.d_e, wl.d), npdt)
        wd = np.empty((wl.E, wl.d, wl.d_e), npdt)

        def one(e):
            a, b, c = self.expert(e)
            wg[e], wu[e], wd[e] = a, b, c

        with _cf.ThreadPoolExecutor(max_workers=threads or _threads()) as ex:
            list(ex.map(one, range(wl.E)))
        return wg, wu, wd


def _threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(16, n))


def make_inputs(wl: Workload | str, seed: int = 0) -> Inputs:
    if isinstance(wl, str):
        wl = get(wl)
    x = _draw(seed, (0,), (wl.T, wl.d), 1.0, wl.dtype)
    w_r = _draw(seed, (1,), (wl.E, wl.d), 1.0 / wl.d, wl.dtype)
    b_r = None
    if wl.router_bias_var is not None:
        b_r = _draw(seed, (2,), (wl.E,), wl.router_bias_var, "f32")
    return Inputs(wl=wl, seed=seed, x=x, w_r=w_r, b_r=b_r)


def as_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of stored inputs (bf16 bits or float32)."""
    if dtype == "bf16":
        return bf16_to_f32(a).astype(np.float64)
    return np.asarray(a, dtype=np.float32).astype(np.float64)
