"""Upload a workload's host inputs into torch device tensors (marshalling only).

bf16 inputs travel as their raw 16-bit patterns and are reinterpreted as
torch.bfloat16 on the device, so the device sees exactly the host bits.  Expert
weights are drawn and copied one expert at a time (threads draw ahead), which
keeps host memory small at the largest workload.
"""
from __future__ import annotations

import concurrent.futures as cf
from dataclasses import dataclass

import numpy as np
import torch

from . import Inputs, _threads


def _to_dev(a: np.ndarray, dtype: str, device) -> torch.Tensor:
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16))
        return t.to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


@dataclass
class DeviceInputs:
    x: torch.Tensor
    w_r: torch.Tensor
    b_r: torch.Tensor | None
    w_gate: torch.Tensor     # [E, d_e, d]
    w_up: torch.Tensor       # [E, d_e, d]
    w_down: torch.Tensor     # [E, d, d_e]
    shared: tuple | None     # (W_g, W_u, W_d) or None
    scales: tuple | None = None         # FP8: (gate [E,d_e], up [E,d_e], down [E,d]) fp32;
                                        # MXFP4: (gate [E,d/32,d_e], up, down [E,d_e/32,d]) uint8
    shared_scales: tuple | None = None  # the shared expert's, with a leading 1


def _upload_quant(inp: Inputs, device, threads) -> DeviceInputs:
    """Quantised expert weights: codes and scales as the workload stores them."""
    wl = inp.wl
    u8, f32 = torch.uint8, torch.float32
    if wl.weights == "fp8_e4m3":
        wg = torch.empty((wl.E, wl.d_e, wl.d), dtype=u8, device=device)
        wu = torch.empty((wl.E, wl.d_e, wl.d), dtype=u8, device=device)
        wd = torch.empty((wl.E, wl.d, wl.d_e), dtype=u8, device=device)
        sg = torch.empty((wl.E, wl.d_e), dtype=f32, device=device)
        su = torch.empty((wl.E, wl.d_e), dtype=f32, device=device)
        sd = torch.empty((wl.E, wl.d), dtype=f32, device=device)
    else:                                    # mxfp4: two codes per byte, E8M0 scales block-major
        wg = torch.empty((wl.E, wl.d_e, wl.d // 2), dtype=u8, device=device)
        wu = torch.empty((wl.E, wl.d_e, wl.d // 2), dtype=u8, device=device)
        wd = torch.empty((wl.E, wl.d, wl.d_e // 2), dtype=u8, device=device)
        sg = torch.empty((wl.E, wl.d // 32, wl.d_e), dtype=u8, device=device)
        su = torch.empty((wl.E, wl.d // 32, wl.d_e), dtype=u8, device=device)
        sd = torch.empty((wl.E, wl.d_e // 32, wl.d), dtype=u8, device=device)
    with cf.ThreadPoolExecutor(max_workers=threads or _threads()) as ex:
        futs = [ex.submit(inp.expert_q, e) for e in range(wl.E)]
        for e, fu in enumerate(futs):
            (qg, s_g), (qu, s_u), (qd, s_d) = fu.result()
            for dst, src in ((wg, qg), (wu, qu), (wd, qd), (sg, s_g), (su, s_u), (sd, s_d)):
                dst[e].copy_(torch.from_numpy(src).to(device))
            futs[e] = None
    shared = shared_scales = None
    sq = inp.shared_q()
    if sq is not None:
        shared = tuple(torch.from_numpy(q).to(device) for q, _ in sq)
        shared_scales = tuple(torch.from_numpy(sc).unsqueeze(0).to(device) for _, sc in sq)
    b_r = None if inp.b_r is None else torch.from_numpy(inp.b_r).to(device)
    return DeviceInputs(_to_dev(inp.x, wl.dtype, device), _to_dev(inp.w_r, wl.dtype, device), b_r,
                        wg, wu, wd, shared, (sg, su, sd), shared_scales)


def upload(inp: Inputs, device="cuda", threads: int | None = None) -> DeviceInputs:
    wl = inp.wl
    if wl.weights != "native":
        return _upload_quant(inp, device, threads)
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    wg = torch.empty((wl.E, wl.d_e, wl.d), dtype=tdt, device=device)
    wu = torch.empty((wl.E, wl.d_e, wl.d), dtype=tdt, device=device)
    wd = torch.empty((wl.E, wl.d, wl.d_e), dtype=tdt, device=device)
    with cf.ThreadPoolExecutor(max_workers=threads or _threads()) as ex:
        futs = [ex.submit(inp.expert, e) for e in range(wl.E)]
        for e, fu in enumerate(futs):
            a, b, c = fu.result()
            wg[e].copy_(_to_dev(a, wl.dtype, device))
            wu[e].copy_(_to_dev(b, wl.dtype, device))
            wd[e].copy_(_to_dev(c, wl.dtype, device))
            futs[e] = None
    sh = inp.shared()
    shared = None if sh is None else tuple(_to_dev(m, wl.dtype, device) for m in sh)
    b_r = None if inp.b_r is None else torch.from_numpy(inp.b_r).to(device)
    return DeviceInputs(_to_dev(inp.x, wl.dtype, device), _to_dev(inp.w_r, wl.dtype, device), b_r,
                        wg, wu, wd, shared)
