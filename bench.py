#!/usr/bin/env python3
"""MoE-layer forward throughput on one MI355X, with roofline and CPU-oracle baseline.

One step = one moe_forward call (router, dispatch, grouped SwiGLU experts, combine)
over one batch of synthetic tokens already resident in device memory.  Default
workload: the Mixtral 8x7B layer shape at a prefill batch of 4096 tokens (bf16
weights and activations, fp32 accumulate).  A decode-batch line (16 tokens, same
weights) rides along as "secondary" (also timed as replays of the call captured in a HIP
graph: ms_per_step_graph), the split ABI's moe_permute (the gather of token
rows into expert order) on the prefill routing as "secondary_permute", the backward pass
of the prefill call as "secondary_backward", and decode with FP8 and MXFP4 expert weights
as "secondary_fp8" and "secondary_mxfp4", and the two HBM-bound prefill-sized workloads -- the
Switch top-1 layer with capacity factor 1.25 and the DeepSeek-V3-shaped layer with 256 routed
experts and a shared expert -- as "secondary_switch" and "secondary_deepseek"; the prefill with
MXFP8 activations on the scaled FP8 MFMA (FP8 and MXFP4 weights) as "secondary_prefill_fp8_mx"
and "secondary_prefill_mxfp4_mx".  Every line
carries routing health (dropped fraction, MaxVio, per-expert counts; with the CPU baseline, the
oracle's near-tie tokens and how many the GPU routed differently).

Prints ONE JSON line.  Timing: W untimed warm-up steps, then K steps bracketed by
torch.cuda.synchronize(); per-stage durations come from HIP events that the library
records on its stream at the stage boundaries (moe_forward's stage_events).
"""
from __future__ import annotations

import argparse
import ctypes as C
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/sec at Mixtral shape; % bf16 MFMA peak / % HBM peak"
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0       # MI355X dense FP8 MFMA (also the rate of FP8 x FP4 products)
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="mixtral_prefill")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--secondaries", default="decode,permute,backward,fp8,mxfp4,prefill_mx,switch,deepseek",
                    help="comma-separated secondary lines to run after the Mixtral prefill line")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU work of the oracle sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (3 times): the reference kernel for "
                         "scaling rocprofv3 FETCH_SIZE / WRITE_SIZE to bytes")
    return ap.parse_args()


def copy_calibration():
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 3}))


class HipEvents:
    """hipEvent_t handles from the process's HIP runtime (the one torch loaded)."""

    def __init__(self):
        self.hip = C.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [C.POINTER(C.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        self.hip.hipEventDestroy.argtypes = [C.c_void_p]

    def create(self, n):
        arr = (C.c_void_p * n)()
        for i in range(n):
            h = C.c_void_p()
            if self.hip.hipEventCreate(C.byref(h)) != 0:
                raise RuntimeError("hipEventCreate failed")
            arr[i] = h
        return arr

    def elapsed_ms(self, a, b) -> float:
        ms = C.c_float()
        if self.hip.hipEventElapsedTime(C.byref(ms), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return ms.value

    def destroy(self, arr):
        for h in arr:
            self.hip.hipEventDestroy(h)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    d = os.path.join(ROOT, "sparse_mixture_experts_17_amd", "csrc")
    for f in sorted(os.listdir(d)):
        h.update(f.encode())
        h.update(open(os.path.join(d, f), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, stage: str):
    """HBM bytes per launch from the committed rocprofv3 PMC summary, if the kernels
    are unchanged since it was taken; else None."""
    try:
        t = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if t.get("source_hash") != kernel_source_hash():
        return None
    return t.get("per_launch_bytes", {}).get(workload, {}).get(stage)


def run_gpu(wl_name, steps, warmup, dev_weights=None, kernel_stage="gate_up", graph=False):
    """Upload a workload and time moe_forward on it.

    Timed region: `steps` calls, each recording HIP events only at the start and end of
    `kernel_stage` (two stream markers per call), bracketed by synchronisations.  A second,
    untimed pass records every stage boundary for the per-stage breakdown, and a third
    records nothing, to show what the markers cost.
    """
    import numpy as np
    import torch

    import sparse_mixture_experts_17_amd as moe
    import workloads as wl
    from workloads.device import upload

    w = wl.get(wl_name)
    inp = wl.make_inputs(w, seed=0)
    t0 = time.time()
    if dev_weights is None:
        dev = upload(inp)
    else:                                    # same experts and router (same streams), new tokens
        import workloads.device as wd
        dev = wd.DeviceInputs(wd._to_dev(inp.x, w.dtype, "cuda"), dev_weights.w_r, dev_weights.b_r,
                              dev_weights.w_gate, dev_weights.w_up, dev_weights.w_down, dev_weights.shared,
                              dev_weights.scales, dev_weights.shared_scales)
    t_up = time.time() - t0
    cap = -1 if w.capacity_factor is None else moe.moe_capacity(w.T, w.k, w.E, w.capacity_factor)
    shape = moe.make_shape(w.T, w.d, w.d_e, w.E, w.k, capacity=cap, renormalize=w.renormalize,
                           d_e_shared=w.d_e_shared, dtype=moe.MOE_BF16 if w.dtype == "bf16" else moe.MOE_F32,
                           scoring=1 if w.scoring == "sigmoid" else 0, n_group=w.n_group, topk_group=w.topk_group,
                           wfmt={"native": moe.MOE_W_NATIVE, "fp8_e4m3": moe.MOE_W_FP8_E4M3,
                                 "mxfp4": moe.MOE_W_MXFP4}[w.weights],
                           afmt={None: moe.MOE_A_NATIVE, "mxfp8": moe.MOE_A_MXFP8}[w.act])
    out = moe.alloc_forward(shape)
    ev = HipEvents()
    nst = moe._lib.MOE_NUM_STAGES
    names = moe._lib.STAGE_NAMES
    ks = names.index(kernel_stage)

    def call(events=None):
        moe.forward(shape, dev.x, dev.w_r, dev.b_r, dev.w_gate, dev.w_up, dev.w_down, dev.shared, out=out,
                    stage_events=events, scales=dev.scales, shared_scales=dev.shared_scales)

    def kernel_events():
        arr = (C.c_void_p * (nst + 1))()
        pair = ev.create(2)
        arr[ks], arr[ks + 1] = pair[0], pair[1]
        return arr, pair

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    marks = [kernel_events() for _ in range(steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    start.record()
    for s in range(steps):
        call(marks[s][0])
    end.record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    total_ms = start.elapsed_time(end)
    kernel_ms = float(np.mean([ev.elapsed_ms(p[0], p[1]) for _, p in marks]))
    for _, p in marks:
        ev.destroy(p)
    # per-stage breakdown (every boundary marked; not the timed region)
    full = [ev.create(nst + 1) for _ in range(steps)]
    for s in range(steps):
        call(full[s])
    torch.cuda.synchronize()
    stage_ms = np.array([[ev.elapsed_ms(e[i], e[i + 1]) for i in range(nst)] for e in full])
    for e in full:
        ev.destroy(e)
    # no markers at all
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for s in range(steps):
        call()
    b.record()
    torch.cuda.synchronize()
    plain_ms = a.elapsed_time(b) / steps
    stages = {n: float(v) for n, v in zip(names, stage_ms.mean(axis=0))}
    graph_ms = None
    if graph:
        # the same call captured once in a HIP graph and replayed (no per-launch host work)
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            call()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            call()
        for _ in range(warmup):
            g.replay()
        torch.cuda.synchronize()
        a.record()
        for s_ in range(steps):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        graph_ms = a.elapsed_time(b) / steps
        del g
    kept = out.kept.cpu().numpy()
    R_kept = int(kept.sum())
    touched = int((kept > 0).sum())
    return dict(w=w, shape=shape, cap=cap, total_ms=total_ms, wall_s=t_wall, stages=stages, kernel_ms=kernel_ms,
                steps=steps,
                plain_ms=plain_ms, graph_ms=graph_ms, R_kept=R_kept, touched=touched, upload_s=t_up, dev=dev, inp=inp,
                out=out)


def run_permute(info, steps, warmup):
    """The split ABI's moe_permute on the forward's routing: histogram, scan, stable rank and the
    gather of every kept assignment's token row into expert order (the fused forward instead
    gathers inside the gate/up product's loads).  Timed with events around each call."""
    import numpy as np
    import torch

    import sparse_mixture_experts_17_amd as moe

    w, shape, dev, out = info["w"], info["shape"], info["dev"], info["out"]
    R = w.T * w.k
    i32 = torch.int32
    kept = torch.empty(w.E, dtype=i32, device="cuda")
    offsets = torch.empty(w.E + 1, dtype=i32, device="cuda")
    row_token = torch.empty(R, dtype=i32, device="cuda")
    row_of = torch.empty((w.T, w.k), dtype=i32, device="cuda")
    x_perm = torch.empty((R, w.d), dtype=dev.x.dtype, device="cuda")

    def call():
        moe.moe_permute(shape, dev.x, out.idx, kept, offsets, row_token, row_of, x_perm, out.ws)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a_, b_ in evs:
        a_.record()
        call()
        b_.record()
    torch.cuda.synchronize()
    ms = float(np.mean([a_.elapsed_time(b_) for a_, b_ in evs]))
    rk = int(kept.sum())
    s = dev.x.element_size()
    nbytes = 2 * rk * w.d * s + R * 4 * 3 + route_chunks(w.T) * w.E * 4 * 2
    gbs = nbytes / (ms / 1e3) / 1e9
    return {"workload": w.name + " (moe_permute, split ABI)", "ms_per_call": ms, "rows": rk,
            "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS,
            "algorithmic": "kept rows x d x elem read + the same written, + idx, row_of, row_token, histograms"}


def route_chunks(T):
    return (T + 15) // 16


def layer_work(w, R_kept, touched):
    """Algorithmic FLOPs and bytes of one layer call (per unit figures x units)."""
    s = 2 if w.dtype == "bf16" else 4
    sw = {"native": s, "fp8_e4m3": 1, "mxfp4": 0.5 + 1 / 32}[w.weights]   # bytes per expert weight
    # (MXFP4: half a byte per element plus one scale byte per 32; FP8: + a 4-byte scale per row)
    flops_gate_up = 4 * w.d * w.d_e * R_kept
    flops_down = 2 * w.d * w.d_e * R_kept
    flops_router = 2 * w.d * w.E * w.T
    flops_shared = 6 * w.d * w.d_e_shared * w.T
    rs = 4 if w.weights == "fp8_e4m3" else 0           # bytes per weight row outside sw
    bytes_gate_up = touched * 2 * w.d_e * (w.d * sw + rs) + R_kept * w.d * s + R_kept * w.d_e * s
    bytes_down = touched * w.d * (w.d_e * sw + rs) + R_kept * w.d_e * s + R_kept * w.d * 4
    bytes_layer = (touched * 3 * w.d * w.d_e * sw + touched * (2 * w.d_e + w.d) * rs + w.E * w.d * s
                   + w.T * w.d * s + w.T * w.d * 4 + w.T * w.k * 8 + 3 * w.d * w.d_e_shared * sw)
    return dict(flops_gate_up=flops_gate_up, flops_down=flops_down, flops_layer=flops_gate_up + flops_down +
                flops_router + flops_shared, bytes_gate_up=bytes_gate_up, bytes_down=bytes_down,
                bytes_layer=bytes_layer)


def health(info):
    """Routing health of a call, from the GPU's own outputs: the dropped fraction of assignments
    (kevinluzbetak.com capacity worked example: the per-layer health check), MaxVio = (busiest
    expert's load - mean load) / mean load over the assignments before capacity
    (jacopoparretti.dev, "A bias"), per-expert counts, and the touched experts."""
    w, out = info["w"], info["out"]
    counts = out.counts.cpu().numpy().astype(int)
    kept = out.kept.cpu().numpy().astype(int)
    R = w.T * w.k
    mean = R / w.E
    return {"dropped_fraction": (R - int(kept.sum())) / R if R else 0.0,
            "dropped_assignments": R - int(kept.sum()),
            "maxvio": (int(counts.max()) - mean) / mean if R else 0.0,
            "experts_touched": int((kept > 0).sum()), "aux": float(out.aux.cpu()[0]),
            "counts": counts.tolist()}


def stage_rates(info):
    """Achieved GB/s of the HBM-bound small stages from their algorithmic bytes (router: x, W_r,
    indices and gates; combine: kept expert rows in fp32 + y, + the shared expert's output)."""
    w, st = info["w"], info["stages"]
    s = 2 if w.dtype == "bf16" else 4
    R = info["R_kept"]
    rb = w.T * w.d * s + w.E * w.d * s + w.T * w.k * 8
    cb = R * w.d * 4 + w.T * w.d * 4 + (w.T * w.d * 4 if w.d_e_shared else 0)
    out = {}
    for name, b in (("router", rb), ("combine", cb)):
        ms = st[name]
        out[name] = {"ms": ms, "algorithmic_bytes": b, "gbs": b / (ms / 1e3) / 1e9 if ms > 0 else None,
                     "frac_hbm": b / (ms / 1e3) / 1e9 / PEAK_HBM_GBS if ms > 0 else None}
    return out


def streaming_line(info, kernel_name):
    """JSON object of an HBM-bound prefill-sized workload (Switch capacity, DeepSeek-V3 shape):
    tokens/s, stage times, the dominant kernel's HBM roofline and the layer's fractions."""
    w = info["w"]
    ms = info["total_ms"] / info["steps"]
    work = layer_work(w, info["R_kept"], info["touched"])
    gu_ms = info["kernel_ms"]
    gb = work["bytes_gate_up"] / (gu_ms / 1e3) / 1e9
    st = info["stages"]
    dn = st["down"]
    return {
        "workload": w.name, "value": w.T / (ms / 1e3), "unit": "tokens/s", "ms_per_step": ms,
        "config": {"T": w.T, "d": w.d, "d_e": w.d_e, "E": w.E, "k": w.k, "capacity": info["cap"],
                   "d_e_shared": w.d_e_shared},
        "stages_ms": st, "ms_per_step_unmarked": info["plain_ms"],
        "roofline": {"kernel": kernel_name, "bound": "hbm", "achieved": gb, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": gb / PEAK_HBM_GBS, "traffic": measured_traffic(w.name, "gate_up"), "avg_ms": gu_ms,
                     "algorithmic": "gate+up weights of touched experts + gathered x rows + h rows"},
        "down": {"gbs": work["bytes_down"] / (dn / 1e3) / 1e9, "frac_hbm": work["bytes_down"] / (dn / 1e3) / 1e9
                 / PEAK_HBM_GBS, "traffic": measured_traffic(w.name, "down")},
        "layer": {"algorithmic_bytes": work["bytes_layer"], "flops": work["flops_layer"],
                  "frac_hbm": work["bytes_layer"] / (ms / 1e3) / 1e9 / PEAK_HBM_GBS,
                  "frac_mfma": work["flops_layer"] / (ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS,
                  "hbm_roofline_ms": work["bytes_layer"] / (PEAK_HBM_GBS * 1e9) * 1e3},
        "stage_rates": stage_rates(info),
        "health": health(info),
    }


def mx_prefill_line(info, fmt):
    """JSON object of a prefill run on the scaled FP8 MFMA (MXFP8 activations): tokens/s, stages and
    the gate/up product against the dense FP8 MFMA peak."""
    w = info["w"]
    ms = info["total_ms"] / info["steps"]
    work = layer_work(w, info["R_kept"], info["touched"])
    gu = info["kernel_ms"]
    tf = work["flops_gate_up"] / (gu / 1e3) / 1e12
    return {
        "workload": w.name, "value": w.T / (ms / 1e3), "unit": "tokens/s", "ms_per_step": ms,
        "stages_ms": info["stages"], "ms_per_step_unmarked": info["plain_ms"],
        "roofline": {"kernel": f"grouped_gemm_mx gate_up (MXFP8 x {fmt}, scaled MFMA)", "bound": "mfma",
                     "achieved": tf, "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s", "frac": tf / PEAK_FP8_TFLOPS,
                     "traffic": measured_traffic(w.name, "gate_up"), "avg_ms": gu,
                     "algorithmic": f"4*d*d_e FLOPs per kept row x {info['R_kept']} rows"},
        "layer_tflops": work["flops_layer"] / (ms / 1e3) / 1e12,
        "health": health(info),
    }


def secondary_line(dec, fmt):
    """JSON object of a decode run with quantised expert weights."""
    wd = dec["w"]
    steps = dec["steps"]
    dwork = layer_work(wd, dec["R_kept"], dec["touched"])
    dms = dec["total_ms"] / steps
    gb = dwork["bytes_gate_up"] / (dec["kernel_ms"] / 1e3) / 1e9
    return {
        "workload": wd.name, "value": wd.T / (dms / 1e3), "unit": "tokens/s", "ms_per_step": dms,
        "stages_ms": dec["stages"], "experts_touched": dec["touched"], "ms_per_step_unmarked": dec["plain_ms"],
        "ms_per_step_graph": dec["graph_ms"],
        "roofline": {"kernel": f"grouped_gemm gate_up (decode tiles, {fmt} weights)", "bound": "hbm",
                     "achieved": gb, "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": gb / PEAK_HBM_GBS,
                     "traffic": measured_traffic(wd.name, "gate_up"), "avg_ms": dec["kernel_ms"]},
        "layer_hbm_frac": dwork["bytes_layer"] / (dms / 1e3) / 1e9 / PEAK_HBM_GBS,
        "health": health(dec),
    }


def run_backward(info, steps, warmup, kernel_stage="dx_expert"):
    """Time moe_backward on the forward's inputs and routing (same weights, dy ~ N(0, 1)).

    As run_gpu: the timed region records HIP events only around `kernel_stage`; a second,
    untimed pass marks every stage boundary.
    """
    import numpy as np
    import torch

    import sparse_mixture_experts_17_amd as moe

    w, shape, dev = info["w"], info["shape"], info["dev"]
    fwd = moe.forward(shape, dev.x, dev.w_r, dev.b_r, dev.w_gate, dev.w_up, dev.w_down, dev.shared)
    dy = torch.from_numpy(info["inp"].dy()).to("cuda")
    out = moe.alloc_backward(shape, dev.b_r is not None)
    ev = HipEvents()
    nst = moe._lib.MOE_NUM_BSTAGES
    names = moe._lib.BSTAGE_NAMES
    ks = names.index(kernel_stage)

    def call(events=None):
        moe.backward(shape, dev.x, dev.w_r, dev.b_r, dev.w_gate, dev.w_up, dev.w_down, fwd, dy, 0.01, dev.shared,
                     out=out, stage_events=events)

    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    marks = []
    for _ in range(steps):
        arr = (C.c_void_p * (nst + 1))()
        pair = ev.create(2)
        arr[ks], arr[ks + 1] = pair[0], pair[1]
        marks.append((arr, pair))
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for s_ in range(steps):
        call(marks[s_][0])
    end.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end)
    kernel_ms = float(np.mean([ev.elapsed_ms(p[0], p[1]) for _, p in marks]))
    for _, p in marks:
        ev.destroy(p)
    full = [ev.create(nst + 1) for _ in range(steps)]
    for s_ in range(steps):
        call(full[s_])
    torch.cuda.synchronize()
    stage_ms = np.array([[ev.elapsed_ms(e[i], e[i + 1]) for i in range(nst)] for e in full])
    for e in full:
        ev.destroy(e)
    R = info["R_kept"]
    ms = total_ms / steps
    # products of the backward: gate/up recompute 4, u = dy W_d 2, dX 4, dW_d 2, dW_g + dW_u 4
    # (x d x d_e FLOPs per kept row); the shared expert adds 16 x d x d_e_shared per token
    flops = 16 * w.d * w.d_e * R + 16 * w.d * w.d_e_shared * w.T
    k_flops = 4 * w.d * w.d_e * R                     # dX = dA W_g + dB W_u (one launch)
    achieved = k_flops / (kernel_ms / 1e3) / 1e12
    return {
        "workload": w.name + " (backward)", "value": w.T / (ms / 1e3), "unit": "tokens/s", "ms_per_step": ms,
        "stages_ms": {n: float(v) for n, v in zip(names, stage_ms.mean(axis=0))},
        "tflops": flops / (ms / 1e3) / 1e12, "frac_mfma": flops / (ms / 1e3) / 1e12 / PEAK_BF16_TFLOPS,
        "roofline": {"kernel": "grouped_gemm dX = [dA|dB] [W_g;W_u] (large tiles)", "bound": "mfma",
                     "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS, "traffic": measured_traffic(w.name, "dx_expert"),
                     "avg_ms": kernel_ms,
                     "algorithmic": f"4*d*d_e FLOPs per kept row x {R} rows"},
    }


def oracle_routing_check(info, idx):
    """CPU-baseline leg: the oracle's routing of the same tokens against the GPU's idx -- the
    near-tie tokens (k-th and (k+1)-th scores within 1e-6) and how many of them the GPU routed
    differently; every other token must match exactly."""
    import numpy as np
    import workloads as wl
    from oracle import moe_oracle as mo
    w, inp = info["w"], info["inp"]
    _, _, own, _, nt = mo.route(wl.as_f64(inp.x, w.dtype), wl.as_f64(inp.w_r, w.dtype), w.k, inp.b_r,
                                w.renormalize, scoring=w.scoring, n_group=w.n_group, topk_group=w.topk_group)
    differ = np.nonzero((own != idx).any(axis=1))[0]
    return {"near_ties": int(len(nt)), "flipped": int(np.isin(differ, nt).sum()),
            "other_mismatches": int((~np.isin(differ, nt)).sum())}


def cpu_baseline(info, target_s):
    """The CPU oracle, unchanged, on the first n tokens of the same workload."""
    import numpy as np
    import workloads as wl
    from oracle import moe_oracle as mo
    try:
        import threadpoolctl
        pools = threadpoolctl.threadpool_info()
        cores = max([p.get("num_threads", 1) for p in pools if p.get("user_api") == "blas"] or [1])
    except Exception:
        cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    w, inp = info["w"], info["inp"]
    x = wl.as_f64(inp.x, w.dtype)
    w_r = wl.as_f64(inp.w_r, w.dtype)
    import concurrent.futures as cf
    with cf.ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
        experts = list(ex.map(lambda e: tuple(wl.as_f64(m, w.dtype) for m in inp.expert(e)), range(w.E)))
    sh = inp.shared()
    sh = None if sh is None else tuple(wl.as_f64(m, w.dtype) for m in sh)
    cap = -1 if w.capacity_factor is None else mo.capacity(w.T, w.k, w.E, w.capacity_factor)
    n = min(w.T, 64)
    while True:                                   # grow the token sample ...
        t0 = time.perf_counter()
        mo.moe_forward(x[:n], w_r, experts, w.k, cap, inp.b_r, w.renormalize, sh)
        dt = time.perf_counter() - t0
        if dt >= target_s / 3 or n >= w.T:
            break
        n = min(w.T, max(n * 2, int(n * target_s / 3 / max(dt, 1e-3))))
    reps, total = 1, dt
    while total < target_s / 2 and n == w.T:      # ... then repeat whole passes
        t0 = time.perf_counter()
        mo.moe_forward(x[:n], w_r, experts, w.k, cap, inp.b_r, w.renormalize, sh)
        total += time.perf_counter() - t0
        reps += 1
    dt = total / reps
    return {"value": n / dt, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "sample": f"first {n} of {w.T} tokens of {w.name} x {reps} pass(es), fp64 NumPy oracle, "
                      f"{dt:.2f} s per pass (weights widened to fp64 beforehand, untimed)"}


def main():
    a = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if a.gpus != 1 or world != 1:
        print(json.dumps({"error": "one GPU only: the layer is measured at its per-GPU shape; expert "
                          "parallelism across GPUs is not implemented", "n_gpus": a.gpus}))
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    if a.copy_calibration:
        copy_calibration()
        return
    print(f"[bench] workload {a.workload}: generating and uploading inputs", file=sys.stderr, flush=True)
    info = run_gpu(a.workload, a.steps, a.warmup)
    w = info["w"]
    work = layer_work(w, info["R_kept"], info["touched"])
    ms = info["total_ms"] / a.steps
    value = w.T / (ms / 1e3)
    st = info["stages"]
    gu_ms = info["kernel_ms"]
    mfma_bound = w.dtype == "bf16" and info["R_kept"] / max(info["touched"], 1) >= 315
    if mfma_bound:
        achieved = work["flops_gate_up"] / (gu_ms / 1e3) / 1e12
        roof = {"kernel": "grouped_gemm gate_up (SiLU*up fused)", "bound": "mfma", "achieved": achieved,
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
                "traffic": measured_traffic(w.name, "gate_up"), "avg_ms": gu_ms,
                "algorithmic": f"4*d*d_e FLOPs per kept row x {info['R_kept']} rows"}
    else:
        achieved = work["bytes_gate_up"] / (gu_ms / 1e3) / 1e9
        roof = {"kernel": "grouped_gemm gate_up (SiLU*up fused)", "bound": "hbm", "achieved": achieved,
                "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS,
                "traffic": measured_traffic(w.name, "gate_up"), "avg_ms": gu_ms,
                "algorithmic": "gate+up weights of touched experts + x_perm rows + h rows"}
    layer = {"tflops": work["flops_layer"] / (ms / 1e3) / 1e12, "gbs": work["bytes_layer"] / (ms / 1e3) / 1e9}
    layer["frac_mfma"] = layer["tflops"] / PEAK_BF16_TFLOPS
    layer["frac_hbm"] = layer["gbs"] / PEAK_HBM_GBS
    line = {
        "metric": METRIC, "value": value, "unit": "tokens/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32", "data": "synthetic",
        "config": {"workload": w.name, "T": w.T, "d": w.d, "d_e": w.d_e, "E": w.E, "k": w.k,
                   "capacity": info["cap"], "d_e_shared": w.d_e_shared, "parallelism": "none (1 GPU)",
                   "weights": "random, seeded (N(0,1/fan_in)), bf16"},
        "roofline": roof,
        "layer": layer,
        "stages_ms": st,
        "ms_per_step_unmarked": info["plain_ms"],
        "stage_rates": stage_rates(info),
        "health": health(info),
    }
    sec_on = set() if a.no_secondary or w.name != "mixtral_prefill" else set(a.secondaries.split(","))
    if "decode" in sec_on:
        print("[bench] secondary: mixtral_decode on the same weights", file=sys.stderr, flush=True)
        dec = run_gpu("mixtral_decode", max(a.steps, 20), a.warmup, dev_weights=info["dev"], graph=True)
        wd = dec["w"]
        dwork = layer_work(wd, dec["R_kept"], dec["touched"])
        dms = dec["total_ms"] / max(a.steps, 20)
        gb = dwork["bytes_gate_up"] / (dec["kernel_ms"] / 1e3) / 1e9
        line["secondary"] = {
            "workload": wd.name, "value": wd.T / (dms / 1e3), "unit": "tokens/s", "ms_per_step": dms,
            "stages_ms": dec["stages"], "experts_touched": dec["touched"], "ms_per_step_unmarked": dec["plain_ms"],
            "ms_per_step_graph": dec["graph_ms"],
            "roofline": {"kernel": "grouped_gemm gate_up (decode tiles)", "bound": "hbm", "achieved": gb,
                         "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": gb / PEAK_HBM_GBS,
                         "traffic": measured_traffic(wd.name, "gate_up"), "avg_ms": dec["kernel_ms"]},
            "layer_hbm_frac": dwork["bytes_layer"] / (dms / 1e3) / 1e9 / PEAK_HBM_GBS,
            "health": health(dec),
        }
    if "permute" in sec_on:
        print("[bench] secondary: moe_permute (split ABI) on the same routing", file=sys.stderr, flush=True)
        line["secondary_permute"] = run_permute(info, max(a.steps, 20), a.warmup)
        torch.cuda.empty_cache()
    if "backward" in sec_on:
        print("[bench] secondary: backward pass on the same inputs", file=sys.stderr, flush=True)
        line["secondary_backward"] = run_backward(info, a.steps, a.warmup)
        torch.cuda.empty_cache()
    if sec_on & {"fp8", "mxfp4", "prefill_mx", "switch", "deepseek"}:
        del info["dev"]
        torch.cuda.empty_cache()
    if "fp8" in sec_on:
        print("[bench] secondary: mixtral_decode_fp8 (FP8 E4M3 expert weights)", file=sys.stderr, flush=True)
        dec = run_gpu("mixtral_decode_fp8", max(a.steps, 20), a.warmup)
        line["secondary_fp8"] = secondary_line(dec, "FP8")
        del dec
    if "mxfp4" in sec_on:
        print("[bench] secondary: mixtral_decode_mxfp4 (MXFP4 expert weights)", file=sys.stderr, flush=True)
        torch.cuda.empty_cache()
        dec = run_gpu("mixtral_decode_mxfp4", max(a.steps, 20), a.warmup, graph=True)
        line["secondary_mxfp4"] = secondary_line(dec, "MXFP4")
        del dec
    if "prefill_mx" in sec_on:
        for key, name, fmt in (("secondary_prefill_fp8_mx", "mixtral_prefill_fp8_mx", "FP8"),
                               ("secondary_prefill_mxfp4_mx", "mixtral_prefill_mxfp4_mx", "MXFP4")):
            print(f"[bench] secondary: {name} (MXFP8 activations, scaled FP8 MFMA)", file=sys.stderr, flush=True)
            torch.cuda.empty_cache()
            sec = run_gpu(name, a.steps, a.warmup)
            line[key] = mx_prefill_line(sec, fmt)
            del sec
    routed = [(line, info, info["out"].idx.cpu().numpy())]
    for key, name, kern in (("secondary_switch", "switch_capacity", "grouped_gemm gate_up (stream tiles)"),
                            ("secondary_deepseek", "deepseek_v3",
                             "grouped_gemm gate_up (stream tiles, 256 routed experts)")):
        if name.split("_")[0] in sec_on:
            print(f"[bench] secondary: {name}", file=sys.stderr, flush=True)
            torch.cuda.empty_cache()
            sec = run_gpu(name, max(a.steps, 10), a.warmup)
            line[key] = streaming_line(sec, kern)
            routed.append((line[key], {"w": sec["w"], "inp": sec["inp"]}, sec["out"].idx.cpu().numpy()))
            del sec
    if not a.no_cpu_baseline:
        print("[bench] CPU oracle baseline", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(info, a.cpu_seconds)
        for obj, inf, idx in routed:
            obj.setdefault("health", {})["oracle_routing"] = oracle_routing_check(inf, idx)
    print(json.dumps(line))


if __name__ == "__main__":
    main()
