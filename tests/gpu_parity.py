"""Shared checks of the HIP path against the CPU oracle (used by the GPU tests).

Protocol
  1. Routing: idx from the GPU equals the oracle's top-k for every token outside the
     near-tie set N (k-th and (k+1)-th oracle probabilities within 1e-6); tokens in N
     are reported and must still hold a valid choice.
  2. Gates within 1e-5 absolute of the oracle's gates for the GPU's idx; counts exact;
     f equal to float32(counts / (T k)); P and aux within 1e-5 relative.
  3. Dispatch (kept, offsets, row_token, row_of, dropped set) bit-exact against the
     oracle's dispatch of the GPU's idx; x_perm rows bit-identical to x rows.
  4. Output: max|y - y_oracle| / rms(y_oracle) <= 1e-4 (fp32) or 2e-2 (bf16) (MXFP8 activations:
     the per-element bound described at MX_EPS), the
     oracle run with the GPU's routing, over every token (at full size too; the oracle
     streams the experts).
  5. Backward: every gradient (dx, dW_r, db_r, dW_g, dW_u, dW_d, the shared expert's, dL/dg)
     against the oracle's backward with the GPU's routing: ||G - G_oracle|| / ||G_oracle||
     <= BWD_FROB and max|G - G_oracle| / max|G_oracle| <= BWD_PEAK per tensor and per expert
     slice of the weight gradients.
"""
from __future__ import annotations

import concurrent.futures as cf
import sys
import time

import numpy as np
import torch

import sparse_mixture_experts_17_amd as moe
import workloads as wl
from oracle import moe_oracle as mo
from workloads.device import upload

TOL = {"f32": 1e-4, "bf16": 2e-2}
# MXFP8 activations (act = "mxfp8"): h is rounded to E4M3 steps of 6-12 %, so an h value within
# the accumulation error of a rounding midpoint may round either way, and an exact oracle cannot
# say which.  The oracle bounds, per output element, what such roundings can change
# (swiglu_mx_deviation) for products accurate to MX_EPS times the sum of their terms'
# magnitudes -- 2^-16, against at most 1.2e-6 measured for the scaled FP8 MFMA on random
# 4,096-term dot products.  Checks: |dy| <= bound + MX_TAU rms(y) everywhere (MX_TAU covers
# the fp32 gates and the combine), and rms(dy) <= MX_RMS rms(y) (a wrong scale or layout moves
# the rms by order one; midpoint roundings by a few 1e-3).
MX_EPS = 2.0 ** -16
MX_TAU = 1e-3
MX_RMS = 1e-2
# Backward bars, per gradient tensor and per expert slice of the weight gradients (an
# expert's gradient is a sum over its rows, few for a small expert, so an element can be a
# sum of a handful of products of heavy-tailed factors and a bar relative to the rms would
# be set by the tail):
#   frob: ||G - G_ref|| / ||G_ref||;   peak: max|G - G_ref| / max|G_ref|.
# In bf16 a gradient's operands carry at most two roundings to bf16 each (2^-9 relative:
# dy, then dA or dB; g dy; h), summed in fp32.  Over many terms the errors add like
# 2^-9 x sqrt(#terms) x (typical term) against a largest element of several times
# sqrt(#terms) x (typical term): a few 1e-3 for both measures, the rms one bar 1e-2.  For a
# one-row expert the slice is an outer product and its largest element carries the
# roundings of both factors in full, up to 4 x 2^-9 ~ 8e-3: the peak bar is 2e-2.  fp32
# (fp32 operands, fp32 accumulation): 1e-5.
BWD_FROB = {"f32": 1e-5, "bf16": 1e-2}
BWD_PEAK = {"f32": 1e-5, "bf16": 2e-2}

# dL/daux of the backward tests: the Switch auxiliary-loss weight (0.01)
D_AUX = 0.01


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def shape_of(w: wl.Workload, T=None):
    cap = -1 if w.capacity_factor is None else moe.moe_capacity(w.T, w.k, w.E, w.capacity_factor)
    return moe.make_shape(w.T if T is None else T, w.d, w.d_e, w.E, w.k, capacity=cap, renormalize=w.renormalize,
                          d_e_shared=w.d_e_shared, dtype=moe.MOE_BF16 if w.dtype == "bf16" else moe.MOE_F32,
                          scoring=1 if w.scoring == "sigmoid" else 0, n_group=w.n_group,
                          topk_group=w.topk_group, wfmt=WFMT[w.weights], afmt=AFMT[w.act]), cap


WFMT = {"native": 0, "fp8_e4m3": 1, "mxfp4": 2}
AFMT = {None: 0, "mxfp8": 1}


def dequant(q, sc, weights):
    """Float64 weights from quantised storage, decoded by the oracle."""
    return mo.dequantize_rows(q, sc) if weights == "fp8_e4m3" else mo.dequantize_mx_rows(q, sc)


def router_kw(w: wl.Workload) -> dict:
    return dict(scoring=w.scoring, n_group=w.n_group, topk_group=w.topk_group)


def oracle_cap(w: wl.Workload) -> int:
    return -1 if w.capacity_factor is None else mo.capacity(w.T, w.k, w.E, w.capacity_factor)


def f64(a, w):
    return wl.as_f64(a, w.dtype)


def expert_f64(inp, e):
    """Float64 weights of routed expert e as the GPU sees them (quantised codes decoded and
    scaled by the oracle)."""
    if inp.wl.weights != "native":
        return tuple(dequant(q, sc, inp.wl.weights) for q, sc in inp.expert_q(e))
    return tuple(f64(m, inp.wl) for m in inp.expert(e))


def shared_f64(inp):
    if inp.wl.weights != "native":
        sq = inp.shared_q()
        return None if sq is None else tuple(dequant(q, sc, inp.wl.weights) for q, sc in sq)
    sh = inp.shared()
    return None if sh is None else tuple(f64(m, inp.wl) for m in sh)


def experts_f64(inp, es, threads=16):
    """{e: float64 weights} for the experts in es, drawn in parallel on the host."""
    def one(e):
        return e, expert_f64(inp, e)
    with cf.ThreadPoolExecutor(max_workers=threads) as ex:
        return dict(ex.map(one, sorted(set(int(e) for e in es))))


class LazyExperts:
    """Float64 routed-expert weights for the oracle, drawn on demand with a bounded window of
    experts drawn ahead in threads, so a full-size check holds about `window` experts in host
    memory at a time (the oracle asks for experts in ascending order)."""

    def __init__(self, inp, window=16, threads=16, tag=""):
        self.inp, self.window, self.tag = inp, window, tag
        self.E = inp.wl.E
        self.pool = cf.ThreadPoolExecutor(max_workers=threads)
        self.futs = {}
        self.t0 = time.time()

    def __len__(self):
        return self.E

    def __getitem__(self, e):
        for f in range(e, min(self.E, e + self.window)):
            if f not in self.futs:
                self.futs[f] = self.pool.submit(expert_f64, self.inp, f)
        for f in [f for f in self.futs if f < e]:
            del self.futs[f]
        out = self.futs.pop(e).result()
        if self.E >= 64 and (e + 1) % 64 == 0:
            log(f"  [{self.tag}] oracle through expert {e + 1}/{self.E} ({time.time() - self.t0:.1f}s)")
        return out

    def close(self):
        self.pool.shutdown(wait=True, cancel_futures=True)
        self.futs.clear()


def check_valid_choice(w, sel, pick, own, slack=mo.NEAR_TIE):
    """A near-tie token's GPU choice `pick` must be a top-k the selection rule could have made
    had the scores moved by less than `slack`: k distinct experts in descending score order,
    none below the oracle's k-th score by more than `slack`, and an allowed set of experts in
    which no unpicked expert scores more than `slack` above the lowest pick.  Without groups
    every expert is allowed.  Under the group limit the allowed set is topk_group groups: the
    groups of the picks, every group whose score clearly beats the topk_group-th group score
    (by more than `slack`), and, to fill up, groups within `slack` of that score; every group in
    it must score at least the topk_group-th group score minus `slack`."""
    pick = np.asarray(pick, np.int64)
    assert len(set(pick.tolist())) == w.k, pick
    assert np.all(np.diff(sel[pick]) <= slack), ("slots not in descending order", pick, sel[pick])
    low = sel[pick].min()
    assert low >= np.sort(sel[np.asarray(own, np.int64)])[0] - slack, ("pick below the oracle's k-th", pick)
    if w.n_group == 1:
        others = np.ones(w.E, bool)
        others[pick] = False
        assert not np.any(sel[others] > low + slack), ("a higher unpicked expert", pick)
        return
    gs = w.E // w.n_group
    gsc = sel.reshape(w.n_group, gs).max(axis=1)
    gth = np.sort(gsc)[::-1][w.topk_group - 1]              # the topk_group-th group score
    must = set((pick // gs).tolist()) | set(np.nonzero(gsc > gth + slack)[0].tolist())
    assert len(must) <= w.topk_group, ("more groups than allowed", pick)
    assert all(gsc[g] >= gth - slack for g in must), ("pick outside the allowed groups", pick, gsc)
    for g in must:                     # inside the allowed groups the picks are the top-k
        members = np.arange(g * gs, (g + 1) * gs)
        rest = members[~np.isin(members, pick)]
        assert not np.any(sel[rest] > low + slack), ("a higher unpicked expert", pick, g)
    fill = [g for g in range(w.n_group) if g not in must and gth - slack <= gsc[g] <= low + slack]
    assert len(fill) >= w.topk_group - len(must), ("allowed groups cannot be completed", pick)


def check_routing(w, inp, idx, gate, counts, f, P, aux):
    """Steps 1-2; returns (p, near-tie tokens, flipped tokens)."""
    x = f64(inp.x, w)
    r, p, own_idx, _, nt = mo.route(x, f64(inp.w_r, w), w.k, inp.b_r, w.renormalize, **router_kw(w))
    mask = np.ones(w.T, bool)
    mask[nt] = False
    assert np.array_equal(idx[mask], own_idx[mask]), \
        f"routing differs on {np.nonzero((idx != own_idx).any(1) & mask)[0][:10]}"
    flipped = [int(t) for t in nt if not np.array_equal(idx[t], own_idx[t])]
    for t in flipped:          # a near tie may go either way, but the choice must be a valid top-k
        sel = p[t] if w.scoring == "softmax" else p[t] + (0 if inp.b_r is None else inp.b_r)
        check_valid_choice(w, sel, idx[t], own_idx[t])
    g_ref = mo.gates(p, idx, w.renormalize)
    assert np.max(np.abs(gate - g_ref)) <= 1e-5, np.max(np.abs(gate - g_ref))
    c_ref, f_ref, P_ref, aux_ref = mo.load_balance_stats(p, idx, w.E)
    assert np.array_equal(counts, c_ref)
    assert np.array_equal(f, f_ref.astype(np.float32))
    assert np.max(np.abs(P - P_ref) / np.maximum(P_ref, 1e-30)) <= 1e-5, np.max(np.abs(P - P_ref) / P_ref)
    assert abs(aux - aux_ref) <= 1e-5 * abs(aux_ref)
    return p, nt, flipped


def check_dispatch(w, idx, cap, kept, offsets, row_token, row_of):
    d = mo.dispatch(idx, w.E, cap)
    assert np.array_equal(kept, d.kept)
    assert np.array_equal(offsets, d.offsets)
    R = int(d.offsets[-1])
    assert np.array_equal(row_token[:R], d.row_token)
    assert np.array_equal(row_of, d.row_of)
    return d


def run_forward(w: wl.Workload, seed=0, sample=None, repeat_check=False, assert_y=True):
    """Forward on the GPU + every protocol check.  sample=None: all tokens' y checked (the oracle
    runs over every expert, a window of experts in memory at a time).  assert_y=False leaves
    the output bound to the caller (the measured error is returned)."""
    t0 = time.time()
    inp = wl.make_inputs(w, seed)
    dev = upload(inp)
    shape, cap = shape_of(w)
    assert cap == oracle_cap(w)
    out = moe.forward(shape, dev.x, dev.w_r, dev.b_r, dev.w_gate, dev.w_up, dev.w_down, dev.shared,
                      scales=dev.scales, shared_scales=dev.shared_scales)
    torch.cuda.synchronize()
    h = {k: getattr(out, k).cpu().numpy() for k in
         ["y", "idx", "gate", "counts", "kept", "f", "P", "aux", "offsets", "row_token", "row_of"]}
    if repeat_check:
        out2 = moe.forward(shape, dev.x, dev.w_r, dev.b_r, dev.w_gate, dev.w_up, dev.w_down, dev.shared,
                           scales=dev.scales, shared_scales=dev.shared_scales)
        torch.cuda.synchronize()
        R = int(h["offsets"][-1])                # row_token past R is left untouched
        for k in h:
            a, b = getattr(out2, k).cpu().numpy(), h[k]
            if k == "row_token":
                a, b = a[:R], b[:R]
            assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), f"second run differs in {k}"
    del dev, out
    torch.cuda.empty_cache()
    p, nt, flipped = check_routing(w, inp, h["idx"], h["gate"], h["counts"], h["f"], h["P"], h["aux"][0])
    disp = check_dispatch(w, h["idx"], cap, h["kept"], h["offsets"], h["row_token"], h["row_of"])
    x = f64(inp.x, w)
    sh = shared_f64(inp)
    mx = w.act == "mxfp8"
    y_bound = None
    if sample is None:
        ex = LazyExperts(inp, tag=w.name)
        try:
            ref = mo.moe_forward(x, f64(inp.w_r, w), ex, w.k, cap, inp.b_r, w.renormalize, sh, idx=h["idx"],
                                 act=w.act, mx_eps=MX_EPS if mx else None, **router_kw(w))
        finally:
            ex.close()
        y_ref, y, y_bound = ref.y, h["y"], ref.y_bound
        del ref
    else:
        toks = np.asarray(sample)
        kept_mask = disp.row_of[toks] >= 0
        need = h["idx"][toks][kept_mask]
        ex = experts_f64(inp, need)
        g_ref = mo.gates(p[toks], h["idx"][toks], w.renormalize)
        y_ref = mo.outputs_for_tokens(x[toks], h["idx"][toks], g_ref, kept_mask, lambda e: ex[e], sh, act=w.act,
                                      mx_eps=MX_EPS if mx else None)
        if mx:
            y_ref, y_bound = y_ref
        y = h["y"][toks]
    err = mo.rel_err(y, y_ref)
    if mx:
        rms = float(np.sqrt(np.mean(y_ref * y_ref)))
        dy = np.abs(y - y_ref)
        room = y_bound + MX_TAU * rms
        rms_ratio = float(np.sqrt(np.mean(dy * dy))) / rms
        log(f"[{w.name}] MXFP8: max |dy| / (bound + tau rms) = {float(np.max(dy / room)):.3f}; rms(dy)/rms(y) = "
            f"{rms_ratio:.2e}; median bound / rms = {float(np.median(y_bound)) / rms:.2e}")
        assert np.all(dy <= room), np.argwhere(dy > room)[:5]
        assert rms_ratio <= MX_RMS, rms_ratio
    dropped = int(disp.dropped.size)
    log(f"[{w.name}] T={w.T} d={w.d} d_e={w.d_e} E={w.E} k={w.k} cap={cap}: max|dy|/rms={err:.3e} "
        f"near_ties={len(nt)} flipped={len(flipped)} dropped={dropped} ({time.time() - t0:.1f}s)")
    if assert_y and not mx:
        assert err <= TOL[w.dtype], err
    return dict(err=err, near_ties=len(nt), flipped=len(flipped), dropped=dropped, host=h)


def run_backward(w: wl.Workload, seed=0, d_aux=D_AUX, repeat_check=False):
    """Forward + backward on the GPU; every gradient against the oracle's backward with the
    GPU's routing (after the forward's routing and dispatch checks)."""
    t0 = time.time()
    inp = wl.make_inputs(w, seed)
    dev = upload(inp)
    shape, cap = shape_of(w)
    out = moe.forward(shape, dev.x, dev.w_r, dev.b_r, dev.w_gate, dev.w_up, dev.w_down, dev.shared)
    dy_h = inp.dy()
    dy = torch.from_numpy(dy_h).to(dev.x.device)
    g = moe.backward(shape, dev.x, dev.w_r, dev.b_r, dev.w_gate, dev.w_up, dev.w_down, out, dy, d_aux, dev.shared)
    torch.cuda.synchronize()
    names = ["dx", "dw_r", "dw_gate", "dw_up", "dw_down", "dgate"] + (["db_r"] if g.db_r is not None else [])
    hg = {k: getattr(g, k).cpu().numpy() for k in names}
    if g.dshared is not None:
        for i, k in enumerate(["dws_gate", "dws_up", "dws_down"]):
            hg[k] = g.dshared[i].cpu().numpy()
    hf = {k: getattr(out, k).cpu().numpy() for k in
          ["idx", "gate", "counts", "f", "P", "aux", "kept", "offsets", "row_token", "row_of"]}
    if repeat_check:
        g2 = moe.backward(shape, dev.x, dev.w_r, dev.b_r, dev.w_gate, dev.w_up, dev.w_down, out, dy, d_aux,
                          dev.shared)
        torch.cuda.synchronize()
        for k in names:
            assert np.array_equal(getattr(g2, k).cpu().numpy().view(np.uint8), hg[k].view(np.uint8)), \
                f"second backward differs in {k}"
    del dev, out, g
    torch.cuda.empty_cache()
    check_routing(w, inp, hf["idx"], hf["gate"], hf["counts"], hf["f"], hf["P"], hf["aux"][0])
    check_dispatch(w, hf["idx"], cap, hf["kept"], hf["offsets"], hf["row_token"], hf["row_of"])
    log(f"[{w.name} backward] GPU done ({time.time() - t0:.1f}s); oracle backward")
    ex = experts_f64(inp, range(w.E))
    ref = mo.moe_backward(f64(inp.x, w), f64(inp.w_r, w), [ex[e] for e in range(w.E)], w.k, dy_h.astype(np.float64),
                          d_aux, cap, inp.b_r, w.renormalize, shared_f64(inp), idx=hf["idx"], **router_kw(w))
    want = {"dx": ref.dx, "dw_r": ref.dw_r, "dw_gate": ref.dw_gate, "dw_up": ref.dw_up, "dw_down": ref.dw_down,
            "dgate": ref.dgate}
    if "db_r" in hg:
        want["db_r"] = ref.db_r
    if ref.dshared is not None:
        want.update(dws_gate=ref.dshared[0], dws_up=ref.dshared[1], dws_down=ref.dshared[2])
    errs = {}
    for k, v in want.items():
        got = hg[k]
        assert got.shape == v.shape, (k, got.shape, v.shape)
        slices = list(range(v.shape[0])) if k in ("dw_gate", "dw_up", "dw_down") else [None]
        frob = peak = 0.0
        for e in slices:
            a, b = (got, v) if e is None else (got[e], v[e])
            if not np.any(b):                   # e.g. an expert with no rows: exactly zero
                assert not np.any(a), (k, e)
                continue
            frob = max(frob, float(np.linalg.norm(a - b)) / float(np.linalg.norm(b)))
            peak = max(peak, float(np.max(np.abs(a - b))) / float(np.max(np.abs(b))))
        errs[k] = (frob, peak)
    log(f"[{w.name} backward] T={w.T} d={w.d} d_e={w.d_e} E={w.E} k={w.k} cap={cap}: "
        + " ".join(f"{k}={f:.1e}/{m:.1e}" for k, (f, m) in errs.items()) + f" ({time.time() - t0:.1f}s)")
    for k, (f, m) in errs.items():
        assert f <= BWD_FROB[w.dtype] and m <= BWD_PEAK[w.dtype], (k, f, m)
    return errs
