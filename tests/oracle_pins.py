"""Pins of the CPU oracle: checks against what the pages and mathematics fix.

Each ``pin_*`` function raises AssertionError when the oracle disagrees with
something outside itself: a number printed on a page (tests/golden), a closed
form, an invariant the pages state, a library routine in a special case that
reduces to it, or the pure-Python brute force.  ``test_oracle.py`` runs them;
``test_oracle_mutations.py`` plants mistakes in the oracle and checks that at
least one pin fails for each.

Functions reach the oracle through module attributes (``mo.softmax`` ...) so that
a planted mistake is seen by every pin.
"""
from __future__ import annotations

import json
import math
import os
from math import comb

import numpy as np

from oracle import bruteforce as bf
from oracle import moe_oracle as mo
from oracle import param_count as pc

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")))


def _rng(seed):
    return np.random.default_rng(seed)


def _logit_inputs(logits):
    """x = e_0 and W_r[:, 0] = logits, so x W_r^T reproduces the logits exactly."""
    logits = np.asarray(logits, np.float64)
    E = logits.size
    d = 4
    x = np.zeros((1, d))
    x[0, 0] = 1.0
    w_r = np.zeros((E, d))
    w_r[:, 0] = logits
    # fill the other columns with values that x does not see
    w_r[:, 1:] = np.arange(E * (d - 1)).reshape(E, d - 1) * 0.37
    return x, w_r


def _tiny_layer(seed, T=5, d=6, d_e=4, E=5, bias=False, shared=False, scale=1.0):
    g = _rng(seed)
    x = g.standard_normal((T, d)) * scale
    w_r = g.standard_normal((E, d))
    experts = [(g.standard_normal((d_e, d)) * 0.7, g.standard_normal((d_e, d)) * 0.7,
                g.standard_normal((d, d_e)) * 0.7) for _ in range(E)]
    b_r = g.standard_normal(E) if bias else None
    sh = None
    if shared:
        sh = (g.standard_normal((3, d)), g.standard_normal((3, d)), g.standard_normal((d, 3)))
    return x, w_r, experts, b_r, sh


# --------------------------------------------------------------------------- printed examples

def pin_router_worked_examples():
    for ex in GOLDEN["router_examples"]:
        if "logits" in ex:
            logits = ex["logits"]
        else:
            logits = [0.0] * ex["E"]
            for e, v in ex["top_logits"].items():
                logits[int(e)] = v
        x, w_r = _logit_inputs(logits)
        r, p, idx, g = mo.route(x, w_r, ex["k"])[:4]
        assert list(idx[0]) == ex["experts"], (ex["source"], idx[0])
        tol = 0.5 * 10 ** (-ex["decimals"])
        assert np.allclose(g[0], ex["gates"], atol=tol + 1e-12), (ex["source"], g[0])
        if "probs" in ex:
            assert np.allclose(p[0], ex["probs"], atol=tol + 1e-12), (ex["source"], p[0])
        # closed form for k = 2: g_0 = 1 / (1 + e^{-(r_a - r_b)})
        ra, rb = logits[ex["experts"][0]], logits[ex["experts"][1]]
        assert abs(g[0, 0] - 1.0 / (1.0 + math.exp(-(ra - rb)))) < 1e-14


def pin_capacity_worked_example():
    c = GOLDEN["capacity_example"]
    cap = mo.capacity(c["T"], c["k"], c["E"], c["C"])
    assert cap == c["slots"], cap
    # Build the routing the page describes: 3000 of the 4096 tokens choose expert 0
    # (as one of their two experts); the rest spread over the others.
    T, E, k = c["T"], c["E"], c["k"]
    idx = np.zeros((T, k), np.int32)
    for t in range(T):
        if t < c["chosen_by"]:
            idx[t] = (0, 1 + t % 3)
        else:
            idx[t] = (1 + t % 3, 1 + (t + 1) % 3)
    disp = mo.dispatch(idx, E, cap)
    assert disp.counts[0] == c["chosen_by"]
    assert disp.counts[0] - disp.kept[0] == c["overflow"]
    # arrival order: the first `cap` of expert 0's assignments survive
    assert np.all(disp.row_of[:cap, 0] >= 0) and np.all(disp.row_of[cap:c["chosen_by"], 0] == -1)
    # the capacity rule at the Switch-style workload: 1.25 * 8192 / 64 = 160
    assert mo.capacity(8192, 1, 64, 1.25) == 160
    assert mo.capacity(10, 1, 4, 1.0) == 2        # 2.5 rounds down


def pin_param_counts():
    for name, pcnt in GOLDEN["param_counts"].items():
        total, active = pc.moe_param_count(pcnt["cfg"])
        assert total == pcnt["total"], (name, total)
        assert active == pcnt["active"], (name, active)
    m = GOLDEN["param_counts"]["mixtral"]
    cfg = m["cfg"]
    assert 2 * 4096 ** 2 + 2 * 4096 * 1024 == cfg["attn"]
    lt, la = pc.layer_params(cfg["d"], cfg["d_e"], cfg["E"], cfg["k"])
    assert lt == m["eight_experts"] + m["router"]
    assert lt + cfg["attn"] + m["norms_per_layer"] == m["per_layer"]
    assert la + cfg["attn"] + m["norms_per_layer"] == m["active_per_layer"]
    assert pc.layer_params(cfg["d"], cfg["d_e"], 1, 1)[0] - cfg["d"] == m["one_expert"]
    ds = GOLDEN["param_counts"]["deepseek_v3"]
    assert pc.layer_params(7168, 2048, 1, 1)[0] - 7168 == ds["one_expert"]


def pin_flop_arithmetic():
    f = GOLDEN["flops"]["router_vs_experts"]
    router = pc.router_flops_per_token(f["d"], f["E"])
    experts = pc.forward_flops_per_token(f["d"], f["d_e"], f["E"], f["experts_run"]) - router
    assert abs(router - f["router_approx"]) / f["router_approx"] < 0.01, router
    assert abs(experts - f["experts_approx"]) / f["experts_approx"] < 0.001, experts
    assert 0.004 < router / experts < 0.006                       # "half a percent"
    fw = GOLDEN["flops"]["forward_per_token"]
    # 2 FLOPs per active matrix parameter: one layer's count equals 2 * its active params
    d, de, E, k = 4096, 14336, 8, 2
    assert pc.forward_flops_per_token(d, de, E, k) == 2 * pc.layer_params(d, de, E, k)[1]
    assert abs(2 * fw["n_active"] / 1e9 - fw["gflops"]) < 1e-9
    tr = GOLDEN["flops"]["train"]
    moe = pc.train_flops(tr["n_active"], tr["tokens"])
    dense = pc.train_flops(tr["n_total"], tr["tokens"])
    assert abs(moe - tr["moe_flops"]) / tr["moe_flops"] < 0.02
    assert abs(dense - tr["dense_flops"]) / tr["dense_flops"] < 0.01
    assert round(pc.flops_ratio(tr["n_total"], tr["n_active"])) == tr["ratio"]


def pin_combinatorics():
    c = GOLDEN["combinatorics"]
    assert comb(8, 2) == c["c_8_2"]
    assert abs(comb(8, 2) ** 32 / c["paths_mixtral_approx"] - 1) < 0.1
    assert comb(256, 8) == c["c_256_8"]


# --------------------------------------------------------------------------- library routines / closed forms

def pin_softmax_library():
    import scipy.special
    g = _rng(1)
    r = g.standard_normal((7, 9)) * 5
    assert np.allclose(mo.softmax(r), scipy.special.softmax(r, axis=1), rtol=1e-13, atol=0)
    # large logits stay finite (max subtraction)
    big = np.array([[1000.0, 999.0, -1000.0]])
    p = mo.softmax(big)
    assert np.all(np.isfinite(p)) and abs(p[0, 0] - 1 / (1 + math.exp(-1))) < 1e-14


def pin_silu():
    import torch
    z = np.linspace(-30, 30, 241)
    ref = torch.nn.functional.silu(torch.tensor(z, dtype=torch.float64)).numpy()
    assert np.allclose(mo.silu(z), ref, rtol=1e-14, atol=1e-300)
    assert mo.silu(np.array([0.0]))[0] == 0.0
    assert abs(mo.silu(np.array([1.0]))[0] - 1 / (1 + math.exp(-1))) < 1e-15


def pin_dense_swiglu_special_case():
    """E = 1, k = 1: the layer is one dense SwiGLU FFN (gate 1)."""
    import torch
    g = _rng(2)
    T, d, de = 6, 5, 7           # non-square everywhere, so a transposed operand fails
    x = g.standard_normal((T, d))
    w_r = g.standard_normal((1, d))
    wg, wu, wd = g.standard_normal((de, d)), g.standard_normal((de, d)), g.standard_normal((d, de))
    res = mo.moe_forward(x, w_r, [(wg, wu, wd)], k=1)
    tx = torch.tensor(x)
    lin = torch.nn.functional.linear
    ref = lin(torch.nn.functional.silu(lin(tx, torch.tensor(wg))) * lin(tx, torch.tensor(wu)),
              torch.tensor(wd)).numpy()
    assert np.allclose(res.y, ref, rtol=1e-12, atol=1e-12)
    assert np.all(res.gate == 1.0) and np.all(res.idx == 0)
    assert np.allclose(mo.swiglu_ffn(x, wg, wu, wd), ref, rtol=1e-12, atol=1e-12)


# --------------------------------------------------------------------------- invariants

def pin_gates_sum_to_one():
    x, w_r, experts, b_r, _ = _tiny_layer(3, T=40, E=7, bias=True)
    for k in (1, 2, 3, 7):
        _, p, idx, g = mo.route(x, w_r, k, b_r)[:4]
        assert np.allclose(g.sum(axis=1), 1.0, atol=1e-14)
        assert np.all(np.diff(g, axis=1) <= 1e-15)       # slots in descending gate order
        # chosen experts are the k most probable
        thr = np.take_along_axis(p, idx.astype(np.int64), axis=1).min(axis=1)
        for t in range(p.shape[0]):
            others = np.delete(p[t], idx[t])
            assert np.all(others <= thr[t] + 0.0)


def pin_tie_break():
    """W_r = 0: every logit is 0, so experts 0..k-1 win with gates 1/k and P = 1/E."""
    g = _rng(4)
    T, d, E = 9, 6, 6
    x = g.standard_normal((T, d))
    w_r = np.zeros((E, d))
    for k in (1, 2, 4):
        _, p, idx, gt = mo.route(x, w_r, k)[:4]
        assert np.all(idx == np.arange(k)[None, :])
        assert np.allclose(gt, 1.0 / k, atol=1e-15)
        counts, f, P, aux = mo.load_balance_stats(p, idx, E)
        assert np.allclose(P, 1.0 / E, atol=1e-15)
    # a tie between two non-top experts also goes to the lower index
    x1, w1 = _logit_inputs([0.5, 1.0, 0.5, 0.5, 2.0])
    _, _, idx, _ = mo.route(x1, w1, 3)[:4]
    assert list(idx[0]) == [4, 1, 0]


def pin_aux_balanced():
    """T = m E, W_r = c [I | 0], x_t = e_{t mod E}: f = P = 1/E and aux = 1 exactly."""
    E, m, d, c = 8, 5, 11, 3.0
    T = m * E
    x = np.zeros((T, d))
    for t in range(T):
        x[t, t % E] = 1.0
    w_r = np.zeros((E, d))
    w_r[:, :E] = c * np.eye(E)
    _, p, idx, _ = mo.route(x, w_r, 1)[:4]
    counts, f, P, aux = mo.load_balance_stats(p, idx, E)
    assert np.all(counts == m)
    assert np.allclose(f, 1.0 / E, atol=1e-15) and np.allclose(P, 1.0 / E, atol=1e-15)
    assert abs(aux - 1.0) < 1e-14
    # unbalanced routing has aux > 1: everything to expert 0
    x0 = np.zeros((T, d))
    x0[:, 0] = 1.0
    _, p0, idx0, _ = mo.route(x0, w_r, 1)[:4]
    assert mo.load_balance_stats(p0, idx0, E)[3] > 1.5
    # f counts all k choices: sums to 1 at any k, and is 1/E when k = E
    x2, w2, _, _, _ = _tiny_layer(5, T=30, E=6)
    _, pE, iE, _ = mo.route(x2, w2, 6)[:4]
    assert np.allclose(mo.load_balance_stats(pE, iE, 6)[1], 1.0 / 6, atol=1e-15)
    for k in (1, 2, 3):
        _, p2, i2, _ = mo.route(x2, w2, k)[:4]
        assert abs(mo.load_balance_stats(p2, i2, 6)[1].sum() - 1.0) < 1e-14
        assert np.allclose(mo.load_balance_stats(p2, i2, 6)[2], p2.mean(axis=0))


def pin_near_ties():
    x, w_r = _logit_inputs([1.0, 1.0 + 5e-7, 0.0, 1.0 + 1e-5])
    _, p, _, _ = mo.route(x, w_r, 2)[:4]
    # p is about 0.3 for the three near-equal logits: the 2nd/3rd gap (experts 1
    # and 0) is about 1.5e-7 < 1e-6, the 1st/2nd gap about 2.8e-6 > 1e-6
    assert list(mo.near_ties(p, 2)) == [0]
    assert list(mo.near_ties(p, 1)) == []
    x2, w2 = _logit_inputs([3.0, 1.0, 0.0])
    _, p2, _, _ = mo.route(x2, w2, 1)[:4]
    assert list(mo.near_ties(p2, 1)) == [] and list(mo.near_ties(p2, 3)) == []


def pin_near_ties_grouped():
    """Near ties under the group limit, on hand-built selection scores.

    Eight experts in four groups of two ({0,1}, {2,3}, {4,5}, {6,7}), two groups allowed.  A token
    is reported when either decision rests on a gap below 1e-6: the topk_group-th against the
    next group score, or the k-th against the next expert score among the allowed experts.
    Gaps elsewhere (between allowed groups, inside excluded groups) must not report it.
    """
    e = 5e-7
    k2 = np.array([
        [0.9, 0.2, 0.5, 0.1, 0.5 + e, 0.3, 0.1, 0.0],    # 2nd vs 3rd group score: reported
        [0.9, 0.7, 0.7 + e, 0.1, 0.2, 0.1, 0.0, 0.05],   # 2nd vs 3rd allowed expert: reported
        [0.9, 0.1, 0.5, 0.3, 0.2, 0.1, 0.05, 0.0],       # no small gap
        [0.9, 0.8, 0.5, 0.0, 0.5 - e, 0.0, 0.1, 0.0],    # 2nd vs 3rd group: reported (the experts agree)
    ])
    assert list(mo.near_ties_grouped(k2, 2, 4, 2)) == [0, 1, 3]
    k3 = np.array([
        [0.9, 0.3, 0.8, 0.1, 0.3 - e, 0.0, 0.0, 0.0],    # tie with an expert of an excluded group only
        [0.9, 0.5, 0.9 - e, 0.0, 0.2, 0.0, 0.1, 0.0],    # 1st vs 2nd (both allowed): not a decision
        [0.9, 0.8, 0.7, 0.6, 0.5, 0.4, 0.3, 0.2],        # no small gap
        [0.9, 0.85, 0.6, 0.55, 0.6 + e, 0.0, 0.1, 0.0],  # 2nd vs 3rd group score: reported
    ])
    assert list(mo.near_ties_grouped(k3, 3, 4, 2)) == [3]
    # every group allowed: only the expert decision counts (row 3's group gap no longer decides)
    assert list(mo.near_ties_grouped(k2[3:4], 2, 4, 4)) == []
    assert list(mo.near_ties_grouped(k2[1:2], 2, 4, 4)) == [0]
    # one group: the plain near-tie rule
    g = _rng(41)
    sc = g.random((200, 8))
    sc[::3, 5] = sc[::3, 2] + 3e-7
    for k in (1, 2, 3):
        assert np.array_equal(mo.near_ties_grouped(sc, k, 1, 1), mo.near_ties(sc, k))
    # tokens not reported keep their chosen set under any perturbation that moves each
    # score by less than a quarter of the threshold
    sc = g.random((400, 12)) * 1e-5                     # many gaps near the threshold
    for k, ng, tg in ((2, 4, 2), (3, 3, 1), (4, 6, 3)):
        nt = set(mo.near_ties_grouped(sc, k, ng, tg).tolist())
        assert 0 < len(nt) < sc.shape[0]
        base = mo.group_limited_top_k(sc, k, ng, tg)
        for trial in range(20):
            pert = sc + (g.random(sc.shape) - 0.5) * 0.5e-6
            moved = mo.group_limited_top_k(pert, k, ng, tg)
            for t in range(sc.shape[0]):
                if t not in nt:
                    assert set(base[t]) == set(moved[t]), (k, ng, tg, t)


def pin_e4m3_encode_library():
    """E4M3 rounding against torch's float8_e4m3fn conversion (round to nearest even): random
    values over the whole range, every midpoint between neighbouring codes (ties must land on
    the even code), every code's own value (exact round trip), saturation above 448."""
    import torch
    g = _rng(51)
    v = g.standard_normal(100000) * np.exp2(g.integers(-14, 10, 100000))
    v = np.clip(v, -448, 448)
    want = torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(mo.e4m3_encode(v), want)
    codes = np.arange(256, dtype=np.uint8)
    vals = mo.e4m3_decode(codes)
    ok = ~np.isnan(vals)
    assert np.array_equal(mo.e4m3_encode(vals[ok]), codes[ok])
    pos = np.sort(vals[ok & (vals > 0)])
    mid = (pos[:-1] + pos[1:]) / 2
    got = mo.e4m3_encode(mid)
    assert np.array_equal(got, torch.from_numpy(mid.astype(np.float32)).to(torch.float8_e4m3fn)
                          .view(torch.uint8).numpy())
    assert np.all(got % 2 == 0)
    assert list(mo.e4m3_encode(np.array([448.0, 463.9, 1e4, -1e4]))) == [0x7E, 0x7E, 0x7E, 0xFE]


def pin_mxfp8_scale_rule():
    """The MX block scale 2^X, X = floor(log2 block max) - 8, on hand-worked blocks, and the
    rounding error bound it implies: at most half a step of E4M3 at the element's size
    (2^-4 relative in the normal range; 2^(X-10) absolute below it), and elements above
    448 * 2^X saturating to exactly that."""
    rows = np.zeros((6, 64))
    rows[0, :32] = 448.0                 # X = 0
    rows[1, 5] = 1.0                     # X = -8
    rows[2, 31] = -0.75                  # floor(log2 0.75) = -1: X = -9
    rows[3, :] = 2.0 ** -140             # below the smallest scale: X clamps to -127
    rows[4, 33] = 3.0                    # second block only: X = -7; first block all zero
    rows[5, :32] = np.arange(32) * 0.25  # max 7.75: X = -6, and 7.75 * 2^6 = 496 saturates to 448
    q, sc = mo.mxfp8_quantize_rows(rows)
    assert sc.tolist() == [[127, 0], [119, 0], [118, 0], [0, 0], [0, 120], [121, 0]], sc.tolist()
    back = mo.dequantize_mxfp8_rows(q, sc)
    assert np.array_equal(back[:3], rows[:3]) and np.array_equal(back[4], rows[4])
    assert back[5, 31] == 7.0 and back[5, 28] == 7.0 and back[5, 4] == 1.0
    g = _rng(52)
    v = g.standard_normal((40, 256)) * np.exp2(g.integers(-20, 20, (40, 1)))
    q, sc = mo.mxfp8_quantize_rows(v)
    back = mo.dequantize_mxfp8_rows(q, sc)
    X = np.repeat(sc.astype(np.int64) - 127, 32, axis=1)
    sat = np.abs(v) > 448.0 * np.exp2(X)               # the block maximum can land in (448, 512) * 2^X
    normal = (np.abs(v) >= np.exp2(X - 6.0)) & ~sat
    sub = np.abs(v) < np.exp2(X - 6.0)
    assert sat.any() and normal.any() and sub.any()
    assert np.all(np.abs(back - v)[normal] <= np.abs(v)[normal] * 2.0 ** -4)
    assert np.all(np.abs(back - v)[sub] <= np.exp2(X[sub] - 10.0))
    assert np.array_equal(np.abs(back)[sat], (448.0 * np.exp2(X))[sat])


def pin_mxfp8_layer_bruteforce():
    """The layer with MXFP8 activations against the pure-Python brute force (table-search
    E4M3 rounding), with capacity, bias, a shared expert and both scorings."""
    for seed, T, d, de, E, k, cap, scoring in [(61, 3, 64, 32, 4, 2, 2, "softmax"), (62, 4, 32, 64, 5, 1, -1,
                                                                                      "sigmoid")]:
        g = _rng(seed)
        x = g.standard_normal((T, d))
        w_r = g.standard_normal((E, d))
        ex = [(g.standard_normal((de, d)) * .3, g.standard_normal((de, d)) * .3, g.standard_normal((d, de)) * .3)
              for _ in range(E)]
        sh = (g.standard_normal((32, d)) * .3, g.standard_normal((32, d)) * .3, g.standard_normal((d, 32)) * .3)
        b = g.standard_normal(E) * 0.2
        res = mo.moe_forward(x, w_r, ex, k, cap, b, True, sh, scoring=scoring, act="mxfp8")
        yb, ib, _ = bf.moe_dense_bruteforce(x.tolist(), w_r.tolist(), [tuple(m.tolist() for m in e) for e in ex], k,
                                            cap, b.tolist(), True, tuple(m.tolist() for m in sh), scoring, act="mxfp8")
        assert np.array_equal(res.idx, np.array(ib))
        assert np.allclose(res.y, np.array(yb), rtol=1e-12, atol=1e-12)
        # the rounding changes the output by about the E4M3 step, not more
        plain = mo.moe_forward(x, w_r, ex, k, cap, b, True, sh, scoring=scoring)
        assert 1e-3 < mo.rel_err(res.y, plain.y) < 0.3


def pin_silu_range():
    """SiLU's minimum sits where its derivative vanishes, and silu_range agrees with a dense scan
    of random intervals (some holding the minimum)."""
    assert abs(mo.silu_grad(np.float64(mo.SILU_ARGMIN))) < 1e-14
    g = _rng(81)
    lo = g.uniform(-4, 3, 300)
    hi = lo + g.uniform(0, 2, 300)
    mn, mx = mo.silu_range(lo, hi)
    for i in range(300):
        z = np.linspace(lo[i], hi[i], 20001)
        v = mo.silu(z)
        assert mn[i] <= v.min() + 1e-15 and abs(mn[i] - v.min()) < 1e-8
        assert abs(mx[i] - v.max()) < 1e-15


def pin_mxfp8_round_interval():
    """Reachable MXFP8 values: a point interval gives the rounding itself; an element at a rounding
    midpoint reaches both neighbours; and every row drawn inside the intervals (each element
    independently, the block scale following the drawn maximum) rounds inside [qlo, qhi] --
    with intervals that straddle midpoints, zero, and block maxima at powers of two."""
    g = _rng(82)
    v = g.standard_normal((6, 64)) * np.exp2(g.integers(-6, 6, (6, 1)))
    qlo, qhi = mo.mxfp8_round_interval(v, v)
    assert np.array_equal(qlo, mo.mxfp8_round_rows(v)) and np.array_equal(qhi, qlo)
    row = np.zeros((1, 32))
    row[0, 0] = 256.0                                  # scale 2^0
    row[0, 1] = 1.0625                                 # midpoint of 1.0 and 1.125
    lo, hi = mo.mxfp8_round_interval(row - 1e-9, row + 1e-9)
    assert lo[0, 1] == 1.0 and hi[0, 1] == 1.125
    for trial in range(40):
        v = g.standard_normal((3, 64)) * np.exp2(g.integers(-4, 4, (3, 1)))
        v[0, 3] = 2.0 ** g.integers(-3, 4)             # a block maximum right at a power of two
        r = np.abs(v) * g.uniform(0, 0.05, v.shape) * (g.random(v.shape) < 0.5)
        lo, hi = v - r, v + r
        qlo, qhi = mo.mxfp8_round_interval(lo, hi)
        for _ in range(25):
            pt = lo + (hi - lo) * g.random(v.shape)
            ends = g.random(v.shape)
            pt = np.where(ends < 0.1, lo, np.where(ends > 0.9, hi, pt))     # some elements at an end
            q = mo.mxfp8_round_rows(pt)
            assert np.all(q >= qlo) and np.all(q <= qhi)
        for ends in (lo, hi):                          # the end points themselves
            q = mo.mxfp8_round_rows(ends)
            assert np.all(q >= qlo) and np.all(q <= qhi)


def pin_swiglu_mx_deviation():
    """The MXFP8 SwiGLU deviation bound holds for products computed with errors up to eps times
    the sum of the terms' magnitudes: random such errors in a and b, h rounded from float32,
    the down product recomputed -- every output within the bound, and some h codes do flip."""
    g = _rng(83)
    m, d, de, eps = 24, 64, 96, 3e-3
    X = mo.mxfp8_round_rows(g.standard_normal((m, d)))
    wg, wu = g.standard_normal((de, d)) / 8, g.standard_normal((de, d)) / 8
    wd = g.standard_normal((d, de)) / 10
    hq, qlo, qhi, bound = mo.swiglu_mx_deviation(X, wg, wu, wd, eps)
    a, b = X @ wg.T, X @ wu.T
    A, B = np.abs(X) @ np.abs(wg).T, np.abs(X) @ np.abs(wu).T
    o = hq @ wd.T
    flips = 0
    for _ in range(60):
        ap = a + eps * A * g.uniform(-1, 1, a.shape)
        bp = b + eps * B * g.uniform(-1, 1, b.shape)
        hp = mo.mxfp8_round_rows((mo.silu(ap) * bp).astype(np.float32))
        assert np.all(hp >= qlo) and np.all(hp <= qhi)
        flips += int((hp != hq).sum())
        assert np.all(np.abs(hp @ wd.T - o) <= bound)
    assert flips > 0
    assert np.all(bound >= 0)


def pin_dispatch_invariants():
    g = _rng(6)
    for (T, E, k, cap) in [(50, 5, 2, -1), (50, 5, 2, 7), (33, 4, 3, 0), (64, 8, 1, 5), (0, 3, 2, 4)]:
        idx = np.stack([g.permutation(E)[:k] for _ in range(T)]) if T else np.zeros((0, k), np.int32)
        d = mo.dispatch(idx, E, cap)
        assert d.counts.sum() == T * k
        assert np.all(d.kept <= (d.counts if cap < 0 else np.minimum(d.counts, cap)))
        assert int(d.kept.sum()) + d.dropped.size == T * k
        assert d.offsets[0] == 0 and np.all(np.diff(d.offsets) == d.kept)
        # each kept row holds its token, rows of an expert are in arrival order
        for e in range(E):
            rows = []
            for a in range(T * k):
                t, j = divmod(a, k)
                if idx[t, j] == e and d.row_of[t, j] >= 0:
                    rows.append((a, d.row_of[t, j]))
            rr = [r for _, r in rows]
            assert rr == list(range(d.offsets[e], d.offsets[e + 1]))
            for a, r in rows:
                assert d.row_token[r] == a // k
        # dropped = beyond the first cap arrivals of each expert
        seen = np.zeros(E, int)
        for a in range(T * k):
            t, j = divmod(a, k)
            e = idx[t, j]
            assert (d.row_of[t, j] < 0) == (cap >= 0 and seen[e] >= cap)
            seen[e] += 1


def pin_bruteforce_agreement():
    """Sparse oracle == pure-Python dense evaluation with zero gates (tiny inputs)."""
    cases = [
        dict(seed=7, T=5, d=6, d_e=4, E=5, k=2, cap=-1),
        dict(seed=8, T=6, d=5, d_e=3, E=4, k=1, cap=-1, bias=True),
        dict(seed=9, T=8, d=4, d_e=5, E=3, k=2, cap=3),
        dict(seed=10, T=7, d=3, d_e=2, E=6, k=3, cap=2, shared=True),
        dict(seed=11, T=4, d=4, d_e=4, E=4, k=4, cap=-1, renorm=False),
        dict(seed=12, T=6, d=5, d_e=3, E=5, k=2, cap=0),
    ]
    for c in cases:
        x, w_r, experts, b_r, sh = _tiny_layer(c["seed"], T=c["T"], d=c["d"], d_e=c["d_e"], E=c["E"],
                                               bias=c.get("bias", False), shared=c.get("shared", False))
        renorm = c.get("renorm", True)
        res = mo.moe_forward(x, w_r, experts, c["k"], c["cap"], b_r, renorm, sh)
        yb, ib, gb = bf.moe_dense_bruteforce(x.tolist(), w_r.tolist(),
                                             [tuple(m.tolist() for m in ex) for ex in experts],
                                             c["k"], c["cap"], None if b_r is None else b_r.tolist(),
                                             renorm, None if sh is None else tuple(m.tolist() for m in sh))
        assert np.array_equal(res.idx, np.array(ib)), c
        assert np.allclose(res.gate, np.array(gb), rtol=0, atol=1e-14), c
        assert np.allclose(res.y, np.array(yb), rtol=1e-12, atol=1e-12), c
        if c["cap"] == 0:
            # every assignment dropped: only the shared expert (absent here) remains
            assert np.all(res.y == 0.0)


def pin_upcycling():
    """E identical experts: y = FFN(x) for any router, since gates sum to one."""
    g = _rng(13)
    T, d, de, E = 12, 6, 5, 4
    x = g.standard_normal((T, d))
    w_r = g.standard_normal((E, d))
    ex = (g.standard_normal((de, d)), g.standard_normal((de, d)), g.standard_normal((d, de)))
    ref = mo.swiglu_ffn(x, *ex)
    for k in (1, 2, 4):
        res = mo.moe_forward(x, w_r, [ex] * E, k)
        assert np.allclose(res.y, ref, rtol=1e-12, atol=1e-12)


def pin_wide_ffn_identity():
    """A wide SwiGLU cut into E consecutive hidden blocks sums back to the wide FFN
    (Zero to Frontier, 'An MoE layer is a wide FFN with blocks switched off');
    with W_r = 0 and k = E every gate is 1/E, so y = FFN_wide(x) / E."""
    g = _rng(14)
    T, d, E, de = 5, 6, 4, 3
    dff = E * de
    x = g.standard_normal((T, d))
    Wg, Wu, Wd = g.standard_normal((dff, d)), g.standard_normal((dff, d)), g.standard_normal((d, dff))
    wide = mo.swiglu_ffn(x, Wg, Wu, Wd)
    experts = [(Wg[i * de:(i + 1) * de], Wu[i * de:(i + 1) * de], Wd[:, i * de:(i + 1) * de]) for i in range(E)]
    assert np.allclose(sum(mo.swiglu_ffn(x, *e) for e in experts), wide, rtol=1e-12, atol=1e-12)
    res = mo.moe_forward(x, np.zeros((E, d)), experts, k=E)
    assert np.allclose(res.y, wide / E, rtol=1e-12, atol=1e-12)


def pin_per_token_path():
    """outputs_for_tokens (per-token form) agrees with the expert-loop form."""
    x, w_r, experts, b_r, sh = _tiny_layer(15, T=9, E=5, bias=True, shared=True)
    res = mo.moe_forward(x, w_r, experts, 2, 3, b_r, True, sh)
    sel = [0, 3, 8]
    y = mo.outputs_for_tokens(x[sel], res.idx[sel], res.gate[sel], res.disp.row_of[sel] >= 0,
                              lambda e: experts[e], sh)
    assert np.allclose(y, res.y[sel], rtol=1e-12, atol=1e-12)


def pin_rel_err():
    a = np.array([[3.0, -4.0]])
    assert abs(mo.rel_err(a + np.array([[0.0, 0.1]]), a) - 0.1 / math.sqrt(12.5)) < 1e-15





# --------------------------------------------------------------------------- DeepSeek-V3 style router

def pin_sigmoid_selects_like_softmax():
    """sigmoid and softmax are both increasing in the logit, so without a bias and group
    limit they choose the same experts in the same order; only the gate values differ."""
    g = _rng(21)
    x, w_r = g.standard_normal((40, 9)), g.standard_normal((16, 9))
    for k in (1, 3, 8):
        i_soft = mo.route(x, w_r, k)[2]
        r, s, i_sig, gt, _ = mo.route(x, w_r, k, scoring="sigmoid")
        assert np.array_equal(i_soft, i_sig)
        sel = 1.0 / (1.0 + np.exp(-np.take_along_axis(r, i_sig.astype(np.int64), axis=1)))
        assert np.allclose(gt, sel / sel.sum(axis=1, keepdims=True), rtol=1e-14, atol=0)
        assert np.allclose(gt.sum(axis=1), 1.0, atol=1e-14)
        raw = mo.route(x, w_r, k, scoring="sigmoid", renormalize=False)[3]
        assert np.allclose(raw, sel, rtol=1e-14, atol=0)


def pin_selection_bias_only():
    """A bias moves the choice but never enters the gate values."""
    x, w_r = _logit_inputs([1.0, 0.5, -0.5, 0.2])
    b = np.array([0.0, 0.0, 10.0, 0.0])
    r, s, idx, gt, _ = mo.route(x, w_r, 2, b_r=b, scoring="sigmoid")
    assert list(idx[0]) == [2, 0]
    s2, s0 = 1 / (1 + math.exp(0.5)), 1 / (1 + math.exp(-1.0))
    assert abs(gt[0, 0] - s2 / (s2 + s0)) < 1e-15 and abs(gt[0, 1] - s0 / (s2 + s0)) < 1e-15
    # P averages the affinities, not the biased scores
    assert np.allclose(s[0], 1 / (1 + np.exp(-np.array([1.0, 0.5, -0.5, 0.2]))), rtol=1e-15)


def pin_group_limit():
    """Group limit: a worked case, and the two limits where it changes nothing."""
    # 8 experts in 4 groups of 2; only the best group may be used
    x, w_r = _logit_inputs([3.0, -2.0, 2.5, 2.4, 0.0, 0.1, -1.0, -3.0])
    for scoring in ("softmax", "sigmoid"):
        idx = mo.route(x, w_r, 2, scoring=scoring, n_group=4, topk_group=1)[2]
        assert list(idx[0]) == [0, 1], (scoring, idx)      # expert 2 (2.5) is in a dropped group
        idx = mo.route(x, w_r, 3, scoring=scoring, n_group=4, topk_group=2)[2]
        assert list(idx[0]) == [0, 2, 3], (scoring, idx)
    g = _rng(22)
    x, w_r, b = g.standard_normal((30, 7)), g.standard_normal((12, 7)), g.standard_normal(12) * 0.1
    for scoring in ("softmax", "sigmoid"):
        free = mo.route(x, w_r, 4, b_r=b, scoring=scoring)[2]
        assert np.array_equal(mo.route(x, w_r, 4, b_r=b, scoring=scoring, n_group=3, topk_group=3)[2], free)
        assert np.array_equal(mo.route(x, w_r, 4, b_r=b, scoring=scoring, n_group=12, topk_group=4)[2], free)


def pin_grouped_bruteforce():
    """Sigmoid scoring, selection bias and group limit against the pure-Python brute force."""
    for seed, T, d, de, E, k, ng, tg, cap in [(31, 6, 5, 3, 8, 2, 4, 2, -1), (32, 7, 4, 4, 6, 3, 3, 2, 3),
                                              (33, 5, 6, 2, 8, 4, 2, 1, -1)]:
        x, w_r, experts, b_r, sh = _tiny_layer(seed, T=T, d=d, d_e=de, E=E, bias=True, shared=(seed == 32))
        b_r = b_r * 0.2
        res = mo.moe_forward(x, w_r, experts, k, cap, b_r, True, sh, scoring="sigmoid", n_group=ng,
                             topk_group=tg)
        yb, ib, gb = bf.moe_dense_bruteforce(x.tolist(), w_r.tolist(),
                                             [tuple(m.tolist() for m in ex) for ex in experts], k, cap,
                                             b_r.tolist(), True, None if sh is None else
                                             tuple(m.tolist() for m in sh), "sigmoid", ng, tg)
        assert np.array_equal(res.idx, np.array(ib))
        assert np.allclose(res.gate, np.array(gb), rtol=0, atol=1e-14)
        assert np.allclose(res.y, np.array(yb), rtol=1e-12, atol=1e-12)


def pin_e4m3_library():
    """Every one of the 256 E4M3 codes decodes as torch's float8_e4m3fn does (an
    independent implementation of the same OCP format), NaN in the same places."""
    import torch
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = mo.e4m3_decode(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert np.array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))   # -0 stays -0


def pin_e4m3_fixed_points():
    """Values the format definition fixes: one, the largest finite value, the smallest
    normal and subnormal, the largest subnormal, NaN, and order along the codes."""
    d = mo.e4m3_decode
    assert d(np.array([0x38]))[0] == 1.0
    assert d(np.array([0x7E]))[0] == 448.0 and d(np.array([0xFE]))[0] == -448.0
    assert d(np.array([0x08]))[0] == 2.0 ** -6
    assert d(np.array([0x01]))[0] == 2.0 ** -9
    assert d(np.array([0x07]))[0] == 7 * 2.0 ** -9
    assert d(np.array([0x40]))[0] == 2.0 and d(np.array([0x3C]))[0] == 1.5
    assert np.isnan(d(np.array([0x7F]))[0]) and np.isnan(d(np.array([0xFF]))[0])
    pos = d(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0)                              # strictly increasing
    assert np.array_equal(d(np.arange(0x80, 0xFF, dtype=np.uint8)), -pos)


def pin_dequantize_rows():
    """Each row is its decoded codes times that row's scale (non-square, so a scale
    applied along the wrong axis fails)."""
    rng = _rng(11)
    codes = rng.integers(0, 0x7F, size=(3, 5)).astype(np.uint8)
    scale = np.array([0.5, 2.0, 0.125], np.float32)
    w = mo.dequantize_rows(codes, scale)
    for n in range(3):
        assert np.array_equal(w[n], mo.e4m3_decode(codes[n]) * float(scale[n]))


def pin_e2m1_table():
    """The 16 E2M1 codes take the magnitudes the format fixes (0, 0.5, 1, 1.5, 2, 3, 4, 6),
    the sign bit negates, and only the low four bits of a byte count."""
    d = mo.e2m1_decode
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    assert list(d(np.arange(8, dtype=np.uint8))) == mags
    neg = d(np.arange(8, 16, dtype=np.uint8))
    assert list(-neg) == mags and np.signbit(neg[0])
    assert np.array_equal(d(np.arange(16, 32, dtype=np.uint8)), d(np.arange(16, dtype=np.uint8)))


def pin_e8m0_library():
    """E8M0 scale bytes decode as torch's float8_e8m0fnu does (independent implementation)."""
    import torch
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = mo.e8m0_decode(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert mo.e8m0_decode(np.array([127]))[0] == 1.0 and mo.e8m0_decode(np.array([130]))[0] == 8.0


def pin_mx_dequantize():
    """Packing and block scales: element 2j in the low nibble of byte j, the scale of block b
    covering elements 32b .. 32b + 31 of its row (rows and blocks differ, so a transposed
    scale or swapped nibbles fail)."""
    rng = _rng(12)
    n, k = 3, 64
    codes = rng.integers(0, 16, size=(n, k)).astype(np.uint8)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    sc = np.array([[120, 127, 131], [125, 129, 133]], np.uint8)        # [k/32, n]
    w = mo.dequantize_mx_rows(packed, sc)
    for r in range(n):
        for j in range(k):
            assert w[r, j] == mo.e2m1_decode(codes[r, j:j + 1])[0] * 2.0 ** (int(sc[j // 32, r]) - 127)


# --------------------------------------------------------------------------- backward

def _loss(x, w_r, experts, k, dy, d_aux, cap, b_r, renorm, sh, idx, scoring, ng, tg):
    """L = sum(dy * y) + d_aux * aux from the (pinned) forward, routing forced to idx."""
    res = mo.moe_forward(x, w_r, experts, k, cap, b_r, renorm, sh, idx, scoring, ng, tg)
    return float(np.sum(dy * res.y) + d_aux * res.aux)


def _fd_check(seed, T, d, de, E, k, cap, renorm, scoring="softmax", ng=1, tg=1, bias=True, shared=True,
              d_aux=0.7, step=1e-6):
    """Central differences of the forward loss, every input element, against moe_backward.

    The routing (idx) is taken from the unperturbed forward and held fixed, which is the
    definition of the backward pass (selection carries no gradient); capacity then drops
    the same assignments at every perturbed point.
    """
    x, w_r, experts, b_r, sh = _tiny_layer(seed, T=T, d=d, d_e=de, E=E, bias=bias, shared=shared)
    if b_r is not None and scoring == "sigmoid":
        b_r = b_r * 0.2
    dy = _rng(seed + 1000).standard_normal((T, d))
    idx = mo.moe_forward(x, w_r, experts, k, cap, b_r, renorm, sh, None, scoring, ng, tg).idx
    G = mo.moe_backward(x, w_r, experts, k, dy, d_aux, cap, b_r, renorm, sh, idx, scoring, ng, tg)
    experts = [list(ex) for ex in experts]
    sh = None if sh is None else list(sh)

    def L():
        return _loss(x, w_r, experts, k, dy, d_aux, cap, b_r, renorm, sh, idx, scoring, ng, tg)

    def fd(arr):
        out = np.zeros_like(arr)
        for i in np.ndindex(arr.shape):
            v = arr[i]
            arr[i] = v + step
            lp = L()
            arr[i] = v - step
            lm = L()
            arr[i] = v
            out[i] = (lp - lm) / (2 * step)
        return out

    checks = [("dx", fd(x), G.dx), ("dw_r", fd(w_r), G.dw_r)]
    if b_r is not None:
        checks.append(("db_r", fd(b_r), G.db_r))
    for e in range(E):
        for m, name, got in ((0, "dw_gate", G.dw_gate[e]), (1, "dw_up", G.dw_up[e]), (2, "dw_down", G.dw_down[e])):
            experts[e][m] = experts[e][m].copy()
            checks.append((f"{name}[{e}]", fd(experts[e][m]), got))
    if sh is not None:
        for m in range(3):
            sh[m] = sh[m].copy()
            checks.append((f"dshared[{m}]", fd(sh[m]), G.dshared[m]))
    for name, want, got in checks:
        assert got is not None and np.shape(got) == np.shape(want), name
        scale = max(1.0, float(np.max(np.abs(want))))
        assert np.max(np.abs(np.asarray(got) - want)) <= 1e-6 * scale, (name, np.max(np.abs(got - want)))
    return G, idx


def pin_backward_fd_softmax():
    """Softmax router with bias, renormalised gates, capacity drops, shared expert, aux term."""
    G, idx = _fd_check(41, T=6, d=5, de=4, E=4, k=2, cap=2, renorm=True)
    # the softmax is unchanged by a common shift of the logits: each dr row sums to zero
    assert np.allclose(G.dlogits.sum(axis=1), 0.0, atol=1e-12)


def pin_backward_fd_raw_gates():
    """Switch-style raw gates at k = 1 with drops, and k = 3 without a bias or shared expert."""
    _fd_check(42, T=7, d=4, de=3, E=3, k=1, cap=2, renorm=False)
    _fd_check(43, T=5, d=4, de=3, E=5, k=3, cap=-1, renorm=True, bias=False, shared=False, d_aux=0.0)


def pin_backward_fd_sigmoid():
    """Sigmoid affinities with a selection-only bias and the group limit."""
    G, _ = _fd_check(44, T=6, d=4, de=3, E=8, k=2, cap=-1, renorm=True, scoring="sigmoid", ng=4, tg=2)
    assert np.array_equal(G.db_r, np.zeros(8))       # the bias only picks experts
    _fd_check(45, T=5, d=4, de=3, E=6, k=3, cap=3, renorm=False, scoring="sigmoid", ng=3, tg=2, shared=False)


def pin_backward_dropped_slots():
    """A dropped slot gets dL/dg = 0 and sends nothing to its expert; a token whose every
    slot is dropped still gets the router's and the shared expert's dx."""
    x, w_r, experts, b_r, sh = _tiny_layer(46, T=6, d=5, d_e=4, E=3, bias=False, shared=True)
    idx = np.zeros((6, 1), dtype=np.int32)               # all on expert 0, capacity 2
    dy = _rng(47).standard_normal((6, 5))
    G = mo.moe_backward(x, w_r, experts, 1, dy, 0.0, 2, None, True, sh, idx)
    assert np.all(G.dgate[2:] == 0.0) and np.all(G.dgate[:2] != 0.0)
    assert np.all(G.dw_gate[1:] == 0.0) and np.all(G.dw_down[1:] == 0.0)
    # k = 1 renormalised: g = 1 whatever p is, so the router gets no gradient from y
    assert np.allclose(G.dlogits, 0.0, atol=1e-15) and np.allclose(G.dw_r, 0.0, atol=1e-15)
    sX = mo.swiglu_backward(x, *sh, dy)[0]
    assert np.allclose(G.dx[2:], sX[2:], rtol=1e-13, atol=1e-13)
    # expert 0 saw tokens 0 and 1 only
    xe = mo.swiglu_backward(x[:2], *experts[0], dy[:2])
    assert np.allclose(G.dw_gate[0], xe[1], rtol=1e-13, atol=1e-13)


def pin_backward_single_expert_autograd():
    """E = 1, k = 1 reduces the layer to one SwiGLU network (g = 1, aux = 1 at any logits):
    the gradients are torch.autograd's of that network, and the router gets none."""
    import torch
    g = _rng(48)
    T, d, de = 7, 6, 5
    x, w_r = g.standard_normal((T, d)), g.standard_normal((1, d))
    wg, wu, wd = g.standard_normal((de, d)), g.standard_normal((de, d)), g.standard_normal((d, de))
    dy = g.standard_normal((T, d))
    G = mo.moe_backward(x, w_r, [(wg, wu, wd)], 1, dy, d_aux=0.9)
    tx, tg, tu, td = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (x, wg, wu, wd))
    y = torch.nn.functional.linear(torch.nn.functional.silu(torch.nn.functional.linear(tx, tg))
                                   * torch.nn.functional.linear(tx, tu), td)
    y.backward(torch.tensor(dy))
    for got, want in ((G.dx, tx.grad), (G.dw_gate[0], tg.grad), (G.dw_up[0], tu.grad), (G.dw_down[0], td.grad)):
        assert np.allclose(got, want.numpy(), rtol=1e-12, atol=1e-12)
    assert np.allclose(G.dw_r, 0.0, atol=1e-15)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
