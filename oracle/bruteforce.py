"""Pure-Python brute force of the MoE layer for tiny inputs (no NumPy arithmetic).

TEST INFRASTRUCTURE (see the package docstring).

It evaluates the dense form that Zero to Frontier §13.1 uses to check its
worked example ("A worked example small enough to check by hand"): run every
expert on every token and multiply the unchosen ones by a zero gate.  It is an
independent second implementation of the same definition: nested loops over
Python floats, ``math.exp``, a selection loop for the top-k, a per-expert
arrival counter for the capacity rule, and a table search for the E4M3 rounding
of MXFP8 activations, so a NumPy slip in the main oracle (a transposed operand, a
wrong axis, a dropped term, a wrong rounding rule) cannot repeat here.
"""
from __future__ import annotations

import math
import struct


def _f32(v):
    """v rounded to the nearest float32 (struct's pack does the rounding)."""
    return struct.unpack("f", struct.pack("f", v))[0]


def _e4m3_table():
    """(value, code) of every non-negative finite E4M3 code, built from the bit fields."""
    out = []
    for ex in range(16):
        for man in range(8):
            if ex == 15 and man == 7:
                continue                                   # NaN
            val = (man / 8.0) * 2.0 ** -6 if ex == 0 else (1.0 + man / 8.0) * 2.0 ** (ex - 7)
            out.append((val, (ex << 3) | man))
    return out


_E4M3 = _e4m3_table()


def _round_e4m3(w):
    """Nearest E4M3 value by search over the table, ties to the even code, saturating."""
    a = min(abs(w), 448.0)
    best = None
    for val, code in _E4M3:
        key = (abs(val - a), code & 1)
        if best is None or key < best[0]:
            best = (key, val)
    return math.copysign(best[1], w)


def _mxfp8_row(row):
    """A row rounded to MXFP8: blocks of 32 share 2^X, X = floor(log2 block max) - 8."""
    out = []
    for b0 in range(0, len(row), 32):
        blk = row[b0:b0 + 32]
        amax = max(abs(v) for v in blk)
        if amax == 0.0:
            x = -127
        else:
            x = max(-127, min(127, math.frexp(amax)[1] - 1 - 8))
        sc = 2.0 ** x
        out.extend(_round_e4m3(v / sc) * sc for v in blk)
    return out


def _matvec(W, v):
    """W [out][in] times v [in]."""
    return [sum(W[o][i] * v[i] for i in range(len(v))) for o in range(len(W))]


def _silu(z):
    return z / (1.0 + math.exp(-z)) if z > -700 else 0.0


def _expert(Wg, Wu, Wd, x, act=None):
    a = _matvec(Wg, x)
    b = _matvec(Wu, x)
    h = [_silu(a[n]) * b[n] for n in range(len(a))]
    if act == "mxfp8":                                     # h enters the down product as MXFP8
        h = _mxfp8_row([_f32(v) for v in h])
    return _matvec(Wd, h)


def _select(score, k, allowed):
    """k rounds of 'best remaining allowed expert', lower index on ties."""
    chosen = []
    for _ in range(k):
        best = -1
        for e in range(len(score)):
            if e in chosen or not allowed[e]:
                continue
            if best < 0 or score[e] > score[best]:
                best = e
        chosen.append(best)
    return chosen


def moe_dense_bruteforce(x, w_r, experts, k, cap=-1, b_r=None, renormalize=True, shared=None,
                         scoring="softmax", n_group=1, topk_group=1, act=None):
    """Returns (y, idx, gates) as nested lists.

    x [T][d]; w_r [E][d]; experts[e] = (Wg [d_e][d], Wu [d_e][d], Wd [d][d_e]);
    b_r [E] or None.  cap < 0: unlimited.  scoring "sigmoid": independent sigmoid
    affinities, b_r used only to choose, gates from the affinities; n_group > 1: only the
    topk_group groups (consecutive blocks of E / n_group experts) with the highest best
    member may be chosen.  act "mxfp8": every expert product takes MXFP8 activations (x
    rounded per token row, h rounded from its float32 value); the router sees x as given.
    """
    T = len(x)
    E = len(w_r)
    d = len(x[0]) if T else 0
    ys, idxs, gs = [], [], []
    seen = [0] * E
    for t in range(T):
        raw = [sum(w_r[e][i] * x[t][i] for i in range(d)) for e in range(E)]
        if scoring == "softmax":
            logits = [raw[e] + (b_r[e] if b_r is not None else 0.0) for e in range(E)]
            mx = max(logits)
            ex = [math.exp(v - mx) for v in logits]
            s = sum(ex)
            p = [v / s for v in ex]
            sel = p
        else:
            p = [1.0 / (1.0 + math.exp(-v)) for v in raw]
            sel = [p[e] + (b_r[e] if b_r is not None else 0.0) for e in range(E)]
        gsz = E // n_group
        best_in = [max(sel[g * gsz:(g + 1) * gsz]) for g in range(n_group)]
        groups = _select(best_in, topk_group, [True] * n_group)
        allowed = [(e // gsz) in groups for e in range(E)]
        chosen = _select(sel, k, allowed)
        if renormalize:
            z = sum(p[e] for e in chosen)
            g_sel = [p[e] / z for e in chosen]
        else:
            g_sel = [p[e] for e in chosen]
        # dense gate vector: zero for unchosen experts and for dropped assignments
        gate_full = [0.0] * E
        for j, e in enumerate(chosen):
            rank = seen[e]
            seen[e] += 1
            if cap < 0 or rank < cap:
                gate_full[e] = g_sel[j]
        xa = x[t] if act is None else _mxfp8_row(list(x[t]))
        y = [0.0] * d
        for e in range(E):                        # every expert runs
            out = _expert(*experts[e], xa, act)
            for i in range(d):
                y[i] += gate_full[e] * out[i]
        if shared is not None:
            out = _expert(*shared, xa, act)
            for i in range(d):
                y[i] += out[i]
        ys.append(y)
        idxs.append(chosen)
        gs.append(g_sel)
    return ys, idxs, gs
