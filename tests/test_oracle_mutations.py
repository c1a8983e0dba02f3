"""Planted mistakes in the CPU oracle must each make at least one pin fail.

The mistakes are planted on the CPU only, by replacing one oracle function at a
time (pytest's monkeypatch restores it afterwards).  Each models a plausible slip:
a dropped term, a wrong sign, a wrong axis or index, a transposed operand, a
wrong tie-break, a wrong capacity rule.
"""
import numpy as np
import pytest

import oracle_pins as pins
from oracle import moe_oracle as mo

_orig = {name: getattr(mo, name) for name in
         ["softmax", "top_k", "gates", "silu", "swiglu_ffn", "router_logits", "load_balance_stats",
          "capacity", "dispatch", "near_ties", "near_ties_grouped", "sigmoid", "group_limited_top_k", "route", "e4m3_decode", "e4m3_encode", "mxfp8_quantize_rows", "mxfp8_round_rows", "silu_range",
          "mxfp8_round_interval", "swiglu_mx_deviation",
          "dequantize_rows", "e2m1_decode", "e8m0_decode", "dequantize_mx_rows", "silu_grad",
          "swiglu_backward", "router_backward", "moe_backward"]}


def _softmax_no_shift(r):
    e = np.exp(r)
    return e / e.sum(axis=1, keepdims=True)


def _softmax_wrong_axis(r):
    m = r.max(axis=0, keepdims=True)
    e = np.exp(r - m)
    return e / e.sum(axis=0, keepdims=True)


def _topk_high_index_wins(p, k):
    E = p.shape[1]
    order = np.argsort(-p[:, ::-1], axis=1, kind="stable")
    return (E - 1 - order[:, :k]).astype(np.int32)


def _topk_smallest(p, k):
    return np.argsort(p, axis=1, kind="stable")[:, :k].astype(np.int32)


def _topk_unsorted_slots(p, k):
    return np.sort(_orig["top_k"](p, k), axis=1).astype(np.int32)


def _gates_never_renorm(p, idx, renormalize=True):
    return _orig["gates"](p, idx, False)


def _silu_is_sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def _silu_sign(z):
    return z / (1.0 + np.exp(z))


def _ffn_no_up(X, w_g, w_u, w_d):
    return mo.silu(np.asarray(X) @ np.asarray(w_g).T) @ np.asarray(w_d).T


def _ffn_swapped(X, w_g, w_u, w_d):
    return _orig["swiglu_ffn"](X, w_u, w_g, w_d)


def _ffn_transposed_down(X, w_g, w_u, w_d):
    X = np.asarray(X, np.float64)
    h = mo.silu(X @ np.asarray(w_g).T) * (X @ np.asarray(w_u).T)
    wd = np.asarray(w_d)
    return h @ (wd if wd.shape[0] == h.shape[1] else wd.reshape(wd.shape[1], wd.shape[0]))


def _router_bias_minus(x, w_r, b_r=None):
    r = np.asarray(x, np.float64) @ np.asarray(w_r, np.float64).T
    return r - (0 if b_r is None else np.asarray(b_r)[None, :])


def _stats_top1_f(p, idx, E):
    counts, f, P, aux = _orig["load_balance_stats"](p, idx, E)
    f = np.bincount(idx[:, 0], minlength=E) / idx.shape[0]
    return counts, f, P, float(E * np.sum(f * P))


def _stats_P_of_chosen(p, idx, E):
    counts, f, P, aux = _orig["load_balance_stats"](p, idx, E)
    P = (np.take_along_axis(p, idx.astype(np.int64), axis=1).sum(axis=0).sum() / p.shape[0]) * np.ones(E) / E
    return counts, f, P, float(E * np.sum(f * P))


def _capacity_no_k(T, k, E, C):
    return int(np.floor(C * T / E))


def _capacity_ceil(T, k, E, C):
    return int(np.ceil(C * T * k / E + 0.5))


def _dispatch_keep_last(idx, E, cap=-1):
    if cap < 0:
        return _orig["dispatch"](idx, E, cap)
    rev = _orig["dispatch"](idx[::-1, ::-1].copy(), E, cap)
    T, k = idx.shape
    row_of = rev.row_of[::-1, ::-1].copy()
    return mo.Dispatch(rev.counts, rev.kept, rev.offsets, rev.row_token, row_of)


def _dispatch_no_cap(idx, E, cap=-1):
    return _orig["dispatch"](idx, E, -1)


def _near_ties_off_by_one(p, k, threshold=mo.NEAR_TIE):
    return _orig["near_ties"](p, k + 1 if k + 1 < p.shape[1] else k, threshold)


def _sigmoid_sign(z):
    return 1.0 / (1.0 + np.exp(z))


def _group_score_sum(score, k, n_group, topk_group):
    T, E = score.shape
    gs = E // n_group
    gscore = score.reshape(T, n_group, gs).sum(axis=2)
    gorder = np.argsort(-gscore, axis=1, kind="stable")[:, :topk_group]
    allowed = np.zeros((T, n_group), dtype=bool)
    np.put_along_axis(allowed, gorder, True, axis=1)
    return mo.top_k(np.where(np.repeat(allowed, gs, axis=1), score, -np.inf), k)


def _group_ignored(score, k, n_group, topk_group):
    return mo.top_k(score, k)


def _group_interleaved(score, k, n_group, topk_group):
    T, E = score.shape
    perm = np.argsort(np.arange(E) % n_group, kind="stable")        # experts of group g: e % n_group == g
    idx = _orig["group_limited_top_k"](score[:, perm], k, n_group, topk_group)
    return perm[idx].astype(np.int32)


def _route_bias_in_gates(x, w_r, k, b_r=None, renormalize=True, idx=None, scoring="softmax", n_group=1,
                         topk_group=1):
    r, p, idx, g, nt = _orig["route"](x, w_r, k, b_r, renormalize, idx, scoring, n_group, topk_group)
    if scoring == "sigmoid" and b_r is not None:
        sel = np.take_along_axis(p + np.asarray(b_r)[None, :], idx.astype(np.int64), axis=1)
        g = sel / sel.sum(axis=1, keepdims=True) if renormalize else sel
    return r, p, idx, g, nt


def _e4m3_bias8(codes):
    return _orig["e4m3_decode"](codes) / 2.0


def _e4m3_no_subnormals(codes):
    c = np.asarray(codes, np.uint8).astype(np.int64)
    v = _orig["e4m3_decode"](codes)
    ex, man = (c >> 3) & 15, c & 7
    sub = (ex == 0) & (man > 0)
    mag = (1.0 + man / 8.0) * 2.0 ** -7
    return np.where(sub, np.where(c >> 7 == 1, -mag, mag), v)


def _e4m3_mantissa_16(codes):
    c = np.asarray(codes, np.uint8).astype(np.int64)
    v = _orig["e4m3_decode"](codes)
    ex, man = (c >> 3) & 15, c & 7
    mag = (1.0 + man / 16.0) * np.exp2(ex - 7.0)
    return np.where((ex > 0) & ~np.isnan(v), np.where(c >> 7 == 1, -mag, mag), v)


def _dequant_columns(codes, scale):
    w = mo.e4m3_decode(codes)
    sc = np.resize(np.asarray(scale, np.float64), w.shape[1])
    return w * sc.reshape(1, -1)


def _e2m1_bias2(nibbles):
    return _orig["e2m1_decode"](nibbles) / 2.0


def _e2m1_no_subnormal(nibbles):
    c = np.asarray(nibbles, np.uint8).astype(np.int64) & 15
    v = _orig["e2m1_decode"](nibbles)
    return np.where(((c >> 1) & 3) == 0, np.where(c >> 3 == 1, -1.0, 1.0) * (c & 1) * 1.0, v)


def _e8m0_bias128(codes):
    return _orig["e8m0_decode"](codes) / 2.0


def _mx_nibbles_swapped(packed, scales, block=32):
    p = np.asarray(packed, np.uint8)
    return _orig["dequantize_mx_rows"](((p >> 4) | (p << 4)).astype(np.uint8), scales, block)


def _mx_scales_transposed(packed, scales, block=32):
    sc = np.asarray(scales, np.uint8)
    return _orig["dequantize_mx_rows"](packed, np.resize(sc.T, sc.shape), block)


def _silu_grad_sigmoid(z):
    return mo.sigmoid(z)


def _silu_grad_sign(z):
    s = mo.sigmoid(z)
    return s * (1.0 - z * (1.0 - s))


def _swb_no_b(X, w_g, w_u, w_d, dO):
    X = np.asarray(X, np.float64)
    a, b = X @ np.asarray(w_g).T, X @ np.asarray(w_u).T
    dh = dO @ np.asarray(w_d)
    da, db = dh * mo.silu_grad(a), dh * mo.silu(a)
    return da @ w_g + db @ w_u, da.T @ X, db.T @ X, dO.T @ (mo.silu(a) * b)


def _swb_dx_no_up(X, w_g, w_u, w_d, dO):
    dX, gg, gu, gd = _orig["swiglu_backward"](X, w_g, w_u, w_d, dO)
    X = np.asarray(X, np.float64)
    a = X @ np.asarray(w_g).T
    db = (dO @ np.asarray(w_d)) * mo.silu(a)
    return dX - db @ np.asarray(w_u), gg, gu, gd


def _swb_swapped(X, w_g, w_u, w_d, dO):
    dX, gg, gu, gd = _orig["swiglu_backward"](X, w_g, w_u, w_d, dO)
    return dX, gu, gg, gd


def _swb_down_transposed(X, w_g, w_u, w_d, dO):
    dX, gg, gu, gd = _orig["swiglu_backward"](X, w_g, w_u, w_d, dO)
    return dX, gg, gu, np.resize(gd.T, gd.shape)


def _rb_no_renorm_term(p, idx, g, dgate, f, d_aux, renormalize=True, scoring="softmax"):
    if renormalize:
        S = np.take_along_axis(p, idx.astype(np.int64), axis=1).sum(axis=1, keepdims=True)
        return _orig["router_backward"](p, idx, g, dgate / S, f, d_aux, False, scoring)
    return _orig["router_backward"](p, idx, g, dgate, f, d_aux, renormalize, scoring)


def _rb_no_aux(p, idx, g, dgate, f, d_aux, renormalize=True, scoring="softmax"):
    return _orig["router_backward"](p, idx, g, dgate, f, 0.0, renormalize, scoring)


def _rb_aux_without_E(p, idx, g, dgate, f, d_aux, renormalize=True, scoring="softmax"):
    return _orig["router_backward"](p, idx, g, dgate, f, d_aux / p.shape[1], renormalize, scoring)


def _rb_softmax_sign(p, idx, g, dgate, f, d_aux, renormalize=True, scoring="softmax"):
    dr = _orig["router_backward"](p, idx, g, dgate, f, d_aux, renormalize, scoring)
    if scoring != "softmax":
        return dr
    # p * (dp + sum p dp) instead of p * (dp - sum p dp)
    dp = dr / p + 0.0
    c = np.sum(p * dp, axis=1, keepdims=True) / (1.0 - np.sum(p * p, axis=1, keepdims=True))
    return dr + 2.0 * p * c


def _rb_sigmoid_no_1mp(p, idx, g, dgate, f, d_aux, renormalize=True, scoring="softmax"):
    dr = _orig["router_backward"](p, idx, g, dgate, f, d_aux, renormalize, scoring)
    return dr / (1.0 - p) if scoring == "sigmoid" else dr


def _bwd_dropped_slots_count(x, w_r, experts, k, dy, d_aux=0.0, cap=-1, *a, **kw):
    return _orig["moe_backward"](x, w_r, experts, k, dy, d_aux, -1, *a, **kw)


def _bwd_no_router_dx(x, w_r, experts, k, dy, *a, **kw):
    G = _orig["moe_backward"](x, w_r, experts, k, dy, *a, **kw)
    G.dx = G.dx - G.dlogits @ np.asarray(w_r, np.float64)
    return G


def _bwd_sigmoid_bias_grad(x, w_r, experts, k, dy, *a, **kw):
    G = _orig["moe_backward"](x, w_r, experts, k, dy, *a, **kw)
    if G.db_r is not None:
        G.db_r = G.dlogits.sum(axis=0)
    return G


def _ntg_excuse_all(score, k, n_group, topk_group, threshold=mo.NEAR_TIE):
    return np.arange(score.shape[0])


def _ntg_report_none(score, k, n_group, topk_group, threshold=mo.NEAR_TIE):
    return np.zeros(0, dtype=np.int64)


def _ntg_mask_ignored(score, k, n_group, topk_group, threshold=mo.NEAR_TIE):
    """Expert decision taken over every expert instead of the allowed ones."""
    grp = _orig["near_ties_grouped"](score, k, n_group, topk_group, threshold)
    out = set(grp.tolist())
    g_only = _orig["near_ties_grouped"](score, k, n_group, n_group, threshold)   # expert gaps, all allowed
    out -= set(g_only.tolist())
    out |= set(mo.near_ties(score, k, threshold).tolist())
    gs = score.shape[1] // n_group
    if topk_group < n_group:
        gsc = -np.sort(-score.reshape(score.shape[0], n_group, gs).max(axis=2), axis=1)
        out |= set(np.nonzero(gsc[:, topk_group - 1] - gsc[:, topk_group] < threshold)[0].tolist())
    return np.array(sorted(out), dtype=np.int64)


def _ntg_group_off_by_one(score, k, n_group, topk_group, threshold=mo.NEAR_TIE):
    """Group decision read between the (topk_group-1)-th and topk_group-th group scores."""
    T, E = score.shape
    gs = E // n_group
    out = set(_orig["near_ties_grouped"](score, k, n_group, n_group, threshold).tolist())
    if topk_group > 1:
        gsc = -np.sort(-score.reshape(T, n_group, gs).max(axis=2), axis=1)
        out |= set(np.nonzero(gsc[:, topk_group - 2] - gsc[:, topk_group - 1] < threshold)[0].tolist())
    return np.array(sorted(out), dtype=np.int64)


def _ntg_no_group_decision(score, k, n_group, topk_group, threshold=mo.NEAR_TIE):
    """Only the expert decision among the allowed experts is checked."""
    T, E = score.shape
    gs = E // n_group
    allowed_sel = mo.group_limited_top_k(score, min(E, topk_group * gs), n_group, topk_group)
    masked = np.full_like(score, -np.inf)
    np.put_along_axis(masked, allowed_sel.astype(np.int64), np.take_along_axis(score, allowed_sel.astype(np.int64),
                                                                                 axis=1), axis=1)
    return mo.near_ties(masked, k, threshold) if k < topk_group * gs else np.zeros(0, dtype=np.int64)


def _enc_ties_away(v):
    v = np.asarray(v, np.float64)
    c = _orig["e4m3_encode"](v)
    lo = mo.e4m3_decode(c)
    up = mo.e4m3_decode(np.where(c % 2 == 0, c + 1, c).astype(np.uint8))
    tie = np.isclose(np.abs(v) - np.abs(lo), np.abs(up) - np.abs(v), rtol=0, atol=0) & (c % 2 == 0) & (np.abs(v) > 0)
    return np.where(tie & (np.abs(v) < 448), c + 1, c).astype(np.uint8)


def _enc_truncate(v):
    v = np.asarray(v, np.float64)
    c = _orig["e4m3_encode"](v)
    over = np.abs(mo.e4m3_decode(c)) > np.abs(v)
    return np.where(over & (c % 128 > 0), c - 1, c).astype(np.uint8)


def _enc_no_saturation(v):
    v = np.asarray(v, np.float64)
    c = _orig["e4m3_encode"](v)
    return np.where(np.abs(v) > 448, np.uint8(0x7F) | (c & 0x80), c).astype(np.uint8)


def _mxq_scale_minus7(v, block=32):
    q, sc = _orig["mxfp8_quantize_rows"](v, block)
    sc = np.minimum(sc.astype(np.int64) + 1, 254).astype(np.uint8)
    vals = np.asarray(v, np.float64) / np.repeat(np.exp2(sc.astype(np.float64) - 127), block, axis=1)
    return mo.e4m3_encode(vals), sc


def _mxq_row_scale(v, block=32):
    v = np.asarray(v, np.float64)
    return _orig["mxfp8_quantize_rows"](v, v.shape[1])[0], np.repeat(
        _orig["mxfp8_quantize_rows"](v, v.shape[1])[1], v.shape[1] // block, axis=1)


def _mxr_identity(v, block=32):
    return np.asarray(v, np.float64)


def _sr_no_interior(lo, hi):
    sl, sh = mo.silu(np.asarray(lo, np.float64)), mo.silu(np.asarray(hi, np.float64))
    return np.minimum(sl, sh), np.maximum(sl, sh)


def _ri_one_scale(lo, hi, block=32):
    lo = np.asarray(lo, np.float64)
    hi = np.asarray(hi, np.float64)
    mid = (lo + hi) / 2
    q, sc = mo.mxfp8_quantize_rows(mid, block)
    s = np.repeat(np.exp2(sc.astype(np.float64) - 127), block, axis=1)
    return mo.e4m3_decode(mo.e4m3_encode(lo / s)) * s, mo.e4m3_decode(mo.e4m3_encode(hi / s)) * s


def _dev_no_flips(X, w_g, w_u, w_d, eps):
    hq, qlo, qhi, _ = _orig["swiglu_mx_deviation"](X, w_g, w_u, w_d, eps)
    return hq, qlo, qhi, eps * (np.abs(hq) @ np.abs(np.asarray(w_d, np.float64)).T)


MUTANTS = [
    ("softmax", _softmax_no_shift), ("softmax", _softmax_wrong_axis),
    ("top_k", _topk_high_index_wins), ("top_k", _topk_smallest), ("top_k", _topk_unsorted_slots),
    ("gates", _gates_never_renorm),
    ("silu", _silu_is_sigmoid), ("silu", _silu_sign),
    ("swiglu_ffn", _ffn_no_up), ("swiglu_ffn", _ffn_swapped), ("swiglu_ffn", _ffn_transposed_down),
    ("router_logits", _router_bias_minus),
    ("load_balance_stats", _stats_top1_f), ("load_balance_stats", _stats_P_of_chosen),
    ("capacity", _capacity_no_k), ("capacity", _capacity_ceil),
    ("dispatch", _dispatch_keep_last), ("dispatch", _dispatch_no_cap),
    ("near_ties", _near_ties_off_by_one),
    ("near_ties_grouped", _ntg_excuse_all), ("near_ties_grouped", _ntg_report_none),
    ("near_ties_grouped", _ntg_mask_ignored), ("near_ties_grouped", _ntg_group_off_by_one),
    ("near_ties_grouped", _ntg_no_group_decision),
    ("sigmoid", _sigmoid_sign), ("group_limited_top_k", _group_score_sum),
    ("group_limited_top_k", _group_ignored), ("group_limited_top_k", _group_interleaved),
    ("route", _route_bias_in_gates),
    ("e4m3_decode", _e4m3_bias8), ("e4m3_decode", _e4m3_no_subnormals), ("e4m3_decode", _e4m3_mantissa_16),
    ("dequantize_rows", _dequant_columns),
    ("e4m3_encode", _enc_ties_away), ("e4m3_encode", _enc_truncate), ("e4m3_encode", _enc_no_saturation),
    ("mxfp8_quantize_rows", _mxq_scale_minus7), ("mxfp8_quantize_rows", _mxq_row_scale),
    ("mxfp8_round_rows", _mxr_identity),
    ("silu_range", _sr_no_interior), ("mxfp8_round_interval", _ri_one_scale),
    ("swiglu_mx_deviation", _dev_no_flips),
    ("e2m1_decode", _e2m1_bias2), ("e2m1_decode", _e2m1_no_subnormal), ("e8m0_decode", _e8m0_bias128),
    ("dequantize_mx_rows", _mx_nibbles_swapped), ("dequantize_mx_rows", _mx_scales_transposed),
    ("silu_grad", _silu_grad_sigmoid), ("silu_grad", _silu_grad_sign),
    ("swiglu_backward", _swb_no_b), ("swiglu_backward", _swb_dx_no_up), ("swiglu_backward", _swb_swapped),
    ("swiglu_backward", _swb_down_transposed),
    ("router_backward", _rb_no_renorm_term), ("router_backward", _rb_no_aux),
    ("router_backward", _rb_aux_without_E), ("router_backward", _rb_softmax_sign),
    ("router_backward", _rb_sigmoid_no_1mp),
    ("moe_backward", _bwd_dropped_slots_count), ("moe_backward", _bwd_no_router_dx),
    ("moe_backward", _bwd_sigmoid_bias_grad),
]


@pytest.mark.parametrize("target,mutant", MUTANTS, ids=[m.__name__ for _, m in MUTANTS])
def test_planted_mistake_is_caught(monkeypatch, target, mutant):
    monkeypatch.setattr(mo, target, mutant)
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin()
        except Exception:            # an assertion or a shape error: either way the pin caught it
            failed.append(pin.__name__)
    assert failed, f"no pin catches the planted mistake {mutant.__name__} in {target}"
