"""Float64 oracle of the forward and backward passes of one sparse MoE FFN layer.

TEST INFRASTRUCTURE (see the package docstring): only tests, the smoke check and
the benchmark's CPU-baseline leg use this module.

The layer, in the notation of Zero to Frontier §13.1 "Why MoE", section "The MoE
layer": for a token row x (the output of the pre-FFN norm), a linear router
gives one logit per expert, r = x W_r; the k largest logits form the set K; the
chosen experts get weights g_i that sum to one; the layer returns
sum_{i in K} g_i FFN_i(x), where each expert is a SwiGLU network
FFN_i(x) = (SiLU(x W_g^i) * x W_u^i) W_d^i.  Unchosen experts are never run.

Storage follows the PyTorch layer of the kevinluzbetak.com "Mixture-Of-Experts"
page (nn.Linear keeps [out, in]): W_r is [E, d], W_g and W_u are [d_e, d] per
expert, W_d is [d, d_e] per expert, so r = x @ W_r.T and so on.

Readings taken where the pages leave a step open (each is listed with its reason
in the design notes of the repository):
  * top-k ties: the lower expert index wins; slots are ordered by descending
    probability (the PyTorch layer's ``topk`` order), so slot 0 is the top-1 choice.
  * softmax over all E, then top-k, then renormalise over the k (the
    kevinluzbetak.com routing paragraph) -- equal in exact arithmetic to the
    softmax over the k chosen logits of the "The MoE layer" gate equation.
  * ``renormalize=False`` keeps the raw softmax probability as the gate (the
    Switch top-1 variant; the kevinluzbetak.com router worked example notes that
    some implementations use the raw probabilities).
  * capacity: each expert keeps at most ``cap`` assignments; assignments are
    taken in arrival order t*k + j and the rest are dropped.  A dropped
    assignment contributes nothing; a surviving gate is not renormalised; a
    token whose every assignment is dropped gets y = 0 (plus the shared expert),
    the caller's residual carrying it through.
  * f_e counts every one of the k choices before capacity, divided by T*k;
    P_e is the mean over all T tokens of the full softmax; aux = E * sum f_e P_e
    (the auxiliary-loss code of the kevinluzbetak.com layer, without alpha).
  * SiLU(z) = z * sigmoid(z) = z / (1 + exp(-z)) (the pages name it, not define it).
  * a shared expert is added with weight one, outside routing, capacity and
    the statistics.
  * backward: the routing (expert choice and capacity drops) and f are constants;
    gradients reach the router only through the chosen gates and through P in
    aux (Moatlab AI-064, "Inside the Router").
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

NEAR_TIE = 1e-6


# --------------------------------------------------------------------------- router

def router_logits(x: np.ndarray, w_r: np.ndarray, b_r: np.ndarray | None = None) -> np.ndarray:
    """r = x W_r (+ b): one logit per expert per token.

    Zero to Frontier §13.1, "The MoE layer": the router is one linear map d -> E.
    The optional per-expert bias b (float32 in storage) is added to the logits
    before the softmax; it is part of the logits for selection, gates and P.
    """
    r = np.asarray(x, np.float64) @ np.asarray(w_r, np.float64).T
    if b_r is not None:
        r = r + np.asarray(b_r, np.float64)[None, :]
    return r


def softmax(r: np.ndarray) -> np.ndarray:
    """p = softmax(r) over the expert axis, computed with the row max subtracted.

    kevinluzbetak.com "Mixture-Of-Experts", routing paragraph: p = softmax(h W_r)
    over the E experts.  Subtracting the row maximum changes nothing in exact
    arithmetic and keeps exp finite.
    """
    m = r.max(axis=1, keepdims=True)
    e = np.exp(r - m)
    return e / e.sum(axis=1, keepdims=True)


def top_k(p: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k most probable experts per token, int32 [T, k].

    A stable sort on -p keeps equal probabilities in ascending expert order, so
    the lower index wins a tie and slot 0 is the most probable expert.
    """
    order = np.argsort(-p, axis=1, kind="stable")
    return order[:, :k].astype(np.int32)


def gates(p: np.ndarray, idx: np.ndarray, renormalize: bool = True) -> np.ndarray:
    """g[t, j] for the chosen experts idx[t, j].

    renormalize: g = p_i / sum_{j in K} p_j (kevinluzbetak.com routing paragraph;
    Zero to Frontier "The MoE layer" gate equation, e^{r_i} / sum_K e^{r_j}).
    Otherwise g = p_i (the raw-probability variant).
    """
    sel = np.take_along_axis(p, idx.astype(np.int64), axis=1)
    if renormalize:
        sel = sel / sel.sum(axis=1, keepdims=True)
    return sel


def near_ties(p: np.ndarray, k: int, threshold: float = NEAR_TIE) -> np.ndarray:
    """Tokens whose k-th and (k+1)-th largest probabilities differ by < threshold.

    For these tokens the choice between the two experts is decided by rounding,
    so a different but equally valid order is accepted and only reported.
    """
    T, E = p.shape
    if k >= E:
        return np.zeros(0, dtype=np.int64)
    s = -np.sort(-p, axis=1)
    return np.nonzero(s[:, k - 1] - s[:, k] < threshold)[0]


# --------------------------------------------------------------------------- statistics

def load_balance_stats(p: np.ndarray, idx: np.ndarray, E: int):
    """(counts, f, P, aux) of the Switch auxiliary term.

    kevinluzbetak.com "Mixture-Of-Experts", load-balancing fixes and the PyTorch
    layer's auxiliary-loss lines: f_e is the fraction of assignments dispatched
    to e, P_e the mean router probability of e, aux = E * sum_e f_e P_e, which is
    smallest under uniform routing and equals 1 when routing is balanced.
    counts are taken over all k choices, before any capacity drop.
    """
    T, k = idx.shape
    counts = np.bincount(idx.ravel().astype(np.int64), minlength=E).astype(np.int64)
    R = T * k
    f = counts / R if R > 0 else np.zeros(E)
    P = p.mean(axis=0) if T > 0 else np.zeros(E)
    aux = float(E * np.sum(f * P))
    return counts, f, P, aux


def capacity(T: int, k: int, E: int, C: float) -> int:
    """Per-expert slot count floor(C * T * k / E).

    Capacity is tokens per batch over experts times a factor (AI Engineering
    Illustrated, "The safety valve is a capacity limit"; "A hard limit" on the
    jacopoparretti.dev page).  The kevinluzbetak.com capacity worked example
    counts top-k slots, C * T * k / E; at k = 1 the two agree.  A non-integer
    product is rounded down.
    """
    return int(math.floor(C * T * k / E))


# --------------------------------------------------------------------------- dispatch

@dataclass
class Dispatch:
    counts: np.ndarray     # int64 [E] assignments per expert, before capacity
    kept: np.ndarray       # int64 [E] assignments kept
    offsets: np.ndarray    # int64 [E+1] exclusive scan of kept
    row_token: np.ndarray  # int64 [sum kept] token of each expert-ordered row
    row_of: np.ndarray     # int64 [T, k] row of assignment (t, j), or -1 if dropped

    @property
    def dropped(self) -> np.ndarray:
        """Flat indices t*k + j of dropped assignments, ascending."""
        return np.nonzero(self.row_of.ravel() < 0)[0]


def dispatch(idx: np.ndarray, E: int, cap: int = -1) -> Dispatch:
    """Group assignments by expert in arrival order, keeping at most cap per expert.

    The layer's per-expert token lists (the PyTorch layer's ``nonzero`` per
    expert) laid out as one expert-contiguous list.  Within an expert, rows are in
    ascending t*k + j.  cap < 0 means no limit.
    """
    T, k = idx.shape
    flat = idx.ravel().astype(np.int64)
    counts = np.bincount(flat, minlength=E).astype(np.int64)
    kept = counts.copy() if cap < 0 else np.minimum(counts, cap)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(kept)
    row_of = np.full(T * k, -1, dtype=np.int64)
    row_token = np.full(int(offsets[-1]), -1, dtype=np.int64)
    seen = np.zeros(E, dtype=np.int64)
    for a in range(T * k):                      # arrival order
        e = flat[a]
        rank = seen[e]
        seen[e] += 1
        if cap < 0 or rank < cap:
            row = offsets[e] + rank
            row_of[a] = row
            row_token[row] = a // k
    return Dispatch(counts, kept, offsets, row_token, row_of.reshape(T, k))


# --------------------------------------------------------------------------- experts

def silu(z: np.ndarray) -> np.ndarray:
    """SiLU(z) = z * sigmoid(z) = z / (1 + e^{-z})."""
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def swiglu_ffn(X: np.ndarray, w_g: np.ndarray, w_u: np.ndarray, w_d: np.ndarray, act: str | None = None) -> np.ndarray:
    """FFN(X) = (SiLU(X W_g) * (X W_u)) W_d for rows X [m, d]; weights stored [out, in].

    Zero to Frontier §13.1, "The MoE layer" (each expert is a SwiGLU network);
    the kevinluzbetak.com layer's SwiGLU module (w1 = gate, w3 = up, w2 = down).
    act="mxfp8": the activations entering each product are MXFP8 values (see
    ``mxfp8_round_rows``): X as given (the caller passes it already rounded), and h rounded
    from its float32 value before the down product.
    """
    X = np.asarray(X, np.float64)
    a = X @ np.asarray(w_g, np.float64).T
    b = X @ np.asarray(w_u, np.float64).T
    h = silu(a) * b
    if act == "mxfp8":
        h = mxfp8_round_rows(h.astype(np.float32))
    elif act is not None:
        raise ValueError(act)
    return h @ np.asarray(w_d, np.float64).T


# --------------------------------------------------------------------------- layer

@dataclass
class Result:
    y: np.ndarray          # [T, d] layer output (without the residual)
    logits: np.ndarray     # [T, E]
    p: np.ndarray          # [T, E]
    idx: np.ndarray        # int32 [T, k]
    gate: np.ndarray       # [T, k]
    counts: np.ndarray
    f: np.ndarray
    P: np.ndarray
    aux: float
    disp: Dispatch
    near_tie: np.ndarray   # token indices
    y_bound: np.ndarray | None = None   # act="mxfp8" with mx_eps: per-element deviation bound of y


# --------------------------------------------------------------------------- DeepSeek-V3 style router

def sigmoid(z: np.ndarray) -> np.ndarray:
    """Per-expert affinity 1 / (1 + e^{-z})."""
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


def group_limited_top_k(score: np.ndarray, k: int, n_group: int, topk_group: int) -> np.ndarray:
    """Top-k of `score` among the experts of each token's topk_group best groups.

    The E experts are cut into n_group consecutive groups of E / n_group.  A group's
    score is the highest expert score in it (reading: the pages say only that a token is
    limited to 4 of its 8 groups -- jacopoparretti.dev, "Smaller experts, more of them").
    Groups and experts are ranked by score, the lower index winning a tie.
    """
    T, E = score.shape
    gs = E // n_group
    gscore = score.reshape(T, n_group, gs).max(axis=2)
    gorder = np.argsort(-gscore, axis=1, kind="stable")[:, :topk_group]
    allowed = np.zeros((T, n_group), dtype=bool)
    np.put_along_axis(allowed, gorder, True, axis=1)
    masked = np.where(np.repeat(allowed, gs, axis=1), score, -np.inf)
    return top_k(masked, k)


def near_ties_grouped(score: np.ndarray, k: int, n_group: int, topk_group: int,
                      threshold: float = NEAR_TIE) -> np.ndarray:
    """Tokens whose group choice or expert choice is decided by a gap < threshold."""
    T, E = score.shape
    gs = E // n_group
    out = np.zeros(T, dtype=bool)
    if topk_group < n_group:
        gscore = -np.sort(-score.reshape(T, n_group, gs).max(axis=2), axis=1)
        out |= gscore[:, topk_group - 1] - gscore[:, topk_group] < threshold
    gscore = score.reshape(T, n_group, gs).max(axis=2)
    gorder = np.argsort(-gscore, axis=1, kind="stable")[:, :topk_group]
    allowed = np.zeros((T, n_group), dtype=bool)
    np.put_along_axis(allowed, gorder, True, axis=1)
    masked = np.where(np.repeat(allowed, gs, axis=1), score, -np.inf)
    if k < topk_group * gs:
        srt = -np.sort(-masked, axis=1)
        out |= srt[:, k - 1] - srt[:, k] < threshold
    return np.nonzero(out)[0]


def route(x, w_r, k: int, b_r=None, renormalize: bool = True, idx=None, scoring: str = "softmax",
          n_group: int = 1, topk_group: int = 1):
    """Router half of the layer: (logits, p, idx, gates, near-tie tokens); idx may be forced.

    scoring="softmax": p = softmax(x W_r + b) and the top-k of p (b is part of the logits).
    scoring="sigmoid": the DeepSeek-V3 rule -- an independent sigmoid affinity s per expert,
    the bias b added to s only to pick the experts, gates from s of the chosen ones
    (AI Engineering Illustrated, "The router is small but it decides everything" and "Fix 2
    nudges a bias instead"; jacopoparretti.dev, "Experts and a router" and "A bias").  Here
    p is the affinity s, which the statistics average as P.
    n_group > 1 limits each token to its topk_group best expert groups.
    """
    if scoring == "softmax":
        r = router_logits(x, w_r, b_r)
        p = softmax(r)
        sel = p
    elif scoring == "sigmoid":
        r = router_logits(x, w_r, None)
        p = sigmoid(r)
        sel = p if b_r is None else p + np.asarray(b_r, np.float64)[None, :]
    else:
        raise ValueError(scoring)
    if idx is None:
        idx = top_k(sel, k) if n_group == 1 else group_limited_top_k(sel, k, n_group, topk_group)
    g = gates(p, idx, renormalize)
    nt = near_ties(sel, k) if n_group == 1 else near_ties_grouped(sel, k, n_group, topk_group)
    return r, p, np.asarray(idx, np.int32), g, nt


def moe_forward(x, w_r, experts, k: int, cap: int = -1, b_r=None, renormalize: bool = True,
                shared=None, idx=None, scoring: str = "softmax", n_group: int = 1,
                topk_group: int = 1, act: str | None = None, mx_eps: float | None = None) -> Result:
    """The whole layer.

    experts: sequence (or any object with ``__getitem__`` and ``__len__``) whose
    item e is (W_g, W_u, W_d) of expert e in float64-convertible form.  The loop
    runs over experts, one batch of that expert's kept rows at a time, the shape
    of the readable PyTorch layer (Zero to Frontier, "In PyTorch").
    shared: (W_g, W_u, W_d) of an always-on expert added with weight 1, or None.
    idx: forced routing (int [T, k]); when given, gates are computed for it.
    scoring, n_group, topk_group: router variant (see ``route``).
    act: None, or "mxfp8": the expert products take MXFP8 activations (x rounded once,
    per token row; h rounded per row inside each expert); the router sees x unrounded.
    mx_eps (with act="mxfp8"): also return y_bound, the per-element bound of
    ``swiglu_mx_deviation`` carried through the gates and the combine.
    """
    x = np.asarray(x, np.float64)
    T, d = x.shape
    E = len(experts)
    r, p, idx, g, nt = route(x, w_r, k, b_r, renormalize, idx, scoring, n_group, topk_group)
    xe = x if act is None else mxfp8_round_rows(x)
    counts, f, P, aux = load_balance_stats(p, idx, E)
    disp = dispatch(idx, E, cap)
    R_kept = int(disp.offsets[-1])
    O = np.zeros((R_kept, d), dtype=np.float64)
    bound = mx_eps is not None and act == "mxfp8"
    OB = np.zeros((R_kept, d), dtype=np.float64) if bound else None
    for e in range(E):
        lo, hi = int(disp.offsets[e]), int(disp.offsets[e + 1])
        if hi == lo:
            continue                              # unchosen experts never run
        toks = disp.row_token[lo:hi]
        wg, wu, wd = experts[e]
        O[lo:hi] = swiglu_ffn(xe[toks], wg, wu, wd, act)
        if bound:
            OB[lo:hi] = swiglu_mx_deviation(xe[toks], wg, wu, wd, mx_eps)[3]
    y = np.zeros((T, d), dtype=np.float64)
    yb = np.zeros((T, d), dtype=np.float64) if bound else None
    for j in range(k):                            # fixed slot order
        rows = disp.row_of[:, j]
        keep = rows >= 0
        y[keep] += g[keep, j:j + 1] * O[rows[keep]]
        if bound:
            yb[keep] += np.abs(g[keep, j:j + 1]) * OB[rows[keep]]
    if shared is not None:
        y += swiglu_ffn(xe, *shared, act=act)
        if bound:
            yb += swiglu_mx_deviation(xe, *shared, mx_eps)[3]
    return Result(y=y, logits=r, p=p, idx=idx, gate=g, counts=counts, f=f, P=P, aux=aux,
                  disp=disp, near_tie=nt, y_bound=yb)


def outputs_for_tokens(x_rows, idx_rows, gate_rows, kept_rows, expert_of, shared=None,
                       act: str | None = None, mx_eps: float | None = None):
    """y for a few tokens, one token at a time, from their routing.

    x_rows [n, d]; idx_rows, gate_rows, kept_rows [n, k] (kept: bool).  expert_of(e)
    returns (W_g, W_u, W_d).  Evaluates sum_j kept * g_j FFN_{idx_j}(x) directly:
    the per-token form of the layer, used to check sampled rows at full size.
    With act="mxfp8" and mx_eps, returns (y, y_bound) (see ``moe_forward``).
    """
    x_rows = np.asarray(x_rows, np.float64)
    if act is not None:
        x_rows = mxfp8_round_rows(x_rows)
    n, d = x_rows.shape
    y = np.zeros((n, d))
    need: dict[int, list] = {}
    for t in range(n):
        for j in range(idx_rows.shape[1]):
            if kept_rows[t, j]:
                need.setdefault(int(idx_rows[t, j]), []).append((t, j))
    bound = mx_eps is not None and act == "mxfp8"
    yb = np.zeros((n, d))
    contrib = np.zeros((n, idx_rows.shape[1], d))
    for e, tj in sorted(need.items()):
        wg, wu, wd = expert_of(e)
        ts = [t for t, _ in tj]
        out = swiglu_ffn(x_rows[ts], wg, wu, wd, act)
        ob = swiglu_mx_deviation(x_rows[ts], wg, wu, wd, mx_eps)[3] if bound else None
        for i, ((t, j), row) in enumerate(zip(tj, out)):
            contrib[t, j] = float(gate_rows[t, j]) * row
            if bound:
                yb[t] += abs(float(gate_rows[t, j])) * ob[i]
    for j in range(idx_rows.shape[1]):            # fixed slot order
        y += contrib[:, j]
    if shared is not None:
        y += swiglu_ffn(x_rows, *shared, act=act)
        if bound:
            yb += swiglu_mx_deviation(x_rows, *shared, mx_eps)[3]
    return (y, yb) if bound else y


# --------------------------------------------------------------------------- FP8 expert weights

def e4m3_decode(codes) -> np.ndarray:
    """Exact value of each one-byte FP8 E4M3 code, float64.

    The pages store expert weights in one byte per parameter (jacopoparretti.dev,
    "Memory": the DeepSeek-V3 weights ship in FP8; AI Engineering Illustrated, "Trade-offs
    to weigh": small-batch MoE is bound by reading weights, which quantising attacks)
    without fixing the encoding.  E4M3 here is the OCP 8-bit float: sign bit, 4 exponent
    bits with bias 7, 3 mantissa bits; exponent 0 holds the subnormals m/8 * 2^-6; there
    are no infinities and S.1111.111 is NaN, so the largest finite value is 448.
    """
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = c >> 7
    ex = (c >> 3) & 15
    man = c & 7
    mag = np.where(ex == 0, (man / 8.0) * 2.0 ** -6, (1.0 + man / 8.0) * np.exp2(ex - 7.0))
    val = np.where(sign == 1, -mag, mag)
    return np.where((ex == 15) & (man == 7), np.nan, val)


def dequantize_rows(codes, scale) -> np.ndarray:
    """W[n, :] = scale[n] * e4m3(codes[n, :]): one fp32 scale per output row (channel).

    The pages do not say how FP8 weights are scaled; one scale per output channel is the
    plainest reading, and a row scale factors out of each output's dot product.
    """
    w = e4m3_decode(codes)
    return w * np.asarray(scale, np.float64).reshape(-1, 1)


def e2m1_decode(nibbles) -> np.ndarray:
    """Exact value of each 4-bit E2M1 element code (the OCP MX FP4 element), float64.

    The pages cite expert weights kept in MXFP4 (AI Engineering Illustrated, "Total
    parameters and active parameters are different budgets"; jacopoparretti.dev, "Speed
    follows active, memory follows total") without defining it.  E2M1: sign bit, 2
    exponent bits with bias 1, 1 mantissa bit; exponent 0 holds 0 and 0.5; the
    magnitudes are 0, 0.5, 1, 1.5, 2, 3, 4, 6; no infinities or NaN.
    """
    c = np.asarray(nibbles, dtype=np.uint8).astype(np.int64) & 15
    sign = c >> 3
    ex = (c >> 1) & 3
    man = c & 1
    mag = np.where(ex == 0, 0.5 * man, (1.0 + 0.5 * man) * np.exp2(ex - 1.0))
    return np.where(sign == 1, -mag, mag)


def e8m0_decode(codes) -> np.ndarray:
    """Value of each E8M0 scale byte (the MX shared block scale): 2^(code - 127), 255 = NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.float64)
    return np.where(c == 255, np.nan, np.exp2(c - 127.0))


def dequantize_mx_rows(packed, scales, block: int = 32) -> np.ndarray:
    """W [n, k] from MXFP4 storage: packed [n, k/2] bytes, element 2j of a row in the low
    nibble of byte j and element 2j+1 in the high nibble; scales [k/block, n] E8M0 bytes,
    scales[b, r] shared by elements block*b .. block*b + block - 1 of row r.
    """
    packed = np.asarray(packed, dtype=np.uint8)
    n, half = packed.shape
    codes = np.empty((n, 2 * half), dtype=np.uint8)
    codes[:, 0::2] = packed & 15
    codes[:, 1::2] = packed >> 4
    sc = e8m0_decode(np.asarray(scales, dtype=np.uint8))          # [k/block, n]
    return e2m1_decode(codes) * np.repeat(sc.T, block, axis=1)


# --------------------------------------------------------------------------- MXFP8 activations

E4M3_MAX = 448.0


def e4m3_encode(v) -> np.ndarray:
    """The E4M3 code (uint8) nearest to each value, ties to the even code, magnitudes above
    448 saturating to 448 (the format has no infinities).

    Written from the format (see ``e4m3_decode``): a magnitude in [2^E, 2^(E+1)) with
    E >= -6 has spacing 2^(E-3); below 2^-6 the subnormals have spacing 2^-9.  The sign is
    kept, also on a value that rounds to zero (-0).  NaN is not an input here.
    """
    v = np.asarray(v, np.float64)
    mag = np.minimum(np.abs(v), E4M3_MAX)
    _, e = np.frexp(mag)                                   # mag = m 2^e, m in [0.5, 1)
    E = np.where(mag > 0, e - 1, -7)
    quantum = np.exp2(np.maximum(E, -6) - 3.0)
    qm = np.round(mag / quantum) * quantum                 # np.round: half to even
    qm = np.minimum(qm, E4M3_MAX)
    # encode qm: exponent field and mantissa
    _, e2 = np.frexp(qm)
    E2 = np.where(qm > 0, e2 - 1, -7)
    normal = E2 >= -6
    expf = np.where(normal, E2 + 7, 0)
    man = np.where(normal, qm / np.exp2(E2) - 1.0, qm / 2.0 ** -6) * 8.0
    code = (expf.astype(np.int64) << 3) | np.round(man).astype(np.int64)
    sign = np.signbit(v)                                   # a negative value that rounds to 0 is -0
    return (code | (sign.astype(np.int64) << 7)).astype(np.uint8)


def _mx_scale_code(amax) -> np.ndarray:
    """E8M0 byte of MX blocks with largest magnitudes amax: floor(log2 amax) - 8 + 127 in [0, 254];
    an all-zero block gets 0."""
    amax = np.asarray(amax, np.float64)
    _, e = np.frexp(amax)
    X = np.where(amax > 0, e - 1 - 8, -127)
    return np.clip(X + 127, 0, 254).astype(np.int64)


def mxfp8_quantize_rows(v, block: int = 32):
    """OCP MXFP8 of the rows of v [n, k]: (codes uint8 [n, k], scales uint8 [n, k/block]).

    Reading for the FP8 product's activations (the pages give FP8 as the storage of
    DeepSeek-V3's weights -- jacopoparretti.dev, "Memory" -- but leave open how the
    activations meet them): every block of 32 consecutive elements of a row shares an E8M0
    scale 2^X with X = floor(log2(max |v| over the block)) - 8 (8 is the largest exponent
    of E4M3, so the block maximum lands in [256, 512) before saturation at 448); each element
    is the E4M3 code nearest v / 2^X.  An all-zero block gets the smallest scale, 2^-127.
    The E8M0 byte is X + 127, kept in [0, 254].
    """
    v = np.asarray(v, np.float64)
    n, kk = v.shape
    blocks = v.reshape(n, kk // block, block)
    sc = _mx_scale_code(np.abs(blocks).max(axis=2))
    scaled = blocks / np.exp2(sc - 127.0)[:, :, None]
    codes = e4m3_encode(scaled).reshape(n, kk)
    return codes, sc.astype(np.uint8)


def dequantize_mxfp8_rows(codes, scales, block: int = 32) -> np.ndarray:
    """Values of MXFP8 rows: e4m3(code) * 2^(scale - 127), scales [n, k/block]."""
    codes = np.asarray(codes, np.uint8)
    sc = e8m0_decode(np.asarray(scales, np.uint8))
    return e4m3_decode(codes) * np.repeat(sc, block, axis=1)


def mxfp8_round_rows(v, block: int = 32) -> np.ndarray:
    """v rounded to its MXFP8 value (quantise, then decode), float64."""
    q, sc = mxfp8_quantize_rows(v, block)
    return dequantize_mxfp8_rows(q, sc, block)


# --------------------------------------------------------------------------- MXFP8: reachable codes

SILU_ARGMIN = -1.2784645427610738       # SiLU's only stationary point (its global minimum)


def silu_range(lo, hi):
    """(min, max) of SiLU over each interval [lo, hi]: SiLU falls to its minimum at SILU_ARGMIN
    and rises after it, so the extremes are the end points and, inside, that minimum."""
    lo = np.asarray(lo, np.float64)
    hi = np.asarray(hi, np.float64)
    sl, sh = silu(lo), silu(hi)
    inside = (lo <= SILU_ARGMIN) & (SILU_ARGMIN <= hi)
    return np.where(inside, silu(np.float64(SILU_ARGMIN)), np.minimum(sl, sh)), np.maximum(sl, sh)


def mxfp8_round_interval(lo, hi, block: int = 32):
    """Lowest and highest MXFP8 value each element of rows [n, k] can round to when every element
    may take any value in its own interval [lo, hi].

    The block scale follows the block maximum, which ranges over [largest lower magnitude, largest
    upper magnitude]; every E8M0 code between the two end codes is reachable.  For a fixed scale
    the rounding (nearest, saturating) never decreases with the value, so an element's extremes
    under that scale are the roundings of lo and hi.
    """
    lo = np.asarray(lo, np.float64)
    hi = np.asarray(hi, np.float64)
    n, kk = lo.shape
    L = lo.reshape(n, kk // block, block)
    H = hi.reshape(n, kk // block, block)
    straddle = (L <= 0) & (H >= 0)
    mlo = np.where(straddle, 0.0, np.minimum(np.abs(L), np.abs(H)))
    mhi = np.maximum(np.abs(L), np.abs(H))
    c_lo = _mx_scale_code(mlo.max(axis=2))
    c_hi = _mx_scale_code(mhi.max(axis=2))
    qlo = np.full(L.shape, np.inf)
    qhi = np.full(L.shape, -np.inf)
    for off in range(int((c_hi - c_lo).max()) + 1 if n * kk else 0):
        c = np.minimum(c_lo + off, c_hi)[:, :, None]
        sc = np.exp2(c - 127.0)
        qlo = np.minimum(qlo, e4m3_decode(e4m3_encode(L / sc)) * sc)
        qhi = np.maximum(qhi, e4m3_decode(e4m3_encode(H / sc)) * sc)
    return qlo.reshape(n, kk), qhi.reshape(n, kk)


def swiglu_mx_deviation(X, w_g, w_u, w_d, eps: float):
    """How far an implementation of the MXFP8 SwiGLU product may land from this oracle's, per
    output element, when each of its dot products is within eps times the sum of its terms'
    magnitudes of the exact value (what a floating-point accumulation gives).

    X [m, d] are MXFP8 values (both sides round x identically, bit for bit).  a and b then lie
    in [a - eps A, a + eps A] with A = |X| |W_g|^T (and the same for b); h = SiLU(a) b lies in the
    range of SiLU over a's interval times b's interval, widened by 2^-20 relative for the fp32
    rounding of h and the hardware exp and reciprocal behind SiLU; its MXFP8 value may be any
    value reachable from that interval (``mxfp8_round_interval``) -- a value near a rounding
    midpoint can go either way.  Returns (hq, qlo, qhi, bound): the oracle's rounded h, the
    reachable range of each element, and per output element of h W_d^T the bound
    sum_j dev_j |W_d[n, j]| + eps sum_j (|hq_j| + dev_j) |W_d[n, j]|, dev_j the larger distance
    from hq_j to its range's ends.
    """
    X = np.asarray(X, np.float64)
    wg, wu, wd = (np.asarray(w, np.float64) for w in (w_g, w_u, w_d))
    a, b = X @ wg.T, X @ wu.T
    da, db = eps * (np.abs(X) @ np.abs(wg).T), eps * (np.abs(X) @ np.abs(wu).T)
    s_lo, s_hi = silu_range(a - da, a + da)
    corners = np.stack([s_lo * (b - db), s_lo * (b + db), s_hi * (b - db), s_hi * (b + db)])
    hlo, hhi = corners.min(axis=0), corners.max(axis=0)
    hlo = hlo - np.abs(hlo) * 2.0 ** -20
    hhi = hhi + np.abs(hhi) * 2.0 ** -20
    hq = mxfp8_round_rows((silu(a) * b).astype(np.float32))
    qlo, qhi = mxfp8_round_interval(hlo, hhi)
    dev = np.maximum(qhi - hq, hq - qlo)
    awd = np.abs(wd)
    return hq, qlo, qhi, dev @ awd.T + eps * ((np.abs(hq) + dev) @ awd.T)


def rel_err(y, y_ref) -> float:
    """max |y - y_ref| / rms(y_ref): the output tolerance measure."""
    y = np.asarray(y, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    rms = math.sqrt(float(np.mean(y_ref * y_ref))) if y_ref.size else 0.0
    if y_ref.size == 0:
        return 0.0
    if rms == 0.0:
        return float(np.max(np.abs(y - y_ref)))
    return float(np.max(np.abs(y - y_ref)) / rms)


# --------------------------------------------------------------------------- backward

@dataclass
class Grads:
    dx: np.ndarray             # [T, d]
    dw_r: np.ndarray           # [E, d]
    db_r: np.ndarray | None    # [E], or None when the layer has no router bias
    dw_gate: np.ndarray        # [E, d_e, d]
    dw_up: np.ndarray          # [E, d_e, d]
    dw_down: np.ndarray        # [E, d, d_e]
    dshared: tuple | None      # (dW_g, dW_u, dW_d) of the shared expert, or None
    dgate: np.ndarray          # [T, k] dL/dg of each slot (0 for a dropped slot)
    dlogits: np.ndarray        # [T, E] dL/dr


def silu_grad(z: np.ndarray) -> np.ndarray:
    """d SiLU(z) / dz = sigma(z) (1 + z (1 - sigma(z))), the derivative of z * sigma(z)."""
    s = sigmoid(z)
    return s * (1.0 + z * (1.0 - s))


def swiglu_backward(X, w_g, w_u, w_d, dO):
    """(dX, dW_g, dW_u, dW_d) of O = (SiLU(X W_g^T) * (X W_u^T)) W_d^T for rows X [m, d].

    The chain rule through the SwiGLU expert of Zero to Frontier §13.1, "The MoE layer",
    with h = SiLU(a) * b, a = X W_g^T, b = X W_u^T:
      dW_d = dO^T h,   dh = dO W_d,
      da = dh * b * SiLU'(a),   db = dh * SiLU(a),
      dW_g = da^T X,   dW_u = db^T X,   dX = da W_g + db W_u.
    """
    X = np.asarray(X, np.float64)
    wg, wu, wd = (np.asarray(w, np.float64) for w in (w_g, w_u, w_d))
    a = X @ wg.T
    b = X @ wu.T
    h = silu(a) * b
    dh = dO @ wd
    da = dh * b * silu_grad(a)
    db = dh * silu(a)
    return da @ wg + db @ wu, da.T @ X, db.T @ X, dO.T @ h


def router_backward(p: np.ndarray, idx: np.ndarray, g: np.ndarray, dgate: np.ndarray, f: np.ndarray,
                    d_aux: float, renormalize: bool = True, scoring: str = "softmax") -> np.ndarray:
    """dL/dr [T, E] from the gate gradients and the auxiliary term, with the choice of
    experts held fixed.

    The top-k choice is a hard selection with no gradient; the gradient reaches the router
    only through the weights of the chosen experts (Moatlab AI-064, "Inside the
    Router").  Steps:
      * renormalised gates g_j = p_{K_j} / S, S = sum_{i in K} p_i, give
        dp_{K_i} = (dg_i - sum_j dg_j g_j) / S; raw gates give dp_{K_i} = dg_i;
      * aux = E sum_e f_e P_e with P_e the mean of p over the T tokens and f_e fixed
        by the counts, so it adds d_aux * E * f_e / T to every dp[t, e];
      * softmax scoring: dr = p * (dp - sum_e p_e dp_e); sigmoid scoring (p is the
        affinity sigma(r)): dr = dp * p * (1 - p).
    """
    T, E = p.shape
    dp = np.zeros((T, E))
    if renormalize:
        S = np.take_along_axis(p, idx.astype(np.int64), axis=1).sum(axis=1, keepdims=True)
        dpk = (dgate - np.sum(dgate * g, axis=1, keepdims=True)) / S
    else:
        dpk = dgate
    rows = np.arange(T)
    for j in range(idx.shape[1]):
        dp[rows, idx[:, j]] += dpk[:, j]
    if T > 0:
        dp += d_aux * E * np.asarray(f, np.float64)[None, :] / T
    if scoring == "softmax":
        return p * (dp - np.sum(p * dp, axis=1, keepdims=True))
    if scoring == "sigmoid":
        return dp * p * (1.0 - p)
    raise ValueError(scoring)


def moe_backward(x, w_r, experts, k: int, dy, d_aux: float = 0.0, cap: int = -1, b_r=None,
                 renormalize: bool = True, shared=None, idx=None, scoring: str = "softmax",
                 n_group: int = 1, topk_group: int = 1) -> Grads:
    """Gradients of L = sum(dy * y) + d_aux * aux for the layer of ``moe_forward``.

    The routing -- which experts each token picked and which assignments capacity
    dropped -- is a constant of the backward pass (Moatlab AI-064, "Inside the
    Router"); f, being counts, is constant too.  A kept slot (t, j) with expert e and row
    r passes g_tj dy_t into expert e's rows (dO_r) and gets dL/dg_tj = dy_t . O_r; a
    dropped slot passes nothing.  Expert gradients follow ``swiglu_backward`` and the
    router's ``router_backward``; dx sums every kept slot's dX row, the router's dr W_r
    and the shared expert's dX.  The router bias is part of the logits under softmax
    scoring (db_r = sum_t dr_t); under sigmoid scoring it only picks experts and gets a
    zero gradient.
    """
    x = np.asarray(x, np.float64)
    dy = np.asarray(dy, np.float64)
    T, d = x.shape
    E = len(experts)
    fwd = moe_forward(x, w_r, experts, k, cap, b_r, renormalize, None, idx, scoring, n_group, topk_group)
    disp, g = fwd.disp, fwd.gate
    dx = np.zeros((T, d))
    dgate = np.zeros((T, k))
    dwg, dwu, dwd = [], [], []
    slot = np.full(int(disp.offsets[-1]), -1, dtype=np.int64)        # slot j of each kept row
    for j in range(k):
        rows = disp.row_of[:, j]
        slot[rows[rows >= 0]] = j
    for e in range(E):
        wg, wu, wd = (np.asarray(w, np.float64) for w in experts[e])
        lo, hi = int(disp.offsets[e]), int(disp.offsets[e + 1])
        if hi == lo:                                 # an expert with no rows gets zero gradients
            dwg.append(np.zeros_like(wg))
            dwu.append(np.zeros_like(wu))
            dwd.append(np.zeros_like(wd))
            continue
        toks, js = disp.row_token[lo:hi], slot[lo:hi]
        X = x[toks]
        O = swiglu_ffn(X, wg, wu, wd)
        dgate[toks, js] = np.sum(dy[toks] * O, axis=1)
        dO = g[toks, js][:, None] * dy[toks]
        dX, gg, gu, gd = swiglu_backward(X, wg, wu, wd, dO)
        dwg.append(gg)
        dwu.append(gu)
        dwd.append(gd)
        np.add.at(dx, toks, dX)
    dr = router_backward(fwd.p, fwd.idx, g, dgate, fwd.f, d_aux, renormalize, scoring)
    w_r64 = np.asarray(w_r, np.float64)
    dx += dr @ w_r64
    dw_r = dr.T @ x
    db_r = None
    if b_r is not None:
        db_r = dr.sum(axis=0) if scoring == "softmax" else np.zeros(E)
    dshared = None
    if shared is not None:
        sX, sg, su, sd = swiglu_backward(x, *shared, dy)
        dx += sX
        dshared = (sg, su, sd)
    return Grads(dx=dx, dw_r=dw_r, db_r=db_r, dw_gate=np.stack(dwg) if E else np.zeros((0,)),
                 dw_up=np.stack(dwu) if E else np.zeros((0,)), dw_down=np.stack(dwd) if E else np.zeros((0,)),
                 dshared=dshared, dgate=dgate, dlogits=dr)
