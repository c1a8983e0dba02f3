"""Parameter and FLOP arithmetic of MoE decoders.

TEST INFRASTRUCTURE (see the package docstring).

Zero to Frontier §13.1, "Total and active parameters" (and its exercise "Total and
active parameters of an MoE model"): a layer's experts are E SwiGLU blocks of three
d x d_e matrices each, plus a d x E router matrix with no bias; a token touches its k
experts and the whole router.  For a whole decoder the counting rules taken from the
same exercise: no linear layer carries a bias; each block has two RMSNorm gain
vectors of length d and the model one more at the end; shared experts count as
active for every token; the first n_dense blocks use a dense SwiGLU FFN of width
d_ff instead of experts; the embedding (and, when untied, the output projection)
counts fully in both totals.

FLOPs: "FLOPs per token, and the 6N rule for MoE" and the dense-vs-MoE table of
the "In PyTorch" section give 2 FLOPs per active matrix parameter per token
forward, i.e. 6 d d_e k + 2 d E for one MoE layer's experts and router.
"""
from __future__ import annotations


def layer_params(d: int, d_e: int, E: int, k: int) -> tuple[int, int]:
    """(total, active) of one MoE layer's experts plus its router."""
    return 3 * d * d_e * E + d * E, 3 * d * d_e * k + d * E


def moe_param_count(cfg: dict) -> tuple[int, int]:
    """(total, active) parameters of a whole decoder described by cfg.

    cfg keys: V, d, L, attn (attention parameters per layer), n_dense, d_ff, E,
    E_shared, k, d_e, tied.
    """
    V, d, L = cfg["V"], cfg["d"], cfg["L"]
    attn, n_dense, d_ff = cfg["attn"], cfg.get("n_dense", 0), cfg.get("d_ff", 0)
    E, Es, k, d_e = cfg["E"], cfg.get("E_shared", 0), cfg["k"], cfg["d_e"]
    norms = 2 * d
    dense_layer = attn + 3 * d * d_ff + norms
    moe_total = attn + 3 * d * d_e * (E + Es) + d * E + norms
    moe_active = attn + 3 * d * d_e * (k + Es) + d * E + norms
    emb = V * d * (1 if cfg.get("tied", False) else 2)
    n_moe = L - n_dense
    total = n_dense * dense_layer + n_moe * moe_total + emb + d
    active = n_dense * dense_layer + n_moe * moe_active + emb + d
    return total, active


def forward_flops_per_token(d: int, d_e: int, E: int, k: int, d_e_shared: int = 0) -> int:
    """Forward FLOPs of one MoE layer per token: 6 d d_e k + 2 d E (+ 6 d d_e_shared)."""
    return 6 * d * d_e * k + 2 * d * E + 6 * d * d_e_shared


def router_flops_per_token(d: int, E: int) -> int:
    """2 d E: the router's share, paid in full by every token."""
    return 2 * d * E


def train_flops(n_active: float, tokens: float) -> float:
    """6 N_active D: training compute of an MoE model on D tokens."""
    return 6.0 * n_active * tokens


def flops_ratio(n_total: float, n_active: float) -> float:
    """How many times more compute a dense model of n_total parameters needs."""
    return n_total / n_active
