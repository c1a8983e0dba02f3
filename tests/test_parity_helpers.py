"""Host logic of the GPU parity protocol, on the CPU: the validity check that a near-tie
token's GPU choice must pass when it differs from the oracle's."""
import numpy as np
import pytest

import gpu_parity as gp
import workloads as wl

W = wl.scaled(wl.get("deepseek_v3_grouped"), name="v", T=1, d=128, d_e=128, E=8, k=2, n_group=4, topk_group=2)
e = 4e-7
# groups {0,1} {2,3} {4,5} {6,7}; groups 1 and 2 tie within 1e-6 for the second place
SEL = np.array([0.9, 0.1, 0.5, 0.0, 0.5 + e, 0.3, 0.2, 0.0])
OWN = [0, 4]          # the oracle keeps groups 0 and 2


@pytest.mark.parametrize("pick", [[0, 4], [0, 2]])
def test_valid_flips_pass(pick):
    gp.check_valid_choice(W, SEL, pick, OWN)


@pytest.mark.parametrize("pick,why", [
    ([0, 6], "expert 6 lies in group 3, which is not within 1e-6 of the second group score"),
    ([4, 0], "slots out of descending order"),
    ([0, 0], "an expert twice"),
    ([0, 5], "expert 4 of the same allowed group scores higher than the pick 5"),
    ([2, 4], "expert 0 of an allowed group scores higher than both picks"),
])
def test_invalid_flips_fail(pick, why):
    with pytest.raises(AssertionError):
        gp.check_valid_choice(W, SEL, pick, OWN)


def test_three_groups_rejected():
    w = wl.scaled(W, k=3, topk_group=2)
    sel = np.array([0.9, 0.1, 0.5, 0.0, 0.5 + e, 0.0, 0.5 - e, 0.0])
    gp.check_valid_choice(w, sel, [0, 2, 1], [0, 4, 1])         # groups 0 and 1 instead of 0 and 2
    with pytest.raises(AssertionError):
        gp.check_valid_choice(w, sel, [0, 4, 2], [0, 4, 1])     # groups 0, 2 and 1: one too many


def test_plain_router():
    w = wl.scaled(wl.get("mixtral_prefill"), name="p", T=1, d=128, d_e=128, E=6, k=2)
    sel = np.array([0.3, 0.2, 0.2 + e, 0.1, 0.1, 0.1])
    gp.check_valid_choice(w, sel, [0, 1], [0, 2])
    with pytest.raises(AssertionError):
        gp.check_valid_choice(w, sel, [0, 3], [0, 2])
