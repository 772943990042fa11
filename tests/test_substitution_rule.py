"""The near-tie substitution check the GPU tests apply ([TO] FusedTopKFwdOp: an expert,
or a group, whose selection score is within 1e-5 relative, a group score also 1e-6
absolute, of the last one kept may be kept in its place). Runs on the CPU: the oracle's
own choices must pass, and choices the rule does not allow must fail."""
import numpy as np

import oracle.moe_oracle as O
from moe_testlib import valid_substitution


def _route(logits, K, G=1, TG=1, bias=None):
    return O.route(np.asarray(logits, np.float64)[None, :], K, "sigmoid", True, 1.0, G, TG,
                   None if bias is None else np.asarray(bias, np.float64))


def _check(r, ids, K, G=1, TG=1):
    gs = None if r.group_scores is None else r.group_scores[0]
    return valid_substitution(r.keys[0], gs, np.asarray(ids), K, G, TG)


def test_oracle_choices_pass():
    rng = np.random.default_rng(1)
    for trial in range(200):
        E, K, G, TG = [(16, 3, 1, 1), (32, 8, 8, 4), (24, 4, 4, 2)][trial % 3]
        z = rng.standard_normal(E)
        bias = rng.uniform(-0.1, 0.1, E) if trial % 2 else None
        r = _route(z, K, G, TG, bias)
        assert _check(r, r.topk_ids[0], K, G, TG) is None


def test_expert_swap_within_and_beyond_tolerance():
    # keys: expert 2 is the K-th kept (K = 3), expert 5 just below it
    z = np.full(8, -3.0)
    z[[0, 1, 2]] = [3.0, 2.0, 1.0]
    s1 = O.sigmoid(1.0)
    for rel, ok in ((3e-6, True), (5e-5, False)):
        target = s1 * (1 - rel)
        z[5] = np.log(target / (1 - target))
        r = _route(z, 3)
        assert list(r.topk_ids[0]) == [0, 1, 2]
        why = _check(r, [0, 1, 5], 3)
        assert (why is None) == ok, (rel, why)
    # a far-away expert is never a valid substitute
    assert _check(r, [0, 1, 7], 3) is not None
    # repeated ids fail
    assert _check(r, [0, 1, 1], 3) is not None


def test_group_swap_within_and_beyond_tolerance():
    # 4 groups of 2 experts, one group kept, K 2, zero bias: a group's score is the sum of
    # its pair's sigmoids. Group 1 scores rel below group 0 (the one the oracle keeps).
    E, G, TG, K = 8, 4, 1, 2
    s1 = O.sigmoid(1.0)
    for rel, ok in ((2e-6, True), (1e-3, False)):
        target = s1 - 2 * s1 * rel
        z = np.full(E, -3.0)
        z[[0, 1, 2]] = 1.0
        z[3] = np.log(target / (1 - target))
        r = _route(z, K, G, TG, np.zeros(E))
        assert list(r.topk_ids[0]) == [0, 1]
        why = _check(r, [2, 3], K, G, TG)
        assert (why is None) == ok, (rel, why)
        assert _check(r, [0, 2], K, G, TG) is not None  # two groups where one is kept
    # a group far below the kept one can never be used
    assert _check(r, [6, 7], K, G, TG) is not None
