"""Helpers shared by the GPU parity tests: tensor conversion, lazy expert access for the
oracle, the tolerances, and the near-tie aware comparison of routing results."""
import dataclasses
import itertools
import sys

import numpy as np
import torch

import oracle.moe_oracle as O

# Tolerances. bf16 outputs: max |err| <= 2e-2 * max |ref|; float32 outputs:
# max |err| <= 1e-4 * max |ref|; float16 outputs: the bf16 bound scaled by the ratio of
# the two formats' unit roundoffs (2^-11 / 2^-8), 2.5e-3 * max |ref|; routing weights:
# 1e-4 relative per element; expert ids bit-exact except on tokens whose selection gap
# is below 1e-6.
TOL = {"bf16": 2e-2, "f32": 1e-4, "f16": 2.5e-3}
WEIGHT_RTOL = 1e-4
TIE_GAP = 1e-6


def say(*a):
    """Progress line naming the case before a GPU step (flushed)."""
    print(*a, file=sys.stderr, flush=True)


def np64(t: torch.Tensor) -> np.ndarray:
    """float64 host copy (widening is exact; done on the tensor's device, so large expert
    slices cross to the host once)."""
    t = t.detach()
    if t.is_floating_point():
        return t.double().cpu().numpy()
    return t.cpu().numpy().astype(np.float64)


class LazyExperts:
    """w[e] -> float64 numpy copy of one expert's slice of a device tensor."""

    def __init__(self, t):
        self.t = t

    def __getitem__(self, e):
        return np64(self.t[int(e)])

    def __len__(self):
        return self.t.shape[0]


def assert_close(got, ref, dtype: str, what: str = ""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    scale = np.max(np.abs(ref)) if ref.size else 0.0
    err = np.max(np.abs(got - ref)) if ref.size else 0.0
    assert err <= TOL[dtype] * max(scale, 1e-30), \
        f"{what}: max|err| {err:.3e} > {TOL[dtype]} * max|ref| {scale:.3e}"
    return err / max(scale, 1e-30)


def near_tie_tokens(r: "O.RouteResult") -> np.ndarray:
    return (r.gap_sel < TIE_GAP) | (r.gap_group < TIE_GAP)


# [TO] FusedTopKFwdOp: an expert whose selection score is within 1e-5 (relative) of the
# last one kept may be kept in its place; a group likewise, its score within 1e-5
# relative or 1e-6 absolute of the last kept group score.
SUB_REL, SUB_GROUP_ABS = 1e-5, 1e-6


def valid_substitution(keys, gscores, ids, K: int, G: int, TG: int):
    """Is `ids` (one token's K chosen experts) a selection the page's substitution rule
    allows, given that token's float32 selection keys [E] and group scores [G] (None
    without groups)? Returns a reason string when it is not, else None.

    The chosen groups must be TG groups, each kept by the reference order or scoring
    within the group tolerance of the last kept group; inside those groups the chosen
    experts must be the top K up to the expert tolerance around the K-th key."""
    ids = np.asarray(ids, dtype=np.int64)
    E = keys.size
    if len(set(ids.tolist())) != K or ids.min() < 0 or ids.max() >= E:
        return "ids repeated or out of range"
    if G > 1:
        group_of = np.arange(E) // (E // G)
        order = O.ranked(gscores)
        last = gscores[order[TG - 1]]
        tol_g = max(SUB_REL * abs(last), SUB_GROUP_ABS)
        allowed = [g for g in range(G) if g in order[:TG] or gscores[g] >= last - tol_g]
        used = set(group_of[ids].tolist())
        if not used <= set(allowed) or len(used) > TG:
            return f"groups {sorted(used)} not within tolerance of the kept groups"
        choices = [set(c) for c in itertools.combinations(allowed, TG) if used <= set(c)]
        eligible_sets = [np.isin(group_of, sorted(c)) for c in choices]
    else:
        eligible_sets = [np.ones(E, dtype=bool)]
    chosen = np.zeros(E, dtype=bool)
    chosen[ids] = True
    for elig in eligible_sets:
        kth = np.sort(keys[elig])[::-1][K - 1]
        tol = SUB_REL * abs(kth)
        rest = keys[elig & ~chosen]
        if keys[ids].min() >= kth - tol and (rest.size == 0 or rest.max() <= kth + tol):
            return None
    return "chosen experts are not a top-k within tolerance"


def check_route(w_gpu, ids_gpu, r: "O.RouteResult", what: str = "", reroute=None,
                G: int = 1, TG: int = 1):
    """Compare GPU routing with the oracle's.

    Tokens whose selection gap is at least 1e-6: ids bit-exact, weights within 1e-4
    relative. Near-tie tokens (gap below 1e-6): the GPU's choice must be one the page's
    substitution rule allows (valid_substitution), and its weights must match the
    oracle's weights for that same choice. `reroute(tokens, ids)` returns the oracle's
    RouteResult for those tokens with the given expert ids (hash-routing form: weights
    from the scores of exactly those experts); it is required when near ties occur.

    Returns (tie mask, RouteResult of the GPU's choice for every token): the oracle's own
    result where the ids agree, the rerouted one on near-tie tokens."""
    ids = ids_gpu.cpu().numpy().astype(np.int64)
    w = w_gpu.cpu().numpy().astype(np.float64)
    tie = near_tie_tokens(r)
    ok = ~tie
    assert np.array_equal(ids[ok], r.topk_ids[ok]), \
        f"{what}: ids differ on {np.sum(np.any(ids[ok] != r.topk_ids[ok], axis=1))} tokens"
    K = ids.shape[1]
    fixed = dataclasses.replace(r)
    tt = np.nonzero(tie)[0]
    if tt.size:
        for t in tt:
            why = valid_substitution(r.keys[t], None if r.group_scores is None
                                     else r.group_scores[t], ids[t], K, G, TG)
            assert why is None, f"{what}: token {t}: {why}"
        assert reroute is not None, f"{what}: {tt.size} near-tie tokens and no reroute"
        rr = reroute(tt, ids[tt])
        fixed.topk_ids = r.topk_ids.copy()
        fixed.topk_weights = r.topk_weights.copy()
        fixed.wn = r.wn.copy()
        fixed.topk_ids[tt] = rr.topk_ids
        fixed.topk_weights[tt] = rr.topk_weights
        fixed.wn[tt] = rr.wn
        if r.router_probs is not None:
            fixed.router_probs = r.router_probs.copy()
            fixed.weight_scale = r.weight_scale.copy()
            fixed.router_probs[tt] = rr.router_probs
            fixed.weight_scale[tt] = rr.weight_scale
    rel = np.abs(w - fixed.topk_weights) / np.maximum(np.abs(fixed.topk_weights), 1e-30)
    assert rel.size == 0 or rel.max() <= WEIGHT_RTOL, f"{what}: weights rel err {rel.max():.2e}"
    return tie, fixed


def route_rerouter(logits, K, scoring, renormalize, rsf, **ep):
    """reroute() for check_route: the oracle's route of the given tokens with the given
    expert ids (float64 host logits; ep = the expert-parallel keyword arguments)."""
    def reroute(tokens, ids):
        return O.route(logits[tokens], K, scoring, renormalize, rsf, expert_ids=ids, **ep)
    return reroute


def guarded(shape, dtype, device="cuda", guard: int = 4096):
    """An output tensor inside a larger buffer whose guard bands hold a sentinel; returns
    (view, check) where check() asserts the guard bands are untouched."""
    n = int(np.prod(shape))
    buf = torch.full((n + 2 * guard,), float("nan") if dtype.is_floating_point else -7,
                     dtype=dtype, device=device)
    if not dtype.is_floating_point:
        buf.fill_(-7)
    else:
        buf.fill_(-12345.0)
    view = buf[guard:guard + n].view(shape)
    before = buf.clone()

    def check():
        assert torch.equal(buf[:guard], before[:guard]), "write before the output"
        assert torch.equal(buf[guard + n:], before[guard + n:]), "write past the output"

    return view, check
