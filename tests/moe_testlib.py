"""Helpers shared by the GPU parity tests: tensor conversion, lazy expert access for the
oracle, the tolerances, and the near-tie aware comparison of routing results."""
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
    t = t.detach()
    if t.dtype in (torch.bfloat16, torch.float16):
        t = t.float()
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


def check_route(w_gpu, ids_gpu, r: "O.RouteResult", what: str = "") -> np.ndarray:
    """Compare GPU routing with the oracle's. Returns the mask of near-tie tokens (whose
    choice may legitimately differ). For those, the GPU's experts must still be a valid
    choice: each one's key within 1e-5 (relative) of the oracle's K-th key."""
    ids = ids_gpu.cpu().numpy().astype(np.int64)
    w = w_gpu.cpu().numpy().astype(np.float64)
    tie = near_tie_tokens(r)
    ok = ~tie
    assert np.array_equal(ids[ok], r.topk_ids[ok]), \
        f"{what}: ids differ on {np.sum(np.any(ids[ok] != r.topk_ids[ok], axis=1))} tokens"
    rel = np.abs(w[ok] - r.topk_weights[ok]) / np.maximum(np.abs(r.topk_weights[ok]), 1e-30)
    assert rel.size == 0 or rel.max() <= WEIGHT_RTOL, f"{what}: weights rel err {rel.max():.2e}"
    for t in np.nonzero(tie)[0]:
        assert len(set(ids[t].tolist())) == ids.shape[1], f"{what}: repeated ids, token {t}"
        # the same expert set, or a set whose members all score near the K-th key
        s = r.scores[t]
        kth = np.min(s[r.topk_ids[t]])
        assert np.all(s[ids[t]] >= kth - 1e-5 * max(abs(kth), 1e-30) - 1e-6), (what, t)
    return tie


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
