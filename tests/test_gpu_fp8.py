"""Block-scaled FP8 grouped GEMM over a masked slab (moe_grouped_gemm_fp8_masked) against
the oracle.

Bound: the page's own for this op, |err| <= atol + rtol |ref| with atol = 2e-2 *
sqrt(max(1, K / 1024)) and rtol = 2e-2 against the dequantized product, and the bf16
bound of every other output, max |err| <= 2e-2 max |ref|. Rows at or past an expert's
count must be left as they were."""
import math

import numpy as np
import pytest
import torch

import oracle.moe_oracle as O
from mixture_experts_ffn_moerouter_amd import binding as B
from mixture_experts_ffn_moerouter_amd import inputs as I
from moe_testlib import assert_close, guarded, np64, say

pytestmark = pytest.mark.gpu
SENTINEL = 12288.0  # 1.5 * 2^13, exactly representable in bf16


def run(d, out=None):
    E, max_m, _ = d["a"].shape
    N = d["b"].shape[1]
    if out is None:
        out = torch.full((E, max_m, N), SENTINEL, dtype=torch.bfloat16, device="cuda")
    B.moe_grouped_gemm_fp8_masked(d["a"], d["a_scale"], d["b"], d["b_scale"], d["counts"],
                                  out=out)
    torch.cuda.synchronize()
    return out


def host(d):
    return {k: v.cpu().numpy() for k, v in d.items()}


def check(got, ref, counts, K, what):
    E, max_m, N = got.shape
    atol = 2e-2 * math.sqrt(max(1.0, K / 1024))
    valid = []
    for g in range(E):
        m = int(min(max(int(counts[g]), 0), max_m))
        gg, rr = got[g, :m], ref[g, :m]
        excess = np.abs(gg - rr) - (atol + 2e-2 * np.abs(rr))
        if (excess > 0).any():
            w = np.unravel_index(np.argmax(excess), excess.shape)
            raise AssertionError(
                f"{what}: expert {g}, {(excess > 0).sum()} elements past the fp8 bound; worst "
                f"at row {w[0]} col {w[1]}: got {gg[w]!r} ref {rr[w]!r} (max|ref| of the expert "
                f"{np.abs(rr).max():.4g})")
        assert np.all(got[g, m:] == SENTINEL), f"{what}: expert {g} wrote rows past its count"
        valid.append((gg, rr))
    if valid:
        assert_close(np.concatenate([v[0].ravel() for v in valid]),
                     np.concatenate([v[1].ravel() for v in valid]), "bf16", what)


def test_fp8_small_all_counts():
    """Empty, single-row, ragged, full and over-full experts; three 128-wide K blocks (an
    odd number of steps) and three weight tiles."""
    cfg = I.FP8_CONFIGS["fp8_small"]
    say(f"[fp8] {cfg.name}")
    d = I.make_fp8_inputs(cfg, device="cuda")
    got = np64(run(d))
    h = host(d)
    ref = O.grouped_gemm_fp8_masked(h["a"], h["a_scale"], h["b"], h["b_scale"], h["counts"])
    check(got, ref, h["counts"], cfg.K, cfg.name)


# (E, max_m, K, N), counts from max_m down to 1: 320 / 160 / 1 rows are two full 160-row
# tiles, one full tile and one row; 161 rows are two tiles (96 + 65)
@pytest.mark.parametrize("shape", [(1, 32, 128, 128), (3, 96, 256, 128), (2, 300, 640, 384),
                                   (4, 128, 1024, 256), (3, 320, 384, 256),
                                   (2, 161, 256, 384)])
def test_fp8_shapes(shape):
    E, max_m, K, N = shape
    say(f"[fp8] shape {shape}")
    counts = tuple(int(c) for c in np.linspace(max_m, 1, E).round())
    cfg = I.Fp8GemmConfig(f"fp8_{E}_{max_m}_{K}_{N}", E=E, max_m=max_m, K=K, N=N,
                          counts=counts)
    d = I.make_fp8_inputs(cfg, seed=3, device="cuda")
    got = np64(run(d))
    h = host(d)
    ref = O.grouped_gemm_fp8_masked(h["a"], h["a_scale"], h["b"], h["b_scale"], h["counts"])
    check(got, ref, h["counts"], K, cfg.name)


def _block_magnitudes(h):
    """sum over k of |a_k| |b_k| a_scale b_scale per output element (float64): the size of
    the products a float32 accumulation adds up, which bounds its rounding (a block sum
    can cancel to far below its products)."""
    A = torch.from_numpy(h["a"]).view(torch.float8_e4m3fn).to(torch.float64)
    Bw = torch.from_numpy(h["b"]).view(torch.float8_e4m3fn).to(torch.float64)
    sa = torch.from_numpy(h["a_scale"]).double()
    sb = torch.from_numpy(h["b_scale"]).double()
    E, M, K = A.shape
    N = Bw.shape[1]
    mag = torch.zeros((E, M, N), dtype=torch.float64)
    nb = torch.arange(N) // 128
    for kb in range(K // 128):
        ks = slice(128 * kb, 128 * (kb + 1))
        part = torch.bmm(A[:, :, ks].abs(), Bw[:, :, ks].abs().transpose(1, 2).contiguous())
        mag += part * sa[:, :, kb, None].abs() * sb[:, nb, kb][:, None, :].abs()
    return mag.numpy()


def test_fp8_scales_span_binades():
    """Scales spread over 2^-8 .. 2^8 per row, per weight block and per K block, so a scale
    applied to the wrong row, weight block or K block shows. Terms then reach ~1e4 while
    some outputs cancel to ~0.1, so the page's absolute bound (set for its own scale
    ranges) is replaced by the float32 accumulation bound of each element's products:
    |err| <= 2e-2 |ref| + 1e-5 * sum_k |a_k b_k| scales (about 128 roundings of 2^-24). A
    misplaced scale is off by at least half of a whole block term, far above that."""
    cfg = I.Fp8GemmConfig("fp8_scales", E=3, max_m=130, K=512, N=256, counts=(130, 64, 7))
    say(f"[fp8] {cfg.name}")
    d = I.make_fp8_inputs(cfg, seed=5, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(7)
    d["a_scale"] *= torch.exp2(torch.randint(-8, 9, d["a_scale"].shape, device="cuda",
                                             generator=g).float())
    d["b_scale"] *= torch.exp2(torch.randint(-8, 9, d["b_scale"].shape, device="cuda",
                                             generator=g).float())
    got = np64(run(d))
    h = host(d)
    ref = O.grouped_gemm_fp8_masked(h["a"], h["a_scale"], h["b"], h["b_scale"], h["counts"])
    mag = _block_magnitudes(h)
    for e in range(cfg.E):
        m = int(h["counts"][e])
        err = np.abs(got[e, :m] - ref[e, :m])
        lim = 2e-2 * np.abs(ref[e, :m]) + 1e-5 * mag[e, :m]
        assert np.all(err <= lim), (e, float((err - lim).max()))
        assert np.all(got[e, m:] == SENTINEL)
    assert_close(got[0, :130], ref[0, :130], "bf16", cfg.name)


def test_fp8_guard_bands_and_repeat():
    """Nothing outside out is written; a second call gives identical bytes."""
    cfg = I.FP8_CONFIGS["fp8_small"]
    d = I.make_fp8_inputs(cfg, device="cuda")
    E, M, N = cfg.E, cfg.max_m, cfg.N
    out, guard_ok = guarded((E, M, N), torch.bfloat16)
    out.fill_(SENTINEL)
    run(d, out)
    guard_ok()
    first = out.clone()
    run(d, out)
    assert torch.equal(first, out)


def boundary_rows(m: int, stride: int = 32) -> np.ndarray:
    """Rows 0 and m - 1 and both sides of every stride-row boundary below m: the first
    and last row of any row tile whose height is a multiple of stride."""
    j = np.arange(stride, m, stride)
    return np.unique(np.concatenate([[0, m - 1], j - 1, j])).astype(np.int64)


@pytest.mark.parametrize("name", ["dsv3_fp8_gate_up", "dsv3_fp8_down"])
def test_fp8_full_size_every_expert(name):
    """The DeepSeek-V3 shapes over masked slabs (E 256, slabs of 256 rows, about 128 valid
    rows per expert): every output computed on the GPU. For every expert, its boundary
    rows (first and last row of every row tile) are compared on one 256-column weight
    tile (expert g takes tile g mod N/256, so every weight tile is compared on 16 or more
    experts), and its rows past the count must be untouched."""
    cfg = I.FP8_CONFIGS[name]
    say(f"[fp8-full] {cfg.name} generating inputs")
    d = I.make_fp8_inputs(cfg, device="cuda")
    say(f"[fp8-full] {cfg.name} gemm")
    out = run(d)
    counts = d["counts"].cpu().numpy()
    nt = cfg.N // 256
    got_all, ref_all = [], []
    for g in range(cfg.E):
        m = int(counts[g])
        if m == 0:
            continue
        rows = boundary_rows(m)
        c0 = 256 * (g % nt)
        rt = torch.as_tensor(rows, device="cuda")
        sub = {"a": d["a"][g:g + 1, rt].cpu().numpy(),
               "a_scale": d["a_scale"][g:g + 1, rt].cpu().numpy(),
               "b": d["b"][g:g + 1, c0:c0 + 256].cpu().numpy(),
               "b_scale": d["b_scale"][g:g + 1, c0 // 128:c0 // 128 + 2].cpu().numpy()}
        ref = O.grouped_gemm_fp8_masked(sub["a"], sub["a_scale"], sub["b"], sub["b_scale"],
                                        np.array([rows.size]))
        got = np64(out[g:g + 1, rt, c0:c0 + 256])
        check(got, ref, np.array([rows.size]), cfg.K, f"{cfg.name} expert {g}")
        assert np.all(np64(out[g, m:]) == SENTINEL), f"expert {g} wrote past its count"
        got_all.append(got.ravel())
        ref_all.append(ref.ravel())
    assert_close(np.concatenate(got_all), np.concatenate(ref_all), "bf16", cfg.name)
