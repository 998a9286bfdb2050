"""GPU parity: the HIP path, called through the C ABI, against the CPU oracle.

Tolerances (max abs error on y): 1e-4 for float32, 2e-2 for bf16 storage with
float32 accumulation. bf16 inputs are the bf16-rounded values both sides see.
"""
import math

import numpy as np
import pytest
import torch

from gpu_helpers import TOL, Gpu, log, max_err, y_numpy
from oracle import pool
from oracle import tri_attn_oracle as O
from triangular_pair_attention_amd import binding as B
from workloads import WORKLOADS, Workload, make_inputs

pytestmark = pytest.mark.gpu

LOG2E = 1.4426950408889634


def run_case(inp, fill=-1e9, slack=0.0, rows=None):
    g = Gpu(inp, fill=fill, slack=slack)
    try:
        y = y_numpy(g.forward())
        torch.cuda.synchronize()
    finally:
        g.close()
    if rows is None:
        ref = O.forward(inp, fill=fill)
        return y, ref
    ref = O.forward_rows(inp, rows, fill=fill)
    return np.stack([y[b, i] for b, i in rows]), ref


def check(y, ref, dtype, what):
    finite = np.isfinite(ref)
    assert (np.isfinite(y) == finite).all(), f"{what}: NaN pattern differs"
    err, idx = max_err(np.where(finite, y, 0), np.where(finite, ref, 0))
    log(f"{what}: max abs err {err:.3e} at {idx}, max|y| {np.abs(ref[finite]).max():.3f}")
    assert err <= TOL[dtype], f"{what}: max abs err {err} > {TOL[dtype]} at {idx}"


# ------------------------------------------------------------------ the five workloads
@pytest.mark.parametrize("k", [1, 2, 3, 4])
def test_workload_full(k):
    w = WORKLOADS[k]
    log(f"workload {w.name}: full oracle comparison")
    inp = make_inputs(w)
    y, ref = run_case(inp)
    check(y, ref, w.dtype, w.name)


def test_workload5_full():
    """B=4, N=512, h=8 (the headline workload, in the benchmark's launch
    configuration): every output element of all 2048 pair rows against the
    oracle, the rows spread over host worker processes."""
    w = WORKLOADS[5]
    log(f"workload {w.name}: full oracle comparison (worker processes)")
    inp = make_inputs(w)
    g = Gpu(inp)
    try:
        y = g.forward().float().cpu().numpy()
        torch.cuda.synchronize()
    finally:
        g.close()
    rows = [(b, i) for b in range(w.B) for i in range(w.N)]
    r = pool.compare_rows(inp, y, rows)["y"]
    log(f"{w.name}: max abs err {r['max_abs_err']:.3e} at {r['where']}, max|y| {r['max_abs_ref']:.3f}")
    assert r["same_nan_pattern"]
    assert r["max_abs_err"] <= TOL[w.dtype]


def recovered_fraction(g):
    """Share of attention work items whose last forward took the
    exact-maximum recovery path (the workspace's per-item flags)."""
    lay = B.tri_attn_get_workspace_layout(g.handle, g.B, g.N)
    flags = g.region(lay.recover_flags, lay.attention_items, torch.uint8).cpu().numpy()
    assert set(np.unique(flags).tolist()) <= {0, 1}
    return float(flags.mean()), lay.attention_items


PEAK = 8.0  # factor on the query and pair-bias weights in the peaked-input tests


def test_workload5_benchmark_inputs_never_recover():
    """The softmax bound of the benchmark inputs is tight enough that no
    attention work item of the headline workload is recomputed."""
    inp = make_inputs(WORKLOADS[5])
    g = Gpu(inp)
    try:
        g.forward()
        torch.cuda.synchronize()
        frac, items = recovered_fraction(g)
    finally:
        g.close()
    log(f"{WORKLOADS[5].name}: {items} attention items, recovered fraction {frac:.4f}")
    assert frac == 0.0


def test_workload5_peaked_full():
    """The headline workload with the query and pair-bias weights scaled by 8
    (peaked softmax, scores and bias 8x larger, so the Cauchy-Schwarz shift
    is much looser): all 2048 rows against the oracle. Tolerance: q and k
    reach the matrix cores in bf16, so each score carries an absolute error
    proportional to its size; scaling the scores by 8 scales that error, and
    to first order the error of y, by 8: 8 x 2e-2. The share of items that
    took the recovery path is logged."""
    w = WORKLOADS[5]
    inp = make_inputs(w)
    inp["w_query"] = inp["w_query"] * PEAK
    inp["w_bias_proj"] = inp["w_bias_proj"] * PEAK
    g = Gpu(inp)
    try:
        y = g.forward().float().cpu().numpy()
        torch.cuda.synchronize()
        frac, items = recovered_fraction(g)
    finally:
        g.close()
    log(f"{w.name} peaked x{PEAK:g}: {items} attention items, recovered fraction {frac:.4f}")
    r = pool.compare_rows(inp, y, [(b, i) for b in range(w.B) for i in range(w.N)])["y"]
    log(f"{w.name} peaked: max abs err {r['max_abs_err']:.3e} at {r['where']}, max|y| {r['max_abs_ref']:.3f}")
    assert r["same_nan_pattern"]
    assert r["max_abs_err"] <= TOL["bf16"] * PEAK


def test_workload5_shape_float32_peaked_sampled_rows():
    """The headline shape (B=4, N=512, D=128, h=8, per-batch padding) in
    float32 with peaked inputs: the float32 head-size-16 attention uses the
    same bounded shift, and float32 keeps the 1e-4 tolerance. Sampled rows."""
    w = Workload("c5shape_f32_peaked", 4, 512, 128, 8, "f32", ("pad_range", 384, 512), seed=1005)
    inp = make_inputs(w)
    inp["w_query"] = inp["w_query"] * PEAK
    inp["w_bias_proj"] = inp["w_bias_proj"] * PEAK
    rows = [(0, 0), (0, 300), (1, 17), (1, 511), (2, 255), (3, 0), (3, 400), (3, 511)]
    g = Gpu(inp)
    try:
        y = y_numpy(g.forward())
        torch.cuda.synchronize()
        frac, items = recovered_fraction(g)
    finally:
        g.close()
    log(f"{w.name}: {items} attention items, recovered fraction {frac:.4f}")
    check(np.stack([y[b, i] for b, i in rows]), O.forward_rows(inp, rows), "f32", w.name)


def gpu_y32(inp):
    g = Gpu(inp)
    try:
        y = g.forward().float().cpu().numpy()
        torch.cuda.synchronize()
    finally:
        g.close()
    return y


@pytest.mark.parametrize("k", [5, 4, 2])
def test_full_size_permutation_equivariance(k):
    """Every output at full size, through a property of the method: one
    permutation pi of all residue axes with a permutation sigma of the batch,
    P'[b,i,j] = P[sigma(b),pi(i),pi(j)] and M'[b,j,k] = M[sigma(b),pi(j),pi(k)],
    gives y'[b,i,j] = y[sigma(b),pi(i),pi(j)] (exact for the oracle; its own
    tests check that). Both GPU results lie within the tolerance of the
    oracle's, so they may differ by at most twice the tolerance. The permuted
    mask scatters the padding, so the permuted run skips no key chunk while
    the plain one does."""
    w = WORKLOADS[k]
    log(f"workload {w.name}: permutation equivariance at full size")
    inp = make_inputs(w)
    rng = np.random.default_rng(7)
    pi, sg = rng.permutation(w.N), rng.permutation(w.B)
    perm = dict(inp)
    for name in ("pair_repr", "pair_mask"):
        perm[name] = np.ascontiguousarray(inp[name][sg][:, pi][:, :, pi])
    y = gpu_y32(inp)
    y2 = gpu_y32(perm)
    want = y[sg][:, pi][:, :, pi]
    assert (np.isfinite(y2) == np.isfinite(want)).all()
    diff = float(np.abs(y2 - want).max())
    log(f"  max |y' - permuted y| {diff:.3e}, max |y| {np.abs(y).max():.3f}")
    assert diff <= 2 * TOL[w.dtype]


@pytest.mark.parametrize("dtype,h", [("bf16", 8), ("bf16", 4), ("f32", 4)])
def test_large_n_sampled_rows(dtype, h):
    """N = 1040 (17 key chunks, the last one ragged): larger than any
    workload, so 64-bit offsets, many key steps and the chunk bookkeeping are
    exercised; compared on sampled rows."""
    w = Workload("largeN", 1, 1040, 128, h, dtype, ("pad", 1000), seed=21)
    log(f"large N {dtype} h={h}: sampled rows")
    inp = make_inputs(w)
    rows = [(0, i) for i in (0, 517, 999, 1000, 1039)]
    y, ref = run_case(inp, rows=rows)
    check(y, ref, dtype, f"large N {dtype} h={h}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_workspace_past_4gib_sampled_rows(dtype):
    """N = 2048, d = 32: the workspace exceeds 4 GiB (bf16 about 4.1 GB,
    float32 9.7 GB with the split keys), so region offsets past 2^32 bytes
    are exercised in every kernel; compared on sampled rows, including the
    last valid row, the first padded one and the last one."""
    w = Workload("ws4g", 1, 2048, 128, 4, dtype, ("pad", 2000), seed=23)
    log(f"workspace past 4 GiB {dtype}: sampled rows")
    inp = make_inputs(w)
    rows = [(0, i) for i in (0, 1023, 1999, 2000, 2047)]
    g = Gpu(inp)
    try:
        log(f"  workspace {g.ws_bytes / 2**30:.2f} GiB")
        assert g.ws_bytes > 2**32
        y = g.forward()
        ys = torch.stack([y[b, i] for b, i in rows]).float().cpu().numpy().astype(np.float64)
        torch.cuda.synchronize()
    finally:
        g.close()
    ref = O.forward_rows(inp, rows)
    check(ys, ref, dtype, f"workspace past 4 GiB {dtype}")


# ------------------------------------------------------------------ small and ragged shapes
SHAPES = [
    (1, 1, 64, 4), (2, 3, 64, 2), (2, 17, 64, 4), (1, 33, 128, 4), (1, 65, 128, 8),
    (2, 100, 64, 2), (1, 130, 128, 4), (1, 70, 128, 8), (3, 64, 128, 8), (1, 129, 64, 4),
]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B%dN%dD%dh%d" % s)
@pytest.mark.parametrize("mask", [("bernoulli", 0.7), ("pad", 0.6)], ids=["bern", "pad"])
def test_small_ragged(shape, dtype, mask):
    B_, N, D, h = shape
    if mask[0] == "pad":
        mask = ("pad", max(1, int(N * mask[1])))
    w = Workload("small", B_, N, D, h, dtype, mask, seed=100 + N + D + h)
    log(f"small {shape} {dtype} {mask}")
    y, ref = run_case(make_inputs(w))
    check(y, ref, dtype, f"{shape} {dtype} {mask}")


def _random_case(n):
    """Seeded random configuration n: batch 1-3, N 1-200, D 64 or 128, head
    size 16 or 32, either dtype, Bernoulli or padding mask, -1e9 fill."""
    rng = np.random.default_rng(5000 + n)
    B_ = int(rng.integers(1, 4))
    N = int(rng.integers(1, 201))
    D = int(rng.choice([64, 128]))
    h = D // int(rng.choice([16, 32]))
    dtype = str(rng.choice(["f32", "bf16"]))
    if rng.random() < 0.5:
        mask = ("bernoulli", float(rng.uniform(0.5, 0.95)))
    else:
        mask = ("pad", int(rng.integers(1, N + 1)))
    return Workload(f"random{n}", B_, N, D, h, dtype, mask, seed=6000 + n)


@pytest.mark.parametrize("n", range(48))
def test_random_shapes(n):
    w = _random_case(n)
    log(f"random case {n}: B={w.B} N={w.N} D={w.D} h={w.h} {w.dtype} {w.mask}")
    y, ref = run_case(make_inputs(w))
    check(y, ref, w.dtype, w.name)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_all_keys_masked(dtype):
    """Mask all zero: every query column is fully masked -> mean of v over all N keys."""
    w = Workload("allmasked", 2, 40, 128, 4, dtype, ("zeros",), seed=5)
    log(f"all masked {dtype}")
    y, ref = run_case(make_inputs(w))
    check(y, ref, dtype, "all masked")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_minus_inf_fill_gives_nan_on_fully_masked_columns(dtype):
    w = Workload("ninf", 1, 50, 64, 4, dtype, ("pad", 30), seed=6)
    log(f"-inf fill {dtype}")
    y, ref = run_case(make_inputs(w), fill=-math.inf)
    assert np.isnan(ref[:, :, 30:]).all() and np.isnan(y[:, :, 30:]).all()
    check(y, ref, dtype, "-inf fill")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dh", [16, 32])
@pytest.mark.parametrize("slack", [100.0, 400.0])
def test_loose_shift_and_recovery_path(dtype, dh, slack):
    """shift_slack loosens the softmax bound. The shift sits 96 below the
    bound (its headroom), so at 100 every shift is positive and bf16 d=32
    waves apply it (they skip it where the shift is at most 0), while every
    column's sum stays far above the recovery threshold; at 400 every sum
    underflows and each item takes the exact-maximum recovery path, which the
    per-item flags record. Neither may change the result."""
    w = Workload("slack", 1, 48, 128, 128 // dh, dtype, ("pad", 40), seed=7)
    log(f"shift slack {slack} {dtype} d={dh}")
    inp = make_inputs(w)
    g = Gpu(inp, slack=slack)
    try:
        y = y_numpy(g.forward())
        torch.cuda.synchronize()
        frac, _ = recovered_fraction(g)
    finally:
        g.close()
    log(f"  recovered fraction {frac:.3f}")
    assert frac == (1.0 if slack > 200 else 0.0)
    check(y, O.forward(inp), dtype, f"slack {slack}")


@pytest.mark.parametrize("dtype,dh", [("bf16", 16), ("bf16", 32), ("f32", 32)])
def test_recovery_on_every_item_of_persistent_workgroups(dtype, dh):
    """N = 300 gives more attention work items than resident workgroups
    (900 to 3000), so each workgroup runs several items back to back, with
    its per-item state double-buffered; slack 400 sends every item through
    the exact-maximum recovery path."""
    w = Workload("slack300", 1, 300, 128, 128 // dh, dtype, ("pad", 290), seed=11)
    log(f"persistent recovery {dtype} d={dh}")
    inp = make_inputs(w)
    rows = [(0, i) for i in (0, 1, 7, 8, 150, 151, 289, 290, 299)]
    y, ref = run_case(inp, slack=400.0, rows=rows)
    check(y, ref, dtype, f"persistent recovery {dtype} d={dh}")


@pytest.mark.parametrize("dtype,h", [("bf16", 4), ("bf16", 2), ("f32", 2)])
def test_d64_two_batches_sampled_rows(dtype, h):
    """D = 64 at N = 300, two batches with their own padding length (a range
    like the largest workload's): more attention items than resident
    workgroups and more projection tiles than workgroups, so the persistent
    attention loop and kernel 1's tile loop both run, with ragged chunks."""
    w = Workload("d64", 2, 300, 64, h, dtype, ("pad_range", 200, 300), seed=12)
    log(f"D=64 two batches {dtype} h={h}")
    inp = make_inputs(w)
    rows = [(0, 0), (0, 5), (0, 199), (0, 250), (1, 3), (1, 150), (1, 298), (1, 299)]
    y, ref = run_case(inp, rows=rows)
    check(y, ref, dtype, f"D=64 two batches {dtype} h={h}")


@pytest.mark.parametrize("h", [4, 2], ids=["d16", "d32"])
def test_large_scores_stay_finite(h):
    """Scaled-up query weights make the scores large (peaked softmax); at
    head size 32 the float32 scores run as split bf16 products."""
    w = Workload("peaked", 1, 40, 64, h, "f32", ("bernoulli", 0.8), seed=8)
    inp = make_inputs(w)
    inp["w_query"] *= 8
    inp["w_bias_proj"] *= 8
    log(f"peaked softmax h={h}")
    y, ref = run_case(inp)
    check(y, ref, "f32", "peaked")


# ------------------------------------------------------------------ stage parity of kernel 1
# Up to one 64-position tile per resident workgroup, kernel 1 runs its straight
# one-tile instantiation; more tiles (the last three shapes: 900, 900 and 1500
# tiles, ragged last chunks) take the persistent loop with its prefetch.
@pytest.mark.parametrize("dtype,shape", [("f32", (2, 40, 64, 4)), ("bf16", (1, 70, 128, 4)),
                                         ("bf16", (1, 66, 128, 8)), ("f32", (1, 64, 128, 4)),
                                         ("f32", (2, 150, 64, 4)), ("bf16", (2, 150, 128, 8)),
                                         ("f32", (1, 300, 128, 4))])
def test_projection_stage(dtype, shape):
    B_, N, D, h = shape
    d = D // h
    inp = make_inputs(Workload("stage", B_, N, D, h, dtype, ("bernoulli", 0.7), seed=9))
    log(f"stage {dtype} {shape}")
    g = Gpu(inp)
    try:
        lay = g.project()
        Np = lay.padded_n
        cap = {}
        O.forward(inp, capture=cap)
        dt = g.dt
        f = lambda off, n, t=dt: g.region(off, n, t).float().cpu().numpy().astype(np.float64)  # noqa: E731
        q = f(lay.q, B_ * N * D * Np).reshape(B_, N, D // 16, Np, 16)[:, :, :, :N].transpose(0, 1, 3, 2, 4)
        k = g.k_region(lay)
        gg = f(lay.g, B_ * N * D * Np).reshape(B_, N, D // 16, Np, 16)[:, :, :, :N].transpose(0, 1, 3, 2, 4)
        vt = f(lay.vt, B_ * N * D * Np).reshape(B_, N, h, d, Np)[..., :N]
        zm = f(lay.zm, B_ * h * N * Np, torch.float32).reshape(B_, h, N, Np)
        zmax = f(lay.zmax, B_ * h * N * (Np // 64), torch.float32).reshape(B_, h, Np // 64, N).transpose(0, 1, 3, 2)
        kmax = f(lay.kmax, B_ * N * (D // 16) * (Np // 64), torch.float32).reshape(B_, N, D // 16, Np // 64)
        vsum = f(lay.vsum, B_ * N * D * (Np // 64), torch.float32).reshape(B_, N, Np // 64, D).transpose(0, 1, 3, 2)
    finally:
        g.close()
    q = q.reshape(B_, N, N, D)
    k = k.reshape(B_, N, N, D)
    gg = gg.reshape(B_, N, N, D)
    rq = O.merge_heads(cap["q"]).reshape(B_, N, N, D) * LOG2E / math.sqrt(d)
    rk = O.merge_heads(cap["k"]).reshape(B_, N, N, D)
    rv = cap["v"].reshape(B_, N, h, N, d)  # (b, i, t, j, u)
    rg = cap["g"].reshape(B_, N, N, D)
    M = inp["pair_mask"]
    rz = np.where(M[:, None] != 0, cap["z"] * LOG2E, -np.inf)  # (b, t, j, k)
    # float32: the products run as six exact bf16 products of split operands;
    # the bound is float32-level (measured errors are about 1e-6)
    atol, rtol = (1e-5, 1e-5) if dtype == "f32" else (2e-2, 1e-2)
    for name, got, ref in (("q", q, rq), ("k", k, rk), ("g", gg, rg), ("v", vt, rv.transpose(0, 1, 2, 4, 3))):
        log(f"  {name}: max abs err {np.abs(got - ref).max():.3e}, max |ref| {np.abs(ref).max():.3f}")
        np.testing.assert_allclose(got, ref, rtol=rtol, atol=atol, err_msg=name)
    fin = np.isfinite(rz)
    assert (np.isfinite(zm[..., :N]) == fin).all()
    np.testing.assert_allclose(zm[..., :N][fin], rz[fin], rtol=rtol, atol=atol)
    assert (zm[..., N:] == -np.inf).all()
    # per-chunk maxima
    pad = np.full((B_, h, N, Np), -np.inf)
    pad[..., :N] = rz
    np.testing.assert_allclose(zmax, pad.reshape(B_, h, N, Np // 64, 64).max(-1), rtol=rtol, atol=atol)
    kn2 = np.zeros((B_, N, D // 16, Np))  # |k|^2 over each 16-channel block, per column
    kn2[..., :N] = (rk.reshape(B_, N, N, D // 16, 16) ** 2).sum(-1).transpose(0, 1, 3, 2)
    np.testing.assert_allclose(kmax, kn2.reshape(B_, N, D // 16, Np // 64, 64).max(-1), rtol=2 * rtol, atol=atol)
    # per-chunk sums of v over the key columns (zero beyond N)
    vs = np.zeros((B_, N, D, Np))
    vs[..., :N] = O.merge_heads(cap["v"]).reshape(B_, N, N, D).transpose(0, 1, 3, 2)
    vs = vs.reshape(B_, N, D, Np // 64, 64).sum(-1)
    np.testing.assert_allclose(vsum, vs, rtol=rtol, atol=atol * 64)


def test_float32_split_products_scale():
    """float32 projections run as six exact bf16 products of split operands:
    their error must stay at float32 level relative to the values' scale,
    here with pair_repr offset by 3e4 (spread 1e4) and weights scaled by 1e3
    and 1e-3."""
    B_, N, D, h = 1, 70, 128, 4
    inp = make_inputs(Workload("scale", B_, N, D, h, "f32", ("bernoulli", 0.8), seed=12))
    inp["pair_repr"] = (inp["pair_repr"] * 1e4 + 3e4).astype(np.float32)
    inp["w_key"] = (inp["w_key"] * 1e3).astype(np.float32)
    inp["w_value"] = (inp["w_value"] * 1e-3).astype(np.float32)
    inp["w_out"] = (inp["w_out"] * 1e3).astype(np.float32)
    inp["b_out"] = (inp["b_out"] * 1e3).astype(np.float32)
    log("float32 split products at scale")
    g = Gpu(inp)
    try:
        lay = g.project()
        Np = lay.padded_n
        f = lambda off, n: g.region(off, n, torch.float32).cpu().numpy().astype(np.float64)  # noqa: E731
        k = g.k_region(lay)
        vt = f(lay.vt, B_ * N * D * Np).reshape(B_, N, h, D // h, Np)[..., :N]
        y = y_numpy(g.forward())
        torch.cuda.synchronize()
    finally:
        g.close()
    cap = {}
    ref = O.forward(inp, capture=cap)
    rk = O.merge_heads(cap["k"]).reshape(B_, N, N, D)
    rv = cap["v"].reshape(B_, N, h, N, D // h).transpose(0, 1, 2, 4, 3)
    for name, got, want, bound in (("k", k.reshape(B_, N, N, D), rk, 1e-5), ("v", vt, rv, 1e-5), ("y", y, ref, 1e-5)):
        rel = float(np.abs(got - want).max() / np.abs(want).max())
        log(f"  {name}: max |ref| {np.abs(want).max():.3e}, max abs err / max |ref| {rel:.2e}")
        assert rel <= bound, f"{name}: relative error {rel} > {bound}"


# ------------------------------------------------------------------ ending-node variant
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape,mask", [((2, 40, 64, 4), ("bernoulli", 0.8)), ((1, 130, 128, 4), ("pad", 100)),
                                        ((1, 150, 128, 8), ("bernoulli", 0.7)), ((2, 33, 64, 2), ("pad", 20))],
                         ids=["B2N40", "N130pad", "N150h8", "B2N33d32"])
def test_ending_node(shape, mask, dtype):
    """Ending-node attention (the other residue axis) against the oracle's
    ending-node forward, element by element."""
    B_, N, D, h = shape
    inp = make_inputs(Workload("ending", B_, N, D, h, dtype, mask, seed=40 + N))
    log(f"ending node {shape} {dtype} {mask}")
    g = Gpu(inp, ending=True)
    try:
        y = y_numpy(g.forward())
        torch.cuda.synchronize()
    finally:
        g.close()
    check(y, O.forward_ending(inp), dtype, f"ending {shape} {dtype}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ending_node_large_sampled_columns(dtype):
    """N = 300 (persistent loops in every kernel), compared on sampled output
    columns y[b, :, j]."""
    w = Workload("ending_large", 1, 300, 128, 4, dtype, ("pad", 270), seed=77)
    inp = make_inputs(w)
    log(f"ending node N=300 {dtype}")
    g = Gpu(inp, ending=True)
    try:
        y = y_numpy(g.forward())
        torch.cuda.synchronize()
    finally:
        g.close()
    cols = [(0, 0), (0, 131), (0, 269), (0, 270), (0, 299)]
    got = np.stack([y[b, :, j] for b, j in cols])
    check(got, O.forward_ending_cols(inp, cols), dtype, f"ending N=300 {dtype} sampled columns")


def test_ending_node_workload5_full():
    """Ending-node handle at B=4, N=512, h=8 bf16 (per-batch padding): every
    output column y[b, :, j] against the oracle's ending-node forward, which
    is its starting-node forward of the pair representation and mask with
    both residue axes swapped (columns spread over host worker processes)."""
    w = WORKLOADS[5]
    log(f"ending node {w.name}: full oracle comparison (worker processes)")
    inp = make_inputs(w)
    g = Gpu(inp, ending=True)
    try:
        y = g.forward().float().cpu().numpy()
        torch.cuda.synchronize()
    finally:
        g.close()
    cols = [(b, j) for b in range(w.B) for j in range(w.N)]
    r = pool.compare_rows(O._transposed(inp), np.ascontiguousarray(np.swapaxes(y, 1, 2)), cols)["y"]
    log(f"ending {w.name}: max abs err {r['max_abs_err']:.3e} at (b, j, i, c) {r['where']}, "
        f"max|y| {r['max_abs_ref']:.3f}")
    assert r["same_nan_pattern"]
    assert r["max_abs_err"] <= TOL[w.dtype]


# ------------------------------------------------------------------ ABI behaviour on the GPU
def test_deterministic_and_stream():
    inp = make_inputs(WORKLOADS[3].replace(N=96))
    log("determinism")
    g = Gpu(inp)
    try:
        a = g.forward().clone()
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            b = g.forward(stream=s)
        s.synchronize()
        assert torch.equal(a, b)
    finally:
        g.close()


@pytest.mark.parametrize("k", [2, 3])
def test_forward_captured_in_hip_graph(k):
    """The forward enqueues kernels only (no memsets, no allocation), so it can
    be captured in a HIP graph; every replay, with eager work of the library
    between replays, must equal the eager forward bit for bit."""
    w = WORKLOADS[k]
    inp = make_inputs(w)
    log(f"HIP graph capture {w.name}")
    g = Gpu(inp)
    try:
        eager = g.forward().clone()
        torch.cuda.synchronize()
        out = torch.empty_like(g.P)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            g.forward(out=out, stream=side)  # warm-up on a side stream before capture
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            g.forward(out=out, stream=torch.cuda.current_stream())
        for r in range(4):
            out.fill_(float("nan"))
            graph.replay()
            torch.cuda.synchronize()
            assert torch.equal(out, eager), f"replay {r} differs from the eager forward"
            other = g.forward()  # eager work between replays
            torch.cuda.synchronize()
            assert torch.equal(other, eager)
        del graph
    finally:
        g.close()


def test_empty_and_error_paths():
    inp = make_inputs(Workload("err", 1, 20, 64, 4, "f32", ("bernoulli", 0.8), 3))
    log("error paths")
    g = Gpu(inp)
    try:
        assert B.tri_attn_workspace_size(g.handle, 0, 20) == 0
        B.tri_attn_forward(g.handle, 0, 0, 0, 0, 20, 0, 0)  # B == 0: no-op
        B.tri_attn_forward(g.handle, 0, 0, 0, 3, 0, 0, 0)  # N == 0: no-op
        out = torch.empty_like(g.P)
        with pytest.raises(B.TriAttnError) as e:
            B.tri_attn_forward(g.handle, g.P, g.M, out, g.B, g.N, g.ws, g.ws_bytes - 1)
        assert e.value.code == B.TRI_ATTN_ERR_WORKSPACE
        with pytest.raises(B.TriAttnError) as e:
            B.tri_attn_forward(g.handle, g.P, g.M, out, g.B, g.N, g.ws.data_ptr() + 8, g.ws_bytes)
        assert e.value.code == B.TRI_ATTN_ERR_WORKSPACE
        with pytest.raises(B.TriAttnError) as e:
            B.tri_attn_forward(g.handle, g.P, g.M, 0, g.B, g.N, g.ws, g.ws_bytes)
        assert e.value.code == B.TRI_ATTN_ERR_INVALID_ARG
        with pytest.raises(B.TriAttnError) as e:
            B.tri_attn_forward(g.handle, g.P, g.M, out, -1, g.N, g.ws, g.ws_bytes)
        assert e.value.code == B.TRI_ATTN_ERR_INVALID_ARG
        torch.cuda.synchronize()
    finally:
        g.close()


def test_stages_equal_forward():
    """project, attend, output in turn give the forward's exact bits."""
    inp = make_inputs(WORKLOADS[1])
    log("project + attend + output")
    g = Gpu(inp)
    try:
        a = g.forward().clone()
        g.project()
        b = torch.empty_like(g.P)
        st = torch.cuda.current_stream()
        B.tri_attn_attend(g.handle, g.B, g.N, g.ws, g.ws_bytes, st)
        B.tri_attn_output(g.handle, b, g.B, g.N, g.ws, g.ws_bytes, st)
        torch.cuda.synchronize()
        assert torch.equal(a, b)
        with pytest.raises(B.TriAttnError) as e:
            B.tri_attn_output(g.handle, 0, g.B, g.N, g.ws, g.ws_bytes)
        assert e.value.code == B.TRI_ATTN_ERR_INVALID_ARG
    finally:
        g.close()


def test_convenience_wrapper_matches_abi():
    from triangular_pair_attention_amd import TriangularAttention
    inp = make_inputs(Workload("wrap", 1, 36, 64, 2, "bf16", ("bernoulli", 0.8), 4))
    log("wrapper")
    g = Gpu(inp)
    try:
        a = g.forward()
        m = TriangularAttention(g.w, num_heads=2)
        b = m(g.P, g.M)
        torch.cuda.synchronize()
        assert torch.equal(a, b)
        m.close()
    finally:
        g.close()
