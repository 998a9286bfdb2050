"""GPU parity of the one-pass variant (tri_attn_forward_onepass: a bias
pre-pass, then one fused kernel per pair row) with the CPU oracle, at the
tolerances of the three-kernel forward (max abs error on y: 1e-4 float32,
2e-2 bf16 storage with float32 accumulation)."""
import math

import numpy as np
import pytest
import torch

from gpu_helpers import TOL, Gpu, log, max_err
from oracle import pool
from oracle import tri_attn_oracle as O
from triangular_pair_attention_amd import binding as B
from workloads import WORKLOADS, Workload, make_inputs

pytestmark = pytest.mark.gpu


def onepass(g, out=None):
    n = B.tri_attn_onepass_workspace_size(g.handle, g.B, g.N)
    ws = torch.empty(max(n, 256), dtype=torch.uint8, device=g.dev)
    if out is None:
        out = torch.empty_like(g.P)
    B.tri_attn_forward_onepass(g.handle, g.P, g.M, out, g.B, g.N, ws, n, torch.cuda.current_stream())
    return out


def run(inp, fill=-1e9, ending=False):
    g = Gpu(inp, fill=fill, ending=ending)
    try:
        y = onepass(g).float().cpu().numpy().astype(np.float64)
        torch.cuda.synchronize()
    finally:
        g.close()
    return y


def check(y, ref, dtype, what):
    finite = np.isfinite(ref)
    assert (np.isfinite(y) == finite).all(), f"{what}: NaN pattern differs"
    err, idx = max_err(np.where(finite, y, 0), np.where(finite, ref, 0))
    log(f"{what}: max abs err {err:.3e} at {idx}, max|y| {np.abs(ref[finite]).max():.3f}")
    assert err <= TOL[dtype], f"{what}: max abs err {err} > {TOL[dtype]} at {idx}"


@pytest.mark.parametrize("k", [1, 2, 3, 4])
def test_onepass_workload_full(k):
    w = WORKLOADS[k]
    log(f"one-pass {w.name}: full oracle comparison")
    inp = make_inputs(w)
    check(run(inp), O.forward(inp), w.dtype, f"one-pass {w.name}")


def test_onepass_workload5_full():
    """B=4, N=512, h=8: all 2048 pair rows against the oracle (worker processes)."""
    w = WORKLOADS[5]
    log(f"one-pass {w.name}: full oracle comparison (worker processes)")
    inp = make_inputs(w)
    g = Gpu(inp)
    try:
        y = onepass(g).float().cpu().numpy()
        torch.cuda.synchronize()
    finally:
        g.close()
    r = pool.compare_rows(inp, y, [(b, i) for b in range(w.B) for i in range(w.N)])["y"]
    log(f"one-pass {w.name}: max abs err {r['max_abs_err']:.3e} at {r['where']}, max|y| {r['max_abs_ref']:.3f}")
    assert r["same_nan_pattern"]
    assert r["max_abs_err"] <= TOL[w.dtype]


SHAPES = [(1, 1, 64, 4), (2, 3, 64, 2), (2, 17, 64, 4), (1, 33, 128, 4), (1, 65, 128, 8), (2, 100, 64, 2),
          (1, 130, 128, 4), (3, 64, 128, 8), (1, 129, 64, 4), (1, 200, 128, 8)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "B%dN%dD%dh%d" % s)
@pytest.mark.parametrize("mask", [("bernoulli", 0.7), ("pad", 0.6)], ids=["bern", "pad"])
def test_onepass_small_ragged(shape, dtype, mask):
    """Ragged N (partial 16-position blocks and 64-key steps), both head
    sizes and widths, padding (fully masked query columns) and Bernoulli masks."""
    B_, N, D, h = shape
    if mask[0] == "pad":
        mask = ("pad", max(1, int(N * mask[1])))
    inp = make_inputs(Workload("op_small", B_, N, D, h, dtype, mask, seed=300 + N + D + h))
    log(f"one-pass {shape} {dtype} {mask}")
    check(run(inp), O.forward(inp), dtype, f"one-pass {shape} {dtype} {mask}")


@pytest.mark.parametrize("dtype,D,h", [("f32", 128, 4), ("f32", 128, 8), ("bf16", 128, 4), ("bf16", 64, 2)])
def test_onepass_largest_rows_sampled(dtype, D, h):
    """N = 512, the largest row the fused kernel takes (four position blocks
    per wave), two batches with their own padding length; sampled rows."""
    w = Workload("op_n512", 2, 512, D, h, dtype, ("pad_range", 380, 512), seed=310 + h)
    inp = make_inputs(w)
    log(f"one-pass N=512 {dtype} D={D} h={h}")
    rows = [(0, 0), (0, 200), (0, 511), (1, 3), (1, 379), (1, 511)]
    g = Gpu(inp)
    try:
        y = onepass(g).float().cpu().numpy().astype(np.float64)
        torch.cuda.synchronize()
    finally:
        g.close()
    check(np.stack([y[b, i] for b, i in rows]), O.forward_rows(inp, rows), dtype, f"one-pass N=512 {dtype}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_onepass_all_keys_masked(dtype):
    """Every query column fully masked: the mean of v over all N keys."""
    inp = make_inputs(Workload("op_allmasked", 2, 40, 128, 4, dtype, ("zeros",), seed=305))
    log(f"one-pass all masked {dtype}")
    check(run(inp), O.forward(inp), dtype, "one-pass all masked")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_onepass_minus_inf_fill(dtype):
    inp = make_inputs(Workload("op_ninf", 1, 50, 64, 4, dtype, ("pad", 30), seed=306))
    log(f"one-pass -inf fill {dtype}")
    y = run(inp, fill=-math.inf)
    ref = O.forward(inp, fill=-math.inf)
    assert np.isnan(ref[:, :, 30:]).all() and np.isnan(y[:, :, 30:]).all()
    check(y, ref, dtype, "one-pass -inf fill")


PEAK = 8.0  # factor on the query and pair-bias weights


def peaked_tolerance(dtype):
    """float32: the workload tolerance. bf16: q and k reach the matrix cores
    rounded to bf16, so each score carries an absolute error proportional to
    its own size; scaling the query and bias weights by PEAK scales the scores,
    hence (to first order) the error of the weights and of y, by PEAK."""
    return TOL[dtype] * (PEAK if dtype == "bf16" else 1.0)


@pytest.mark.parametrize("dtype,h", [("f32", 4), ("f32", 2), ("bf16", 8)])
def test_onepass_peaked_scores(dtype, h):
    """Query and bias weights scaled by 8 (peaked softmax): the running
    maximum needs no bound."""
    inp = make_inputs(Workload("op_peaked", 1, 90, 64 if h < 8 else 128, h, dtype, ("bernoulli", 0.8), seed=307))
    inp["w_query"] *= PEAK
    inp["w_bias_proj"] *= PEAK
    log(f"one-pass peaked {dtype} h={h}")
    y, ref = run(inp), O.forward(inp)
    assert (np.isfinite(y) == np.isfinite(ref)).all()
    err, idx = max_err(y, ref)
    log(f"one-pass peaked {dtype}: max abs err {err:.3e} at {idx}, max|y| {np.abs(ref).max():.3f}")
    assert err <= peaked_tolerance(dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape,mask", [((2, 40, 64, 4), ("bernoulli", 0.8)), ((1, 130, 128, 4), ("pad", 100)),
                                        ((1, 150, 128, 8), ("bernoulli", 0.7)), ((2, 33, 64, 2), ("pad", 20))],
                         ids=["B2N40", "N130pad", "N150h8", "B2N33d32"])
def test_onepass_ending_node(shape, mask, dtype):
    B_, N, D, h = shape
    inp = make_inputs(Workload("op_ending", B_, N, D, h, dtype, mask, seed=320 + N))
    log(f"one-pass ending node {shape} {dtype}")
    check(run(inp, ending=True), O.forward_ending(inp), dtype, f"one-pass ending {shape} {dtype}")


def test_onepass_deterministic_and_matches_three_kernel_path():
    """Two calls give the same bits; the three-kernel forward agrees within
    twice the tolerance (both lie within it of the oracle)."""
    w = WORKLOADS[3]
    inp = make_inputs(w)
    g = Gpu(inp)
    try:
        a = onepass(g).float().cpu().numpy()
        b = onepass(g).float().cpu().numpy()
        c = g.forward().float().cpu().numpy()
        torch.cuda.synchronize()
    finally:
        g.close()
    assert np.array_equal(a, b)
    diff = float(np.abs(a - c).max())
    log(f"one-pass vs three-kernel forward {w.name}: max diff {diff:.3e}")
    assert diff <= 2 * TOL[w.dtype]


def test_onepass_errors():
    inp = make_inputs(Workload("op_err", 1, 20, 64, 4, "f32", ("bernoulli", 0.8), 309))
    g = Gpu(inp)
    try:
        assert B.tri_attn_onepass_workspace_size(g.handle, 0, 20) == 0
        assert B.tri_attn_onepass_workspace_size(g.handle, 1, 20) == 1 * 4 * 20 * 64 * 4
        with pytest.raises(B.TriAttnError) as e:
            B.tri_attn_onepass_workspace_size(g.handle, 1, 513)
        assert e.value.code == B.TRI_ATTN_ERR_UNSUPPORTED
        n = B.tri_attn_onepass_workspace_size(g.handle, g.B, g.N)
        ws = torch.empty(n + 512, dtype=torch.uint8, device=g.dev)
        out = torch.empty_like(g.P)
        B.tri_attn_forward_onepass(g.handle, 0, 0, 0, 0, 20, 0, 0)  # B == 0: no-op
        with pytest.raises(B.TriAttnError) as e:
            B.tri_attn_forward_onepass(g.handle, g.P, g.M, out, g.B, g.N, ws, n - 1)
        assert e.value.code == B.TRI_ATTN_ERR_WORKSPACE
        with pytest.raises(B.TriAttnError) as e:
            B.tri_attn_forward_onepass(g.handle, g.P, g.M, out, g.B, g.N, ws.data_ptr() + 8, n)
        assert e.value.code == B.TRI_ATTN_ERR_WORKSPACE
        with pytest.raises(B.TriAttnError) as e:
            B.tri_attn_forward_onepass(g.handle, g.P, g.M, 0, g.B, g.N, ws, n)
        assert e.value.code == B.TRI_ATTN_ERR_INVALID_ARG
        torch.cuda.synchronize()
    finally:
        g.close()
