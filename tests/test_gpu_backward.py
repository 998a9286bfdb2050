"""GPU parity of the training-mode backward (tri_attn_backward_train) with
the backward oracle (hand back-propagation in float64, itself pinned by
finite differences and autograd): dL/d(pair_repr) and dL/d(every parameter)
for the same dropout decisions.

Tolerance: the GPU computes every step in float32 from the same inputs,
the attention products as split bf16 products (about 2^-16 relative error),
so each gradient tensor must agree with the oracle's to 1e-3 of its largest
magnitude (the longest float32 sums run over all B*N*N positions; their
rounding error grows like sqrt(B*N*N) * 2^-24 relative, about 2e-5 at
B*N*N = 65536; both well inside the bound)."""
import math

import numpy as np
import pytest
import torch

from gpu_helpers import Gpu, log
from oracle import tri_attn_backward_oracle as BO
from oracle import tri_attn_oracle as O
from triangular_pair_attention_amd import binding as B
from workloads import WORKLOADS, Workload, make_inputs

pytestmark = pytest.mark.gpu

RTOL = 1e-3
SHAPE = {"d_pair_repr": "pair_repr", "d_ln_weight": "ln_weight", "d_ln_bias": "ln_bias", "d_w_query": "w_query",
         "d_w_key": "w_key", "d_w_value": "w_value", "d_w_gate": "w_gate", "d_b_gate": "b_gate",
         "d_w_bias_proj": "w_bias_proj", "d_w_out": "w_out", "d_b_out": "b_out"}


def run_backward(inp, dy, rate, seed, offset, fill=-1e9, ending=False, dz_ranges=0):
    g = Gpu(inp, fill=fill, ending=ending)
    try:
        if dz_ranges:
            B.tri_attn_set_backward_dz_ranges(g.handle, dz_ranges)
        grads = {k: torch.zeros(np.shape(inp[v]), dtype=torch.float32, device=g.dev) for k, v in SHAPE.items()}
        n = B.tri_attn_backward_workspace_size(g.handle, g.B, g.N)
        ws = torch.empty(max(n, 256), dtype=torch.uint8, device=g.dev)
        dyt = torch.from_numpy(dy).to(g.dev).to(g.dt).contiguous()
        B.tri_attn_backward_train(g.handle, g.P, g.M, dyt, g.B, g.N, rate, seed, offset, grads, ws, n,
                                  torch.cuda.current_stream())
        torch.cuda.synchronize()
        return {k: v.double().cpu().numpy() for k, v in grads.items()}
    finally:
        g.close()


def make_dy(inp, seed):
    rng = np.random.default_rng(seed)
    dy = rng.standard_normal(np.shape(inp["pair_repr"])).astype(np.float32)
    if inp["dtype"] == "bf16":
        from workloads import round_to_bf16
        dy = round_to_bf16(dy)
    return dy


def check_backward(inp, rate, seed, offset, what, fill=-1e9, dz_ranges=0):
    dy = make_dy(inp, 99)
    got = run_backward(inp, dy, rate, seed, offset, fill, dz_ranges=dz_ranges)
    ref = BO.backward_train(inp, dy.astype(np.float64), rate, seed, offset, fill=fill)
    worst = 0.0
    for k in SHAPE:
        r, gk = ref[k], got[k]
        assert r.shape == gk.shape, k
        fin = np.isfinite(r)
        assert (np.isfinite(gk) == fin).all(), f"{what} {k}: NaN pattern differs"
        scale = float(np.abs(r[fin]).max()) if fin.any() else 0.0
        err = float(np.abs(gk[fin] - r[fin]).max()) if fin.any() else 0.0
        rel = err / scale if scale > 0 else err
        worst = max(worst, rel)
        log(f"{what} {k}: max abs err {err:.3e}, max |ref| {scale:.3e}, relative {rel:.2e}")
        assert err <= RTOL * scale + 1e-12, f"{what} {k}: error {err} > {RTOL} * {scale}"
    return worst


SHAPES = [((2, 20, 64, 4), ("bernoulli", 0.8)), ((1, 33, 128, 4), ("pad", 25)), ((1, 40, 128, 8), ("pad", 31)),
          ((2, 17, 64, 2), ("bernoulli", 0.6)), ((1, 70, 128, 4), ("bernoulli", 0.9))]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape,mask", SHAPES, ids=lambda s: str(s))
@pytest.mark.parametrize("rate", [0.0, 0.3])
def test_backward_small(shape, mask, dtype, rate):
    """Small and ragged shapes, both head sizes, fully masked columns (padding)."""
    Bn, N, D, h = shape
    inp = make_inputs(Workload("bwd", Bn, N, D, h, dtype, mask, seed=81 + N))
    check_backward(inp, rate, seed=2**35 + 3, offset=5, what=f"backward {dtype} {shape} {mask} rate {rate}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("ranges", [1, 3, 1000])
def test_backward_pair_bias_step_row_ranges(dtype, ranges):
    """The pair-bias gradient step sums over rows i in ranges whose partial
    sums are added in order afterwards; small sizes choose several ranges,
    large ones (from 2048 (query, key) tiles up, workload 5) a single range
    written directly. Forcing 1, 3 and N ranges (1000 is clamped to N) here
    runs every one of those paths against the oracle."""
    inp = make_inputs(Workload("bwd_ranges", 1, 45, 128, 4, dtype, ("pad", 38), seed=88))
    check_backward(inp, 0.2, seed=17, offset=2, what=f"backward {dtype} {ranges} row ranges", dz_ranges=ranges)


def test_backward_row_range_setter_errors_and_workspace():
    inp = make_inputs(Workload("bwd_ranges_err", 1, 45, 64, 4, "f32", ("ones",), seed=89))
    g = Gpu(inp)
    try:
        with pytest.raises(B.TriAttnError) as e:
            B.tri_attn_set_backward_dz_ranges(g.handle, -1)
        assert e.value.code == B.TRI_ATTN_ERR_INVALID_ARG
        n_auto = B.tri_attn_backward_workspace_size(g.handle, 1, 45)
        B.tri_attn_set_backward_dz_ranges(g.handle, 1)
        n_one = B.tri_attn_backward_workspace_size(g.handle, 1, 45)
        B.tri_attn_set_backward_dz_ranges(g.handle, 5)
        n_five = B.tri_attn_backward_workspace_size(g.handle, 1, 45)
        # one range needs no partial sums; five ranges need five B*h*N*N float32 slices
        assert n_one < n_auto
        assert n_five - n_one >= 5 * 4 * 45 * 45 * 4
    finally:
        g.close()


@pytest.mark.parametrize("k", [1, 2, 3, 4])
def test_backward_workload(k):
    """Workloads 1-4 in full (B=2 N=32 D=64 h=4 f32; B=1 N=128 D=128 h=4 f32;
    B=1 N=256 D=128 h=4 bf16 with 16 padded residues; B=1 N=384 D=128 h=4
    bf16, Bernoulli mask), dropout 0.1."""
    w = WORKLOADS[k]
    log(f"backward {w.name}")
    check_backward(make_inputs(w), 0.1, seed=4242, offset=1, what=f"backward {w.name}")


def test_backward_workload5_sampled_positions():
    """Workload 5 (B=4 N=512 D=128 h=8 bf16, per-batch padding), the size and
    launch configuration the benchmark times, dropout 0.1: the whole
    backward runs on the GPU; dL/d(pair_repr) is compared with the
    position-sampled backward oracle at 24 positions (per batch: the first
    and the last valid position, a position in a padded row, one in a padded
    column, the last position, a random valid one). Each such gradient draws
    on every step of the backward: the gate, dq of its query column, dk and
    dv of its key, and the pair bias's gradient summed over all 512 rows.
    The parameter gradients are sums over all positions; at this size they
    are checked for finiteness (workloads 1-4 compare them in full), and the
    output bias's, which is the plain column sum of dy over every position,
    against that sum in float64."""
    w = WORKLOADS[5]
    inp = make_inputs(w)
    M = np.asarray(inp["pair_mask"])
    rng = np.random.default_rng(505)
    pos = []
    for b in range(w.B):
        L = int(M[b].any(axis=1).sum())  # valid length: rows and columns >= L are padding
        pos += [(b, 0, 0), (b, L - 1, L - 1), (b, min(L, w.N - 1), 3), (b, 7, min(L + 1, w.N - 1)),
                (b, w.N - 1, w.N - 1), (b, int(rng.integers(0, L)), int(rng.integers(0, L)))]
    log(f"backward {w.name}: GPU backward, then the oracle at {len(pos)} positions")
    dy = make_dy(inp, 99)
    got = run_backward(inp, dy, 0.1, 4242, 1)
    for k in SHAPE:
        assert np.isfinite(got[k]).all(), k
    dbo = dy.astype(np.float64).reshape(-1, w.D).sum(axis=0)
    err_bo = float(np.abs(got["d_b_out"] - dbo).max())
    log(f"backward {w.name} d_b_out against the column sums of dy: max abs err {err_bo:.3e}, "
        f"max |ref| {np.abs(dbo).max():.3e}")
    assert err_bo <= RTOL * float(np.abs(dbo).max())
    ref = BO.pair_repr_grad_at(inp, dy.astype(np.float64), 0.1, 4242, 1, pos)
    gk = np.stack([got["d_pair_repr"][p] for p in pos])
    scale = float(np.abs(ref).max())
    err = np.abs(gk - ref).max(axis=1)
    worst = int(err.argmax())
    log(f"backward {w.name} d_pair_repr at {len(pos)} positions: max abs err {err[worst]:.3e} at {pos[worst]}, "
        f"max |ref| {scale:.3e}, relative {err[worst] / scale:.2e}")
    assert err[worst] <= RTOL * scale, f"error {err[worst]} at {pos[worst]} > {RTOL} * {scale}"


@pytest.mark.parametrize("dtype,h", [("f32", 4), ("bf16", 8)])
def test_backward_ragged_several_blocks(dtype, h):
    """N = 300 with 30 padded residues (fully masked query columns): three
    128-key blocks in the dk/dv step and five 64-key chunks in the others,
    the last of each ragged; five 64 x 64 pair-bias tiles per side."""
    inp = make_inputs(Workload("bwd_n300", 1, 300, 128, h, dtype, ("pad", 270), seed=87))
    check_backward(inp, 0.2, seed=23, offset=4, what=f"backward N=300 {dtype} h={h}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape,mask", [((1, 2, 64, 4), ("ones",)), ((2, 3, 64, 2), ("pad", 2)),
                                        ((1, 5, 128, 8), ("bernoulli", 0.5))], ids=["N2", "B2N3pad", "N5bern"])
def test_backward_tiny(shape, mask, dtype):
    """Sizes far below one tile: two keys per row, a padded (fully masked)
    column among three, a sparse mask. (N = 1 is left out: a single key has
    weight 1 whatever its score, so the query, key and pair-bias gradients
    are exactly 0 only by cancellation, da * scale - D = 0; any float32
    evaluation returns rounding-level values there, which a bar relative to
    an exact 0 cannot take.)"""
    Bn, N, D, h = shape
    inp = make_inputs(Workload("bwd_tiny", Bn, N, D, h, dtype, mask, seed=90 + N))
    check_backward(inp, 0.25, seed=31, offset=2, what=f"backward tiny {dtype} {shape} {mask}")


def test_backward_minus_inf_fill():
    """-inf fill on a mask where every query column keeps a valid key."""
    inp = make_inputs(Workload("bwd_ninf", 1, 24, 64, 4, "f32", ("bernoulli", 0.7), seed=83))
    check_backward(inp, 0.2, seed=7, offset=0, what="backward -inf fill", fill=-math.inf)


def test_backward_deterministic():
    """Two calls give the same bits (fixed-order sums, no atomics)."""
    inp = make_inputs(Workload("bwd_det", 1, 40, 128, 4, "bf16", ("pad", 33), seed=84))
    dy = make_dy(inp, 5)
    a = run_backward(inp, dy, 0.2, 9, 0)
    b = run_backward(inp, dy, 0.2, 9, 0)
    for k in SHAPE:
        assert np.array_equal(a[k], b[k]), k


def test_backward_back_to_back_calls_on_one_workspace():
    """The keep bits are made on the handle's second stream: calls issued back
    to back on one stream and one workspace, with different seeds and no
    synchronisation between them, must each give the bits of a call made on
    its own (the fork orders a call's keep bits after the previous call's
    attention steps, the join orders its attention steps after them)."""
    inp = make_inputs(Workload("bwd_b2b", 1, 128, 128, 8, "bf16", ("pad", 100), seed=86))
    dy = make_dy(inp, 6)
    seeds = (9, 10, 9)
    alone = {sd: run_backward(inp, dy, 0.3, sd, 0) for sd in set(seeds)}
    g = Gpu(inp)
    try:
        n = B.tri_attn_backward_workspace_size(g.handle, g.B, g.N)
        ws = torch.empty(n, dtype=torch.uint8, device=g.dev)
        dyt = torch.from_numpy(dy).to(g.dev).to(g.dt).contiguous()
        outs = []
        for sd in seeds:
            grads = {k: torch.zeros(np.shape(inp[v]), dtype=torch.float32, device=g.dev) for k, v in SHAPE.items()}
            B.tri_attn_backward_train(g.handle, g.P, g.M, dyt, g.B, g.N, 0.3, sd, 0, grads, ws, n,
                                      torch.cuda.current_stream())
            outs.append(grads)
        torch.cuda.synchronize()
        for sd, grads in zip(seeds, outs):
            for k in SHAPE:
                assert np.array_equal(grads[k].double().cpu().numpy(), alone[sd][k]), (sd, k)
        log("back-to-back backward calls on one workspace: bit-identical to separate calls")
    finally:
        g.close()


def test_backward_captured_in_hip_graph():
    """The backward enqueues kernels and events only (no memsets, no
    allocation), its keep bits on the handle's second stream forked from and
    joined to the capturing stream, so it can be captured in a HIP graph;
    every replay, with eager backward calls of other seeds on the same
    workspace between replays, must equal the eager backward bit for bit."""
    inp = make_inputs(Workload("bwd_graph", 1, 64, 128, 4, "bf16", ("pad", 50), seed=87))
    dy = make_dy(inp, 7)
    eager = run_backward(inp, dy, 0.2, 21, 3)
    g = Gpu(inp)
    try:
        n = B.tri_attn_backward_workspace_size(g.handle, g.B, g.N)
        ws = torch.empty(n, dtype=torch.uint8, device=g.dev)
        dyt = torch.from_numpy(dy).to(g.dev).to(g.dt).contiguous()
        mk = lambda: {k: torch.zeros(np.shape(inp[v]), dtype=torch.float32, device=g.dev) for k, v in SHAPE.items()}
        grads, other = mk(), mk()
        call = lambda gr, sd, st: B.tri_attn_backward_train(g.handle, g.P, g.M, dyt, g.B, g.N, 0.2, sd, 3, gr, ws, n, st)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            call(grads, 21, side)  # warm-up on a side stream before capture
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            call(grads, 21, torch.cuda.current_stream())
        for r in range(3):
            for v in grads.values():
                v.fill_(float("nan"))
            graph.replay()
            torch.cuda.synchronize()
            for k in SHAPE:
                assert np.array_equal(grads[k].double().cpu().numpy(), eager[k]), (r, k)
            call(other, 22 + r, torch.cuda.current_stream())  # eager work between replays
            torch.cuda.synchronize()
        del graph
        log("backward captured in a HIP graph: every replay equals the eager backward")
    finally:
        g.close()


def test_backward_argument_errors():
    inp = make_inputs(Workload("bwd_err", 1, 8, 64, 4, "f32", ("ones",), seed=85))
    g = Gpu(inp)
    try:
        n = B.tri_attn_backward_workspace_size(g.handle, g.B, g.N)
        ws = torch.empty(n, dtype=torch.uint8, device=g.dev)
        grads = {k: torch.zeros(np.shape(inp[v]), dtype=torch.float32, device=g.dev) for k, v in SHAPE.items()}
        dy = torch.zeros_like(g.P)
        for rate in (1.0, -0.5, float("nan")):
            with pytest.raises(B.TriAttnError) as e:
                B.tri_attn_backward_train(g.handle, g.P, g.M, dy, g.B, g.N, rate, 1, 0, grads, ws, n)
            assert e.value.code == B.TRI_ATTN_ERR_INVALID_ARG
        with pytest.raises(B.TriAttnError) as e:
            B.tri_attn_backward_train(g.handle, g.P, g.M, dy, g.B, g.N, 0.1, 1, 0, grads, ws, n - 1)
        assert e.value.code == B.TRI_ATTN_ERR_WORKSPACE
        bad = dict(grads)
        bad["d_w_out"] = 0
        with pytest.raises(B.TriAttnError) as e:
            B.tri_attn_backward_train(g.handle, g.P, g.M, dy, g.B, g.N, 0.1, 1, 0, bad, ws, n)
        assert e.value.code == B.TRI_ATTN_ERR_INVALID_ARG
        B.tri_attn_backward_train(g.handle, 0, 0, 0, 0, g.N, 0.1, 1, 0, grads, 0, 0)  # B == 0: no-op
        torch.cuda.synchronize()
    finally:
        g.close()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape,mask", [((2, 20, 64, 4), ("bernoulli", 0.8)), ((1, 33, 128, 4), ("pad", 25)),
                                        ((1, 40, 128, 8), ("pad", 31))], ids=["B2N20", "N33pad", "N40h8"])
def test_backward_ending_node(shape, mask, dtype):
    """Ending-node handles: the ending-node forward is the starting-node one
    of the problem with both residue axes swapped (dropout counters
    included), so its gradients are the backward oracle's on the swapped
    pair_repr, mask and dy, with dL/d(pair_repr) swapped back and every
    parameter gradient unchanged."""
    Bn, N, D, h = shape
    inp = make_inputs(Workload("bwd_end", Bn, N, D, h, dtype, mask, seed=86 + N))
    dy = make_dy(inp, 98)
    got = run_backward(inp, dy, 0.25, 3, 1, ending=True)
    ref = BO.backward_train(O._transposed(inp), np.swapaxes(dy, 1, 2).astype(np.float64), 0.25, 3, 1)
    ref["d_pair_repr"] = np.swapaxes(ref["d_pair_repr"], 1, 2)
    for k in SHAPE:
        r, gk = ref[k], got[k]
        scale = float(np.abs(r).max())
        err = float(np.abs(gk - r).max())
        log(f"backward ending {dtype} {shape} {k}: max abs err {err:.3e}, relative {err / scale:.2e}")
        assert err <= RTOL * scale + 1e-12, k
