"""GPU parity of the training-mode forward (tri_attn_forward_train) with the
training oracle: the same dropout decisions (integers, compared through the
outputs they select), y within the inference tolerances, and the saved
log-sum-exp."""
import math

import numpy as np
import pytest
import torch

from gpu_helpers import TOL, Gpu, log, max_err, y_numpy
from oracle import pool
from oracle import tri_attn_oracle as O
from oracle import tri_attn_train_oracle as TO
from triangular_pair_attention_amd import binding as B
from workloads import WORKLOADS, Workload, make_inputs

pytestmark = pytest.mark.gpu

LSE_TOL = {"f32": 1e-4, "bf16": 5e-2}  # on columns with a valid key (|lse| of order 10)


def run_train(inp, rate, seed, offset, fill=O.MASK_FILL):
    g = Gpu(inp, fill=fill)
    try:
        h = g.h
        lse = torch.empty((g.B, g.N, h, g.N), dtype=torch.float32, device=g.dev)
        out = torch.empty_like(g.P)
        B.tri_attn_forward_train(g.handle, g.P, g.M, out, lse, g.B, g.N, rate, seed, offset, g.ws, g.ws_bytes,
                                 torch.cuda.current_stream())
        torch.cuda.synchronize()
        return y_numpy(out), lse.double().cpu().numpy(), y_numpy(g.forward())
    finally:
        g.close()


def check_train(inp, rate, seed, offset, what, fill=O.MASK_FILL):
    dtype = inp["dtype"]
    y, lse, y_inf = run_train(inp, rate, seed, offset, fill)
    ref, ref_lse = TO.forward_train(inp, rate, seed, offset, fill=fill)
    fin = np.isfinite(ref)
    assert (np.isfinite(y) == fin).all(), f"{what}: NaN pattern of y differs"
    err, idx = max_err(np.where(fin, y, 0), np.where(fin, ref, 0))
    log(f"{what}: y max abs err {err:.3e} at {idx}")
    assert err <= TOL[dtype], f"{what}: y error {err}"
    live = np.asarray(inp["pair_mask"]).any(-1)  # (b, j): the column has a valid key
    live = np.broadcast_to(live[:, None, None, :], ref_lse.shape)
    lerr = float(np.abs(lse - ref_lse)[live].max()) if live.any() else 0.0
    log(f"{what}: lse max abs err {lerr:.3e} on columns with a valid key")
    assert lerr <= LSE_TOL[dtype]
    dead = ~live
    if dead.any():
        if math.isfinite(fill):
            np.testing.assert_allclose(lse[dead], ref_lse[dead], rtol=1e-6)
        else:
            assert np.isnan(lse[dead]).all()
    return y, y_inf


SHAPES = [((2, 40, 64, 4), ("bernoulli", 0.8)), ((1, 70, 128, 4), ("pad", 50)),
          ((1, 66, 128, 8), ("pad", 60)), ((2, 37, 128, 4), ("bernoulli", 0.6)), ((1, 5, 64, 2), ("pad", 3))]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("shape,mask", SHAPES, ids=lambda s: str(s))
@pytest.mark.parametrize("rate", [0.0, 0.3])
def test_train_small(shape, mask, dtype, rate):
    Bn, N, D, h = shape
    inp = make_inputs(Workload("train", Bn, N, D, h, dtype, mask, seed=71))
    y, y_inf = check_train(inp, rate, seed=2**33 + 5, offset=7, what=f"train {dtype} {shape} {mask} rate {rate}")
    if rate == 0.0:
        # no weight dropped: the inference forward's output, within both tolerances
        assert np.abs(y - y_inf)[np.isfinite(y)].max() <= 2 * TOL[dtype]


@pytest.mark.parametrize("k", [2, 3])
def test_train_workload(k):
    w = WORKLOADS[k]
    log(f"train {w.name}")
    check_train(make_inputs(w), 0.15, seed=12345, offset=0, what=f"train {w.name}")


def check_train_pool(inp, rows, rate, seed, offset, what):
    """The training forward (y and lse) on the listed rows against the
    training oracle, the rows spread over host worker processes."""
    dtype = inp["dtype"]
    y, lse, _ = run_train(inp, rate, seed, offset)
    r = pool.compare_rows(inp, y.astype(np.float32), rows, train={"rate": rate, "seed": seed, "offset": offset},
                          lse=lse.astype(np.float32))
    log(f"{what}: y max abs err {r['y']['max_abs_err']:.3e} at {r['y']['where']}; lse max abs err "
        f"{r['lse']['max_abs_err']:.3e} on columns with a valid key, max rel err "
        f"{r['lse_dead_rel']['max_abs_err']:.1e} on fully masked ones")
    assert r["y"]["same_nan_pattern"] and r["lse"]["same_nan_pattern"]
    assert r["y"]["max_abs_err"] <= TOL[dtype]
    assert r["lse"]["max_abs_err"] <= LSE_TOL[dtype]
    assert r["lse_dead_rel"]["max_abs_err"] <= 1e-6


def test_train_workload4_full():
    """B=1, N=384, h=4 (d = 32): every row, so the attention kernel's second
    256-column query block of each row is compared too."""
    w = WORKLOADS[4]
    log(f"train {w.name}: all rows (worker processes)")
    check_train_pool(make_inputs(w), [(0, i) for i in range(w.N)], 0.1, 777, 3, f"train {w.name}")


def test_train_workload5_full():
    """B=4, N=512, h=8 (d = 16): all 2048 rows (every column and head of
    each, y and lse), the rows spread over host worker processes."""
    w = WORKLOADS[5]
    rows = [(b, i) for b in range(w.B) for i in range(w.N)]
    log(f"train {w.name}: all {len(rows)} rows (worker processes)")
    check_train_pool(make_inputs(w), rows, 0.1, 2**40 + 17, 0, f"train {w.name}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_train_ragged_300(dtype):
    """N = 300, padded to 270, head size 32: two 256-column query blocks per
    row (the second ragged), dropout 0.2, every row."""
    w = Workload("train300", 1, 300, 128, 4, dtype, ("pad", 270), seed=75)
    log(f"train N=300 {dtype}")
    check_train_pool(make_inputs(w), [(0, i) for i in range(w.N)], 0.2, 5, 1, f"train N=300 {dtype}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_train_minus_inf_fill(dtype):
    inp = make_inputs(Workload("train", 1, 20, 64, 4, dtype, ("pad", 14), seed=72))
    check_train(inp, 0.25, seed=3, offset=1, what=f"train -inf fill {dtype}", fill=-math.inf)


def test_train_argument_errors():
    inp = make_inputs(Workload("train", 1, 8, 64, 4, "f32", ("ones",), seed=73))
    g = Gpu(inp)
    try:
        out = torch.empty_like(g.P)
        for bad in (1.0, -0.1, float("nan")):
            rc = B.raw_call("tri_attn_forward_train", g.handle, g.P.data_ptr(), g.M.data_ptr(), out.data_ptr(), None,
                            g.B, g.N, B.ctypes.c_double(bad), B.ctypes.c_uint64(1), B.ctypes.c_uint32(0),
                            g.ws.data_ptr(), g.ws_bytes, None)
            assert rc == B.TRI_ATTN_ERR_INVALID_ARG
    finally:
        g.close()


@pytest.mark.parametrize("dtype,shape,mask", [("f32", (2, 40, 64, 4), ("bernoulli", 0.8)),
                                              ("bf16", (1, 70, 128, 4), ("pad", 50)),
                                              ("f32", (1, 66, 128, 8), ("pad", 60))])
def test_train_ending_node(dtype, shape, mask):
    """Ending-node handles: the transposed problem's decisions and lse."""
    Bn, N, D, h = shape
    inp = make_inputs(Workload("train_end", Bn, N, D, h, dtype, mask, seed=74))
    e = Gpu(inp, ending=True)
    try:
        lse = torch.empty((e.B, e.N, e.h, e.N), dtype=torch.float32, device=e.dev)
        out = torch.empty_like(e.P)
        B.tri_attn_forward_train(e.handle, e.P, e.M, out, lse, e.B, e.N, 0.3, 99, 5, e.ws, e.ws_bytes,
                                 torch.cuda.current_stream())
        torch.cuda.synchronize()
        y, lse = y_numpy(out), lse.double().cpu().numpy()
    finally:
        e.close()
    ref, ref_lse = TO.forward_train_ending(inp, 0.3, 99, 5)
    err, idx = max_err(y, ref)
    log(f"train ending node {dtype} {shape}: y max abs err {err:.3e} at {idx}")
    assert err <= TOL[dtype]
    live = np.swapaxes(np.asarray(inp["pair_mask"]), 1, 2).any(-1)  # the transposed problem's columns
    live = np.broadcast_to(live[:, None, None, :], ref_lse.shape)
    assert np.abs(lse - ref_lse)[live].max() <= LSE_TOL[dtype]
