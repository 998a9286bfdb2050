"""Pins for the CPU oracle, independent of its own code.

Each test checks the oracle against something it does not share code with:
library routines on special cases (torch LayerNorm, torch scaled-dot-product
attention, torch Linear), closed forms, invariants of the definition, and a
brute-force scalar evaluation of the per-element formula on tiny inputs.
The last group plants the index mistakes the FW-GLM-5-1 l2_p6 transcript made
(bias and mask indexed by the row, LayerNorm over the wrong extent, output
projection reading one value, -inf fill on fully masked columns) into the
oracle and checks that the pins catch each of them.
"""

import itertools
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle.tri_attn_oracle as O
from workloads import Workload, make_inputs, round_to_bf16

WEIGHTS = ("ln_weight", "ln_bias", "w_query", "w_key", "w_value", "w_gate", "b_gate",
           "w_bias_proj", "w_out", "b_out")


def small(B=2, N=5, D=8, h=2, mask=("bernoulli", 0.7), seed=7, dtype="f32"):
    return make_inputs(Workload("t", B, N, D, h, dtype, mask, seed))


def t64(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float64))


# ------------------------------------------------------------------ independent torch pipeline
def torch_pipeline(inp, fill=O.MASK_FILL):
    """The method assembled from torch library calls in float64, batched over
    all rows at once with scaled_dot_product_attention doing steps (5)-(7).

    The pair bias and the mask enter SDPA as one additive (B, 1, h, N, N)
    float mask broadcast over rows. Masked entries get -inf added, which equals
    replacement by a very negative FILL on every query column with at least one
    valid key (the callers only use such masks).
    """
    P = t64(inp["pair_repr"])
    B, N, _, D = P.shape
    h = inp["num_heads"]
    d = D // h
    w = {k: t64(inp[k]) for k in WEIGHTS}
    x = F.layer_norm(P, (D,), w["ln_weight"], w["ln_bias"], eps=O.LN_EPS)
    g = torch.sigmoid(F.linear(x, w["w_gate"], w["b_gate"]))
    z = F.linear(x, w["w_bias_proj"]).permute(0, 3, 1, 2)  # (B, h, j, k)

    def heads(t):  # (B, i, j, D) -> (B, i, h, j, d)
        return t.unflatten(-1, (h, d)).transpose(2, 3)

    q = heads(F.linear(x, w["w_query"]))
    k = heads(F.linear(x, w["w_key"]))
    v = heads(F.linear(x, w["w_value"]))
    m = torch.from_numpy(np.asarray(inp["pair_mask"])).bool()  # (B, j, k)
    add = z[:, None] + torch.where(m, 0.0, -math.inf).to(torch.float64)[:, None, None]
    o = F.scaled_dot_product_attention(q, k, v, attn_mask=add)  # (B, i, h, j, d)
    o = o.transpose(2, 3).flatten(-2)
    return F.linear(g * o, w["w_out"], w["b_out"]).numpy()


# ------------------------------------------------------------------ scalar brute force
def brute_force(inp, fill=O.MASK_FILL):
    """Per-element formula with Python loops and math.exp (tiny shapes only)."""
    P = np.asarray(inp["pair_repr"], dtype=np.float64)
    M = np.asarray(inp["pair_mask"])
    B, N, _, D = P.shape
    h = inp["num_heads"]
    d = D // h
    W = {k: np.asarray(inp[k], dtype=np.float64) for k in WEIGHTS}
    x = np.zeros_like(P)
    for b, i, j in itertools.product(range(B), range(N), range(N)):
        mu = sum(P[b, i, j, c] for c in range(D)) / D
        var = sum((P[b, i, j, c] - mu) ** 2 for c in range(D)) / D
        for c in range(D):
            x[b, i, j, c] = (P[b, i, j, c] - mu) / math.sqrt(var + O.LN_EPS) * W["ln_weight"][c] + W["ln_bias"][c]

    def dot(wrow, vec):
        return sum(wrow[e] * vec[e] for e in range(D))

    y = np.zeros_like(P)
    for b, i in itertools.product(range(B), range(N)):
        q = [[dot(W["w_query"][c], x[b, i, j]) for c in range(D)] for j in range(N)]
        kk = [[dot(W["w_key"][c], x[b, i, j]) for c in range(D)] for j in range(N)]
        v = [[dot(W["w_value"][c], x[b, i, j]) for c in range(D)] for j in range(N)]
        for j in range(N):
            g = [1.0 / (1.0 + math.exp(-(dot(W["w_gate"][c], x[b, i, j]) + W["b_gate"][c]))) for c in range(D)]
            o = [0.0] * D
            for t in range(h):
                s = []
                for k_ in range(N):
                    if M[b, j, k_] == 0:
                        s.append(fill)
                        continue
                    qk = sum(q[j][t * d + u] * kk[k_][t * d + u] for u in range(d)) / math.sqrt(d)
                    s.append(qk + dot(W["w_bias_proj"][t], x[b, j, k_]))
                mx = max(s)
                e = [math.exp(sv - mx) for sv in s]
                tot = sum(e)
                for u in range(d):
                    o[t * d + u] = sum(e[k_] / tot * v[k_][t * d + u] for k_ in range(N))
            for c in range(D):
                y[b, i, j, c] = sum(W["w_out"][c][e] * g[e] * o[e] for e in range(D)) + W["b_out"][c]
    return y


def brute_force_ending(inp, fill=O.MASK_FILL):
    """Ending-node per-element formula with Python loops (tiny shapes only):
    position (i, j) attends over k with q[i,j].k[k,j]/sqrt(d) + Wz[t].x[k,i],
    FILL where mask[k,i] == 0, values v[k,j]."""
    P = np.asarray(inp["pair_repr"], dtype=np.float64)
    M = np.asarray(inp["pair_mask"])
    B, N, _, D = P.shape
    h = inp["num_heads"]
    d = D // h
    W = {k: np.asarray(inp[k], dtype=np.float64) for k in WEIGHTS}
    x = np.zeros_like(P)
    for b, i, j in itertools.product(range(B), range(N), range(N)):
        mu = sum(P[b, i, j, c] for c in range(D)) / D
        var = sum((P[b, i, j, c] - mu) ** 2 for c in range(D)) / D
        for c in range(D):
            x[b, i, j, c] = (P[b, i, j, c] - mu) / math.sqrt(var + O.LN_EPS) * W["ln_weight"][c] + W["ln_bias"][c]

    def dot(wrow, vec):
        return sum(wrow[e] * vec[e] for e in range(D))

    y = np.zeros_like(P)
    for b, i, j in itertools.product(range(B), range(N), range(N)):
        q = [dot(W["w_query"][c], x[b, i, j]) for c in range(D)]
        g = [1.0 / (1.0 + math.exp(-(dot(W["w_gate"][c], x[b, i, j]) + W["b_gate"][c]))) for c in range(D)]
        kk = [[dot(W["w_key"][c], x[b, k_, j]) for c in range(D)] for k_ in range(N)]
        v = [[dot(W["w_value"][c], x[b, k_, j]) for c in range(D)] for k_ in range(N)]
        o = [0.0] * D
        for t in range(h):
            s = []
            for k_ in range(N):
                if M[b, k_, i] == 0:
                    s.append(fill)
                    continue
                qk = sum(q[t * d + u] * kk[k_][t * d + u] for u in range(d)) / math.sqrt(d)
                s.append(qk + dot(W["w_bias_proj"][t], x[b, k_, i]))
            mx = max(s)
            e = [math.exp(sv - mx) for sv in s]
            tot = sum(e)
            for u in range(d):
                o[t * d + u] = sum(e[k_] / tot * v[k_][t * d + u] for k_ in range(N))
        for c in range(D):
            y[b, i, j, c] = sum(W["w_out"][c][e] * g[e] * o[e] for e in range(D)) + W["b_out"][c]
    return y


# ================================================================== library special cases
def test_layer_norm_matches_torch():
    inp = small(B=2, N=4, D=16)
    x = O.layer_norm(inp["pair_repr"], inp["ln_weight"], inp["ln_bias"])
    ref = F.layer_norm(t64(inp["pair_repr"]), (16,), t64(inp["ln_weight"]), t64(inp["ln_bias"]), eps=1e-5)
    np.testing.assert_allclose(x, ref.numpy(), rtol=0, atol=1e-13)


def test_layer_norm_per_element_moments():
    """mean_c((x-beta)/gamma) = 0 and mean_c(((x-beta)/gamma)^2) = var/(var+eps)."""
    inp = small(B=1, N=3, D=32)
    p = inp["pair_repr"].astype(np.float64) * 0.05  # small variance makes eps visible
    x = O.layer_norm(p, inp["ln_weight"], inp["ln_bias"])
    xh = (x - inp["ln_bias"]) / inp["ln_weight"]
    var = p.var(axis=-1)
    np.testing.assert_allclose(xh.mean(-1), 0.0, atol=1e-13)
    np.testing.assert_allclose((xh ** 2).mean(-1), var / (var + 1e-5), rtol=1e-12)


def test_constant_pair_repr_gives_beta():
    inp = small(B=1, N=3, D=8)
    p = np.broadcast_to(np.arange(9, dtype=np.float64).reshape(1, 3, 3, 1), (1, 3, 3, 8))
    x = O.layer_norm(p, inp["ln_weight"], inp["ln_bias"])
    np.testing.assert_array_equal(x, np.broadcast_to(inp["ln_bias"].astype(np.float64), x.shape))


@pytest.mark.parametrize("mask", [("ones",), ("bernoulli", 0.6), ("pad", 4)])
@pytest.mark.parametrize("shape", [(2, 5, 8, 2), (1, 7, 12, 3), (2, 6, 16, 4)])
def test_matches_torch_sdpa_pipeline(mask, shape):
    """The whole forward against torch LayerNorm + Linear + SDPA with the bias
    and mask as an additive float mask (every query column keeps a valid key)."""
    B, N, D, h = shape
    inp = small(B=B, N=N, D=D, h=h, mask=mask, seed=11 + N)
    M = inp["pair_mask"]
    if mask[0] == "pad":  # keep only queries with a valid key for the -inf SDPA form
        M[:, 4:, :] = 1
    assert (M.max(axis=-1) == 1).all()
    np.testing.assert_allclose(O.forward(inp), torch_pipeline(inp), rtol=0, atol=1e-12)


def test_sdpa_textbook_case_no_bias_no_mask():
    """Wz = 0 and mask = 1: each (b, i, head) is plain scaled-dot-product
    attention over the row; compare the oracle's o with torch SDPA directly."""
    inp = small(B=2, N=6, D=8, h=2, mask=("ones",))
    inp["w_bias_proj"][:] = 0
    cap = {}
    O.forward(inp, capture=cap)
    q, k, v = (t64(cap[n]) for n in ("q", "k", "v"))  # (B*N, h, N, d)
    ref = F.scaled_dot_product_attention(q, k, v)
    np.testing.assert_allclose(O.split_heads(cap["o"], 2), ref.numpy(), rtol=0, atol=1e-13)


# ================================================================== brute force
@pytest.mark.parametrize("fill", [O.MASK_FILL, -1e4])
@pytest.mark.parametrize("shape,mask", [((1, 3, 4, 2), ("bernoulli", 0.6)),
                                        ((2, 3, 6, 3), ("pad", 2)),
                                        ((1, 4, 4, 1), ("bernoulli", 0.5))])
def test_brute_force_tiny_ending_node(shape, mask, fill):
    B, N, D, h = shape
    inp = small(B=B, N=N, D=D, h=h, mask=mask, seed=5 + D)
    np.testing.assert_allclose(O.forward_ending(inp, fill=fill), brute_force_ending(inp, fill=fill), rtol=0,
                               atol=1e-12)


def test_ending_node_columns_and_difference():
    """forward_ending_cols gives columns of forward_ending; on a generic input
    the ending-node output differs from the starting-node one."""
    inp = small(B=2, N=5, D=8, h=2, mask=("bernoulli", 0.7), seed=21)
    y = O.forward_ending(inp)
    cols = [(0, 1), (1, 4)]
    np.testing.assert_allclose(O.forward_ending_cols(inp, cols), np.stack([y[b, :, j] for b, j in cols]),
                               rtol=0, atol=1e-13)
    assert np.abs(y - O.forward(inp)).max() > 1e-3


@pytest.mark.parametrize("fill", [O.MASK_FILL, -1e4])
@pytest.mark.parametrize("shape,mask", [((1, 3, 4, 2), ("bernoulli", 0.6)),
                                        ((2, 3, 6, 3), ("pad", 2)),
                                        ((1, 4, 4, 1), ("bernoulli", 0.5))])
def test_brute_force_tiny(shape, mask, fill):
    B, N, D, h = shape
    inp = small(B=B, N=N, D=D, h=h, mask=mask, seed=3 + D)
    np.testing.assert_allclose(O.forward(inp, fill=fill), brute_force(inp, fill=fill), rtol=0, atol=1e-12)


# ================================================================== closed forms
def test_zero_value_weight_gives_output_bias():
    inp = small()
    inp["w_value"][:] = 0
    y = O.forward(inp)
    np.testing.assert_array_equal(y, np.broadcast_to(inp["b_out"].astype(np.float64), y.shape))


def test_single_residue():
    """N = 1: the only weight is 1, so y = Wo (g * v) + bo."""
    inp = small(B=3, N=1, D=8, h=2, mask=("ones",))
    x = O.layer_norm(inp["pair_repr"], inp["ln_weight"], inp["ln_bias"])
    w = {k: np.asarray(inp[k], np.float64) for k in WEIGHTS}
    g = 1 / (1 + np.exp(-(np.einsum("bijd,cd->bijc", x, w["w_gate"]) + w["b_gate"])))
    v = np.einsum("bijd,cd->bijc", x, w["w_value"])
    ref = np.einsum("bijd,cd->bijc", g * v, w["w_out"]) + w["b_out"]
    np.testing.assert_allclose(O.forward(inp), ref, rtol=0, atol=1e-13)


def test_uniform_weights_over_valid_keys():
    """Wq = 0 and Wz = 0: every valid key gets weight 1/(number of valid keys)."""
    inp = small(B=2, N=6, D=8, h=2, mask=("bernoulli", 0.5))
    inp["w_query"][:] = 0
    inp["w_bias_proj"][:] = 0
    cap = {}
    O.forward(inp, capture=cap)
    M = inp["pair_mask"].astype(np.float64)  # (B, j, k)
    N = 6
    for r in range(2 * N):
        b = r // N
        expect = M[b] / M[b].sum(-1, keepdims=True)
        for t in range(2):
            np.testing.assert_allclose(cap["a"][r, t], expect, atol=1e-15)


def test_fully_masked_column_gets_mean_of_all_values():
    """Reading of FILL: with the -1e9 replacement, a query column with no valid
    key attends uniformly to all N keys (padded ones included)."""
    inp = small(B=1, N=5, D=8, h=2, mask=("pad", 3))
    cap = {}
    O.forward(inp, capture=cap)
    for r in range(5):
        for j in (3, 4):  # fully masked query columns
            np.testing.assert_allclose(cap["a"][r, :, j, :], 0.2, atol=1e-15)
            np.testing.assert_allclose(cap["o"][r, j], O.merge_heads(cap["v"][r].mean(axis=1, keepdims=True))[0],
                                       atol=1e-13)


def test_minus_inf_fill_gives_nan_on_fully_masked_columns_only():
    inp = small(B=1, N=5, D=8, h=2, mask=("pad", 3))
    y_inf = O.forward(inp, fill=-np.inf)
    y_fin = O.forward(inp)
    assert np.isnan(y_inf[:, :, 3:]).all()
    np.testing.assert_allclose(y_inf[:, :, :3], y_fin[:, :, :3], atol=1e-13)


# ================================================================== invariants
def test_softmax_rows_sum_to_one_and_masked_keys_get_zero():
    inp = small(B=2, N=7, D=8, h=2, mask=("bernoulli", 0.6))
    cap = {}
    O.forward(inp, capture=cap)
    a = cap["a"]  # (B*N, h, N, N)
    np.testing.assert_allclose(a.sum(-1), 1.0, atol=1e-12)
    M = inp["pair_mask"]
    for r in range(a.shape[0]):
        b = r // 7
        assert (a[r][:, M[b] == 0] == 0).all()


def test_residue_permutation_equivariance():
    """One permutation of all residue axes: P'[b,i,j] = P[b,pi(i),pi(j)] and
    M'[b,j,k] = M[b,pi(j),pi(k)] give y'[b,i,j] = y[b,pi(i),pi(j)]."""
    inp = small(B=2, N=6, D=8, h=2, mask=("bernoulli", 0.6))
    pi = np.random.default_rng(0).permutation(6)
    inp2 = dict(inp)
    inp2["pair_repr"] = inp["pair_repr"][:, pi][:, :, pi]
    inp2["pair_mask"] = inp["pair_mask"][:, pi][:, :, pi]
    y = O.forward(inp)
    np.testing.assert_allclose(O.forward(inp2), y[:, pi][:, :, pi], atol=1e-12)


def test_row_permutation_with_fixed_bias():
    """With the pair bias off (Wz = 0), permuting the rows i of pair_repr
    permutes the output rows: rows attend independently of each other."""
    inp = small(B=1, N=6, D=8, h=2, mask=("bernoulli", 0.6))
    inp["w_bias_proj"][:] = 0
    pi = np.random.default_rng(1).permutation(6)
    inp2 = dict(inp)
    inp2["pair_repr"] = inp["pair_repr"][:, pi]
    np.testing.assert_allclose(O.forward(inp2), O.forward(inp)[:, pi], atol=1e-12)


def test_batch_permutation_equivariance():
    inp = small(B=3, N=4, D=8, h=2)
    pi = np.array([2, 0, 1])
    inp2 = dict(inp)
    inp2["pair_repr"] = inp["pair_repr"][pi]
    inp2["pair_mask"] = inp["pair_mask"][pi]
    np.testing.assert_allclose(O.forward(inp2), O.forward(inp)[pi], atol=1e-13)


def test_forward_rows_matches_forward():
    inp = small(B=2, N=6, D=8, h=2)
    y = O.forward(inp)
    rows = [(1, 5), (0, 0), (1, 2)]
    np.testing.assert_array_equal(O.forward_rows(inp, rows), np.stack([y[b, i] for b, i in rows]))


# ================================================================== generator
def test_bf16_rounding_matches_torch():
    a = np.random.default_rng(5).standard_normal(10000).astype(np.float32) * 10
    a[:4] = [1.00390625, 1.01171875, -1.00390625, 3.0]  # exact ties
    ref = torch.from_numpy(a).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(round_to_bf16(a), ref)


def test_workload_masks():
    from workloads import WORKLOADS
    w5 = WORKLOADS[5].replace(N=16, B=6, mask=("pad_range", 9, 16))
    m = make_inputs(w5)["pair_mask"]
    for b in range(6):
        L = int(m[b].diagonal().sum())
        assert 9 <= L <= 16
        assert (m[b, :L, :L] == 1).all() and m[b, L:].sum() == 0 and m[b, :, L:].sum() == 0
    m1 = make_inputs(WORKLOADS[1])["pair_mask"]
    assert (m1[:, np.arange(32), np.arange(32)] == 1).all()
    assert 0.85 < m1.mean() < 0.95
    m3 = make_inputs(WORKLOADS[3].replace(N=256))["pair_mask"]
    assert m3[0, :240, :240].all() and m3[0, 240:].sum() == 0


def test_generator_is_deterministic_and_bf16_exact():
    from workloads import WORKLOADS
    w = WORKLOADS[3].replace(N=8)
    a, b = make_inputs(w), make_inputs(w)
    for k in a:
        if isinstance(a[k], np.ndarray):
            np.testing.assert_array_equal(a[k], b[k])
            if a[k].dtype == np.float32:
                np.testing.assert_array_equal(round_to_bf16(a[k]), a[k])


# ================================================================== planted mistakes
MUTANTS = {}


def mutant(name):
    def deco(fn):
        MUTANTS[name] = fn
        return fn
    return deco


@mutant("MT1_bias_indexed_by_row")
def _mt1(monkeypatch):
    monkeypatch.setattr(O, "row_bias", lambda z_b, i: np.broadcast_to(z_b[:, i:i + 1, :], z_b.shape))


@mutant("MT2_mask_indexed_by_row")
def _mt2(monkeypatch):
    monkeypatch.setattr(O, "row_mask", lambda m_b, i: np.broadcast_to(m_b[i:i + 1, :], m_b.shape))


@mutant("MT3_layernorm_wrong_extent")
def _mt3(monkeypatch):
    def ln(p, gamma, beta, eps=O.LN_EPS):
        p = np.asarray(p, np.float64)
        mu = p.mean(axis=(-2, -1), keepdims=True)
        var = ((p - mu) ** 2).mean(axis=(-2, -1), keepdims=True)
        return (p - mu) / np.sqrt(var + eps) * gamma + beta
    monkeypatch.setattr(O, "layer_norm", ln)


@mutant("MT4_out_proj_one_value")
def _mt4(monkeypatch):
    monkeypatch.setattr(O, "output_projection",
                        lambda go, w, b: O.linear(np.broadcast_to(go[..., :1], go.shape), w, b))


@mutant("MT5_minus_inf_fill")
def _mt5(monkeypatch):
    orig = O.apply_mask
    monkeypatch.setattr(O, "apply_mask", lambda s, m, fill=O.MASK_FILL: orig(s, m, -np.inf))


@mutant("transposed_scores")
def _mt6(monkeypatch):
    orig = O.row_scores
    monkeypatch.setattr(O, "row_scores", lambda q, k, z: np.swapaxes(orig(q, k, np.swapaxes(z, -1, -2)), -1, -2))


@mutant("no_score_scale")
def _mt7(monkeypatch):
    monkeypatch.setattr(O, "row_scores", lambda q, k, z: q @ np.swapaxes(k, -1, -2) + z)


def _pins_pass():
    """Run the cheap pins; return False as soon as one detects a difference."""
    checks = []
    inp = small(B=2, N=5, D=8, h=2, mask=("bernoulli", 0.6), seed=21)
    inp["pair_mask"][:, np.arange(5), np.arange(5)] = 1
    checks.append(lambda: np.allclose(O.forward(inp), torch_pipeline(inp), atol=1e-10))
    pad = small(B=1, N=5, D=8, h=2, mask=("pad", 3), seed=22)

    def fully_masked_uniform():
        cap = {}
        y = O.forward(pad, capture=cap)
        return np.isfinite(y).all() and np.allclose(cap["a"][:, :, 3:, :], 0.2)
    checks.append(fully_masked_uniform)
    tiny = small(B=1, N=3, D=4, h=2, mask=("bernoulli", 0.6), seed=23)
    checks.append(lambda: np.allclose(O.forward(tiny), brute_force(tiny), atol=1e-10))
    for c in checks:
        with np.errstate(all="ignore"):
            if not c():
                return False
    return True


def test_pins_pass_on_the_oracle():
    assert _pins_pass()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, monkeypatch):
    MUTANTS[name](monkeypatch)
    assert not _pins_pass(), f"planted mistake {name} went undetected"
