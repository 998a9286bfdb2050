"""Pins for the backward oracle (gradients of the training-mode forward),
independent of its own code.

* Central finite differences in float64 of L = sum(dy * y), with y from the
  training forward oracle (a row-by-row formulation the backward does not
  use), for every element of pair_repr and of every parameter, on tiny
  inputs with a partly masked and a fully masked query column.
* torch autograd (float64) on a torch transcription of the forward written
  here, with the dropout decisions taken from the forward oracle.
* Planted mistakes in a copy of the backward oracle (the pair bias's
  gradient from one row instead of the sum over rows; the dropout mask left
  out of the backward) that the finite-difference pin must reject.
* The position-sampled form (pair_repr_grad_at, for sizes where the whole
  backward does not fit in memory) equals the whole backward's
  dL/d(pair_repr) at every position of small inputs: padding with fully
  masked columns, Bernoulli masks, the -inf fill, both dtypes' inputs.
"""
import math

import numpy as np
import pytest
import torch

import oracle.tri_attn_oracle as O
import oracle.tri_attn_train_oracle as TO
from oracle.tri_attn_backward_oracle import backward_train, pair_repr_grad_at
from workloads import Workload, make_inputs

backward_train_ref = backward_train  # restored after the planted-mistake tests

NAMES = ("pair_repr", "ln_weight", "ln_bias", "w_query", "w_key", "w_value", "w_gate", "b_gate",
         "w_bias_proj", "w_out", "b_out")


def tiny(B=1, N=3, D=4, h=2, mask=("pad", 2), seed=31):
    inp = make_inputs(Workload("t", B, N, D, h, "f32", mask, seed))
    return {k: (v.astype(np.float64) if isinstance(v, np.ndarray) and k != "pair_mask" else v)
            for k, v in inp.items()}


def loss(inp, dy, rate, seed, offset=0):
    y, _ = TO.forward_train(inp, rate, seed, offset)
    return float((dy * y).sum())


@pytest.mark.parametrize("rate,mask", [(0.3, ("pad", 2)), (0.0, ("bernoulli", 0.6)), (0.5, ("ones",))])
def test_finite_differences(rate, mask):
    inp = tiny(mask=mask)
    rng = np.random.default_rng(4)
    dy = rng.standard_normal(np.shape(inp["pair_repr"]))
    cap = {}
    gr = backward_train(inp, dy, rate, seed=9, capture=cap)
    y, _ = TO.forward_train(inp, rate, 9)
    np.testing.assert_allclose(cap["y"], y, rtol=0, atol=1e-12)
    eps = 1e-5
    for name in NAMES:
        base = inp[name]
        num = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            plus, minus = dict(inp), dict(inp)
            plus[name] = base.copy()
            minus[name] = base.copy()
            plus[name][idx] += eps
            minus[name][idx] -= eps
            num[idx] = (loss(plus, dy, rate, 9) - loss(minus, dy, rate, 9)) / (2 * eps)
        np.testing.assert_allclose(gr["d_" + name], num, rtol=1e-6, atol=1e-7, err_msg=name)


def torch_forward(w, M, keep, scale, h, fill=O.MASK_FILL):
    """The forward in torch float64 ops, batched over rows, dropout mask given."""
    P = w["pair_repr"]
    B, N, _, D = P.shape
    d = D // h
    x = torch.nn.functional.layer_norm(P, (D,), w["ln_weight"], w["ln_bias"], eps=O.LN_EPS)
    g = torch.sigmoid(x @ w["w_gate"].T + w["b_gate"])
    split = lambda t: t.reshape(B, N, N, h, d).permute(0, 1, 3, 2, 4)  # noqa: E731
    q, k, v = split(x @ w["w_query"].T), split(x @ w["w_key"].T), split(x @ w["w_value"].T)
    z = (x @ w["w_bias_proj"].T).permute(0, 3, 1, 2)  # (b, t, j, k)
    s = q @ k.transpose(-1, -2) / math.sqrt(d) + z.unsqueeze(1)
    s = s.masked_fill(M.unsqueeze(1).unsqueeze(1) == 0, fill)
    a = torch.softmax(s, dim=-1) * keep * scale
    o = (a @ v).permute(0, 1, 3, 2, 4).reshape(B, N, N, D)
    return (g * o) @ w["w_out"].T + w["b_out"]


@pytest.mark.parametrize("rate", [0.0, 0.25])
def test_torch_autograd(rate):
    inp = tiny(B=2, N=6, D=8, h=2, mask=("pad", 4), seed=41)
    B, N, _, D = inp["pair_repr"].shape
    h = inp["num_heads"]
    dy = np.random.default_rng(5).standard_normal((B, N, N, D))
    gr = backward_train(inp, dy, rate, seed=17, offset=2)
    w = {n: torch.tensor(inp[n], dtype=torch.float64, requires_grad=True) for n in NAMES}
    keep = np.stack([np.stack([TO.row_uniforms(b, i, N, h, 17, 2) for i in range(N)]) for b in range(B)])
    keep = torch.tensor(keep >= np.uint32(TO.drop_threshold(rate)), dtype=torch.float64)
    y = torch_forward(w, torch.tensor(inp["pair_mask"]), keep, TO.keep_scale(rate), h)
    (y * torch.tensor(dy)).sum().backward()
    for n in NAMES:
        np.testing.assert_allclose(gr["d_" + n], w[n].grad.numpy(), rtol=0, atol=1e-10, err_msg=n)


# ------------------------------------------------------------------ planted mistakes
@pytest.mark.parametrize("old,new", [
    ("dz = dsm.sum(1)", "dz = dsm[:, 0]"),  # the pair bias's gradient from one row only
    ("da = np.where(f[\"keep\"], da_drop * f[\"scale\"], 0.0)", "da = da_drop * f[\"scale\"]"),  # mask dropped
], ids=["bias-one-row", "no-dropout-mask"])
def test_planted_mistakes_are_caught(old, new, tmp_path):
    import importlib.util

    import oracle.tri_attn_backward_oracle as BW
    src = open(BW.__file__).read()
    assert src.count(old) == 1
    path = tmp_path / "bw_planted.py"
    path.write_text(src.replace(old, new))
    spec = importlib.util.spec_from_file_location("bw_planted", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    inp = tiny(B=2, N=6, D=8, h=2, mask=("pad", 4), seed=41)
    B, N, _, D = inp["pair_repr"].shape
    dy = np.random.default_rng(5).standard_normal((B, N, N, D))
    good = backward_train(inp, dy, 0.25, seed=17)
    bad = mod.backward_train(inp, dy, 0.25, seed=17)
    assert max(np.abs(good[k] - bad[k]).max() for k in good) > 1e-3
    with pytest.raises(AssertionError):
        # the finite-difference pin rejects the planted version
        globals()["backward_train"] = mod.backward_train
        try:
            test_finite_differences(0.3, ("pad", 2))
        finally:
            globals()["backward_train"] = backward_train_ref


# ------------------------------------------------------------------ position-sampled form
@pytest.mark.parametrize("shape,mask,dtype,rate,fill", [
    ((2, 20, 64, 4), ("bernoulli", 0.8), "f32", 0.3, O.MASK_FILL),
    ((1, 33, 128, 4), ("pad", 25), "bf16", 0.0, O.MASK_FILL),
    ((1, 17, 64, 2), ("pad", 12), "f32", 0.5, O.MASK_FILL),
    ((2, 13, 64, 4), ("bernoulli", 0.7), "f32", 0.2, -math.inf),
], ids=["B2N20bern", "N33pad-bf16", "N17pad-d32", "B2N13-inf"])
def test_position_sampled_gradient_equals_whole_backward(shape, mask, dtype, rate, fill):
    """Every position (b, r, c) of the inputs, in an order that switches batch
    more than once, against the whole backward's dL/d(pair_repr)."""
    B, N, D, h = shape
    inp = make_inputs(Workload("sampled", B, N, D, h, dtype, mask, seed=5 + N))
    dy = np.random.default_rng(3).standard_normal((B, N, N, D))
    whole = backward_train(inp, dy, rate, 77, 2, fill=fill)["d_pair_repr"]
    pos = [(b, r, c) for r in range(N) for c in range(N) for b in range(B)]
    got = pair_repr_grad_at(inp, dy, rate, 77, 2, pos, fill=fill)
    ref = np.array([whole[p] for p in pos])
    assert (np.isfinite(got) == np.isfinite(ref)).all()
    fin = np.isfinite(ref)
    assert np.abs(got[fin] - ref[fin]).max() <= 1e-12 * max(1.0, np.abs(ref[fin]).max())
