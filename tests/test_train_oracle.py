"""Pins for the training-mode oracle (dropout on the attention weights and the
saved log-sum-exp), independent of its own code.

* The generator against the published Philox4x32-10 known-answer vectors
  (tests/golden/philox4x32_10_kat.txt), for the oracle's vectorised version
  and for a scalar one written here.
* A brute-force per-element evaluation on tiny inputs: Python loops, the
  scalar generator and math.exp, with the inference steps computed directly
  with numpy, not through the oracle.
* Properties: rate 0 is the inference forward; the mean over many seeds is
  the inference output (the rescale keeps the expectation); the keep
  fraction and the uniformity of the generator's words; the log-sum-exp
  normalises the scores, and a fully masked column has FILL + ln N.
* Planted mistakes (all heads sharing one dropout mask, no rescale of the
  kept weights) that the pins must catch.
"""
import itertools
import math
import os

import numpy as np
import pytest

import oracle.tri_attn_oracle as O
import oracle.tri_attn_train_oracle as TO
from workloads import Workload, make_inputs

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "philox4x32_10_kat.txt")


def kat_vectors():
    rows = []
    with open(GOLDEN) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                words = [int(w, 16) for w in line.split()]
                assert len(words) == 10
                rows.append((words[:4], words[4:6], words[6:]))
    assert len(rows) == 3
    return rows


def philox_scalar(ctr, key):
    """Philox4x32-10 on Python integers, from the generator's definition."""
    c0, c1, c2, c3 = ctr
    k0, k1 = key
    for _ in range(10):
        p0, p1 = c0 * 0xD2511F53, c2 * 0xCD9E8D57
        c0, c1, c2, c3 = (p1 >> 32) ^ c1 ^ k0, p1 & 0xFFFFFFFF, (p0 >> 32) ^ c3 ^ k1, p0 & 0xFFFFFFFF
        k0, k1 = (k0 + 0x9E3779B9) & 0xFFFFFFFF, (k1 + 0xBB67AE85) & 0xFFFFFFFF
    return [c0, c1, c2, c3]


def small(B=2, N=5, D=8, h=2, mask=("bernoulli", 0.7), seed=11):
    return make_inputs(Workload("t", B, N, D, h, "f32", mask, seed))


# ------------------------------------------------------------------ the generator
def test_philox_known_answers():
    for ctr, key, want in kat_vectors():
        assert philox_scalar(ctr, key) == want
        got = TO.philox4x32_10(np.array(ctr, np.uint32), np.array(key, np.uint32))
        assert [int(w) for w in got] == want


def test_philox_vectorised_matches_scalar_on_random_counters():
    rng = np.random.default_rng(3)
    ctr = rng.integers(0, 2**32, size=(64, 4), dtype=np.uint64).astype(np.uint32)
    key = rng.integers(0, 2**32, size=(64, 2), dtype=np.uint64).astype(np.uint32)
    got = TO.philox4x32_10(ctr, key)
    for n in range(64):
        assert [int(w) for w in got[n]] == philox_scalar([int(c) for c in ctr[n]], [int(k) for k in key[n]])


# ------------------------------------------------------------------ brute force
def brute_force_train(inp, rate, seed, offset=0, fill=O.MASK_FILL):
    """y and lse from the per-element definition (tiny shapes only)."""
    P = np.asarray(inp["pair_repr"], np.float64)
    M = np.asarray(inp["pair_mask"])
    B, N, _, D = P.shape
    h = inp["num_heads"]
    d = D // h
    W = {k: np.asarray(inp[k], np.float64) for k in ("ln_weight", "ln_bias", "w_query", "w_key", "w_value",
                                                       "w_gate", "b_gate", "w_bias_proj", "w_out", "b_out")}
    mu = P.mean(-1, keepdims=True)
    var = ((P - mu) ** 2).mean(-1, keepdims=True)
    x = (P - mu) / np.sqrt(var + O.LN_EPS) * W["ln_weight"] + W["ln_bias"]
    q, kk, v = x @ W["w_query"].T, x @ W["w_key"].T, x @ W["w_value"].T
    g = 1.0 / (1.0 + np.exp(-(x @ W["w_gate"].T + W["b_gate"])))
    z = x @ W["w_bias_proj"].T  # z[b, j, k, t]
    thr = min(int(round(rate * 2**32)), 2**32 - 1)
    scale = 2**32 / (2**32 - thr)
    key = (seed & 0xFFFFFFFF, seed >> 32)
    y = np.zeros_like(P)
    lse = np.zeros((B, N, h, N))
    for b, i, j in itertools.product(range(B), range(N), range(N)):
        o = np.zeros(D)
        for t in range(h):
            s = []
            for k in range(N):
                if M[b, j, k] == 0:
                    s.append(fill)
                else:
                    qk = sum(q[b, i, j, t * d + u] * kk[b, i, k, t * d + u] for u in range(d)) / math.sqrt(d)
                    s.append(qk + z[b, j, k, t])
            mx = max(s)
            tot = sum(math.exp(sv - mx) for sv in s)
            lse[b, i, t, j] = mx + math.log(tot)
            for k in range(N):
                u32 = philox_scalar([k // 4, j, (b * N + i) * h + t, offset], key)[k % 4]
                a = math.exp(s[k] - mx) / tot
                a_drop = a * scale if u32 >= thr else 0.0
                o[t * d:(t + 1) * d] += a_drop * v[b, i, k, t * d:(t + 1) * d]
        y[b, i, j] = W["w_out"] @ (g[b, i, j] * o) + W["b_out"]
    return y, lse


@pytest.mark.parametrize("rate,seed,offset", [(0.3, 5, 0), (0.7, 2**40 + 17, 3), (0.05, 99, 2**31)])
def test_brute_force_tiny(rate, seed, offset):
    inp = small()  # N = 5: the last group of four keys is ragged
    y, lse = TO.forward_train(inp, rate, seed, offset)
    yb, lb = brute_force_train(inp, rate, seed, offset)
    np.testing.assert_allclose(y, yb, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lb, rtol=0, atol=1e-12)


def test_rows_equal_whole_forward():
    inp = small(B=2, N=6)
    y, lse = TO.forward_train(inp, 0.4, 21)
    rows = [(1, 5), (0, 0), (1, 2)]
    yr, lr = TO.forward_train_rows(inp, rows, 0.4, 21)
    for r, (b, i) in enumerate(rows):
        np.testing.assert_array_equal(yr[r], y[b, i])
        np.testing.assert_array_equal(lr[r], lse[b, i])


# ------------------------------------------------------------------ properties
def test_rate_zero_is_the_inference_forward():
    inp = small(B=2, N=7, D=16, h=4, mask=("pad", 5))
    y, _ = TO.forward_train(inp, 0.0, 1234)
    np.testing.assert_allclose(y, O.forward(inp), rtol=0, atol=1e-13)


def test_mean_over_seeds_is_the_inference_output():
    """E[a'] = a, and y is affine in a: the mean of y over many seeds must
    approach the inference y within the sampling error."""
    inp = small(B=1, N=4, D=8, h=2, mask=("ones",))
    ref = O.forward(inp)
    S = 1500
    ys = np.stack([TO.forward_train(inp, 0.5, s)[0] for s in range(S)])
    mean, sd = ys.mean(0), ys.std(0)
    assert (np.abs(mean - ref) <= 6 * sd / math.sqrt(S) + 1e-12).all()
    assert sd.max() > 0.01  # dropout does act


def test_keep_fraction_and_uniform_words():
    u = np.concatenate([TO.row_uniforms(b, i, 64, 8, 77).ravel() for b, i in ((0, 0), (0, 63), (1, 5), (3, 17))])
    assert u.size == 4 * 8 * 64 * 64
    for rate in (0.1, 0.5):
        frac = float((u >= np.uint32(TO.drop_threshold(rate))).mean())
        assert abs(frac - (1 - rate)) <= 6 * math.sqrt(rate * (1 - rate) / u.size)
    counts = np.bincount((u >> np.uint32(24)).astype(np.int64), minlength=256)
    chi2 = float(((counts - u.size / 256) ** 2 / (u.size / 256)).sum())
    assert chi2 < 255 + 6 * math.sqrt(2 * 255)


def test_column_uniforms_are_the_row_uniforms():
    """u of one query column in every row equals that column of each row's u."""
    B, N, h, seed, offset = 3, 13, 3, 2**33 + 9, 4
    for b in range(B):
        rows = np.stack([TO.row_uniforms(b, i, N, h, seed, offset) for i in range(N)])  # (i, t, j, k)
        for j in (0, 5, N - 1):
            assert np.array_equal(TO.column_uniforms(b, j, N, h, seed, offset), rows[:, :, j, :])


def test_decisions_depend_on_seed_offset_row_and_head():
    base = TO.row_uniforms(1, 2, 8, 2, 5, 0)
    assert np.array_equal(base, TO.row_uniforms(1, 2, 8, 2, 5, 0))
    for other in (TO.row_uniforms(1, 2, 8, 2, 6, 0), TO.row_uniforms(1, 2, 8, 2, 5 + 2**32, 0),
                  TO.row_uniforms(1, 2, 8, 2, 5, 1), TO.row_uniforms(1, 3, 8, 2, 5, 0),
                  TO.row_uniforms(0, 2, 8, 2, 5, 0)):
        assert (other != base).mean() > 0.99
    assert (base[0] != base[1]).mean() > 0.99


def test_lse_normalises_scores_and_fully_masked_columns():
    inp = small(B=1, N=9, D=16, h=2, mask=("pad", 6))  # columns j >= 6 have no valid key
    cap = {}
    _, lse = TO.forward_train_rows(inp, [(0, 0), (0, 7)], 0.2, 3, capture=cap)
    s = cap["s"]  # (rows, h, N, N)
    tot = np.exp(s - lse[..., None]).sum(-1)
    np.testing.assert_allclose(tot[..., :6], 1.0, rtol=0, atol=1e-12)
    # all scores FILL = -1e9: s - lse loses ~1e-7 to the magnitude
    np.testing.assert_allclose(tot[..., 6:], 1.0, rtol=0, atol=1e-6)
    assert (lse >= s.max(-1) - 1e-12).all()
    np.testing.assert_allclose(lse[..., 6:], TO.lse_fully_masked(9), rtol=0, atol=1e-6)
    assert not cap["keep"].all() and cap["keep"].any()


def test_ending_node_rate_zero_is_the_inference_ending_forward():
    inp = small(B=2, N=6, D=8, h=2, mask=("pad", 4))
    y, lse = TO.forward_train_ending(inp, 0.0, 8)
    np.testing.assert_allclose(y, O.forward_ending(inp), rtol=0, atol=1e-13)
    _, lse_t = TO.forward_train(O._transposed(inp), 0.0, 8)
    np.testing.assert_array_equal(lse, lse_t)


def test_rate_and_seed_validation():
    with pytest.raises(ValueError):
        TO.drop_threshold(1.0)
    with pytest.raises(ValueError):
        TO.drop_threshold(-0.1)
    with pytest.raises(ValueError):
        TO.seed_key(2**64)
    assert TO.drop_threshold(0.0) == 0 and TO.keep_scale(0.0) == 1.0
    assert TO.drop_threshold(0.25) == 2**30


# ------------------------------------------------------------------ planted mistakes
def test_planted_shared_head_mask_is_caught(monkeypatch):
    orig = TO.row_uniforms
    monkeypatch.setattr(TO, "row_uniforms",
                        lambda b, i, N, h, seed, offset=0: np.repeat(orig(b, i, N, 1, seed, offset), h, axis=0))
    inp = small()
    y, _ = TO.forward_train(inp, 0.3, 5)
    yb, _ = brute_force_train(inp, 0.3, 5)
    assert np.abs(y - yb).max() > 1e-3


def test_planted_missing_rescale_is_caught(monkeypatch):
    monkeypatch.setattr(TO, "keep_scale", lambda rate: 1.0)
    inp = small(B=1, N=4, D=8, h=2, mask=("ones",))
    ref = O.forward(inp)
    S = 1500
    ys = np.stack([TO.forward_train(inp, 0.5, s)[0] for s in range(S)])
    mean, sd = ys.mean(0), ys.std(0)
    assert not (np.abs(mean - ref) <= 6 * sd / math.sqrt(S) + 1e-12).all()
