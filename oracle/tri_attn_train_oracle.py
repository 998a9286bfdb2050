"""CPU oracle: starting-node triangular self-attention, training-mode forward.

TEST INFRASTRUCTURE ONLY, like tri_attn_oracle (whose steps it reuses): only
the tests may import it; the library never does and shares no code with it.

What differs from inference is dropout on the attention weights. Sources:

* "FW-GLM-5-1 / l2_p6" transcript, the forward as the agent restates it:
  dropout acts on the attention weights right after the softmax over the key
  axis and before their product with v.
* "Kimi-K2.6 / l2_p6" transcript, the layer list: the module holds a dropout
  layer, which is the identity in evaluation mode.

The pages fix neither the random numbers nor a statistic saved for a
backward pass. The readings here (the numbers are drawn from a published
counter-based generator so that any implementation can reproduce every
decision) are:

  (6') a'[b,i,t,j,k] = a[b,i,t,j,k] * keep[b,i,t,j,k] * 2^32 / (2^32 - thr)
       keep = (u[b,i,t,j,k] >= thr),  thr = min(round(rate * 2^32), 2^32 - 1)
       u[b,i,t,j,k] = word (k mod 4) of Philox4x32-10 with
         counter = (k div 4, j, (b*N + i)*h + t, offset)   (32-bit words)
         key     = (seed mod 2^32, seed div 2^32)
  (7') o uses a' in place of a; steps (1)-(5) and (8) are the inference ones.
  lse[b,i,t,j] = ln sum_k exp(s[b,i,t,j,k]), over the masked scores of step (5).

The scale 2^32 / (2^32 - thr) makes the expectation of a' equal a exactly
(the drop probability is thr / 2^32, rate rounded to 2^-32). Four consecutive
keys share one generator call.

Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as
easy as 1, 2, 3", SC 2011): ten rounds on a counter of four 32-bit words
(c0, c1, c2, c3) and a key (k0, k1). A round forms the two 64-bit products
c0 * 0xD2511F53 and c2 * 0xCD9E8D57 and maps the counter to
(hi(c2 product) ^ c1 ^ k0, lo(c2 product), hi(c0 product) ^ c3 ^ k1,
lo(c0 product)); between rounds the key is bumped by (0x9E3779B9, 0xBB67AE85)
modulo 2^32. The published known-answer vectors pin it.
"""
import math
from typing import Optional, Sequence, Tuple

import numpy as np

from oracle import tri_attn_oracle as O

_M0, _M1 = np.uint64(0xD2511F53), np.uint64(0xCD9E8D57)
_W0, _W1 = 0x9E3779B9, 0xBB67AE85
_MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(counter: np.ndarray, key: np.ndarray) -> np.ndarray:
    """Philox4x32-10 on uint32 arrays: counter (..., 4), key (..., 2) or (2,).
    Returns the four output words (..., 4) uint32."""
    counter = np.asarray(counter, dtype=np.uint32)
    key = np.broadcast_to(np.asarray(key, dtype=np.uint32), counter.shape[:-1] + (2,))
    c0, c1, c2, c3 = (counter[..., n].astype(np.uint64) for n in range(4))
    k0, k1 = key[..., 0].astype(np.uint64), key[..., 1].astype(np.uint64)
    for _ in range(10):
        p0 = c0 * _M0  # < 2^64: exact in uint64
        p1 = c2 * _M1
        c0, c1, c2, c3 = (p1 >> np.uint64(32)) ^ c1 ^ k0, p1 & _MASK32, (p0 >> np.uint64(32)) ^ c3 ^ k1, p0 & _MASK32
        k0 = (k0 + np.uint64(_W0)) & _MASK32
        k1 = (k1 + np.uint64(_W1)) & _MASK32
    return np.stack([c0, c1, c2, c3], axis=-1).astype(np.uint32)


def seed_key(seed: int) -> np.ndarray:
    """The generator key of a 64-bit seed: (low word, high word)."""
    if not 0 <= int(seed) < 2**64:
        raise ValueError("seed must be in [0, 2^64)")
    return np.array([int(seed) & 0xFFFFFFFF, int(seed) >> 32], dtype=np.uint32)


def drop_threshold(rate: float) -> int:
    """thr = min(round(rate * 2^32), 2^32 - 1): a weight is kept iff u >= thr."""
    if not 0.0 <= rate < 1.0:
        raise ValueError("dropout rate must be in [0, 1)")
    return min(int(round(rate * 2.0**32)), 2**32 - 1)


def keep_scale(rate: float) -> float:
    """2^32 / (2^32 - thr): the factor on kept weights (expectation preserved)."""
    return 2.0**32 / (2.0**32 - drop_threshold(rate))


def row_uniforms(b: int, i: int, N: int, h: int, seed: int, offset: int = 0) -> np.ndarray:
    """u[t, j, k] (h, N, N) uint32 of pair row (b, i), as defined in (6')."""
    Nk = (N + 3) // 4
    t = np.arange(h, dtype=np.uint64)[:, None, None]
    j = np.arange(N, dtype=np.uint64)[None, :, None]
    kg = np.arange(Nk, dtype=np.uint64)[None, None, :]
    ctr = np.empty((h, N, Nk, 4), dtype=np.uint32)
    ctr[..., 0] = kg
    ctr[..., 1] = j
    ctr[..., 2] = (np.uint64((b * N + i) * h) + t) & _MASK32
    ctr[..., 3] = np.uint32(int(offset) & 0xFFFFFFFF)
    words = philox4x32_10(ctr, seed_key(seed))  # (h, N, Nk, 4): word k mod 4 of call k div 4
    return words.reshape(h, N, Nk * 4)[:, :, :N]


def column_uniforms(b: int, j: int, N: int, h: int, seed: int, offset: int = 0) -> np.ndarray:
    """u[i, t, k] (N, h, N) uint32 of query column j in every pair row i of
    batch b, as defined in (6'): the words row_uniforms(b, i, ...)[t, j, k]."""
    Nk = (N + 3) // 4
    i = np.arange(N, dtype=np.uint64)[:, None, None]
    t = np.arange(h, dtype=np.uint64)[None, :, None]
    kg = np.arange(Nk, dtype=np.uint64)[None, None, :]
    ctr = np.empty((N, h, Nk, 4), dtype=np.uint32)
    ctr[..., 0] = kg
    ctr[..., 1] = np.uint32(j)
    ctr[..., 2] = ((np.uint64(b * N) + i) * np.uint64(h) + t) & _MASK32
    ctr[..., 3] = np.uint32(int(offset) & 0xFFFFFFFF)
    words = philox4x32_10(ctr, seed_key(seed))  # (N, h, Nk, 4)
    return words.reshape(N, h, Nk * 4)[:, :, :N]


def row_attention_train(x_row, z_b, mask_b, prm, h, u, rate, fill=O.MASK_FILL, capture=None):
    """Steps (2), (4)-(8) of one pair row with dropout (6') on the attention
    weights; u holds the row's uniforms (h, N, N). Returns (y (N, D), lse (h, N))."""
    g = O.sigmoid(O.linear(x_row, prm["w_gate"], prm["b_gate"]))
    q = O.split_heads(O.linear(x_row, prm["w_query"]), h)
    k = O.split_heads(O.linear(x_row, prm["w_key"]), h)
    v = O.split_heads(O.linear(x_row, prm["w_value"]), h)
    s = O.apply_mask(O.row_scores(q, k, z_b), mask_b, fill)  # (h, N, N)
    a = O.softmax(s, axis=-1)
    keep = u >= np.uint32(drop_threshold(rate))
    a_drop = np.where(keep, a * keep_scale(rate), 0.0)
    o = O.merge_heads(a_drop @ v)
    y = O.output_projection(g * o, prm["w_out"], prm["b_out"])
    m = s.max(axis=-1)
    with np.errstate(invalid="ignore", divide="ignore"):
        lse = m + np.log(np.exp(s - m[..., None]).sum(axis=-1))
    if capture is not None:
        capture.update(s=s, a=a, keep=keep, a_drop=a_drop, lse=lse)
    return y, lse


def forward_train_rows(
    inp: dict,
    rows: Sequence[Tuple[int, int]],
    rate: float,
    seed: int,
    offset: int = 0,
    fill: float = O.MASK_FILL,
    eps: float = O.LN_EPS,
    capture: Optional[dict] = None,
):
    """(y (len(rows), N, D), lse (len(rows), h, N)) float64 for the listed rows.
    With ``capture``, the per-row s, a, keep, a_drop and lse stacked over rows."""
    P = inp["pair_repr"]  # widened per batch by layer_norm
    M = np.asarray(inp["pair_mask"])
    h = int(inp["num_heads"])
    prm = O._params(inp)
    B, N, _, D = P.shape
    if D % h:
        raise ValueError("pair_dim must be divisible by num_heads")
    drop_threshold(rate)  # validates the rate
    y = np.empty((len(rows), N, D))
    lse = np.empty((len(rows), h, N))
    xz = {}
    per_row = {} if capture is not None else None
    for r, (b, i) in enumerate(rows):
        if b not in xz:
            x_b = O.layer_norm(P[b], prm["ln_weight"], prm["ln_bias"], eps)
            xz[b] = (x_b, O.pair_bias(x_b, prm["w_bias_proj"]))
        x_b, z_b = xz[b]
        u = row_uniforms(b, i, N, h, seed, offset)
        cap = {} if per_row is not None else None
        y[r], lse[r] = row_attention_train(x_b[i], O.row_bias(z_b, i), O.row_mask(M[b], i), prm, h, u, rate, fill,
                                           cap)
        if per_row is not None:
            for key, val in cap.items():
                per_row.setdefault(key, []).append(val)
    if capture is not None:
        for key, vals in per_row.items():
            capture[key] = np.stack(vals)
    return y, lse


def forward_train(inp: dict, rate: float, seed: int, offset: int = 0, fill: float = O.MASK_FILL,
                  eps: float = O.LN_EPS, capture: Optional[dict] = None):
    """The whole training-mode forward: y (B, N, N, D) and lse (B, N, h, N),
    float64; lse[b, i, t, j] is the natural log-sum-exp of the masked scores
    of query column j of row (b, i), head t."""
    B, N, _, D = np.shape(inp["pair_repr"])
    h = int(inp["num_heads"])
    rows = [(b, i) for b in range(B) for i in range(N)]
    y, lse = forward_train_rows(inp, rows, rate, seed, offset, fill, eps, capture)
    return y.reshape(B, N, N, D), lse.reshape(B, N, h, N)


def forward_train_ending(inp: dict, rate: float, seed: int, offset: int = 0, fill: float = O.MASK_FILL,
                         eps: float = O.LN_EPS):
    """Ending-node training forward: the starting-node training forward of
    the pair representation and mask with both residue axes swapped, y
    swapped back. The dropout counters and lse use the indices of that
    swapped problem: lse[b, j, t, i] belongs to output position (b, i, j)."""
    y, lse = forward_train(O._transposed(inp), rate, seed, offset, fill, eps)
    return np.swapaxes(y, 1, 2), lse


def lse_fully_masked(N: int, fill: float = O.MASK_FILL) -> float:
    """lse of a query column whose keys are all masked: every score is FILL."""
    return fill + math.log(N)
