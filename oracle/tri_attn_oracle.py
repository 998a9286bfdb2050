"""CPU oracle: starting-node triangular self-attention, inference forward.

TEST INFRASTRUCTURE ONLY. This module is the ground truth the GPU path is
checked against. Only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it; the library itself never
does, and shares no code with it.

It is a plain, slow float64 evaluation of the definition, one pair row at a
time, with numpy matmuls as the only library primitive. Sources (the l2_p6
transcripts of the POPCORNBENCH kernel benchmark):

* "FW-GLM-5-1 / l2_p6" transcript: the module's forward as the agent
  restates it while debugging (reshape of x to (B*N, N, D), the head split
  ``view(B*N, N, h, d).transpose(1, 2)``, the pair bias broadcast over rows
  through ``unsqueeze(1)``, the mask broadcast ``(B,1,1,N,N)``, softmax over
  the key axis, the ``transpose(1, 2).reshape(B, N, N, D)`` merge).
* "Kimi-K2.6 / l2_p6" transcript: the forward listing, the layer list
  (query/key/value/bias_proj without bias, gate and out_proj with bias,
  ``head_dim = pair_dim // num_heads``), eval-mode dropout, and the kernels'
  LayerNorm (biased variance, eps = 1e-5).

In index notation (b batch, i row, j query column, k key column, t head,
u channel within a head, d = D / h):

  (1) x[b,i,j]      = LayerNorm_D(P[b,i,j])                       (gamma, beta, eps)
  (2) g[b,i,j,c]    = sigmoid(x[b,i,j] . Wg[c] + bg[c])
  (3) z[b,t,j,k]    = x[b,j,k] . Wz[t]        (pair bias, shared by every row i)
  (4) q[b,i,t,j,u]  = x[b,i,j] . Wq[t*d+u]    (k, v likewise with Wk, Wv)
  (5) s[b,i,t,j,k]  = q[b,i,t,j] . k[b,i,t,k] / sqrt(d) + z[b,t,j,k];
                      s := FILL where mask[b,j,k] == 0  (replacement)
  (6) a             = softmax over k of s    (dropout is the identity)
  (7) o[b,i,j,t*d+u]= sum_k a[b,i,t,j,k] v[b,i,t,k,u]
  (8) y[b,i,j]      = Wo (g[b,i,j] * o[b,i,j]) + bo

Ending-node counterpart (``forward_ending``): the transcripts name only the
starting-node variant; its counterpart along the other residue axis is read
here as the same computation on the transposed pair representation and mask,
transposed back. In index notation: s[b,t,i,j,k] = q[b,i,j] . k[b,k,j] /
sqrt(d) + z_t(x[b,k,i]), FILL where mask[b,k,i] == 0, softmax over k,
o[b,i,j] = sum_k a v[b,k,j], y[b,i,j] = Wo (g[b,i,j] * o[b,i,j]) + bo.

Readings of points the pages leave open (each is listed with its reason in
the design notes): FILL defaults to -1e9, so a query column whose keys are
all masked gets uniform weights over all N keys; FILL = -inf reproduces the
quoted module literally and gives NaN there. The mask and the pair bias are
indexed by (query column j, key column k) and shared over rows i and heads.

Parity: every step is pinned by tests that do not reuse this code (library
LayerNorm and scaled-dot-product attention on special cases, closed forms,
invariants, brute force on tiny inputs, planted mistakes).
"""

from __future__ import annotations

import math
from typing import Iterable, Optional, Sequence, Tuple

import numpy as np

LN_EPS = 1e-5
MASK_FILL = -1e9

__all__ = [
    "LN_EPS",
    "MASK_FILL",
    "layer_norm",
    "linear",
    "sigmoid",
    "softmax",
    "split_heads",
    "merge_heads",
    "pair_bias",
    "row_bias",
    "row_mask",
    "row_scores",
    "output_projection",
    "apply_mask",
    "row_attention",
    "forward",
    "forward_rows",
]


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


# ---------------------------------------------------------------- step (1)
def layer_norm(p: np.ndarray, gamma: np.ndarray, beta: np.ndarray, eps: float = LN_EPS) -> np.ndarray:
    """Step (1): normalise each pair position over its D channels.

    Mean and biased variance (divide by D) over the last axis, then the
    affine gamma, beta, as nn.LayerNorm(pair_dim) does with its default eps.
    """
    p = _f64(p)
    mu = p.mean(axis=-1, keepdims=True)
    var = ((p - mu) ** 2).mean(axis=-1, keepdims=True)
    return (p - mu) / np.sqrt(var + eps) * _f64(gamma) + _f64(beta)


# ---------------------------------------------------------------- steps (2)-(4)
def linear(x: np.ndarray, w: np.ndarray, b: Optional[np.ndarray] = None) -> np.ndarray:
    """nn.Linear convention: weight is (out, in), y = x W^T + b."""
    y = _f64(x) @ _f64(w).T
    if b is not None:
        y = y + _f64(b)
    return y


def sigmoid(x: np.ndarray) -> np.ndarray:
    return 1.0 / (1.0 + np.exp(-x))


def split_heads(y: np.ndarray, h: int) -> np.ndarray:
    """(..., N, D) -> (..., h, N, d): channel c = t*d + u goes to head t."""
    n, D = y.shape[-2:]
    d = D // h
    return np.swapaxes(y.reshape(y.shape[:-1] + (h, d)), -2, -3)


def merge_heads(o: np.ndarray) -> np.ndarray:
    """(..., h, N, d) -> (..., N, D): inverse of split_heads."""
    h, n, d = o.shape[-3:]
    return np.swapaxes(o, -2, -3).reshape(o.shape[:-3] + (n, h * d))


def pair_bias(x_b: np.ndarray, w_bias: np.ndarray) -> np.ndarray:
    """Step (3) for one batch: z[t, j, k] = x[j, k] . Wz[t].

    x_b is (N, N, D); the result (h, N, N) is indexed by the pair (j, k) of the
    LayerNorm output and is added to the scores of every row i.
    """
    return np.moveaxis(linear(x_b, w_bias), -1, 0)


def row_bias(z_b: np.ndarray, i: int) -> np.ndarray:
    """The pair bias seen by row i: the same (h, N, N) tensor z[t, j, k] for every i.

    Both transcripts broadcast the (B, h, N, N) bias over the row axis of the
    (B, N, h, N, N) scores (``unsqueeze(1)``); the bias index is the
    (query column, key column) pair, never the row.
    """
    return z_b


def row_mask(mask_b: np.ndarray, i: int) -> np.ndarray:
    """The mask seen by row i: mask[j, k] of the batch, the same for every row and head
    (the transcripts broadcast it as (B, 1, 1, N, N))."""
    return mask_b


# ---------------------------------------------------------------- step (5)
def row_scores(q: np.ndarray, k: np.ndarray, z_b: np.ndarray) -> np.ndarray:
    """Step (5) before masking, one row: s[t, j, k] = q_j . k_k / sqrt(d) + z[t, j, k]."""
    d = q.shape[-1]
    return q @ np.swapaxes(k, -1, -2) / math.sqrt(d) + z_b


def apply_mask(s: np.ndarray, mask_b: np.ndarray, fill: float = MASK_FILL) -> np.ndarray:
    """Replace the score by FILL wherever mask[j, k] == 0 (same for all heads)."""
    return np.where(np.asarray(mask_b)[None] == 0, fill, s)


# ---------------------------------------------------------------- step (6)
def softmax(s: np.ndarray, axis: int = -1) -> np.ndarray:
    """Softmax with the maximum subtracted first (the value is unchanged by it)."""
    m = s.max(axis=axis, keepdims=True)
    with np.errstate(invalid="ignore"):
        e = np.exp(s - m)
        return e / e.sum(axis=axis, keepdims=True)


# ---------------------------------------------------------------- steps (4)-(8), one row
def row_attention(
    x_row: np.ndarray,
    z_b: np.ndarray,
    mask_b: np.ndarray,
    prm: dict,
    h: int,
    fill: float = MASK_FILL,
    capture: Optional[dict] = None,
) -> np.ndarray:
    """Steps (2), (4)-(8) for one pair row (b, i).

    x_row is the LayerNorm output x[b, i, :, :] (N, D); z_b the pair bias of
    batch b (h, N, N); mask_b the mask of batch b (N, N). Returns y[b, i] (N, D).
    """
    g = sigmoid(linear(x_row, prm["w_gate"], prm["b_gate"]))  # (N, D)
    q = split_heads(linear(x_row, prm["w_query"]), h)  # (h, N, d)
    k = split_heads(linear(x_row, prm["w_key"]), h)
    v = split_heads(linear(x_row, prm["w_value"]), h)
    s = apply_mask(row_scores(q, k, z_b), mask_b, fill)  # (h, N, N)
    a = softmax(s, axis=-1)
    o = merge_heads(a @ v)  # (N, D)
    y = output_projection(g * o, prm["w_out"], prm["b_out"])
    if capture is not None:
        capture.update(g=g, q=q, k=k, v=v, a=a, o=o)
    return y


def output_projection(go: np.ndarray, w_out: np.ndarray, b_out: np.ndarray) -> np.ndarray:
    """Step (8): y = Wo (g * o) + bo, per position."""
    return linear(go, w_out, b_out)


def _params(inp: dict) -> dict:
    return {k: _f64(inp[k]) for k in (
        "ln_weight", "ln_bias", "w_query", "w_key", "w_value",
        "w_gate", "b_gate", "w_bias_proj", "w_out", "b_out")}


def forward(inp: dict, fill: float = MASK_FILL, eps: float = LN_EPS, capture: Optional[dict] = None) -> np.ndarray:
    """The whole forward: y (B, N, N, D) in float64.

    ``inp`` holds ``pair_repr`` (B,N,N,D), ``pair_mask`` (B,N,N; 0 = masked),
    ``num_heads`` and the parameters named as in nn.LayerNorm / nn.Linear.
    With ``capture`` (a dict), the per-step intermediates of every row are
    stored in it: x, z, and g, q, k, v, a, o stacked over (b, i).
    """
    B, N, _, D = np.shape(inp["pair_repr"])
    rows = [(b, i) for b in range(B) for i in range(N)]
    y = forward_rows(inp, rows, fill=fill, eps=eps, capture=capture)
    return y.reshape(B, N, N, D)


def forward_rows(
    inp: dict,
    rows: Sequence[Tuple[int, int]],
    fill: float = MASK_FILL,
    eps: float = LN_EPS,
    capture: Optional[dict] = None,
) -> np.ndarray:
    """y[b, i] for the listed rows (b, i) only: (len(rows), N, D) float64.

    A row needs the LayerNorm of its own N positions and the pair bias of its
    batch, which comes from all N*N positions of that batch. Only the batches
    the rows touch are read (and widened to float64 by layer_norm).
    """
    P = inp["pair_repr"]
    M = np.asarray(inp["pair_mask"])
    h = int(inp["num_heads"])
    prm = _params(inp)
    B, N, _, D = P.shape
    if D % h:
        raise ValueError("pair_dim must be divisible by num_heads")
    out = np.empty((len(rows), N, D), dtype=np.float64)
    x_cache = {}
    z_cache = {}
    per_row = {} if capture is not None else None
    for r, (b, i) in enumerate(rows):
        if b not in z_cache:
            x_b = layer_norm(P[b], prm["ln_weight"], prm["ln_bias"], eps)  # (N, N, D)
            x_cache[b] = x_b
            z_cache[b] = pair_bias(x_b, prm["w_bias_proj"])  # (h, N, N)
        row_cap = {} if per_row is not None else None
        out[r] = row_attention(x_cache[b][i], row_bias(z_cache[b], i), row_mask(M[b], i), prm, h, fill, row_cap)
        if per_row is not None:
            for key, val in row_cap.items():
                per_row.setdefault(key, []).append(val)
    if capture is not None:
        capture["x"] = np.stack([x_cache[b] for b in sorted(x_cache)])
        capture["z"] = np.stack([z_cache[b] for b in sorted(z_cache)])
        for key, vals in per_row.items():
            capture[key] = np.stack(vals)
    return out


def _transposed(inp: dict) -> dict:
    t = dict(inp)
    t["pair_repr"] = np.ascontiguousarray(np.swapaxes(np.asarray(inp["pair_repr"]), 1, 2))
    t["pair_mask"] = np.ascontiguousarray(np.swapaxes(np.asarray(inp["pair_mask"]), 1, 2))
    return t


def forward_ending(inp: dict, fill: float = MASK_FILL, eps: float = LN_EPS) -> np.ndarray:
    """Ending-node forward, y (B, N, N, D) in float64: the starting-node
    forward of the pair representation and mask with both residue axes
    swapped, swapped back (see the module notes for the index form)."""
    return np.swapaxes(forward(_transposed(inp), fill=fill, eps=eps), 1, 2)


def forward_ending_cols(inp: dict, cols: Sequence[Tuple[int, int]], fill: float = MASK_FILL,
                        eps: float = LN_EPS) -> np.ndarray:
    """Ending-node y[b, :, j] for the listed columns (b, j): (len(cols), N, D)."""
    return forward_rows(_transposed(inp), cols, fill=fill, eps=eps)

