"""CPU oracle: gradients of the training-mode forward (starting-node
triangular self-attention with dropout on the attention weights).

TEST INFRASTRUCTURE ONLY, like the forward oracles: only the tests may import
it; the library never does and shares no code with it.

Given dy = dL/dy for the output of ``tri_attn_train_oracle.forward_train``
(same rate, seed and offset, so the same dropout decisions), this returns
dL/d(pair_repr) and dL/d(every parameter), by back-propagation through the
steps of the forward in reverse, in float64:

  (8) y = Wo (g * o) + bo       dWo = sum dy (g*o)^T, dbo = sum dy,
                                d(g*o) = Wo^T dy
      g*o                        dg = d(g*o) * o,  do = d(g*o) * g
  (2) g = sigmoid(Wg x + bg)     dgp = dg * g (1 - g); dWg, dbg, dx += Wg^T dgp
  (7) o = sum_k a' v             da'[j,k] = do[j] . v[k];  dv[k] = sum_j a'[j,k] do[j]
  (6') a' = a * keep * scale     da = da' * keep * scale
  (6) a = softmax_k(s)           ds = a * (da - sum_k a da)
  (5) s = q.k/sqrt(d) + z, or    only unmasked entries pass the gradient on
      FILL where masked          (FILL is a constant): dsm = ds * mask
                                 dq[j] = sum_k dsm[j,k] k[k] / sqrt(d)
                                 dk[k] = sum_j dsm[j,k] q[j] / sqrt(d)
  (3) z[b,t,j,k] = x[b,j,k].Wz[t], shared by every row i:
                                 dz[b,t,j,k] = sum_i dsm[b,i,t,j,k]
                                 dWz[t] = sum dz x,  dx[b,j,k] += sum_t dz Wz[t]
  (4) q, k, v = Wq x, Wk x, Wv x dW* = sum d*^T x,  dx += W*^T d*
  (1) x = gamma * xhat + beta, xhat = (P - mean) / sqrt(var + eps), biased var:
                                 dgamma = sum dx xhat, dbeta = sum dx,
                                 dP = (dxh - mean(dxh) - xhat mean(dxh xhat)) / sqrt(var + eps),
                                 dxh = dx * gamma
"""
import math
from typing import Optional, Sequence, Tuple

import numpy as np

from oracle import tri_attn_oracle as O
from oracle import tri_attn_train_oracle as TO


def _forward_tensors(inp: dict, rate: float, seed: int, offset: int, fill: float, eps: float) -> dict:
    """Every intermediate of the training forward, whole tensors (float64)."""
    P = O._f64(inp["pair_repr"])
    M = np.asarray(inp["pair_mask"])
    h = int(inp["num_heads"])
    prm = O._params(inp)
    B, N, _, D = P.shape
    d = D // h
    mu = P.mean(-1, keepdims=True)
    var = ((P - mu) ** 2).mean(-1, keepdims=True)
    rstd = 1.0 / np.sqrt(var + eps)
    xhat = (P - mu) * rstd
    x = xhat * prm["ln_weight"] + prm["ln_bias"]
    gp = x @ prm["w_gate"].T + prm["b_gate"]
    g = 1.0 / (1.0 + np.exp(-gp))
    heads = lambda y: y.reshape(B, N, N, h, d).transpose(0, 1, 3, 2, 4)  # noqa: E731  (b, i, t, j, u)
    q, k, v = heads(x @ prm["w_query"].T), heads(x @ prm["w_key"].T), heads(x @ prm["w_value"].T)
    z = np.einsum("bjkc,tc->btjk", x, prm["w_bias_proj"])  # (b, t, j, k)
    valid = (M != 0)[:, None, None]  # (b, 1, 1, j, k): broadcast over rows and heads
    s = np.where(valid, q @ np.swapaxes(k, -1, -2) / math.sqrt(d) + z[:, None], fill)  # (b, i, t, j, k)
    a = O.softmax(s, axis=-1)
    keep = np.stack([np.stack([TO.row_uniforms(b, i, N, h, seed, offset) for i in range(N)]) for b in range(B)])
    keep = keep >= np.uint32(TO.drop_threshold(rate))
    scale = TO.keep_scale(rate)
    a_drop = np.where(keep, a * scale, 0.0)
    o = (a_drop @ v).transpose(0, 1, 3, 2, 4).reshape(B, N, N, D)
    y = (g * o) @ prm["w_out"].T + prm["b_out"]
    return dict(P=P, prm=prm, h=h, d=d, xhat=xhat, rstd=rstd, x=x, g=g, q=q, k=k, v=v, valid=valid, a=a,
                keep=keep, scale=scale, a_drop=a_drop, o=o, y=y)


def backward_train(inp: dict, dy: np.ndarray, rate: float, seed: int, offset: int = 0,
                   fill: float = O.MASK_FILL, eps: float = O.LN_EPS, capture: Optional[dict] = None) -> dict:
    """Gradients of L = sum(dy * y) with respect to ``pair_repr`` and every
    parameter, keyed ``d_<name>`` (float64, the shapes of the inputs).
    With ``capture``, the forward's y is stored under "y"."""
    f = _forward_tensors(inp, rate, seed, offset, fill, eps)
    prm, h, d = f["prm"], f["h"], f["d"]
    B, N, _, D = f["P"].shape
    dy = np.asarray(dy, np.float64)
    sq = lambda t: t.reshape(-1, t.shape[-1])  # noqa: E731  positions flattened
    heads = lambda t: t.reshape(B, N, N, h, d).transpose(0, 1, 3, 2, 4)  # noqa: E731
    merge = lambda t: t.transpose(0, 1, 3, 2, 4).reshape(B, N, N, D)  # noqa: E731
    gr = {}
    # (8)
    go = f["g"] * f["o"]
    gr["d_w_out"] = sq(dy).T @ sq(go)
    gr["d_b_out"] = sq(dy).sum(0)
    dgo = dy @ prm["w_out"]
    dg = dgo * f["o"]
    do = heads(dgo * f["g"])  # (b, i, t, j, u)
    # (2)
    dgp = dg * f["g"] * (1.0 - f["g"])
    gr["d_w_gate"] = sq(dgp).T @ sq(f["x"])
    gr["d_b_gate"] = sq(dgp).sum(0)
    dx = dgp @ prm["w_gate"]
    # (7), (6'), (6)
    da_drop = do @ np.swapaxes(f["v"], -1, -2)  # (b, i, t, j, k)
    dv = np.swapaxes(f["a_drop"], -1, -2) @ do  # (b, i, t, k, u)
    da = np.where(f["keep"], da_drop * f["scale"], 0.0)
    ds = f["a"] * (da - (f["a"] * da).sum(-1, keepdims=True))
    # (5)
    dsm = np.where(f["valid"], ds, 0.0)
    dq = dsm @ f["k"] / math.sqrt(d)
    dk = np.swapaxes(dsm, -1, -2) @ f["q"] / math.sqrt(d)
    dz = dsm.sum(1)  # (b, t, j, k): summed over rows i
    # (3)
    gr["d_w_bias_proj"] = np.einsum("btjk,bjkc->tc", dz, f["x"])
    dx = dx + np.einsum("btjk,tc->bjkc", dz, prm["w_bias_proj"])
    # (4)
    for name, dt in (("w_query", dq), ("w_key", dk), ("w_value", dv)):
        dtm = merge(dt)
        gr["d_" + name] = sq(dtm).T @ sq(f["x"])
        dx = dx + dtm @ prm[name]
    # (1)
    gr["d_ln_weight"] = sq(dx * f["xhat"]).sum(0)
    gr["d_ln_bias"] = sq(dx).sum(0)
    dxh = dx * prm["ln_weight"]
    gr["d_pair_repr"] = (dxh - dxh.mean(-1, keepdims=True)
                         - f["xhat"] * (dxh * f["xhat"]).mean(-1, keepdims=True)) * f["rstd"]
    if capture is not None:
        capture["y"] = f["y"]
    return gr


def pair_repr_grad_at(inp: dict, dy: np.ndarray, rate: float, seed: int, offset: int = 0,
                      positions: Sequence[Tuple[int, int, int]] = (), fill: float = O.MASK_FILL,
                      eps: float = O.LN_EPS) -> np.ndarray:
    """dL/d(pair_repr) at the listed positions (b, r, c) only, (len, D)
    float64: the steps of backward_train restricted to what those positions
    need, for sizes where its whole (B, N, h, N, N) tensors do not fit in
    memory. Position (b, r, c) enters pair row r as query column c (q and
    the gate), as key c (k and v), and through the pair bias z[b, :, r, c]
    every row i, as the score of query column r and key c."""
    P = O._f64(inp["pair_repr"])
    M = np.asarray(inp["pair_mask"])
    h = int(inp["num_heads"])
    prm = O._params(inp)
    B, N, _, D = P.shape
    d = D // h
    dy = np.asarray(dy, np.float64)
    thr = np.uint32(TO.drop_threshold(rate))
    scale = TO.keep_scale(rate)
    out = np.empty((len(positions), D))
    cur, f = None, None
    for n, (b, r, c) in enumerate(positions):
        if b != cur:  # every tensor of batch b, positions (i, j)
            cur = b
            mu = P[b].mean(-1, keepdims=True)
            var = ((P[b] - mu) ** 2).mean(-1, keepdims=True)
            rstd = 1.0 / np.sqrt(var + eps)
            xhat = (P[b] - mu) * rstd
            x = xhat * prm["ln_weight"] + prm["ln_bias"]
            g = 1.0 / (1.0 + np.exp(-(x @ prm["w_gate"].T + prm["b_gate"])))
            heads = lambda y: y.reshape(N, N, h, d).transpose(0, 2, 1, 3)  # noqa: E731  (i, t, j, u)
            dgo = dy[b] @ prm["w_out"]
            f = dict(xhat=xhat, rstd=rstd, g=g, dgo=dgo, q=heads(x @ prm["w_query"].T), k=heads(x @ prm["w_key"].T),
                     v=heads(x @ prm["w_value"].T), do=heads(dgo * g),
                     z=np.moveaxis(x @ prm["w_bias_proj"].T, -1, 0), valid=M[b] != 0)
        q, k, v, do, valid = f["q"], f["k"], f["v"], f["do"], f["valid"]
        # row r: (7), (6'), (6), (5) for every query column j and key of the row
        s = np.where(valid[None], q[r] @ np.swapaxes(k[r], -1, -2) / math.sqrt(d) + f["z"], fill)  # (t, j, k)
        a = O.softmax(s, axis=-1)
        keep = TO.row_uniforms(b, r, N, h, seed, offset) >= thr
        a_drop = np.where(keep, a * scale, 0.0)
        o_c = np.einsum("tk,tku->tu", a_drop[:, c, :], v[r]).reshape(D)  # o of query column c, channel t*d + u
        da = np.where(keep, (do[r] @ np.swapaxes(v[r], -1, -2)) * scale, 0.0)
        ds = a * (da - (a * da).sum(-1, keepdims=True))
        dsm = np.where(valid[None], ds, 0.0)
        dq_c = np.einsum("tk,tku->tu", dsm[:, c, :], k[r]) / math.sqrt(d)  # (t, u): query column c
        dk_c = np.einsum("tj,tju->tu", dsm[:, :, c], q[r]) / math.sqrt(d)  # key c
        dv_c = np.einsum("tj,tju->tu", a_drop[:, :, c], do[r])  # key c
        # (8), (2): the gate of position (r, c)
        g_c = f["g"][r, c]
        dgp = f["dgo"][r, c] * o_c * g_c * (1.0 - g_c)
        dx = dgp @ prm["w_gate"]
        # (4)
        for name, dt in (("w_query", dq_c), ("w_key", dk_c), ("w_value", dv_c)):
            dx = dx + dt.reshape(D) @ prm[name]
        # (3): dz[t, r, c] = sum over rows i of dsm[i, t, r, c] (query column r, key c)
        qk = (q[:, :, r, None, :] @ np.swapaxes(k, -1, -2))[:, :, 0, :]  # (i, t, k)
        s_col = np.where(valid[r][None, None], qk / math.sqrt(d) + f["z"][None, :, r, :], fill)
        a_col = O.softmax(s_col, axis=-1)
        keep_col = TO.column_uniforms(b, r, N, h, seed, offset) >= thr
        da_col = np.where(keep_col, (do[:, :, r, None, :] @ np.swapaxes(v, -1, -2))[:, :, 0, :] * scale, 0.0)
        ds_col = a_col * (da_col - (a_col * da_col).sum(-1, keepdims=True))
        dz = ds_col[:, :, c].sum(0) if valid[r, c] else np.zeros(h)
        dx = dx + dz @ prm["w_bias_proj"]
        # (1)
        dxh = dx * prm["ln_weight"]
        xh = f["xhat"][r, c]
        out[n] = (dxh - dxh.mean() - xh * (dxh * xh).mean()) * f["rstd"][r, c, 0]
    return out
