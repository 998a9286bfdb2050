"""Starting-node triangular self-attention forward for MI355X (gfx950).

The compute lives in libtri_attn.so (hand-written HIP kernels behind the C ABI
of include/tri_attn.h). ``binding`` mirrors that ABI with the same names;
``TriangularAttention`` below only owns a handle and a torch-allocated
workspace, and marshals tensors to pointers.
"""
from __future__ import annotations

import math

from .binding import (  # noqa: F401
    TRI_ATTN_BF16,
    TRI_ATTN_F32,
    TriAttnError,
    WEIGHT_FIELDS,
    load_library,
    tri_attn_attend,
    tri_attn_config,
    tri_attn_create,
    tri_attn_destroy,
    tri_attn_forward,
    tri_attn_get_workspace_layout,
    tri_attn_output,
    tri_attn_project,
    tri_attn_strerror,
    tri_attn_workspace_size,
)

__all__ = ["TriangularAttention", "TriAttnError", "TRI_ATTN_F32", "TRI_ATTN_BF16"]


class TriangularAttention:
    """Handle + workspace around the C ABI.

    weights: dict of device tensors named as in WEIGHT_FIELDS (nn.Linear
    layout, dtype float32 or bfloat16). Calls run on torch's current stream.
    """

    def __init__(self, weights: dict, num_heads: int, ln_eps: float = 1e-5, mask_fill: float = -1e9,
                 ending_node: bool = False):
        import torch

        w0 = weights["w_query"]
        self.dtype = w0.dtype
        if w0.dtype == torch.float32:
            code = TRI_ATTN_F32
        elif w0.dtype == torch.bfloat16:
            code = TRI_ATTN_BF16
        else:
            raise TypeError(f"unsupported dtype {w0.dtype}")
        self.D = int(w0.shape[0])
        self.h = int(num_heads)
        self.device = w0.device
        for k in WEIGHT_FIELDS:
            t = weights[k]
            if t.dtype != w0.dtype or not t.is_contiguous() or t.device != w0.device:
                raise ValueError(f"weight {k} must be contiguous {w0.dtype} on {w0.device}")
        cfg = tri_attn_config(pair_dim=self.D, num_heads=self.h, dtype=code, ln_eps=ln_eps,
                              mask_fill=mask_fill if math.isfinite(mask_fill) else -math.inf,
                              ending_node=int(bool(ending_node)))
        self._weights = weights  # kept alive until create has copied them
        self.handle = tri_attn_create(cfg, weights, torch.cuda.current_stream(self.device))
        self._ws = None

    def workspace(self, B: int, N: int):
        import torch

        n = tri_attn_workspace_size(self.handle, B, N)
        if self._ws is None or self._ws.numel() < n:
            self._ws = torch.empty(max(n, 256), dtype=torch.uint8, device=self.device)
        return self._ws, n

    def __call__(self, pair_repr, pair_mask, out=None):
        import torch

        B, N, N2, D = pair_repr.shape
        if N2 != N or D != self.D or pair_repr.dtype != self.dtype or not pair_repr.is_contiguous():
            raise ValueError("pair_repr must be contiguous (B, N, N, D) in the handle's dtype")
        if pair_mask.shape != (B, N, N) or pair_mask.dtype != torch.uint8 or not pair_mask.is_contiguous():
            raise ValueError("pair_mask must be contiguous uint8 (B, N, N)")
        if out is None:
            out = torch.empty_like(pair_repr)
        ws, n = self.workspace(B, N)
        tri_attn_forward(self.handle, pair_repr, pair_mask, out, B, N, ws, n,
                         torch.cuda.current_stream(self.device))
        return out

    def close(self):
        if getattr(self, "handle", None):
            tri_attn_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
