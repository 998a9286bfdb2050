"""Helpers shared by the GPU tests: move seeded inputs to the device, run the
library through its C ABI, and compare with the oracle."""
import math
import sys

import numpy as np
import torch

from triangular_pair_attention_amd import binding as B
from workloads import WEIGHT_NAMES

TOL = {"f32": 1e-4, "bf16": 2e-2}  # max abs error on y


def torch_dtype(name):
    return torch.float32 if name == "f32" else torch.bfloat16


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


class Gpu:
    """One library handle built from seeded inputs (numpy dict from workloads)."""

    def __init__(self, inp, fill=-1e9, slack=0.0, device="cuda", ending=False):
        self.inp = inp
        self.dt = torch_dtype(inp["dtype"])
        self.dev = torch.device(device)
        self.w = {k: torch.from_numpy(inp[k]).to(self.dev).to(self.dt).contiguous() for k in WEIGHT_NAMES}
        P = inp["pair_repr"]
        self.B, self.N = int(P.shape[0]), int(P.shape[1])
        self.D, self.h = int(P.shape[3]), int(inp["num_heads"])
        self.P = torch.from_numpy(P).to(self.dev).to(self.dt).contiguous()
        self.M = torch.from_numpy(inp["pair_mask"]).to(self.dev).contiguous()
        code = B.TRI_ATTN_F32 if inp["dtype"] == "f32" else B.TRI_ATTN_BF16
        self.cfg = B.tri_attn_config(self.D, self.h, code, 1e-5, fill if math.isfinite(fill) else -math.inf,
                                     int(ending))
        self.handle = B.tri_attn_create(self.cfg, self.w, torch.cuda.current_stream())
        if slack:
            B.tri_attn_set_shift_slack(self.handle, slack)
        self.ws_bytes = B.tri_attn_workspace_size(self.handle, self.B, self.N)
        self.ws = torch.empty(max(self.ws_bytes, 256), dtype=torch.uint8, device=self.dev)

    def forward(self, out=None, stream=None):
        if out is None:
            out = torch.empty_like(self.P)
        B.tri_attn_forward(self.handle, self.P, self.M, out, self.B, self.N, self.ws, self.ws_bytes,
                           stream or torch.cuda.current_stream())
        return out

    def project(self):
        B.tri_attn_project(self.handle, self.P, self.M, self.B, self.N, self.ws, self.ws_bytes,
                           torch.cuda.current_stream())
        torch.cuda.synchronize()
        return B.tri_attn_get_workspace_layout(self.handle, self.B, self.N)

    def k_region(self, lay):
        """k from the workspace as float64 [B, N, N(key), D]: float32 handles
        with d = 32 hold it as three bf16 parts [b][i][t][p][s][G][r][e]
        (channel 8G + e of head t, key 16s + r), summed here exactly."""
        Bn, N, D, h, Np = self.B, self.N, self.D, self.h, lay.padded_n
        if self.inp["dtype"] == "f32" and D // h == 32:
            raw = self.region(lay.k, Bn * N * D * Np * 3, torch.int16).cpu().numpy().astype(np.uint16)
            parts = (raw.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
            parts = parts.reshape(Bn, N, h, 3, Np // 16, 4, 16, 8).sum(3)  # b i t s G r e
            k = parts.transpose(0, 1, 3, 5, 2, 4, 6).reshape(Bn, N, Np, D)  # b i (s r) (t G e)
            return k[:, :, :N]
        k = self.region(lay.k, Bn * N * D * Np, self.dt).float().cpu().numpy().astype(np.float64)
        return k.reshape(Bn, N, D // 16, Np, 16)[:, :, :, :N].transpose(0, 1, 3, 2, 4).reshape(Bn, N, N, D)

    def region(self, off, count, dtype):
        elem = torch.tensor([], dtype=dtype).element_size()
        return self.ws[off:off + count * elem].view(dtype)

    def close(self):
        if self.handle:
            B.tri_attn_destroy(self.handle)
            self.handle = None


def y_numpy(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def max_err(a, b):
    d = np.abs(a - b)
    i = np.unravel_index(np.argmax(d), d.shape)
    return float(d[i]), i
