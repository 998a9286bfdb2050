"""The allocation-free forward (tri_attn_forward_noalloc, workspace in the
library's static device array) against tri_attn_forward with a caller
workspace: same kernels, so the same bits; two calls in a row on one handle,
the second smaller, so the shared array carries the first call's contents
into the second; and the size limit."""
import numpy as np
import pytest
import torch

from gpu_helpers import TOL, Gpu, log, y_numpy
from triangular_pair_attention_amd import binding as B
from workloads import WORKLOADS, Workload, make_inputs

pytestmark = pytest.mark.gpu

MAX_BYTES = 256 << 20  # TRI_ATTN_NOALLOC_MAX_BYTES


def _pair(w):
    """(forward output, noalloc output) of one workload on one handle."""
    inp = make_inputs(w)
    g = Gpu(inp)
    try:
        assert g.ws_bytes <= MAX_BYTES
        ref = g.forward()
        out = torch.full_like(g.P, float("nan"))
        B.tri_attn_forward_noalloc(g.handle, g.P, g.M, out, g.B, g.N, torch.cuda.current_stream())
        torch.cuda.synchronize()
        return ref, out, inp
    finally:
        g.close()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_equals_forward_twice_second_smaller(dtype):
    big = Workload("noalloc_big", 2, 160, 128, 8 if dtype == "bf16" else 4, dtype, ("pad_range", 120, 160), 31)
    small = Workload("noalloc_small", 1, 37, 128, 8 if dtype == "bf16" else 4, dtype, ("bernoulli", 0.8), 32)
    for w in (big, small):
        log(f"noalloc {dtype} B={w.B} N={w.N}")
        ref, out, inp = _pair(w)
        assert torch.equal(out, ref), f"{w.name}: noalloc output differs from the forward's"
        # and within the parity bar of the oracle-checked forward
        assert float(np.abs(y_numpy(out) - y_numpy(ref)).max()) <= TOL[dtype]


def test_noalloc_on_one_handle_two_sizes():
    """One handle, the larger problem then a smaller one (the array keeps the
    larger call's bytes beyond the smaller call's workspace)."""
    w = WORKLOADS[3]  # B=1, N=256, bf16, workspace about 68 MB
    inp = make_inputs(w)
    g = Gpu(inp)
    try:
        st = torch.cuda.current_stream()
        out = torch.empty_like(g.P)
        B.tri_attn_forward_noalloc(g.handle, g.P, g.M, out, g.B, g.N, st)
        ref = g.forward()
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        n = 100
        P2 = g.P[:, :n, :n].contiguous()
        M2 = g.M[:, :n, :n].contiguous()
        out2 = torch.empty_like(P2)
        B.tri_attn_forward_noalloc(g.handle, P2, M2, out2, g.B, n, st)
        ws2 = torch.empty(B.tri_attn_workspace_size(g.handle, g.B, n), dtype=torch.uint8, device=g.dev)
        ref2 = torch.empty_like(P2)
        B.tri_attn_forward(g.handle, P2, M2, ref2, g.B, n, ws2, ws2.numel(), st)
        torch.cuda.synchronize()
        assert torch.equal(out2, ref2)
    finally:
        g.close()


def test_noalloc_rejects_sizes_past_the_array():
    w = Workload("noalloc_limit", 1, 8, 128, 8, "bf16", ("ones",), 33)
    g = Gpu(make_inputs(w))
    try:
        # B=4, N=512 needs about 1.1 GB of workspace: refused before any launch
        need = B.tri_attn_workspace_size(g.handle, 4, 512)
        assert need > MAX_BYTES
        with pytest.raises(B.TriAttnError) as e:
            B.tri_attn_forward_noalloc(g.handle, 0, 0, 0, 4, 512)
        assert e.value.code == B.TRI_ATTN_ERR_WORKSPACE
        B.tri_attn_forward_noalloc(g.handle, 0, 0, 0, 0, 512)  # empty: no-op
        torch.cuda.synchronize()
    finally:
        g.close()
