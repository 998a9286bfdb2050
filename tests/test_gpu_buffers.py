"""Buffer discipline on the GPU, through the C ABI: every entry point writes
only inside the buffers it is given (canary bytes on both sides of the
output, lse, gradients and workspace stay intact), and a create whose device
allocation fails returns TRI_ATTN_ERR_OOM without leaking device memory."""
import numpy as np
import pytest
import torch

from gpu_helpers import Gpu, log
from triangular_pair_attention_amd import binding as B
from workloads import WEIGHT_NAMES, Workload, make_inputs

pytestmark = pytest.mark.gpu

CANARY = 0xA5
PAD = 4096  # bytes of canary on each side (keeps the 256-byte alignment)


class Padded:
    """A device buffer of `nbytes` with PAD canary bytes before and after it."""

    def __init__(self, nbytes, dev="cuda"):
        self.n = int(nbytes)
        self.raw = torch.full((self.n + 2 * PAD,), CANARY, dtype=torch.uint8, device=dev)

    @property
    def ptr(self):
        return self.raw.data_ptr() + PAD

    def view(self, dtype, shape):
        return self.raw[PAD:PAD + self.n].view(dtype).view(shape)

    def intact(self):
        r = self.raw.cpu().numpy()
        return bool((r[:PAD] == CANARY).all() and (r[PAD + self.n:] == CANARY).all())


SHAPES = [((1, 70, 128, 4), "bf16", ("pad", 50)), ((2, 33, 64, 2), "f32", ("bernoulli", 0.8)),
          ((1, 300, 128, 8), "bf16", ("pad", 270)), ((1, 17, 128, 8), "f32", ("pad", 9))]
IDS = ["N70bf16", "B2N33f32", "N300bf16", "N17f32"]


def inputs(shape, dtype, mask, seed=90):
    Bn, N, D, h = shape
    return make_inputs(Workload("canary", Bn, N, D, h, dtype, mask, seed=seed + N))


@pytest.mark.parametrize("shape,dtype,mask", SHAPES, ids=IDS)
def test_forward_and_stages_stay_inside_their_buffers(shape, dtype, mask):
    g = Gpu(inputs(shape, dtype, mask))
    try:
        out = Padded(g.P.numel() * g.P.element_size())
        ws = Padded(g.ws_bytes)
        B.tri_attn_forward(g.handle, g.P, g.M, out.ptr, g.B, g.N, ws.ptr, ws.n)
        torch.cuda.synchronize()
        assert out.intact() and ws.intact()
        ref = g.forward()
        torch.cuda.synchronize()
        assert torch.equal(out.view(g.P.dtype, g.P.shape), ref)
        out2 = Padded(out.n)
        B.tri_attn_project(g.handle, g.P, g.M, g.B, g.N, ws.ptr, ws.n)
        B.tri_attn_attend(g.handle, g.B, g.N, ws.ptr, ws.n)
        B.tri_attn_output(g.handle, out2.ptr, g.B, g.N, ws.ptr, ws.n)
        torch.cuda.synchronize()
        assert out2.intact() and ws.intact()
        assert torch.equal(out2.view(g.P.dtype, g.P.shape), ref)
        log(f"canary forward {shape} {dtype}: intact")
    finally:
        g.close()


@pytest.mark.parametrize("shape,dtype,mask", SHAPES, ids=IDS)
def test_onepass_stays_inside_its_buffers(shape, dtype, mask):
    g = Gpu(inputs(shape, dtype, mask))
    try:
        n = B.tri_attn_onepass_workspace_size(g.handle, g.B, g.N)
        out = Padded(g.P.numel() * g.P.element_size())
        ws = Padded(n)
        B.tri_attn_forward_onepass(g.handle, g.P, g.M, out.ptr, g.B, g.N, ws.ptr, ws.n)
        torch.cuda.synchronize()
        assert out.intact() and ws.intact()
    finally:
        g.close()


@pytest.mark.parametrize("shape,dtype,mask", SHAPES, ids=IDS)
def test_training_forward_and_backward_stay_inside_their_buffers(shape, dtype, mask):
    inp = inputs(shape, dtype, mask)
    g = Gpu(inp)
    try:
        out = Padded(g.P.numel() * g.P.element_size())
        lse = Padded(g.B * g.N * g.h * g.N * 4)
        ws = Padded(g.ws_bytes)
        B.tri_attn_forward_train(g.handle, g.P, g.M, out.ptr, lse.ptr, g.B, g.N, 0.2, 11, 3, ws.ptr, ws.n)
        torch.cuda.synchronize()
        assert out.intact() and lse.intact() and ws.intact()
        shapes = {"d_pair_repr": g.P.shape, "d_ln_weight": (g.D,), "d_ln_bias": (g.D,), "d_w_query": (g.D, g.D),
                  "d_w_key": (g.D, g.D), "d_w_value": (g.D, g.D), "d_w_gate": (g.D, g.D), "d_b_gate": (g.D,),
                  "d_w_bias_proj": (g.h, g.D), "d_w_out": (g.D, g.D), "d_b_out": (g.D,)}
        grads = {k: Padded(int(np.prod(v)) * 4) for k, v in shapes.items()}
        nb = B.tri_attn_backward_workspace_size(g.handle, g.B, g.N)
        wsb = Padded(nb)
        dy = torch.randn(g.P.shape, device=g.dev).to(g.dt)
        B.tri_attn_backward_train(g.handle, g.P, g.M, dy, g.B, g.N, 0.2, 11, 3, {k: v.ptr for k, v in grads.items()},
                                  wsb.ptr, wsb.n)
        torch.cuda.synchronize()
        assert wsb.intact()
        for k, v in grads.items():
            assert v.intact(), k
            assert torch.isfinite(v.view(torch.float32, shapes[k])).all(), k
    finally:
        g.close()


def test_noalloc_stays_inside_its_output():
    g = Gpu(inputs((1, 70, 128, 4), "bf16", ("pad", 50)))
    try:
        out = Padded(g.P.numel() * g.P.element_size())
        B.tri_attn_forward_noalloc(g.handle, g.P, g.M, out.ptr, g.B, g.N)
        torch.cuda.synchronize()
        assert out.intact()
    finally:
        g.close()


def _create(inp):
    dt = torch.float32 if inp["dtype"] == "f32" else torch.bfloat16
    w = {k: torch.from_numpy(inp[k]).cuda().to(dt).contiguous() for k in WEIGHT_NAMES}
    D = int(inp["pair_repr"].shape[3])
    cfg = B.tri_attn_config(D, int(inp["num_heads"]), B.TRI_ATTN_F32 if inp["dtype"] == "f32" else B.TRI_ATTN_BF16,
                            1e-5, -1e9, 0)
    return B.tri_attn_create(cfg, w, torch.cuda.current_stream()), w


@pytest.mark.parametrize("dtype,nalloc", [("f32", 4), ("bf16", 3)])
def test_failed_device_allocation_in_create_returns_oom_and_leaks_nothing(dtype, nalloc):
    inp = inputs((1, 16, 128, 4), dtype, ("ones",))
    h, w = _create(inp)  # first create: runtime and static array set up before the baseline
    B.tri_attn_destroy(h)
    torch.cuda.synchronize()
    free0 = torch.cuda.mem_get_info()[0]
    for nth in range(1, nalloc + 1):
        for _ in range(20):
            B.tri_attn_set_alloc_fault(nth)
            with pytest.raises(B.TriAttnError) as e:
                _create(inp)
            assert e.value.code == B.TRI_ATTN_ERR_OOM
    torch.cuda.synchronize()
    free1 = torch.cuda.mem_get_info()[0]
    log(f"alloc fault {dtype}: device free memory {free0} -> {free1}")
    # 20 leaked handles per fault point would be well over 4 MB
    assert free0 - free1 < (4 << 20)
    # past the last allocation nothing fails, and the hook is disarmed after one create
    B.tri_attn_set_alloc_fault(nalloc + 1)
    h, _ = _create(inp)
    B.tri_attn_destroy(h)
    h, _ = _create(inp)
    B.tri_attn_destroy(h)
    with pytest.raises(B.TriAttnError) as e:
        B.tri_attn_set_alloc_fault(-1)
    assert e.value.code == B.TRI_ATTN_ERR_INVALID_ARG
