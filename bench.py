#!/usr/bin/env python3
"""Benchmark of the starting-node triangular self-attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config k]

A step is one tri_attn_forward (kernel 1: LayerNorm + fused projection;
kernel 2: attention + gate; kernel 3: output projection) over one batch of
seeded synthetic inputs already resident in HBM. Prints ONE JSON line.

The default workload is the largest of the five: B=4, N=512, D=128, h=8
(d=16), bf16 storage with float32 accumulation, a per-batch valid length
L_b in [384, 512] masking the trailing rows and columns. `--config k`
selects another of the five workloads (1..5). Each kernel is also timed
through its stage entry point (tri_attn_project / tri_attn_attend /
tri_attn_output), one launch at a time between HIP events on the stream it
runs on, each on the data its predecessors just wrote; the slowest one is
reported in `roofline`.

`--copy-probe` runs only a plain device copy of a known size (the reference
for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE counters to bytes).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "pair-positions/sec + TFLOP/s, triangular-attn fwd; % MFMA/HBM roofline"
PEAK = {  # MI355X published dense peaks
    "hbm_GBps": 8000.0,
    "mfma_f32_TFLOPs": 157.3,
    "mfma_bf16_TFLOPs": 2500.0,
    "valu_f32_TFLOPs": 157.3,  # fp32 vector FMA (packed), 256 CUs at 2.4 GHz
}
# Rates measured on one MI355X by triangular_pair_attention_amd/calib/calib.hip
# (tri_attn_calib): the attention kernel's exponentials and matrix-core work
# do not overlap, so its floor is the sum of the two at these rates.
CALIB = {
    "v_exp_f32_Gops": 13224.7,
    "mfma_bf16_random_TFLOPs": 1655.4,
    "mfma_f32_random_TFLOPs": 148.2,
}
KERNEL_SOURCES = {
    "k1_ln_proj": "triangular_pair_attention_amd/csrc/k1_ln_proj.hip",
    "k2_attention": "triangular_pair_attention_amd/csrc/k2_attention.hip",
    "k3_out_proj": "triangular_pair_attention_amd/csrc/k3_out_proj.hip",
}
# kernels of the one-pass variant (tri_attn_forward_onepass)
VARIANT_SOURCES = {
    "op_bias": "triangular_pair_attention_amd/csrc/onepass.hip",
    "op_fused": "triangular_pair_attention_amd/csrc/onepass.hip",
}
# float32 tensors run kernel 1 from its own source (split products)
F32_SOURCES = {"k1_ln_proj": "triangular_pair_attention_amd/csrc/k1_split.hip"}
# float32 kernels whose products run as six bf16 products each (three-way split
# operands): their matrix-core ceiling is the bf16 peak / 6
SPLIT_KERNELS = ("k1_ln_proj", "k3_out_proj")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.md")


def _code_only(text: str) -> str:
    """Source text without comments and with whitespace collapsed, so that a
    comment edit does not invalidate counters taken on the same code."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source(kernel: str, dtype: str = "bf16") -> str:
    src = KERNEL_SOURCES.get(kernel) or VARIANT_SOURCES[kernel]
    return F32_SOURCES.get(kernel, src) if dtype == "f32" else src


def source_hash(kernel: str, dtype: str = "bf16") -> str:
    """sha256 (first 16 hex digits) of the kernel's code and device_common.h."""
    h = hashlib.sha256()
    for rel in (kernel_source(kernel, dtype), "triangular_pair_attention_amd/csrc/device_common.h"):
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
    return h.hexdigest()[:16]


def work_model(w):
    """Algorithmic flops and bytes of each kernel per launch (dense counts)."""
    B, N, D, h = w.B, w.N, w.D, w.h
    s = 2 if w.dtype == "bf16" else 4
    P = B * N * N
    return {
        "positions": P,
        # LayerNorm + projection: read pair_repr and mask, write q, k, v, gate and the fp32 bias+mask tile
        "k1_ln_proj": {"flops": 2 * P * D * (4 * D + h), "bytes": P * D * s + P + 4 * P * D * s + 4 * B * h * N * N},
        # attention: q.k and p.v; read q, k, v, gate and the bias tile once, write g*o
        "k2_attention": {"flops": 4 * B * N ** 3 * D, "bytes": 4 * P * D * s + 4 * B * h * N * N + P * D * s},
        # output projection: read g*o, write y
        "k3_out_proj": {"flops": 2 * P * D * D, "bytes": 2 * P * D * s},
        # one-pass variant: the bias pre-pass reads pair_repr and the mask and
        # writes the float32 bias+mask tile; the fused row kernel reads
        # pair_repr and that tile once and writes y
        "op_bias": {"flops": 2 * P * D * h, "bytes": P * D * s + P + 4 * B * h * N * N},
        "op_fused": {"flops": 2 * P * D * 4 * D + 4 * B * N ** 3 * D + 2 * P * D * D,
                     "bytes": 2 * P * D * s + 4 * B * h * N * N},
    }


def roofline_of(kernel, w, m, ms, mask=None):
    """The bound of one kernel: HBM where its arithmetic intensity is below the
    ridge of its dtype's matrix-core peak, else the matrix cores. For the
    attention kernel with a mask, `achieved` counts the valid (j, k) score
    pairs only (the work that must be computed); the dense rate is kept as
    `achieved_dense`."""
    mfma = PEAK["mfma_f32_TFLOPs"] if w.dtype == "f32" else PEAK["mfma_bf16_TFLOPs"]
    ridge = mfma * 1e12 / (PEAK["hbm_GBps"] * 1e9)
    fl, by = m[kernel]["flops"], m[kernel]["bytes"]
    if kernel != "k2_attention" and fl / by < ridge:
        r = {"bound": "hbm", "achieved": by / (ms * 1e-3) / 1e9, "peak": PEAK["hbm_GBps"], "unit": "GB/s"}
    else:
        r = {"bound": "mfma", "achieved": fl / (ms * 1e-3) / 1e12, "peak": mfma, "unit": "TFLOP/s"}
    r["frac"] = r["achieved"] / r["peak"]
    if kernel == "k2_attention" and mask is not None:
        # the work that must be computed: the valid (j, k) score pairs only
        # (a fully masked query column has a closed form); `achieved` and
        # `frac` count those, the dense counts stay beside them
        valid = int((mask != 0).sum())  # (b, j, k) pairs, each scored for all N rows i
        r["achieved_dense"], r["frac_dense"] = r["achieved"], r["frac"]
        r["achieved"] = 4 * w.N * w.D * valid / (ms * 1e-3) / 1e12
        r["frac"] = r["achieved"] / r["peak"]
        r["count"] = "valid (j, k) score pairs"
    if w.dtype == "f32" and kernel in SPLIT_KERNELS and r["bound"] == "mfma":
        # the matrix cores run six bf16 products per float32 product
        ceil = PEAK["mfma_bf16_TFLOPs"] / 6
        r["split_products"] = {"bf16_products_per_f32_product": 6, "ceiling": ceil,
                               "frac_of_ceiling": r["achieved"] / ceil}
    return r


def attention_floor(w, m, ms, mask=None):
    """Kernel 2 against its binding floor: the exponentials (one per score,
    B*h*N^3) plus the matrix-core work at the calibrated rates, serially.
    With a mask, also the TFLOP/s on the valid (j, k) score pairs only."""
    B, N, h = w.B, w.N, w.h
    exps = B * h * N ** 3
    mfma = CALIB["mfma_f32_random_TFLOPs"] if w.dtype == "f32" else CALIB["mfma_bf16_random_TFLOPs"]
    t_exp = exps / (CALIB["v_exp_f32_Gops"] * 1e9)
    t_mfma = m["k2_attention"]["flops"] / (mfma * 1e12)
    r = {"exps": exps, "exp_Gops": exps / (ms * 1e-3) / 1e9, "floor_ms": (t_exp + t_mfma) * 1e3,
         "frac_of_floor": (t_exp + t_mfma) * 1e3 / ms}
    if mask is not None:
        valid = int((mask != 0).sum())  # (b, j, k) pairs, each scored for all N rows i
        r["valid_tflops"] = 4 * N * w.D * valid / (ms * 1e-3) / 1e12
    return r


def stored_traffic(workload: str, kernel: str, dtype: str = "bf16"):
    """HBM bytes per launch from the committed rocprofv3 counter runs (the
    table in profiles/hbm_traffic.md), if they were taken on the current
    kernel source; else None. Table row:
    | workload | kernel | source sha256[:16] | FETCH_SIZE KiB | WRITE_SIZE KiB | fetch scale | write scale |"""
    try:
        with open(TRAFFIC_FILE) as f:
            lines = f.read().splitlines()
    except OSError:
        return None
    for line in lines:
        cells = [c.strip() for c in line.strip().strip("|").split("|")]
        if len(cells) != 7 or cells[0] != workload or cells[1] != kernel:
            continue
        if cells[2] != source_hash(kernel, dtype):
            return None
        try:
            fetch, write, fs, ws = (float(c) for c in cells[3:7])
        except ValueError:
            return None
        return fetch * 1024 * fs + write * 1024 * ws
    return None


def cpu_baseline(inp, w, seconds, ending_node=False):
    """The oracle as it stands, on the host's cores: all N rows of batch 0
    (all N columns for the ending-node variant), one contiguous chunk of rows
    per worker process (each worker computes its batch's LayerNorm and pair
    bias once per pass, as one oracle call does), passes repeated until
    `seconds` elapse. `cores` is the number of worker processes, each
    single-threaded. A short single-process run is reported beside it."""
    from oracle import pool
    from oracle.tri_attn_oracle import forward_ending_cols, forward_rows

    rows = [(0, i) for i in range(w.N)]
    r = pool.time_rows(inp, rows, seconds, ending=ending_node)
    pos = r["rows"] * w.N
    what = "columns" if ending_node else "rows"
    result = {
        "value": pos / r["seconds"],
        "unit": "pair-positions/s",
        "cores": r["workers"],
        "kind": "oracle",
        "sample": f"{r['passes']} x all {w.N} {what} of batch 0 of {w.name} ({pos} pair positions, "
                  f"{r['seconds']:.1f} s wall; float64 numpy on {r['workers']} worker processes, one BLAS "
                  f"thread each, one contiguous chunk of {what} per worker per pass)",
    }
    fn = forward_ending_cols if ending_node else forward_rows
    try:
        from threadpoolctl import threadpool_limits
    except Exception:
        return result
    sub = rows[:8]
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        fn(inp, sub)
        el = time.perf_counter() - t0
    result["single_process"] = {
        "value": len(sub) * w.N / el, "unit": "pair-positions/s", "cores": 1,
        "sample": f"the first {len(sub)} {what} of batch 0 in one oracle call on one thread, with their batch's "
                  f"LayerNorm and pair bias ({len(sub) * w.N} pair positions, {el:.1f} s)",
    }
    return result


def copy_probe(mib: int = 256, reps: int = 5):
    import torch

    a = torch.empty(mib << 20, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty_like(a)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": mib << 20, "reps": reps}))


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=5, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-train", action="store_true", help="skip timing the training-mode forward")
    ap.add_argument("--copy-probe", action="store_true")
    ap.add_argument("--ending-node", action="store_true",
                    help="the ending-node variant (attention along the other residue axis)")
    ap.add_argument("--peaked", type=float, default=1.0,
                    help="scale the query and pair-bias weights by this factor (peaked softmax: a looser "
                         "bound for the attention kernel's shift; the share of recomputed items is reported)")
    ap.add_argument("--no-onepass", action="store_true", help="skip timing the one-pass variant")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build runs on one GPU only; the multi-GPU path is a design "
              "(row sharding with an all-gather of the pair bias), not built. Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_probe:
        copy_probe()
        return

    from triangular_pair_attention_amd import binding as B
    from workloads import WEIGHT_NAMES, WORKLOADS, make_inputs

    w = WORKLOADS[args.config]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    dt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    inp = make_inputs(w)
    if args.peaked != 1.0:
        inp["w_query"] = inp["w_query"] * args.peaked
        inp["w_bias_proj"] = inp["w_bias_proj"] * args.peaked
    wname = w.name + ("_ending_node" if args.ending_node else "")
    weights = {k: torch.from_numpy(inp[k]).to(dev).to(dt).contiguous() for k in WEIGHT_NAMES}
    P = torch.from_numpy(inp["pair_repr"]).to(dev).to(dt).contiguous()
    M = torch.from_numpy(inp["pair_mask"]).to(dev).contiguous()
    out = torch.empty_like(P)
    stream = torch.cuda.current_stream(dev)
    cfg = B.tri_attn_config(w.D, w.h, B.TRI_ATTN_F32 if w.dtype == "f32" else B.TRI_ATTN_BF16, 1e-5, -1e9,
                            int(args.ending_node))
    h = B.tri_attn_create(cfg, weights, stream)
    nws = B.tri_attn_workspace_size(h, w.B, w.N)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev)

    def fwd():
        B.tri_attn_forward(h, P, M, out, w.B, w.N, ws, nws, stream)

    def k1():
        B.tri_attn_project(h, P, M, w.B, w.N, ws, nws, stream)

    def k2():
        B.tri_attn_attend(h, w.B, w.N, ws, nws, stream)

    def k3():
        B.tri_attn_output(h, out, w.B, w.N, ws, nws, stream)

    def timed(fn, steps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps  # ms per call

    for _ in range(args.warmup):
        fwd()
    torch.cuda.synchronize()
    # the timed region: exactly `steps` forwards, synchronised on both sides
    t0 = time.perf_counter()
    ms_fwd_ev = timed(fwd, args.steps)
    wall = time.perf_counter() - t0
    ms_fwd = max(ms_fwd_ev, 0.0)
    # the attention work items of the last forward that found their softmax
    # bound too loose and were recomputed with the exact maximum
    lay = B.tri_attn_get_workspace_layout(h, w.B, w.N)
    flags = ws[lay.recover_flags:lay.recover_flags + lay.attention_items].cpu()
    recovery = {"items": lay.attention_items, "recovered": int(flags.sum()),
                "recovered_fraction": float(flags.float().mean())}
    # each kernel alone through its stage entry point, for the roofline: one
    # launch at a time between HIP events on the kernels' stream, each on the
    # data its predecessors just wrote (the attention kernel consumes the gate
    # region, so every timed attention or output launch follows fresh
    # projections, as inside a forward)
    def per_launch(before, fn, steps):
        tot = 0.0
        for _ in range(steps):
            before()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            e1.synchronize()
            tot += e0.elapsed_time(e1)
        return tot / steps

    nk = max(10, min(args.steps, 200))
    ms_k1 = per_launch(lambda: None, k1, nk)
    ms_k2 = per_launch(k1, k2, nk)
    ms_k3 = per_launch(lambda: (k1(), k2()), k3, nk)
    torch.cuda.synchronize()
    # the same forward replayed from a captured HIP graph (a serving loop's
    # launch path), for comparison; `value` stays the direct forward call
    ms_graph = None
    try:
        side = torch.cuda.Stream(dev)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            B.tri_attn_forward(h, P, M, out, w.B, w.N, ws, nws, side)
        stream.wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            B.tri_attn_forward(h, P, M, out, w.B, w.N, ws, nws, torch.cuda.current_stream(dev))
        for _ in range(args.warmup):
            graph.replay()
        ms_graph = timed(graph.replay, args.steps)
        del graph
    except RuntimeError as e:  # capture unsupported: report no graph timing
        print(f"bench.py: graph timing skipped ({e})", file=sys.stderr)
    torch.cuda.synchronize()
    # cold: a 512 MiB buffer is written before every timed forward, so that
    # neither the MALL (256 MB) nor the L2 caches hold the inputs
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    reps = max(5, min(50, args.steps // 10))
    cold = 0.0
    for _ in range(reps):
        flush.fill_(1)
        c0 = torch.cuda.Event(enable_timing=True)
        c1 = torch.cuda.Event(enable_timing=True)
        c0.record(stream)
        fwd()
        c1.record(stream)
        torch.cuda.synchronize()
        cold += c0.elapsed_time(c1)
    ms_cold = cold / reps
    del flush
    # the training-mode forward (dropout 0.1, log-sum-exp saved) on the same
    # workload, for comparison; `value` stays the inference forward
    train = None
    if not args.ending_node and not args.no_train:
        lse = torch.empty((w.B, w.N, w.h, w.N), dtype=torch.float32, device=dev)

        def trn():
            B.tri_attn_forward_train(h, P, M, out, lse, w.B, w.N, 0.1, 12345, 0, ws, nws, stream)

        for _ in range(3):
            trn()
        ms_train = timed(trn, max(1, args.steps // 5))
        train = {"dropout_rate": 0.1, "ms_per_step": ms_train, "ratio_to_inference": ms_train / ms_fwd}
        del lse
        # the backward (all gradients) of the same training step
        nbw = B.tri_attn_backward_workspace_size(h, w.B, w.N)
        wsb = torch.empty(nbw, dtype=torch.uint8, device=dev)
        shapes = {"d_pair_repr": P.shape, "d_ln_weight": (w.D,), "d_ln_bias": (w.D,), "d_w_query": (w.D, w.D),
                  "d_w_key": (w.D, w.D), "d_w_value": (w.D, w.D), "d_w_gate": (w.D, w.D), "d_b_gate": (w.D,),
                  "d_w_bias_proj": (w.h, w.D), "d_w_out": (w.D, w.D), "d_b_out": (w.D,)}
        grads = {k: torch.empty(v, dtype=torch.float32, device=dev) for k, v in shapes.items()}
        dy = torch.randn(P.shape, device=dev, dtype=torch.float32).to(dt)

        def bwd():
            B.tri_attn_backward_train(h, P, M, dy, w.B, w.N, 0.1, 12345, 0, grads, wsb, nbw, stream)

        bwd()
        train["backward_ms_per_step"] = timed(bwd, 2)
        train["backward_workspace_bytes"] = nbw
        del wsb, grads, dy
    # the one-pass variant (bias pre-pass, then one fused kernel per pair row)
    onepass = None
    if not args.no_onepass and w.N <= 512:
        nop = B.tri_attn_onepass_workspace_size(h, w.B, w.N)
        wso = torch.empty(max(nop, 256), dtype=torch.uint8, device=dev)

        def op():
            B.tri_attn_forward_onepass(h, P, M, out, w.B, w.N, wso, nop, stream)

        for _ in range(3):
            op()
        ms_op = timed(op, max(1, args.steps // 5))
        s_ = 2 if w.dtype == "bf16" else 4
        tb = [stored_traffic(wname, k, w.dtype) for k in VARIANT_SOURCES]
        t3 = [stored_traffic(wname, k, w.dtype) for k in KERNEL_SOURCES]
        onepass = {"ms_per_step": ms_op, "value": w.B * w.N * w.N / (ms_op * 1e-3),
                   "ratio_to_three_kernel": ms_op / ms_fwd,
                   "hbm_bytes": None if None in tb else sum(tb),
                   "three_kernel_hbm_bytes": None if None in t3 else sum(t3),
                   "min_bytes": 2 * w.B * w.N * w.N * w.D * s_ + w.B * w.N * w.N}
        del wso
    torch.cuda.synchronize()
    B.tri_attn_destroy(h)

    m = work_model(w)
    pos_per_s = m["positions"] / (ms_fwd * 1e-3)
    total_flops = sum(m[k]["flops"] for k in KERNEL_SOURCES)
    tflops = total_flops / (ms_fwd * 1e-3) / 1e12
    ms_k = {"k1_ln_proj": ms_k1, "k2_attention": ms_k2, "k3_out_proj": ms_k3}
    dom = max(ms_k, key=ms_k.get)
    roof = roofline_of(dom, w, m, ms_k[dom], inp["pair_mask"])
    roof["traffic"] = stored_traffic(wname, dom, w.dtype)
    roof["kernel"] = dom
    roof["kernel_ms"] = ms_k[dom]

    result = {
        "metric": METRIC,
        "value": pos_per_s,
        "unit": "pair-positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_fwd,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if w.dtype == "f32" else "bf16",
        "data": "synthetic",
        "config": {"workload": wname + (f"_peaked{args.peaked:g}" if args.peaked != 1.0 else ""), "B": w.B,
                   "N": w.N, "D": w.D, "h": w.h, "d": w.d, "mask": list(w.mask), "seed": w.seed,
                   "peaked": args.peaked,
                   "variant": "ending-node" if args.ending_node else "starting-node",
                   "parallelism": "none (1 GPU)"},
        "tflops": tflops,
        "ms_per_step_graph_replay": ms_graph,
        "ms_per_step_cold": ms_cold,
        "kernels_ms": ms_k,
        "kernels_roofline": {k: roofline_of(k, w, m, v, inp["pair_mask"]) for k, v in ms_k.items()},
        "attention_floor": attention_floor(w, m, ms_k2, inp["pair_mask"]),
        "wall_s_timed": wall,
        "roofline": roof,
        "train": train,
        "onepass": onepass,
        "recovery": recovery,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(inp, w, args.cpu_seconds, args.ending_node)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
