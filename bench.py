"""Benchmark of the MoE expert hot path on one MI355X.

A step is one pass of the path over one batch of the skewed ~35B-A3B-shaped
layer (T=8192 tokens, H=2048, E=256 experts, top-8, I=512, Zipf(1.2)-biased
routing): moe_permute -> moe_grouped_gemm_swiglu -> moe_unpermute_combine ->
moe_unpermute_grad (backward of the combine). Inputs are synthetic and
resident in HBM before timing starts. `value` is tokens/s of that step.

The same run also times every call at the other workloads (permute/combine
at T=4096 H=2048 E=64 K=6; reorder + special-expert combine of the R=8 x 32
receive buffer; the unpermute backward at T=16384 H=4096), each after a 1 GiB
read that flushes the caches before every timed launch, and the CPU oracle on a bounded sample
of the layer workload (`cpu_baseline`). One JSON line goes to stdout.

    python bench.py [--steps K] [--warmup W] [--no-ops] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
BF16_DENSE_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, published
METRIC = "MoE layer tokens/s; permute/combine HBM GB/s; grouped-GEMM TFLOP/s"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # the first ~25 steps after setup run about 7 % slower than the steady
    # state (0.889 against 0.825 ms per step), so the default warms up past them
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--op-iters", type=int, default=20)
    ap.add_argument("--no-ops", action="store_true", help="skip the per-workload op table")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=6144)
    ap.add_argument("--copy-probe", type=int, default=0, metavar="N",
                    help="only run N device copies of 256 MiB (counter calibration) and exit")
    return ap.parse_args()


# ----------------------------------------------------------------------------- helpers

def dbf(a, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)) \
        .view(torch.bfloat16).to(dev)


def dt(a, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


class Flusher:
    """Reads 1 GiB between timed launches, so no input sits in the 256 MB
    Infinity Cache or the L2s when a timed launch starts and no dirty line is
    left there either: a flush that writes (a 1 GiB fill) leaves up to the
    caches' size in dirty lines, whose write-back to HBM then lands inside the
    next timed launch and is charged to it."""

    def __init__(self, dev):
        import torch
        self.buf = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        self.sink = torch.empty((), dtype=torch.float32, device=dev)

    def __call__(self):
        import torch
        torch.sum(self.buf, dim=0, out=self.sink)


def time_op(fn, iters, flush=None, warm=2):
    """Median / min device time (us) of fn() bracketed by events on the current stream."""
    import torch
    for _ in range(warm):
        fn()
    times = []
    for _ in range(iters):
        if flush is not None:
            flush()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        b.synchronize()
        times.append(a.elapsed_time(b) * 1e3)
    return float(np.median(times)), float(np.min(times))


def op_entry(name, us_med, us_min, nbytes=None, flops=None):
    e = {"op": name, "us_median": round(us_med, 2), "us_min": round(us_min, 2)}
    if nbytes is not None:
        gbs = nbytes / (us_med * 1e-6) / 1e9
        e.update(algorithmic_bytes=int(nbytes), gbs=round(gbs, 1),
                 hbm_frac=round(gbs / HBM_PEAK_GBS, 4))
    if flops is not None:
        tf = flops / (us_med * 1e-6) / 1e12
        e.update(flops=int(flops), tflops=round(tf, 1),
                 mfma_frac=round(tf / BF16_DENSE_PEAK_TFLOPS, 4))
    return e


# ----------------------------------------------------------------------------- algorithmic work

def permute_bytes(T, K, H, N):
    return T * K * 4 + T * H * 2 + N * H * 2 + 2 * T * K * 4 + 0


def row_move_bytes(T, K, H, N):
    """x read once, N rows written, the routing read."""
    return T * H * 2 + N * H * 2 + T * K * 4


def combine_bytes(T, K, H, N, extra_rows=0):
    return N * H * 2 + 3 * T * K * 4 + T * H * 2 + extra_rows * H * 2


def grad_bytes(T, K, H, N):
    return T * H * 2 + 2 * N * H * 2 + 2 * T * K * 4 + T * K * 4


def permute_grad_bytes(T, K, H, N):
    return N * H * 2 + T * K * 4 + T * H * 2


def combine_grad_bytes(T, K, H, N, n_routed, need_ori, num_const):
    """grad_out read; each routed row read and its gradient written; ori_x read
    where a copy / const slot needs it; d_ori_x written for every token; the
    slot metadata, row map and d_probs; const_v read and its gradient written;
    per-token alpha read and its gradient written."""
    return (T * H * 2 + 2 * n_routed * H * 2 + need_ori * H * 2 + T * H * 2 + 3 * T * K * 4
            + N * 4 + T * K * 4 + 2 * num_const * H * 2 + 4 * T * 4)


def reorder_bytes(N, H):
    return 2 * N * H * 2 + 2 * N * 4


def gemm_flops(N, H, I):
    return 6 * N * H * I


def gemm_bytes(N, H, I, active_experts):
    """x read, h written and read back, y written, and the gate/up/down weights
    of every expert that owns at least one row (each counted once)."""
    return 2 * (N * H + 2 * N * I + N * H) + active_experts * 3 * H * I * 2


def gemm_traffic_record():
    """HBM bytes per grouped-GEMM call measured by rocprofv3 counters, if the
    kernel source is unchanged since they were taken (else None)."""
    import hashlib
    rec_path = os.path.join(ROOT, "profiles", "gemm_traffic_skewed_layer.json")
    try:
        rec = json.load(open(rec_path))
        src = open(os.path.join(ROOT, rec["source"]), "rb").read()
    except (OSError, ValueError, KeyError):
        return None
    if hashlib.sha256(src).hexdigest() != rec.get("source_sha256"):
        return None
    return rec


# ----------------------------------------------------------------------------- the layer step

def layer_setup(dev):
    import torch
    import moe_workloads as W
    import unpermute_combine_moe_amd as moe

    g = W.gen_c3()
    c = g["cfg"]
    T, H, E, K, I = c["T"], c["H"], c["E"], c["K"], c["I"]
    S = T * K
    d = dict(cfg=c, host=g)
    d["x"] = dbf(g["x"], dev)
    d["ids"] = dt(g["expert_ids"], dev)
    d["probs"] = dt(g["probs"], dev)
    d["wg"], d["wu"], d["wd"] = (dbf(g[k], dev) for k in ("w_gate", "w_up", "w_down"))
    d["grad_out"] = dbf(W.normal_bf16(W.rng_for(3 * 1000 + 7), (T, H)), dev)
    bf = torch.bfloat16
    d["permuted"] = torch.empty((S, H), dtype=bf, device=dev)
    d["sorted_slot"] = torch.empty(S, dtype=torch.int32, device=dev)
    d["row_of_slot"] = torch.empty((T, K), dtype=torch.int32, device=dev)
    d["counts"] = torch.empty(E, dtype=torch.int32, device=dev)
    d["offsets"] = torch.empty(E + 1, dtype=torch.int32, device=dev)
    d["h"] = torch.empty((S, I), dtype=bf, device=dev)
    d["y"] = torch.empty((S, H), dtype=bf, device=dev)
    d["out"] = torch.empty((T, H), dtype=bf, device=dev)
    d["d_perm"] = torch.empty((S, H), dtype=bf, device=dev)
    d["d_probs"] = torch.empty((T, K), dtype=torch.float32, device=dev)
    d["ws_p"] = moe.workspace(moe.moe_permute_workspace_size(T, K, E), dev)
    d["ws_g"] = moe.workspace(moe.moe_grouped_gemm_swiglu_workspace_size(E, S, H, I), dev)
    return d


def step_calls(d):
    import unpermute_combine_moe_amd as moe

    c = d["cfg"]
    T, H, E, K, I = c["T"], c["H"], c["E"], c["K"], c["I"]
    S = T * K

    def permute():
        moe.moe_permute(d["x"], d["ids"], T, H, K, E, d["permuted"], d["sorted_slot"],
                        d["row_of_slot"], d["counts"], d["offsets"], d["ws_p"])

    def gemm():
        moe.moe_grouped_gemm_swiglu(d["permuted"], d["offsets"], E, S, H, I, d["wg"], d["wu"],
                                    d["wd"], d["h"], d["y"], d["ws_g"])

    def combine():
        moe.moe_unpermute_combine(d["y"], S, d["row_of_slot"], None, d["ids"], d["probs"], T, K, H,
                                  E, None, None, d["out"])

    def grad():
        moe.moe_unpermute_grad(d["grad_out"], d["y"], S, d["row_of_slot"], d["probs"], T, K, H,
                               d["d_perm"], d["d_probs"])

    return permute, gemm, combine, grad


def gemm_grad_ops(args, d, n_rows):
    """The grouped GEMM backward on the layer's own tensors (dy is the unpermute
    backward's d_permuted, h the forward's), twice: recomputing the gate/up
    pre-activations, and taking them from a forward that kept them (that
    forward is timed too). FLOPs counted: 12 N H I (dh, dx and the three weight
    gradients; the recompute, 4 N H I more, is not)."""
    import torch
    import unpermute_combine_moe_amd as moe

    c = d["cfg"]
    T, H, E, K, I = c["T"], c["H"], c["E"], c["K"], c["I"]
    S = T * K
    bf = torch.bfloat16
    dev = d["x"].device
    dx = torch.empty((S, H), dtype=bf, device=dev)
    dwg = torch.empty((E, H, I), dtype=bf, device=dev)
    dwu = torch.empty((E, H, I), dtype=bf, device=dev)
    dwd = torch.empty((E, I, H), dtype=bf, device=dev)
    ws = moe.workspace(moe.moe_grouped_gemm_swiglu_grad_workspace_size(E, S, H, I), dev)
    pre = torch.empty((S, 2 * I), dtype=torch.float32, device=dev)
    ops = []
    fwd = lambda: moe.moe_grouped_gemm_swiglu(d["permuted"], d["offsets"], E, S, H, I, d["wg"],
                                              d["wu"], d["wd"], d["h"], d["y"], d["ws_g"],
                                              preact=pre)
    us, usmin = time_op(fwd, args.op_iters, None)
    ops.append(op_entry("grouped_gemm_swiglu_keep_preact", us, usmin,
                        flops=gemm_flops(n_rows, H, I)))
    for name, p in (("grouped_gemm_swiglu_grad", None),
                    ("grouped_gemm_swiglu_grad_saved_preact", pre)):
        f = lambda: moe.moe_grouped_gemm_swiglu_grad(d["permuted"], d["offsets"], E, S, H, I,
                                                     d["wg"], d["wu"], d["wd"], d["h"],
                                                     d["d_perm"], dx, dwg, dwu, dwd, ws, preact=p)
        us, usmin = time_op(f, args.op_iters, None)
        ops.append(op_entry(name, us, usmin, flops=12 * n_rows * H * I))
    return ops


def graph_step_ops(args, d, n_tokens):
    """The layer step captured once as a HIP graph (torch.cuda.CUDAGraph) and
    replayed, beside the eager step timed the same way (one step between two
    events, synchronised after each): the same kernels without per-launch host
    work."""
    import torch

    permute, gemm, combine, grad = step_calls(d)

    def step():
        permute(); gemm(); combine(); grad()

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    out = []
    for name, fn in (("layer_step_eager", step), ("layer_step_graph_replay", g.replay)):
        us, usmin = time_op(fn, args.op_iters, None)
        e = op_entry(name, us, usmin)
        e["tokens_per_s"] = round(n_tokens / (us * 1e-6), 1)
        out.append(e)
    return out


def run_layer(args, dev):
    import torch

    d = layer_setup(dev)
    permute, gemm, combine, grad = step_calls(d)
    for _ in range(args.warmup):
        permute(); gemm(); combine(); grad()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        e = ev[i]
        e[0].record(); permute(); e[1].record(); gemm(); e[2].record(); combine(); e[3].record()
        grad(); e[4].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    seg = np.array([[e[j].elapsed_time(e[j + 1]) * 1e3 for j in range(4)] for e in ev])  # us
    n_rows = int(d["offsets"][-1].item())
    return d, wall, seg, n_rows


# ----------------------------------------------------------------------------- per-workload ops

def run_ops(args, dev, flush):
    import torch
    import moe_workloads as W
    import unpermute_combine_moe_amd as moe

    ops = []
    # the tiny full path, T=64 H=128 E=8 K=2 I=64: permute -> grouped SwiGLU GEMM
    # -> combine; launch-bound (no roofline target), reported per pass
    g = W.gen_c1()
    c = g["cfg"]
    T, H, E, K, I = c["T"], c["H"], c["E"], c["K"], c["I"]
    x1, ids1, probs1 = dbf(g["x"], dev), dt(g["expert_ids"], dev), dt(g["probs"], dev)
    wg1, wu1, wd1 = (dbf(g[k], dev) for k in ("w_gate", "w_up", "w_down"))
    p1 = moe.permute_alloc(x1, ids1, E)
    ws_p1 = moe.workspace(moe.moe_permute_workspace_size(T, K, E), dev)
    ws_g1 = moe.workspace(moe.moe_grouped_gemm_swiglu_workspace_size(E, T * K, H, I), dev)
    h1 = torch.empty((T * K, I), dtype=torch.bfloat16, device=dev)
    y1 = torch.empty((T * K, H), dtype=torch.bfloat16, device=dev)
    out1 = torch.empty((T, H), dtype=torch.bfloat16, device=dev)

    def f_c1():
        moe.moe_permute(x1, ids1, T, H, K, E, p1["permuted"], p1["sorted_slot"], p1["row_of_slot"],
                        p1["expert_counts"], p1["expert_offsets"], ws_p1)
        moe.moe_grouped_gemm_swiglu(p1["permuted"], p1["expert_offsets"], E, T * K, H, I, wg1, wu1,
                                    wd1, h1, y1, ws_g1)
        moe.moe_unpermute_combine(y1, T * K, p1["row_of_slot"], None, ids1, probs1, T, K, H, E,
                                  None, None, out1)
    us, usmin = time_op(f_c1, args.op_iters, None, warm=5)
    e1 = op_entry("full_path_forward", us, usmin, flops=gemm_flops(T * K, H, I))
    e1["tokens_per_s"] = round(T / (us * 1e-6), 1)
    ops.append(dict(workload=c["name"], timing="three calls, caches warm", **e1))
    # the same three calls captured once as a HIP graph: launch-bound work without
    # the per-launch host cost
    s1 = torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s1):
        f_c1()
    torch.cuda.current_stream().wait_stream(s1)
    torch.cuda.synchronize()
    g1 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g1):
        f_c1()
    us, usmin = time_op(g1.replay, args.op_iters, None, warm=5)
    e1 = op_entry("full_path_forward_graph_replay", us, usmin, flops=gemm_flops(T * K, H, I))
    e1["tokens_per_s"] = round(T / (us * 1e-6), 1)
    ops.append(dict(workload=c["name"], timing="graph replays, caches warm", **e1))
    del g1
    del x1, p1, h1, y1, out1
    # permute / combine, T=4096 H=2048 E=64 K=6
    g = W.gen_c2()
    c = g["cfg"]
    T, H, E, K = c["T"], c["H"], c["E"], c["K"]
    x, ids, probs = dbf(g["x"], dev), dt(g["expert_ids"], dev), dt(g["probs"], dev)
    p = moe.permute_alloc(x, ids, E)
    ws = moe.workspace(moe.moe_permute_workspace_size(T, K, E), dev)
    N = int(p["expert_offsets"][-1].item())
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    f_perm = lambda: moe.moe_permute(x, ids, T, H, K, E, p["permuted"], p["sorted_slot"],
                                     p["row_of_slot"], p["expert_counts"], p["expert_offsets"], ws)
    f_comb = lambda: moe.moe_unpermute_combine(p["permuted"], T * K, p["row_of_slot"], None, ids,
                                               probs, T, K, H, E, None, None, out)
    ops.append(dict(workload=c["name"], **op_entry("permute", *time_op(f_perm, args.op_iters, flush),
                                                   nbytes=permute_bytes(T, K, H, N))))
    ops.append(dict(workload=c["name"], **op_entry("unpermute_combine",
                                                   *time_op(f_comb, args.op_iters, flush),
                                                   nbytes=combine_bytes(T, K, H, N))))
    # the permute's row move alone (moe_permute_rows with the routing just built)
    f_rows = lambda: moe.moe_permute_rows(x, p["row_of_slot"], T, H, K, T * K, p["permuted"])
    ops.append(dict(workload=c["name"], **op_entry("permute_row_move",
                                                   *time_op(f_rows, args.op_iters, flush),
                                                   nbytes=row_move_bytes(T, K, H, N))))
    # the same with x_active_mask: a [T, K] slot mask with 10% of the slots off
    m_np = np.random.default_rng(22).random((T, K)) < 0.9
    mask = torch.from_numpy(m_np).to(dev)
    pm = moe.permute_alloc(x, ids, E, active_mask=mask)
    Nm = int(pm["expert_offsets"][-1].item())
    f_permm = lambda: moe.moe_permute(x, ids, T, H, K, E, pm["permuted"], pm["sorted_slot"],
                                      pm["row_of_slot"], pm["expert_counts"],
                                      pm["expert_offsets"], ws, active_mask=mask)
    f_combm = lambda: moe.moe_unpermute_combine(pm["permuted"], T * K, pm["row_of_slot"], None, ids,
                                                probs, T, K, H, E, None, None, out,
                                                active_mask=mask)
    ops.append(dict(workload=c["name"] + "_slotmask90", **op_entry(
        "permute_masked", *time_op(f_permm, args.op_iters, flush),
        nbytes=permute_bytes(T, K, H, Nm) + T * K)))
    ops.append(dict(workload=c["name"] + "_slotmask90", **op_entry(
        "unpermute_combine_masked", *time_op(f_combm, args.op_iters, flush),
        nbytes=combine_bytes(T, K, H, Nm) + T * K)))
    del x, p, pm, out
    # reorder + combine with special experts, R=8 x E_local=32, N=32768, H=4096
    g = W.gen_c4()
    c = g["cfg"]
    R, El, N, H, T, K = c["R"], c["E_local"], c["N"], c["H"], c["T"], c["K"]
    xr, counts = dbf(g["x_rank_major"], dev), dt(g["counts"], dev)
    r = moe.reorder_alloc(xr, counts, R, El)
    wsr = moe.workspace(moe.moe_rank_to_expert_reorder_workspace_size(R, El), dev)
    f_reo = lambda: moe.moe_rank_to_expert_reorder(xr, counts, R, El, N, H, r["y"], r["perm"],
                                                   r["inv_perm"], r["tokens_per_expert"],
                                                   r["expert_offsets"], wsr)
    keep = [dbf(g["ori_x"], dev), dt(g["alpha1"], dev), dt(g["alpha2"], dev),
            dbf(g["const_v"], dev)]
    sp = moe.make_special(c["num_zero"], c["num_copy"], c["num_const"], keep[0], keep[1], keep[2],
                          (1, 0, 0), keep[3])
    shared = dbf(g["shared_x"], dev)
    src, ids4, probs4 = dt(g["slot_src_row"], dev), dt(g["expert_ids"], dev), dt(g["probs"], dev)
    out4 = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    f_comb4 = lambda: moe.moe_unpermute_combine(r["y"], N, src, r["inv_perm"], ids4, probs4, T, K,
                                                H, El, sp, shared, out4)
    ids_np = g["expert_ids"]
    need_ori = int(np.any((ids_np >= El + c["num_zero"]) & (ids_np < El + 12), axis=1).sum())
    n_routed = int((ids_np < El).sum())
    ops.append(dict(workload=c["name"], **op_entry("rank_to_expert_reorder",
                                                   *time_op(f_reo, args.op_iters, flush),
                                                   nbytes=reorder_bytes(N, H))))
    ops.append(dict(workload=c["name"], **op_entry(
        "unpermute_combine_special", *time_op(f_comb4, args.op_iters, flush),
        nbytes=n_routed * H * 2 + 4 * T * K * 4 + 2 * T * H * 2 + need_ori * H * 2 + N * 4)))
    # backward of that combine: every input's gradient (special experts included)
    g4 = dbf(W.normal_bf16(np.random.default_rng(44), (T, H)), dev)
    d_eo = torch.empty((N, H), dtype=torch.bfloat16, device=dev)
    d_pr = torch.empty((T, K), dtype=torch.float32, device=dev)
    d_ori = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    d_a1 = torch.empty(T, dtype=torch.float32, device=dev)
    d_a2 = torch.empty(T, dtype=torch.float32, device=dev)
    d_cv = torch.empty((c["num_const"], H), dtype=torch.bfloat16, device=dev)
    wsg = moe.workspace(moe.moe_unpermute_combine_grad_workspace_size(T, H, c["num_const"]), dev)
    f_cgrad = lambda: moe.moe_unpermute_combine_grad(g4, r["y"], N, src, r["inv_perm"], ids4,
                                                     probs4, T, K, H, El, sp, d_eo, d_pr, d_ori,
                                                     d_a1, d_a2, d_cv, wsg)
    ops.append(dict(workload=c["name"], **op_entry(
        "unpermute_combine_grad_special", *time_op(f_cgrad, args.op_iters, flush),
        nbytes=combine_grad_bytes(T, K, H, N, n_routed, need_ori, c["num_const"]))))
    del xr, r, keep, shared, out4, g4, d_eo, d_ori
    # unpermute backward, T=16384 H=4096 E=128 K=8
    g = W.gen_c5()
    c = g["cfg"]
    T, H, E, K = c["T"], c["H"], c["E"], c["K"]
    ids5 = dt(g["expert_ids"], dev)
    p5 = moe.permute_alloc(None, ids5, E, rows=False)
    gout, perm5, probs5 = dbf(g["grad_out"], dev), dbf(g["permuted"], dev), dt(g["probs"], dev)
    dperm = torch.empty_like(perm5)
    dprobs = torch.empty((T, K), dtype=torch.float32, device=dev)
    N = T * K
    f_grad = lambda: moe.moe_unpermute_grad(gout, perm5, N, p5["row_of_slot"], probs5, T, K, H,
                                            dperm, dprobs)
    ops.append(dict(workload=c["name"], **op_entry("unpermute_grad",
                                                   *time_op(f_grad, args.op_iters, flush),
                                                   nbytes=grad_bytes(T, K, H, N))))
    # permute backward on the same routing: the gradient of the permuted rows summed per token
    dx = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    f_pgrad = lambda: moe.moe_permute_grad(dperm, N, p5["row_of_slot"], T, K, H, dx)
    ops.append(dict(workload=c["name"], **op_entry("permute_grad",
                                                   *time_op(f_pgrad, args.op_iters, flush),
                                                   nbytes=permute_grad_bytes(T, K, H, N))))
    del dx
    del gout, perm5, dperm
    # deredundency: dispatch indices and whiteboard combine of one outer step
    g = W.gen_dered()
    c = g["cfg"]
    cnt = dt(g["counts"], dev)
    n_sel, G, H = g["n_selected"], g["G"], c["H"]
    di = moe.dered_indices_alloc(cnt, c["expert_start"], c["iep"], c["El"], capacity=n_sel)
    wsi = moe.workspace(moe.moe_deredundency_dispatch_indices_workspace_size(
        c["oep"], c["E"], c["iep"], c["El"]), dev)
    f_di = lambda: moe.moe_deredundency_dispatch_indices(
        cnt, c["oep"], c["E"], c["expert_start"], c["iep"], c["El"], n_sel, di["indices"],
        di["counts_by_dest"], di["total"], wsi)
    src, coeff = dbf(g["outer_output"], dev), dt(g["router_coeff"], dev)
    wb = torch.empty((G, H), dtype=torch.bfloat16, device=dev)
    wsc = moe.workspace(moe.moe_deredundency_combine_workspace_size(n_sel, G), dev)
    f_dc = lambda: moe.moe_deredundency_combine(src, coeff, di["indices"], n_sel, H, G, wb, wsc)
    ops.append(dict(workload=c["name"], **op_entry(
        "deredundency_dispatch_indices", *time_op(f_di, args.op_iters, flush),
        nbytes=c["oep"] * c["E"] * 4 + n_sel * 4)))
    ops.append(dict(workload=c["name"], **op_entry(
        "deredundency_combine", *time_op(f_dc, args.op_iters, flush),
        nbytes=n_sel * H * 2 + G * H * 2 + n_sel * 8 + G * 8)))
    del src, wb
    # device-to-device copy of 1 GiB for reference
    a = torch.empty(1 << 29, dtype=torch.bfloat16, device=dev)
    b = torch.empty_like(a)
    us, usmin = time_op(lambda: b.copy_(a), 10, flush)
    ops.append(dict(workload="d2d_copy_1GiB", **op_entry("torch_copy", us, usmin,
                                                         nbytes=2 * a.numel() * 2)))
    del a, b
    # every memory-bound entry above was timed alone, each launch after the flush
    for e in ops:
        if "hbm_frac" in e and flush is not None:
            e.setdefault("timing", "alone, caches flushed by a 1 GiB read")
    # for scale: the vendor GEMM (torch.matmul, hipBLASLt) on dense bf16 matrices
    # of the skewed layer's two passes, all 65,536 rows as one matrix (no expert
    # groups, no SwiGLU), weights [k][n] as the grouped call takes them
    for name, (M, Kd, Nc) in (("dense_gemm_gate_up_reference", (65536, 2048, 1024)),
                              ("dense_gemm_down_reference", (65536, 512, 2048))):
        xa = torch.randn(M, Kd, device=dev, dtype=torch.bfloat16)
        wa = torch.randn(Kd, Nc, device=dev, dtype=torch.bfloat16) * 0.02
        us, usmin = time_op(lambda: torch.matmul(xa, wa), args.op_iters, None, warm=3)
        ops.append(dict(workload=f"dense_{M}x{Kd}x{Nc}", **op_entry(name, us, usmin,
                                                                   flops=2 * M * Kd * Nc)))
        del xa, wa
    return ops


# ----------------------------------------------------------------------------- CPU baseline

def cpu_baseline(d, n_tok):
    """The CPU oracle timed on the first n_tok tokens of the layer workload:
    permute -> fp64 SwiGLU FFN of their rows -> combine -> combine backward."""
    import oracle

    g = d["host"]
    c = d["cfg"]
    E = c["E"]
    n_tok = min(n_tok, c["T"])
    x, ids, probs = g["x"][:n_tok], g["expert_ids"][:n_tok], g["probs"][:n_tok]
    import moe_workloads as W
    gout = W.normal_bf16(W.rng_for(3 * 1000 + 7), (c["T"], c["H"]))[:n_tok]
    t0 = time.perf_counter()
    p = oracle.permute(x, ids, E)
    _, y64 = oracle.grouped_swiglu(p["permuted"], p["expert_offsets"], g["w_gate"], g["w_up"],
                                   g["w_down"], want_h=False)
    y = oracle.f64_to_bf16(y64)
    oracle.combine(y, p["row_of_slot"], ids, probs, E)
    oracle.unpermute_grad(gout, y, p["row_of_slot"], probs)
    el = time.perf_counter() - t0
    return {"value": round(n_tok / el, 2), "unit": "tokens/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"first {n_tok} of {c['T']} tokens of the layer workload "
                      f"({n_tok * c['K']} routed rows), same step: permute, fp64 SwiGLU FFN, "
                      f"combine, combine backward; {el:.1f} s on {cpu_model()} "
                      f"({os.cpu_count()} logical CPUs visible, OMP_NUM_THREADS="
                      f"{os.environ.get('OMP_NUM_THREADS', 'unset')})"}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "host"


# ----------------------------------------------------------------------------- main

def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); this library has no "
              "multi-GPU path", file=sys.stderr)
        sys.exit(2)
    import torch

    import __graft_entry__ as ge
    ge._ensure_built()
    import unpermute_combine_moe_amd as moe
    moe.load()
    dev = torch.device("cuda:0")
    log(f"device: {torch.cuda.get_device_name(0)}")
    if args.copy_probe:
        a = torch.ones(1 << 27, dtype=torch.bfloat16, device=dev)   # 256 MiB
        b = torch.empty_like(a)
        for _ in range(args.copy_probe):
            b.copy_(a)
        torch.cuda.synchronize()
        log(f"copy probe: {args.copy_probe} x 256 MiB read + 256 MiB written")
        return

    d, wall, seg, n_rows = run_layer(args, dev)
    c = d["cfg"]
    T, H, K, I = c["T"], c["H"], c["K"], c["I"]
    ms_step = wall / args.steps * 1e3
    seg_med = np.median(seg, axis=0)
    log(f"layer step {ms_step:.3f} ms; permute {seg_med[0]:.1f} us, gemm {seg_med[1]:.1f} us, "
        f"combine {seg_med[2]:.1f} us, grad {seg_med[3]:.1f} us")
    g_us = float(np.mean(seg[:, 1]))
    g_tf = gemm_flops(n_rows, H, I) / (g_us * 1e-6) / 1e12
    active = int((d["counts"] > 0).sum().item())
    rec = gemm_traffic_record()
    roofline = {"bound": "mfma", "kernel": "moe_grouped_gemm_swiglu (gate/up + down)",
                "achieved": round(g_tf, 1), "peak": BF16_DENSE_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(g_tf / BF16_DENSE_PEAK_TFLOPS, 4),
                "traffic": rec["traffic_bytes"] if rec else None,
                "avg_us": round(g_us, 2), "flops_per_launch": gemm_flops(n_rows, H, I),
                "algorithmic_bytes_per_launch": gemm_bytes(n_rows, H, I, active),
                "hbm_gbs_algorithmic": round(gemm_bytes(n_rows, H, I, active) / (g_us * 1e-6) / 1e9, 1),
                # the call's own roofline time, max(F / peak, bytes / 8 TB/s), over its time
                "attainable_frac": round(max(gemm_flops(n_rows, H, I) / (BF16_DENSE_PEAK_TFLOPS * 1e12),
                                             gemm_bytes(n_rows, H, I, active) / (HBM_PEAK_GBS * 1e9))
                                         / (g_us * 1e-6), 4)}
    # per-op figures of the layer's memory-bound calls: each call timed alone with
    # a 1 GiB write between launches (nothing left in the 256 MB Infinity Cache);
    # with --no-ops, the in-step times instead (marked as such)
    permute, _, combine, grad = step_calls(d)
    flush = None if args.no_ops else Flusher(dev)
    import unpermute_combine_moe_amd as moe
    row_move = lambda: moe.moe_permute_rows(d["x"], d["row_of_slot"], T, H, K, T * K,
                                            d["permuted"])
    mem_ops = (("permute", permute, 0, permute_bytes(T, K, H, n_rows)),
               ("unpermute_combine", combine, 2, combine_bytes(T, K, H, n_rows)),
               ("unpermute_grad", grad, 3, grad_bytes(T, K, H, n_rows)),
               ("permute_row_move", row_move, None, row_move_bytes(T, K, H, n_rows)))
    layer_ops = []
    for name, fn, col, nbytes in mem_ops:
        if flush is not None:
            us, usmin = time_op(fn, args.op_iters, flush)
            timing = "alone, caches flushed by a 1 GiB read"
        elif col is None:
            continue
        else:
            us, usmin = float(np.median(seg[:, col])), float(np.min(seg[:, col]))
            timing = "in the layer step"
        layer_ops.append(dict(workload=c["name"], timing=timing,
                              **op_entry(name, us, usmin, nbytes=nbytes)))
    layer_ops.insert(1, dict(workload=c["name"], timing="in the layer step",
                             **op_entry("grouped_gemm_swiglu", float(np.median(seg[:, 1])),
                                        float(np.min(seg[:, 1])),
                                        flops=gemm_flops(n_rows, H, I))))
    ops = layer_ops
    if not args.no_ops:
        ops += [dict(workload=c["name"], **o) for o in gemm_grad_ops(args, d, n_rows)]
        ops += [dict(workload=c["name"], timing="one step per timing, caches warm", **o)
                for o in graph_step_ops(args, d, T)]
        ops = ops + run_ops(args, dev, flush)
        del flush
    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        cpu = cpu_baseline(d, args.cpu_sample_tokens)
    line = {
        "metric": METRIC, "value": round(T / (ms_step * 1e-3), 1), "unit": "tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": c["name"], "T": T, "H": H, "E": c["E"], "K": K, "I": I,
                   "routing": "Zipf(1.2)-biased softmax top-8, renormalised",
                   "step": "permute + grouped SwiGLU GEMM + combine + combine backward",
                   "parallelism": "single GPU"},
        "roofline": roofline, "cpu_baseline": cpu, "ops": ops,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
