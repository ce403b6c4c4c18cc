"""The library's calls under HIP graph capture (torch.cuda.CUDAGraph): they
allocate nothing and issue no memset, so a captured step replays the eager
step's bits. Each test replays its graph several times, with eager work that
overwrites every output and a synchronisation between replays, and checks
every replay against the eager result."""
import numpy as np
import pytest
import torch

import bench
import moe_workloads as W
from helpers import to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu


def _capture(fn):
    # warm up on a side stream first, as torch requires before a capture
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def _replay_and_check(g, outs, ref, reps=3):
    for rep in range(reps):
        for t in outs.values():
            t.fill_(-3)  # eager work between the replays: every output overwritten
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, t in outs.items():
            assert torch.equal(t, ref[k]), f"replay {rep}: {k} differs from the eager step"


def test_layer_step_graph_replays(moe_lib):
    """The skewed layer's step (permute -> grouped GEMM -> combine -> unpermute
    backward) as one graph."""
    dev = torch.device("cuda:0")
    d = bench.layer_setup(dev)
    permute, gemm, combine, grad = bench.step_calls(d)

    def step():
        permute(); gemm(); combine(); grad()

    print("skewed layer step under graph capture", flush=True)
    step()
    torch.cuda.synchronize()
    keys = ("permuted", "sorted_slot", "row_of_slot", "counts", "offsets", "h", "y", "out",
            "d_perm", "d_probs")
    ref = {k: d[k].clone() for k in keys}
    g = _capture(step)
    _replay_and_check(g, {k: d[k] for k in keys}, ref)


def test_noalloc_permute_graph_replays(moe_lib):
    """moe_permute_noalloc (no workspace argument) captured on the T=4096,
    E=64, K=6 workload's shape."""
    moe = moe_lib
    T, K, E, H = 4096, 6, 64, 2048
    rng = np.random.default_rng(61)
    ids = np.argsort(rng.random((T, E)), axis=1)[:, :K].astype(np.int32)
    dev = torch.device("cuda:0")
    x, idd = to_dev_bf16(W.normal_bf16(rng, (T, H))), to_dev(ids)
    S = T * K
    outs = dict(permuted=torch.empty((S, H), dtype=torch.bfloat16, device=dev),
                sorted_slot=torch.empty(S, dtype=torch.int32, device=dev),
                row_of_slot=torch.empty((T, K), dtype=torch.int32, device=dev),
                expert_counts=torch.empty(E, dtype=torch.int32, device=dev),
                expert_offsets=torch.empty(E + 1, dtype=torch.int32, device=dev))

    def call():
        moe.moe_permute_noalloc(x, idd, T, H, K, E, outs["permuted"], outs["sorted_slot"],
                                outs["row_of_slot"], outs["expert_counts"],
                                outs["expert_offsets"])

    print(f"permute_noalloc under graph capture T={T} K={K} E={E} H={H}", flush=True)
    call()
    torch.cuda.synchronize()
    ref = {k: t.clone() for k, t in outs.items()}
    g = _capture(call)
    _replay_and_check(g, outs, ref)
