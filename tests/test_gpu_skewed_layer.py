"""Full-size GPU parity of the skewed layer workload (T=8192 tokens, H=2048,
E=256 experts with Zipf(1.2)-biased top-8 routing, I=512), run with the
benchmark's own buffers and calls: every one of the 65,536 routed rows of the
grouped GEMM, all 8,192 tokens of the layer output and of the combine, the
unpermute backward at H=2048 (its two-waves-per-token instance), and the
complete grouped GEMM backward (every dx row, every expert's weight
gradients), each against the fp64 oracle. Inputs of the oracle come from the
seeded generators or from the oracle itself, never from the GPU."""
import numpy as np
import pytest
import torch

import bench
import moe_workloads as W
import oracle
import unpermute_combine_moe_amd as moe
from helpers import (assert_h_within_ulp, assert_rel, bits, f64, ffn_grad_worst, gemm_tol,
                     to_dev, to_dev_bf16)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def layer(moe_lib):
    """One layer step (permute -> grouped GEMM -> combine) of the benchmark,
    on its own buffers; host copies of the outputs."""
    dev = torch.device("cuda:0")
    d = bench.layer_setup(dev)
    permute, gemm, combine, _ = bench.step_calls(d)
    print("skewed layer: permute -> GEMM -> combine", flush=True)
    permute(); gemm(); combine()
    torch.cuda.synchronize()
    out = {k: d[k].cpu().numpy() for k in ("sorted_slot", "row_of_slot", "counts", "offsets")}
    for k in ("permuted", "h", "y", "out"):
        out[k] = bits(d[k])
    out["d"] = d
    return out


@pytest.fixture(scope="module")
def ref(layer):
    """The oracle on the same seeded inputs: permute, then the fp64 FFN of all rows."""
    g = layer["d"]["host"]
    c = layer["d"]["cfg"]
    print("oracle: permute + fp64 FFN of all routed rows", flush=True)
    p = oracle.permute(g["x"], g["expert_ids"], c["E"])
    h64, y64 = oracle.grouped_swiglu(p["permuted"], p["expert_offsets"], g["w_gate"],
                                     g["w_up"], g["w_down"])
    return dict(p=p, h64=h64, y64=y64)


def test_layer_permute_exact(layer, ref):
    p = ref["p"]
    np.testing.assert_array_equal(layer["counts"], p["expert_counts"])
    np.testing.assert_array_equal(layer["offsets"], p["expert_offsets"])
    np.testing.assert_array_equal(layer["sorted_slot"], p["sorted_slot"])
    np.testing.assert_array_equal(layer["row_of_slot"], p["row_of_slot"])
    np.testing.assert_array_equal(layer["permuted"], p["permuted"])


def test_layer_gemm_every_row(layer, ref):
    c = layer["d"]["cfg"]
    n = int(ref["p"]["expert_offsets"][-1])
    assert n == c["T"] * c["K"]
    err = np.abs(f64(layer["y"][:n]) - ref["y64"])
    tol = gemm_tol(c["H"])
    print(f"skewed layer GEMM, {n} rows: max |y - ref| {err.max():.3e} (bound {tol:.3e}), "
          f"rows over half the bound: {int((err.max(axis=1) > tol / 2).sum())}")
    assert err.max() <= tol
    assert_h_within_ulp(layer["h"][:n], ref["h64"])


def test_layer_output_every_token(layer, ref):
    """permute -> GEMM -> combine on the GPU against the oracle chain in fp64
    (the fp64 expert rows, weighted and summed in fp64)."""
    g = layer["d"]["host"]
    c = layer["d"]["cfg"]
    ros = ref["p"]["row_of_slot"]
    want = np.zeros((c["T"], c["H"]))
    for k in range(c["K"]):
        want += g["probs"][:, k:k + 1].astype(np.float64) * ref["y64"][ros[:, k]]
    err = np.abs(f64(layer["out"]) - want)
    tol = gemm_tol(c["H"])
    print(f"skewed layer output, {c['T']} tokens: max err {err.max():.3e} (bound {tol:.3e})")
    assert err.max() <= tol


def test_layer_combine_every_token(layer, ref):
    """The combine call of the step on the oracle's bf16 expert rows against
    the oracle combine of the same rows."""
    g = layer["d"]["host"]
    c = layer["d"]["cfg"]
    T, K, H, E = c["T"], c["K"], c["H"], c["E"]
    yb = oracle.f64_to_bf16(ref["y64"])
    ros = ref["p"]["row_of_slot"]
    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    moe.moe_unpermute_combine(to_dev_bf16(yb), T * K, to_dev(ros), None, to_dev(g["expert_ids"]),
                              to_dev(g["probs"]), T, K, H, E, None, None, out)
    torch.cuda.synchronize()
    want_bits, want64 = oracle.combine(yb, ros, g["expert_ids"], g["probs"], E)
    got = bits(out)
    print(f"skewed layer combine: {float(np.mean(got == want_bits)):.4f} of elements "
          f"bit-equal to the oracle's rounding")
    assert_rel(f64(got), want64, 1e-2, "combine")


def test_layer_unpermute_grad_h2048(layer, ref):
    """The step's unpermute backward (T=8192, K=8, H=2048: two waves per token,
    two 64-chunk rows each) on the oracle's bf16 expert rows."""
    d = layer["d"]
    g = d["host"]
    c = d["cfg"]
    T, K, H = c["T"], c["K"], c["H"]
    yb = oracle.f64_to_bf16(ref["y64"])
    ros = ref["p"]["row_of_slot"]
    # the step's synthetic grad_out, from the same seeded generator
    gout = W.normal_bf16(W.rng_for(3 * 1000 + 7), (T, H))
    dperm = torch.zeros((T * K, H), dtype=torch.bfloat16, device="cuda")
    dprobs = torch.empty((T, K), dtype=torch.float32, device="cuda")
    moe.moe_unpermute_grad(to_dev_bf16(gout), to_dev_bf16(yb), T * K, to_dev(ros),
                           to_dev(g["probs"]), T, K, H, dperm, dprobs)
    torch.cuda.synchronize()
    rdp, _, _, rdpr64 = oracle.unpermute_grad(gout, yb, ros, g["probs"])
    np.testing.assert_array_equal(bits(dperm), rdp)
    assert_rel(dprobs.cpu().numpy(), rdpr64, 1e-2, "d_probs")


def test_layer_gemm_grad_complete(layer, ref):
    """The grouped GEMM backward at the layer's shapes: every dx row and the
    weight gradients of every expert (the empty ones must be zero), and the
    same bits from the path that takes the forward's saved pre-activations."""
    d = layer["d"]
    g = d["host"]
    c = d["cfg"]
    E, H, I = c["E"], c["H"], c["I"]
    p = ref["p"]
    off = p["expert_offsets"]
    x = p["permuted"]
    dy = W.normal_bf16(np.random.default_rng(12), x.shape)
    xd, od, dyd = to_dev_bf16(x), to_dev(off), to_dev_bf16(dy)
    h, _, pre = moe.grouped_gemm_alloc(xd, od, d["wg"], d["wu"], d["wd"], keep_preact=True)
    got_t = moe.grouped_gemm_grad_alloc(xd, od, d["wg"], d["wu"], d["wd"], h, dyd)
    # the path that takes the forward's pre-activations gives the same bits
    saved = moe.grouped_gemm_grad_alloc(xd, od, d["wg"], d["wu"], d["wd"], h, dyd, preact=pre)
    torch.cuda.synchronize()
    n = int(off[-1])
    for k in got_t:
        a, b = (got_t[k][:n], saved[k][:n]) if k == "dx" else (got_t[k], saved[k])
        assert torch.equal(a, b), f"{k}: saved pre-activations differ from recomputation"
    del saved, pre
    got = {k: f64(bits(v)) for k, v in got_t.items()}
    del got_t, h
    print("oracle: fp64 FFN backward of all routed rows", flush=True)
    r = oracle.grouped_swiglu_grad(x, off, g["w_gate"], g["w_up"], g["w_down"], dy)
    counts = np.diff(off)
    live = np.flatnonzero(counts)
    worst = ffn_grad_worst(got, r, x, off, g["w_gate"], g["w_up"], g["w_down"], dy, ref["h64"],
                           live)
    print("skewed layer GEMM backward, worst err/bound: " +
          ", ".join(f"{k} {v:.3f}" for k, v in worst.items()), flush=True)
    empty = counts == 0
    assert not got["dw_gate"][empty].any() and not got["dw_up"][empty].any()
    assert not got["dw_down"][empty].any()
