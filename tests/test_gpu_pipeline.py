"""End-to-end parity of permute -> grouped SwiGLU GEMM -> combine against the
oracle chain run on the same inputs (no GPU intermediate fed to the oracle)."""
import numpy as np
import pytest
import torch

import moe_workloads as W
import oracle
from helpers import assert_rel, bits, f64, gemm_tol, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu


def test_config1_full_path(moe_lib):
    g = W.gen_c1()
    c = g["cfg"]
    E = c["E"]
    ids, probs = to_dev(g["expert_ids"]), to_dev(g["probs"])
    p = moe_lib.permute_alloc(to_dev_bf16(g["x"]), ids, E)
    _, y = moe_lib.grouped_gemm_alloc(p["permuted"], p["expert_offsets"], to_dev_bf16(g["w_gate"]),
                                      to_dev_bf16(g["w_up"]), to_dev_bf16(g["w_down"]))
    out = moe_lib.combine_alloc(y, p["row_of_slot"], ids, probs, E)
    torch.cuda.synchronize()
    op = oracle.permute(g["x"], g["expert_ids"], E)
    _, y64 = oracle.grouped_swiglu(op["permuted"], op["expert_offsets"], g["w_gate"], g["w_up"],
                                   g["w_down"])
    # the oracle combine in fp64 on the fp64 expert output
    T, K = g["expert_ids"].shape
    ref = np.zeros((T, c["H"]))
    ros = op["row_of_slot"]
    for t in range(T):
        for k in range(K):
            ref[t] += float(g["probs"][t, k]) * y64[ros[t, k]]
    got = f64(bits(out))
    tol = gemm_tol(c["H"])
    err = np.max(np.abs(got - ref))
    print(f"config 1 layer output: max err {err:.3e}")
    assert err <= tol

