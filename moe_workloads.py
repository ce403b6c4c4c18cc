"""Seeded synthetic inputs for the MoE permute / expert / combine path.

This module only *constructs inputs*: token rows, router output (expert ids and
probabilities), expert weights and the special-expert operands. It holds none
of the arithmetic of the path itself (no bucketing, no prefix sums over expert
counts, no GEMM, no combine). Both the GPU path and the CPU oracle consume the
exact same bits produced here.

Conventions
-----------
* bf16 tensors are numpy ``uint16`` arrays holding bfloat16 bit patterns,
  obtained from float32 draws by round-to-nearest-even.
* Index tensors are ``int32``; probabilities and special-expert coefficients
  are ``float32``.
* Every draw comes from ``numpy.random.Generator(PCG64(seed))`` in the order
  written in each function, so a config is reproduced exactly from its seed.

The router used to make routing inputs is softmax over fp32 logits, then top-K
by logit (larger logit first; on equal logits the lower expert id first), then
optional renormalisation of the K selected probabilities.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_from_f32", "f32_from_bf16", "rng_for", "normal_bf16", "uniform_bf16",
    "route_topk", "make_routing", "make_tokens", "make_expert_weights",
    "make_rank_major_counts", "CONFIGS", "gen_c1", "gen_c2", "gen_c3", "gen_c4",
    "gen_c5", "generate", "DERED", "gen_dered",
]


# ---------------------------------------------------------------------------
# bf16 bit handling (input construction only)
# ---------------------------------------------------------------------------

def bf16_from_f32(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bits, round to nearest, ties to even (finite inputs)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    rounded = u + np.uint32(0x7FFF) + lsb
    return (rounded >> np.uint32(16)).astype(np.uint16)


def f32_from_bf16(b: np.ndarray) -> np.ndarray:
    """bfloat16 bits -> float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def rng_for(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def normal_bf16(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return bf16_from_f32(a)


def uniform_bf16(rng: np.random.Generator, shape, lo: float, hi: float) -> np.ndarray:
    a = rng.uniform(lo, hi, size=shape).astype(np.float32)
    return bf16_from_f32(a)


# ---------------------------------------------------------------------------
# Router (produces the routing *input* of the path)
# ---------------------------------------------------------------------------

def route_topk(logits: np.ndarray, K: int, renorm: bool):
    """softmax -> top-K -> optional renormalisation.

    Returns ``expert_ids`` int32 [T,K] (descending probability, ties to the
    lower id) and ``probs`` float32 [T,K].
    """
    lg = np.asarray(logits, dtype=np.float32)
    T, E = lg.shape
    if not (0 < K <= E):
        raise ValueError(f"K={K} must be in (0, E={E}]")
    # stable argsort of the negated logits: larger logit first, lower id on ties
    order = np.argsort(-lg, axis=1, kind="stable")[:, :K].astype(np.int32)
    l64 = lg.astype(np.float64)
    m = np.max(l64, axis=1, keepdims=True)
    e = np.exp(l64 - m)
    p = e / np.sum(e, axis=1, keepdims=True)
    top = np.take_along_axis(p, order.astype(np.int64), axis=1)
    if renorm:
        top = top / np.sum(top, axis=1, keepdims=True)
    return order, top.astype(np.float32)


def make_routing(T: int, E: int, K: int, seed: int, *, logits: str = "normal",
                 renorm: bool = True, empty_experts: int = 0, zipf_s: float = 0.0):
    """Random routing for T tokens over E experts.

    ``logits``: "normal" (N(0,1)) or "uniform" (U(0,1)). ``zipf_s`` > 0 adds a
    per-expert bias ``-s * ln(rank_e)`` with ``rank`` a seeded permutation of
    1..E (the log of a Zipf(s) pmf), so a few experts take most tokens.
    ``empty_experts`` experts (seeded choice) get logit -inf and receive none.
    """
    rng = rng_for(seed)
    if logits == "normal":
        lg = rng.standard_normal(size=(T, E), dtype=np.float32)
    elif logits == "uniform":
        lg = rng.uniform(0.0, 1.0, size=(T, E)).astype(np.float32)
    else:
        raise ValueError(logits)
    if zipf_s > 0.0:
        rank = rng.permutation(E) + 1
        lg = lg + (-zipf_s * np.log(rank.astype(np.float64))).astype(np.float32)[None, :]
    if empty_experts > 0:
        dead = rng.choice(E, size=empty_experts, replace=False)
        lg[:, dead] = -np.inf
    return route_topk(lg, K, renorm)


def make_tokens(T: int, H: int, seed: int, std: float = 1.0) -> np.ndarray:
    return normal_bf16(rng_for(seed), (T, H), std)


def make_expert_weights(E: int, H: int, I: int, seed: int, std: float = 0.02):
    """w_gate, w_up [E,H,I] and w_down [E,I,H], bf16 bits, N(0, std^2)."""
    rng = rng_for(seed)
    wg = normal_bf16(rng, (E, H, I), std)
    wu = normal_bf16(rng, (E, H, I), std)
    wd = normal_bf16(rng, (E, I, H), std)
    return wg, wu, wd


def make_rank_major_counts(R: int, E_local: int, N: int, seed: int, alpha: float = 0.5):
    """counts[r*E_local + e] ~ Multinomial(N, Dirichlet(alpha * 1))."""
    rng = rng_for(seed)
    pv = rng.dirichlet(np.full(R * E_local, alpha))
    return rng.multinomial(N, pv).astype(np.int32)


# ---------------------------------------------------------------------------
# The five named workloads
# ---------------------------------------------------------------------------

CONFIGS = {
    1: dict(name="tiny_full_path", T=64, H=128, E=8, K=2, I=64, seed=1),
    2: dict(name="permute_unpermute_T4096_H2048_E64_K6", T=4096, H=2048, E=64, K=6, seed=2),
    3: dict(name="skewed_layer_T8192_H2048_E256_K8_I512", T=8192, H=2048, E=256, K=8, I=512, seed=3),
    4: dict(name="rank_major_reorder_combine_R8_E32_N32768_H4096", R=8, E_local=32, N=32768,
            H=4096, T=4608, K=8, num_zero=4, num_copy=4, num_const=4, n_special_slots=4096,
            seed=4),
    5: dict(name="unpermute_grad_T16384_H4096_E128_K8", T=16384, H=4096, E=128, K=8,
            empty_experts=13, seed=5),
}


def gen_c1(with_weights: bool = True):
    """T=64, H=128, E=8, K=2, I=64; normal logits, top-2, renormalised."""
    c = CONFIGS[1]
    rng = rng_for(c["seed"])
    x = normal_bf16(rng, (c["T"], c["H"]))
    lg = rng.standard_normal(size=(c["T"], c["E"]), dtype=np.float32)
    ids, probs = route_topk(lg, c["K"], renorm=True)
    out = dict(cfg=c, x=x, expert_ids=ids, probs=probs)
    if with_weights:
        out["w_gate"] = normal_bf16(rng, (c["E"], c["H"], c["I"]), 0.02)
        out["w_up"] = normal_bf16(rng, (c["E"], c["H"], c["I"]), 0.02)
        out["w_down"] = normal_bf16(rng, (c["E"], c["I"], c["H"]), 0.02)
    return out


def gen_c2():
    """T=4096, H=2048, E=64, K=6; uniform logits U(0,1), top-6, renormalised."""
    c = CONFIGS[2]
    rng = rng_for(c["seed"])
    x = normal_bf16(rng, (c["T"], c["H"]))
    lg = rng.uniform(0.0, 1.0, size=(c["T"], c["E"])).astype(np.float32)
    ids, probs = route_topk(lg, c["K"], renorm=True)
    return dict(cfg=c, x=x, expert_ids=ids, probs=probs)


def gen_c3(with_weights: bool = True, with_x: bool = True):
    """T=8192, H=2048, E=256, K=8, I=512; Zipf(1.2)-biased normal logits."""
    c = CONFIGS[3]
    rng = rng_for(c["seed"])
    lg = rng.standard_normal(size=(c["T"], c["E"]), dtype=np.float32)
    rank = rng.permutation(c["E"]) + 1
    lg = lg + (-1.2 * np.log(rank.astype(np.float64))).astype(np.float32)[None, :]
    ids, probs = route_topk(lg, c["K"], renorm=True)
    out = dict(cfg=c, expert_ids=ids, probs=probs)
    # x and the weights come from their own streams so that a caller can skip them
    if with_x:
        out["x"] = normal_bf16(rng_for(c["seed"] * 1000 + 1), (c["T"], c["H"]))
    if with_weights:
        wr = rng_for(c["seed"] * 1000 + 2)
        out["w_gate"] = normal_bf16(wr, (c["E"], c["H"], c["I"]), 0.02)
        out["w_up"] = normal_bf16(wr, (c["E"], c["H"], c["I"]), 0.02)
        out["w_down"] = normal_bf16(wr, (c["E"], c["I"], c["H"]), 0.02)
    return out


def gen_c4(with_rows: bool = True):
    """One GPU's rank-major receive buffer (R=8 source segments x 32 local
    experts, 32768 rows of H=4096) and a combine over T=4608 tokens x K=8 slots.

    Of the 36864 slots, 4096 (uniform choice) carry special ids uniform over
    [32, 44): zero [32,36), copy [36,40), const [40,44). The other 32768 slots
    take the rank-major rows in a seeded random bijection; their expert id is
    the local expert of the block the row sits in. ``slot_src_row`` holds that
    rank-major row (-1 for special slots).
    """
    c = CONFIGS[4]
    R, El, N, H, T, K = c["R"], c["E_local"], c["N"], c["H"], c["T"], c["K"]
    rng = rng_for(c["seed"])
    counts = rng.multinomial(N, rng.dirichlet(np.full(R * El, 0.5))).astype(np.int32)
    # label of each rank-major row: the buffer is laid out block (r, e) after block
    # (r, e-1), so the local expert of each row is e repeated counts[r*El+e] times
    row_expert = np.repeat(np.tile(np.arange(El, dtype=np.int32), R), counts)
    n_slots = T * K
    special_slots = rng.choice(n_slots, size=c["n_special_slots"], replace=False)
    special_ids = rng.integers(El, El + c["num_zero"] + c["num_copy"] + c["num_const"],
                               size=c["n_special_slots"]).astype(np.int32)
    is_special = np.zeros(n_slots, dtype=bool)
    is_special[special_slots] = True
    real_slots = np.flatnonzero(~is_special)
    assert real_slots.size == N
    bij = rng.permutation(N).astype(np.int32)
    slot_src_row = np.full(n_slots, -1, dtype=np.int32)
    slot_src_row[real_slots] = bij
    expert_ids = np.empty(n_slots, dtype=np.int32)
    expert_ids[real_slots] = row_expert[bij]
    expert_ids[special_slots] = special_ids
    p = rng.uniform(0.0, 1.0, size=(T, K))
    probs = (p / p.sum(axis=1, keepdims=True)).astype(np.float32)
    alpha1 = rng.uniform(0.0, 1.0, size=T).astype(np.float32)
    alpha2 = rng.uniform(0.0, 1.0, size=T).astype(np.float32)
    const_v = uniform_bf16(rng, (c["num_const"], H), -1.0, 1.0)
    out = dict(cfg=c, counts=counts, slot_src_row=slot_src_row.reshape(T, K),
               expert_ids=expert_ids.reshape(T, K), probs=probs, alpha1=alpha1,
               alpha2=alpha2, const_v=const_v)
    if with_rows:
        rr = rng_for(c["seed"] * 1000 + 1)
        out["x_rank_major"] = normal_bf16(rr, (N, H))
        out["shared_x"] = normal_bf16(rr, (T, H))
        out["ori_x"] = normal_bf16(rr, (T, H))
    return out


def gen_c5(with_rows: bool = True):
    """T=16384, H=4096, E=128, K=8; 13 experts (10%) never chosen; probs are
    the softmax values of the top-8 (not renormalised)."""
    c = CONFIGS[5]
    T, H, E, K = c["T"], c["H"], c["E"], c["K"]
    rng = rng_for(c["seed"])
    lg = rng.standard_normal(size=(T, E), dtype=np.float32)
    dead = rng.choice(E, size=c["empty_experts"], replace=False)
    lg[:, dead] = -np.inf
    ids, probs = route_topk(lg, K, renorm=False)
    out = dict(cfg=c, expert_ids=ids, probs=probs, dead_experts=np.sort(dead).astype(np.int32))
    if with_rows:
        rr = rng_for(c["seed"] * 1000 + 1)
        out["grad_out"] = normal_bf16(rr, (T, H))
        out["permuted"] = normal_bf16(rr, (T * K, H))
    return out


DERED = dict(name="deredundency_oep8_E256_H2048", oep=8, E=256, rows_per_source=8192, H=2048,
             expert_start=0, iep=8, El=32, seed=6)


def gen_dered(with_rows: bool = True):
    """One outer step of the deredundency combine at the skewed layer's sizes:
    8 source ranks, each with 1024 tokens x top-8 = 8192 routed rows over
    256 experts drawn with the Zipf(1.2) popularity of the skewed layer
    (counts[s] ~ Multinomial(8192, p), p_e proportional to rank_e^-1.2 with a
    seeded rank permutation); the outer range takes all 256 experts as
    8 destinations x 32 local experts. router_coeff ~ U(0, 1) per selected row,
    outer_output bf16 N(0, 1)."""
    c = DERED
    rng = rng_for(c["seed"])
    rank = rng.permutation(c["E"]) + 1
    pv = rank.astype(np.float64) ** -1.2
    pv /= pv.sum()
    counts = np.stack([rng.multinomial(c["rows_per_source"], pv)
                       for _ in range(c["oep"])]).astype(np.int32)
    n = int(counts[:, c["expert_start"]:c["expert_start"] + c["iep"] * c["El"]].sum())
    out = dict(cfg=c, counts=counts, n_selected=n, G=int(counts.sum()),
               router_coeff=rng.uniform(0.0, 1.0, size=n).astype(np.float32))
    if with_rows:
        out["outer_output"] = normal_bf16(rng_for(c["seed"] * 1000 + 1), (n, c["H"]))
    return out


def generate(cfg_id: int, **kw):
    return {1: gen_c1, 2: gen_c2, 3: gen_c3, 4: gen_c4, 5: gen_c5}[cfg_id](**kw)
