"""numpy front end of the CPU oracle (oracle/moe_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg, never by the GPU library or its binding. It
shares no code with the GPU path. bf16 arrays are numpy uint16 bit patterns.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libmoe_oracle.so")
_lib = None

_i32p = ctypes.POINTER(ctypes.c_int32)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_f32p = ctypes.POINTER(ctypes.c_float)
_u8p = ctypes.POINTER(ctypes.c_uint8)
_f64p = ctypes.POINTER(ctypes.c_double)
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _b
        _b.build()
    lib = ctypes.CDLL(_LIB_PATH)
    lib.orc_bf16_to_f64.argtypes = [ctypes.c_uint16]
    lib.orc_bf16_to_f64.restype = ctypes.c_double
    lib.orc_f64_to_bf16.argtypes = [ctypes.c_double]
    lib.orc_f64_to_bf16.restype = ctypes.c_uint16
    lib.orc_f64_to_bf16_array.argtypes = [_f64p, _u16p, _i64]
    lib.orc_f64_to_bf16_array.restype = None
    lib.orc_permute.argtypes = [_u16p, _i32p, _i64, _i32, _i32, _i32, _u16p, _i32p, _i32p,
                                _i32p, _i32p]
    lib.orc_reorder_loop.argtypes = [_u16p, _i32p, _i32, _i32, _i64, _i32, _u16p, _i32p, _i32p,
                                     _i32p, _i32p]
    lib.orc_reorder_index_vectorized.argtypes = [_i32p, _i32, _i32, _i64, _i32p, _i32p]
    lib.orc_swiglu_row.argtypes = [_u16p, _i32, _i32, _u16p, _u16p, _u16p, _f64p, _f64p]
    lib.orc_grouped_swiglu.argtypes = [_u16p, _i32p, _i32, _i64, _i32, _i32, _u16p, _u16p,
                                       _u16p, _f64p, _f64p]
    lib.orc_combine.argtypes = [_u16p, _i64, _i32p, _i32p, _i32p, _f32p, _i64, _i32, _i32, _i32,
                                _i32, _i32, _i32, _u16p, _f32p, _f32p, _i64, _i64, _i64, _u16p,
                                _u16p, _u16p, _f64p]
    lib.orc_unpermute_grad.argtypes = [_u16p, _u16p, _i64, _i32p, _f32p, _i64, _i32, _i32, _u16p,
                                       _f32p, _f64p, _f64p]
    lib.orc_permute_grad.argtypes = [_u16p, _i64, _i32p, _i64, _i32, _i32, _u16p, _f64p]
    lib.orc_combine_grad.argtypes = [_u16p, _u16p, _i64, _i32p, _i32p, _i32p, _f32p, _i64, _i32,
                                     _i32, _i32, _i32, _i32, _i32, _u16p, _f32p, _f32p, _i64,
                                     _i64, _i64, _i64, _u16p, _f64p, _u8p, _f64p, _f64p, _f64p,
                                     _f64p, _f64p, _f64p]
    _i64p = ctypes.POINTER(ctypes.c_int64)
    for name in ("orc_dered_indices_loop", "orc_dered_indices_vectorized"):
        getattr(lib, name).argtypes = [_i32p, _i32, _i32, _i32, _i32, _i32, _i64, _i32p, _i32p,
                                       _i64p]
        getattr(lib, name).restype = ctypes.c_int
    lib.orc_scatter_add_rows.argtypes = [_u16p, _f32p, _i32p, _i64, _i32, _i64, _u16p, _f64p]
    lib.orc_scatter_add_rows.restype = ctypes.c_int
    lib.orc_grouped_swiglu_grad.argtypes = [_u16p, _i32p, _i32, _i64, _i32, _i32, _u16p, _u16p,
                                            _u16p, _u16p, _f64p, _f64p, _f64p, _f64p, _f64p,
                                            _f64p, _f64p]
    lib.orc_grouped_swiglu_grad.restype = ctypes.c_int
    lib.orc_num_threads.argtypes = []
    for name in ("orc_permute", "orc_reorder_loop", "orc_reorder_index_vectorized",
                 "orc_swiglu_row", "orc_grouped_swiglu", "orc_combine", "orc_unpermute_grad",
                 "orc_permute_grad", "orc_combine_grad", "orc_num_threads"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a, ctype):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctype))


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (rc={rc})")


def num_threads() -> int:
    return int(_load().orc_num_threads())


# --------------------------------------------------------------------------- bf16

def bf16_to_f64(bits) -> np.ndarray:
    b = _c(bits, np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def f64_to_bf16(values) -> np.ndarray:
    v = _c(values, np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    _load().orc_f64_to_bf16_array(_ptr(v, ctypes.c_double), _ptr(out, ctypes.c_uint16), v.size)
    return out


def f64_to_bf16_scalar(value: float) -> int:
    return int(_load().orc_f64_to_bf16(float(value)))


# --------------------------------------------------------------------------- permute

def _mask_slots(expert_ids, active_mask):
    """x_active_mask ("torch_npu.npu_moe_distribute_combine_v2", 参数说明): a
    [T] mask marks whole tokens, a [T, K] mask single slots, as taking part in
    the exchange. A slot that does not take part is never sent to its expert
    and never comes back: it is a dropped slot, id -1 (no row, no term)."""
    ids = _c(expert_ids, np.int32)
    if active_mask is None:
        return ids
    m = np.asarray(active_mask).astype(bool)
    if m.ndim == 1:
        m = np.repeat(m[:, None], ids.shape[1], axis=1)
    assert m.shape == ids.shape, (m.shape, ids.shape)
    return np.where(m, ids, np.int32(-1)).astype(np.int32)


def permute(x, expert_ids, E: int, *, rows: bool = True, active_mask=None):
    """Stable expert-major permute. Returns dict(permuted, sorted_slot,
    row_of_slot, expert_counts, expert_offsets). Slots outside active_mask
    (optional, [T] or [T, K]) are not routed."""
    ids = _mask_slots(expert_ids, active_mask)
    T, K = ids.shape
    xx = _c(x, np.uint16) if rows else None
    H = xx.shape[1] if rows else 1
    S = T * K
    permuted = np.zeros((S, H), dtype=np.uint16) if rows else None
    sorted_slot = np.empty(S, dtype=np.int32)
    row_of_slot = np.empty(S, dtype=np.int32)
    counts = np.empty(E, dtype=np.int32)
    offsets = np.empty(E + 1, dtype=np.int32)
    rc = _load().orc_permute(_ptr(xx, ctypes.c_uint16), _ptr(ids, ctypes.c_int32), T, H, K, E,
                             _ptr(permuted, ctypes.c_uint16), _ptr(sorted_slot, ctypes.c_int32),
                             _ptr(row_of_slot, ctypes.c_int32), _ptr(counts, ctypes.c_int32),
                             _ptr(offsets, ctypes.c_int32))
    _check(rc, "permute")
    return dict(permuted=permuted, sorted_slot=sorted_slot, row_of_slot=row_of_slot.reshape(T, K),
                expert_counts=counts, expert_offsets=offsets)


# --------------------------------------------------------------------------- reorder

def reorder(x, counts, R: int, E_local: int, N: int | None = None, *, rows: bool = True):
    """Rank-major -> expert-major reorder (block-loop form)."""
    cnt = _c(counts, np.int32)
    xx = _c(x, np.uint16) if rows else None
    if N is None:
        N = int(xx.shape[0]) if rows else int(cnt.sum())
    H = xx.shape[1] if rows else 1
    y = np.zeros((N, H), dtype=np.uint16) if rows else None
    perm = np.empty(N, dtype=np.int32)
    inv = np.empty(N, dtype=np.int32)
    tpe = np.empty(E_local, dtype=np.int32)
    off = np.empty(E_local + 1, dtype=np.int32)
    rc = _load().orc_reorder_loop(_ptr(xx, ctypes.c_uint16), _ptr(cnt, ctypes.c_int32), R,
                                  E_local, N, H, _ptr(y, ctypes.c_uint16),
                                  _ptr(perm, ctypes.c_int32), _ptr(inv, ctypes.c_int32),
                                  _ptr(tpe, ctypes.c_int32), _ptr(off, ctypes.c_int32))
    _check(rc, "reorder")
    return dict(y=y, perm=perm, inv_perm=inv, tokens_per_expert=tpe, expert_offsets=off)


def reorder_index_vectorized(counts, R: int, E_local: int, N: int | None = None):
    cnt = _c(counts, np.int32)
    if N is None:
        N = int(cnt.sum())
    perm = np.empty(N, dtype=np.int32)
    tpe = np.empty(E_local, dtype=np.int32)
    rc = _load().orc_reorder_index_vectorized(_ptr(cnt, ctypes.c_int32), R, E_local, N,
                                              _ptr(perm, ctypes.c_int32), _ptr(tpe, ctypes.c_int32))
    _check(rc, "reorder_index_vectorized")
    return dict(perm=perm, tokens_per_expert=tpe)


# --------------------------------------------------------------------------- expert FFN

def swiglu_row(x_row, wg_e, wu_e, wd_e):
    xr = _c(x_row, np.uint16)
    wg, wu, wd = _c(wg_e, np.uint16), _c(wu_e, np.uint16), _c(wd_e, np.uint16)
    H, I = wg.shape
    h = np.empty(I, dtype=np.float64)
    y = np.empty(H, dtype=np.float64)
    rc = _load().orc_swiglu_row(_ptr(xr, ctypes.c_uint16), H, I, _ptr(wg, ctypes.c_uint16),
                                _ptr(wu, ctypes.c_uint16), _ptr(wd, ctypes.c_uint16),
                                _ptr(h, ctypes.c_double), _ptr(y, ctypes.c_double))
    _check(rc, "swiglu_row")
    return h, y


def grouped_swiglu(x, expert_offsets, w_gate, w_up, w_down, *, want_h: bool = True):
    """fp64 SwiGLU FFN per expert group. Returns (h [N,I] or None, y [N,H])."""
    xx = _c(x, np.uint16)
    off = _c(expert_offsets, np.int32)
    wg, wu, wd = _c(w_gate, np.uint16), _c(w_up, np.uint16), _c(w_down, np.uint16)
    E, H, I = wg.shape
    N = xx.shape[0]
    h = np.zeros((N, I), dtype=np.float64) if want_h else None
    y = np.zeros((N, H), dtype=np.float64)
    rc = _load().orc_grouped_swiglu(_ptr(xx, ctypes.c_uint16), _ptr(off, ctypes.c_int32), E, N, H,
                                    I, _ptr(wg, ctypes.c_uint16), _ptr(wu, ctypes.c_uint16),
                                    _ptr(wd, ctypes.c_uint16), _ptr(h, ctypes.c_double),
                                    _ptr(y, ctypes.c_double))
    _check(rc, "grouped_swiglu")
    return h, y


def grouped_swiglu_grad(x, expert_offsets, w_gate, w_up, w_down, dy):
    """fp64 backward of grouped_swiglu. Returns dict(dx [N,H], dwg, dwu [E,H,I],
    dwd [E,I,H], dh, dg, du [N,I])."""
    xx = _c(x, np.uint16)
    off = _c(expert_offsets, np.int32)
    wg, wu, wd = _c(w_gate, np.uint16), _c(w_up, np.uint16), _c(w_down, np.uint16)
    g = _c(dy, np.uint16)
    E, H, I = wg.shape
    N = xx.shape[0]
    r = dict(dx=np.zeros((N, H)), dwg=np.zeros((E, H, I)), dwu=np.zeros((E, H, I)),
             dwd=np.zeros((E, I, H)), dh=np.zeros((N, I)), dg=np.zeros((N, I)),
             du=np.zeros((N, I)))
    rc = _load().orc_grouped_swiglu_grad(
        _ptr(xx, ctypes.c_uint16), _ptr(off, ctypes.c_int32), E, N, H, I,
        _ptr(wg, ctypes.c_uint16), _ptr(wu, ctypes.c_uint16), _ptr(wd, ctypes.c_uint16),
        _ptr(g, ctypes.c_uint16), *(_ptr(r[k], ctypes.c_double)
                                    for k in ("dx", "dwg", "dwu", "dwd", "dh", "dg", "du")))
    _check(rc, "grouped_swiglu_grad")
    return r


# --------------------------------------------------------------------------- combine

def combine(expert_out, row_of_slot, expert_ids, probs, E: int, *, row_map=None,
            num_zero: int = 0, num_copy: int = 0, num_const: int = 0, ori_x=None,
            alpha1=None, alpha2=None, alpha_strides=(0, 0, 0), const_v=None, shared_x=None,
            H: int | None = None, active_mask=None):
    """Weighted unpermute-combine. Returns (out bf16 bits [T,H], out_f64 [T,H]).
    Slots outside active_mask (optional, [T] or [T, K]) add no term; the
    shared row is still added."""
    ids = _mask_slots(expert_ids, active_mask)
    T, K = ids.shape
    ros = _c(row_of_slot, np.int32)
    pr = _c(probs, np.float32)
    eo = _c(expert_out, np.uint16) if expert_out is not None else None
    if H is None:
        H = eo.shape[1]
    N = eo.shape[0] if eo is not None else 0
    rm = _c(row_map, np.int32) if row_map is not None else None
    ox = _c(ori_x, np.uint16) if ori_x is not None else None
    a1 = _c(alpha1, np.float32) if alpha1 is not None else None
    a2 = _c(alpha2, np.float32) if alpha2 is not None else None
    cv = _c(const_v, np.uint16) if const_v is not None else None
    sx = _c(shared_x, np.uint16) if shared_x is not None else None
    out = np.empty((T, H), dtype=np.uint16)
    out64 = np.empty((T, H), dtype=np.float64)
    st, sc, sh = (int(v) for v in alpha_strides)
    rc = _load().orc_combine(_ptr(eo, ctypes.c_uint16), N, _ptr(ros, ctypes.c_int32),
                             _ptr(rm, ctypes.c_int32), _ptr(ids, ctypes.c_int32),
                             _ptr(pr, ctypes.c_float), T, K, H, E, num_zero, num_copy, num_const,
                             _ptr(ox, ctypes.c_uint16), _ptr(a1, ctypes.c_float),
                             _ptr(a2, ctypes.c_float), st, sc, sh, _ptr(cv, ctypes.c_uint16),
                             _ptr(sx, ctypes.c_uint16), _ptr(out, ctypes.c_uint16),
                             _ptr(out64, ctypes.c_double))
    _check(rc, "combine")
    return out, out64


# --------------------------------------------------------------------------- backward

def unpermute_grad(grad_out, permuted, row_of_slot, probs, *, d_permuted_init=None):
    """Returns (d_permuted bf16 [N,H], d_probs fp32 [T,K], d_permuted_f64, d_probs_f64)."""
    g = _c(grad_out, np.uint16)
    pm = _c(permuted, np.uint16)
    ros = _c(row_of_slot, np.int32)
    pr = _c(probs, np.float32)
    T, K = pr.shape
    H = g.shape[1]
    N = pm.shape[0]
    dperm = (np.array(d_permuted_init, dtype=np.uint16, copy=True) if d_permuted_init is not None
             else np.zeros((N, H), dtype=np.uint16))
    dperm64 = np.zeros((N, H), dtype=np.float64)
    dprobs = np.empty((T, K), dtype=np.float32)
    dprobs64 = np.empty((T, K), dtype=np.float64)
    rc = _load().orc_unpermute_grad(_ptr(g, ctypes.c_uint16), _ptr(pm, ctypes.c_uint16), N,
                                    _ptr(ros, ctypes.c_int32), _ptr(pr, ctypes.c_float), T, K, H,
                                    _ptr(dperm, ctypes.c_uint16), _ptr(dprobs, ctypes.c_float),
                                    _ptr(dperm64, ctypes.c_double),
                                    _ptr(dprobs64, ctypes.c_double))
    _check(rc, "unpermute_grad")
    return dperm, dprobs, dperm64, dprobs64


def permute_grad(d_permuted, row_of_slot):
    """Permute backward: returns (d_x bf16 [T,H], d_x_f64 [T,H]);
    d_x[t] = sum over the token's slots with a row of d_permuted[row]."""
    dp = _c(d_permuted, np.uint16)
    ros = _c(row_of_slot, np.int32)
    T, K = ros.shape
    N, H = dp.shape
    dx = np.empty((T, H), dtype=np.uint16)
    dx64 = np.empty((T, H), dtype=np.float64)
    rc = _load().orc_permute_grad(_ptr(dp, ctypes.c_uint16), N, _ptr(ros, ctypes.c_int32), T, K,
                                  H, _ptr(dx, ctypes.c_uint16), _ptr(dx64, ctypes.c_double))
    _check(rc, "permute_grad")
    return dx, dx64


def combine_grad(grad_out, expert_out, row_of_slot, expert_ids, probs, E: int, *, row_map=None,
                 num_zero: int = 0, num_copy: int = 0, num_const: int = 0, ori_x=None,
                 alpha1=None, alpha2=None, alpha_strides=(0, 0, 0), const_v=None,
                 active_mask=None):
    """Backward of combine() (special and shared experts included), all in fp64.
    Returns a dict: d_expert_out [N,H] (0 in rows no slot references), row_written
    [N] bool, d_probs [T,K], d_ori_x [T,H], d_alpha1 / d_alpha2 (alpha's flat
    layout), d_const_v [num_const,H], d_shared [T,H]."""
    g = _c(grad_out, np.uint16)
    ids = _mask_slots(expert_ids, active_mask)
    T, K = ids.shape
    H = g.shape[1]
    ros = _c(row_of_slot, np.int32)
    pr = _c(probs, np.float32)
    eo = _c(expert_out, np.uint16) if expert_out is not None else None
    N = eo.shape[0] if eo is not None else 0
    rm = _c(row_map, np.int32) if row_map is not None else None
    ox = _c(ori_x, np.uint16) if ori_x is not None else None
    a1 = _c(alpha1, np.float32).reshape(-1) if alpha1 is not None else None
    a2 = _c(alpha2, np.float32).reshape(-1) if alpha2 is not None else None
    n_alpha = a1.size if a1 is not None else 0
    cv = _c(const_v, np.uint16) if const_v is not None else None
    st, sc, sh = (int(v) for v in alpha_strides)
    out = dict(d_expert_out=np.zeros((N, H)), row_written=np.zeros(N, np.uint8),
               d_probs=np.zeros((T, K)), d_ori_x=np.zeros((T, H)), d_alpha1=np.zeros(n_alpha),
               d_alpha2=np.zeros(n_alpha), d_const_v=np.zeros((num_const, H)),
               d_shared=np.zeros((T, H)))
    rc = _load().orc_combine_grad(
        _ptr(g, ctypes.c_uint16), _ptr(eo, ctypes.c_uint16), N, _ptr(ros, ctypes.c_int32),
        _ptr(rm, ctypes.c_int32), _ptr(ids, ctypes.c_int32), _ptr(pr, ctypes.c_float), T, K, H, E,
        num_zero, num_copy, num_const, _ptr(ox, ctypes.c_uint16), _ptr(a1, ctypes.c_float),
        _ptr(a2, ctypes.c_float), st, sc, sh, n_alpha, _ptr(cv, ctypes.c_uint16),
        *(_ptr(out[k], ctypes.c_uint8 if k == "row_written" else ctypes.c_double)
          for k in ("d_expert_out", "row_written", "d_probs", "d_ori_x", "d_alpha1", "d_alpha2",
                    "d_const_v", "d_shared")))
    _check(rc, "combine_grad")
    out["row_written"] = out["row_written"].astype(bool)
    return out


# --------------------------------------------------------------------------- deredundency

def dered_indices(counts_by_source, expert_start: int, iep_size: int, num_local: int, *,
                  capacity: int | None = None, form: str = "loop"):
    """Deredundency dispatch indices. Returns (indices [capacity] int32 with -1
    past the total, counts_by_dest [iep_size*num_local], total)."""
    c = _c(counts_by_source, np.int32)
    oep, E = c.shape
    if capacity is None:
        capacity = int(np.maximum(c, 0).sum())
    idx = np.empty(capacity, dtype=np.int32)
    cbd = np.empty(iep_size * num_local, dtype=np.int32)
    tot = ctypes.c_int64(0)
    fn = {"loop": _load().orc_dered_indices_loop,
          "vectorized": _load().orc_dered_indices_vectorized}[form]
    rc = fn(_ptr(c, ctypes.c_int32), oep, E, expert_start, iep_size, num_local, capacity,
            _ptr(idx, ctypes.c_int32), _ptr(cbd, ctypes.c_int32), ctypes.byref(tot))
    _check(rc, "dered_indices")
    return idx, cbd, int(tot.value)


def scatter_add_rows(src, indices, G: int, coeff=None):
    """whiteboard = zeros[G, H]; whiteboard[indices[j]] += coeff[j] * src[j].
    Returns (bf16 bits [G, H], fp64 [G, H])."""
    sr = _c(src, np.uint16)
    n, H = sr.shape
    ix = _c(indices, np.int32)
    cf = _c(coeff, np.float32) if coeff is not None else None
    out = np.empty((G, H), dtype=np.uint16)
    out64 = np.empty((G, H), dtype=np.float64)
    rc = _load().orc_scatter_add_rows(_ptr(sr, ctypes.c_uint16), _ptr(cf, ctypes.c_float),
                                      _ptr(ix, ctypes.c_int32), n, H, G,
                                      _ptr(out, ctypes.c_uint16), _ptr(out64, ctypes.c_double))
    _check(rc, "scatter_add_rows")
    return out, out64
