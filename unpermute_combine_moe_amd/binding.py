"""ctypes binding of libmoeperm (include/libmoeperm.h).

Argument marshalling only: every function here checks that the torch tensors it
is handed have the dtype / device / contiguity the C ABI expects, passes their
device pointers and the current HIP stream, and turns a non-OK status into a
MoeError. All computation happens in the HIP kernels of libmoeperm.so; if the
library is missing this module raises instead of computing anything itself.

Functions named like the C entry points take every output buffer explicitly;
the ``*_alloc`` helpers allocate outputs and workspace with torch first.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoeperm.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_str(status)} ({status})")


class MoeSpecialExperts(ctypes.Structure):
    _fields_ = [
        ("num_zero", _i32), ("num_copy", _i32), ("num_const", _i32),
        ("ori_x", _vp), ("alpha1", _vp), ("alpha2", _vp),
        ("alpha_stride_t", _i64), ("alpha_stride_c", _i64), ("alpha_stride_h", _i64),
        ("const_v", _vp),
    ]


EXPORTS = (
    "moe_status_str", "moe_abi_version",
    "moe_permute_workspace_size", "moe_permute", "moe_permute_noalloc", "moe_permute_rows",
    "moe_rank_to_expert_reorder_workspace_size", "moe_rank_to_expert_reorder",
    "moe_grouped_gemm_swiglu_workspace_size", "moe_grouped_gemm_swiglu",
    "moe_unpermute_combine", "moe_unpermute_grad", "moe_permute_grad",
    "moe_unpermute_combine_grad_workspace_size", "moe_unpermute_combine_grad",
    "moe_deredundency_dispatch_indices_workspace_size", "moe_deredundency_dispatch_indices",
    "moe_deredundency_combine_workspace_size", "moe_deredundency_combine",
    "moe_grouped_gemm_swiglu_grad_workspace_size", "moe_grouped_gemm_swiglu_grad",
)

_lib = None


def load(path: str = LIB_PATH):
    """Load libmoeperm.so and declare its signatures. Raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"libmoeperm is not built ({path} missing); run "
                          "`python -c 'import __graft_entry__ as g; g.build()'` first")
    lib = ctypes.CDLL(path)
    lib.moe_status_str.argtypes = [ctypes.c_int]
    lib.moe_status_str.restype = ctypes.c_char_p
    lib.moe_abi_version.argtypes = []
    lib.moe_abi_version.restype = _i32
    sz = ctypes.POINTER(ctypes.c_size_t)
    lib.moe_permute_workspace_size.argtypes = [_i64, _i32, _i32, sz]
    lib.moe_permute.argtypes = [_vp, _vp, _vp, _i32, _i64, _i32, _i32, _i32, _vp, _vp, _vp, _vp,
                                _vp, _vp, ctypes.c_size_t, _vp]
    lib.moe_permute_rows.argtypes = [_vp, _vp, _i64, _i32, _i32, _i64, _vp, _vp]
    lib.moe_permute_noalloc.argtypes = [_vp, _vp, _vp, _i32, _i64, _i32, _i32, _i32, _vp, _vp,
                                        _vp, _vp, _vp, _vp]
    lib.moe_rank_to_expert_reorder_workspace_size.argtypes = [_i32, _i32, sz]
    lib.moe_rank_to_expert_reorder.argtypes = [_vp, _vp, _i32, _i32, _i64, _i32, _vp, _vp, _vp,
                                               _vp, _vp, _vp, ctypes.c_size_t, _vp]
    lib.moe_grouped_gemm_swiglu_workspace_size.argtypes = [_i32, _i64, _i32, _i32, sz]
    lib.moe_grouped_gemm_swiglu.argtypes = [_vp, _vp, _i32, _i64, _i32, _i32, _vp, _vp, _vp, _vp,
                                            _vp, _vp, _vp, ctypes.c_size_t, _vp]
    lib.moe_unpermute_combine.argtypes = [_vp, _i64, _vp, _vp, _vp, _vp, _vp, _i32, _i64, _i32,
                                          _i32, _i32, ctypes.POINTER(MoeSpecialExperts), _vp, _vp,
                                          _vp]
    lib.moe_unpermute_grad.argtypes = [_vp, _vp, _i64, _vp, _vp, _i64, _i32, _i32, _vp, _vp, _vp]
    lib.moe_permute_grad.argtypes = [_vp, _i64, _vp, _i64, _i32, _i32, _vp, _vp]
    lib.moe_unpermute_combine_grad_workspace_size.argtypes = [_i64, _i32, _i32, sz]
    lib.moe_unpermute_combine_grad.argtypes = [
        _vp, _vp, _i64, _vp, _vp, _vp, _vp, _vp, _i32, _i64, _i32, _i32, _i32,
        ctypes.POINTER(MoeSpecialExperts), _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
    lib.moe_deredundency_dispatch_indices_workspace_size.argtypes = [_i32, _i32, _i32, _i32, sz]
    lib.moe_deredundency_dispatch_indices.argtypes = [_vp, _i32, _i32, _i32, _i32, _i32, _i64,
                                                      _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]
    lib.moe_deredundency_combine_workspace_size.argtypes = [_i64, _i64, sz]
    lib.moe_deredundency_combine.argtypes = [_vp, _vp, _vp, _i64, _i32, _i64, _vp, _vp,
                                             ctypes.c_size_t, _vp]
    lib.moe_grouped_gemm_swiglu_grad_workspace_size.argtypes = [_i32, _i64, _i32, _i32, sz]
    lib.moe_grouped_gemm_swiglu_grad.argtypes = [_vp, _vp, _i32, _i64, _i32, _i32, _vp, _vp, _vp,
                                                 _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                                 ctypes.c_size_t, _vp]
    for name in EXPORTS[2:]:
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def status_str(status: int) -> str:
    return load().moe_status_str(int(status)).decode()


def _check(status: int, where: str):
    if status != MOE_OK:
        raise MoeError(status, where)


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _ptr(t, dtype=None, name="tensor"):
    """Device pointer of a contiguous tensor (None -> NULL)."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if t.numel() > 0 and not t.is_cuda:
        raise ValueError(f"{name}: expected a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous tensor")
    return t.data_ptr() if t.numel() > 0 else None


_BF16 = torch.bfloat16
_I32 = torch.int32
_F32 = torch.float32


# --------------------------------------------------------------------------- workspaces

def moe_permute_workspace_size(T: int, K: int, E: int) -> int:
    n = ctypes.c_size_t(0)
    _check(load().moe_permute_workspace_size(T, K, E, ctypes.byref(n)), "moe_permute_workspace_size")
    return n.value


def moe_unpermute_combine_grad_workspace_size(T: int, H: int, num_const: int) -> int:
    n = ctypes.c_size_t(0)
    _check(load().moe_unpermute_combine_grad_workspace_size(T, H, num_const, ctypes.byref(n)),
           "moe_unpermute_combine_grad_workspace_size")
    return n.value


def moe_rank_to_expert_reorder_workspace_size(R: int, E_local: int) -> int:
    n = ctypes.c_size_t(0)
    _check(load().moe_rank_to_expert_reorder_workspace_size(R, E_local, ctypes.byref(n)),
           "moe_rank_to_expert_reorder_workspace_size")
    return n.value


def moe_grouped_gemm_swiglu_workspace_size(E: int, N_cap: int, H: int, I: int) -> int:
    n = ctypes.c_size_t(0)
    _check(load().moe_grouped_gemm_swiglu_workspace_size(E, N_cap, H, I, ctypes.byref(n)),
           "moe_grouped_gemm_swiglu_workspace_size")
    return n.value


def workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 16), dtype=torch.uint8, device=device)


# --------------------------------------------------------------------------- calls

def _mask(active_mask, T, K):
    """(pointer, per_slot) of an optional x_active_mask: bool or uint8, [T] or [T, K]."""
    if active_mask is None:
        return None, 0
    if active_mask.dtype not in (torch.bool, torch.uint8):
        raise TypeError(f"active_mask: expected bool or uint8, got {active_mask.dtype}")
    if tuple(active_mask.shape) == (T,):
        per_slot = 0
    elif tuple(active_mask.shape) == (T, K):
        per_slot = 1
    else:
        raise ValueError(f"active_mask: expected shape ({T},) or ({T}, {K}), "
                         f"got {tuple(active_mask.shape)}")
    return _ptr(active_mask, None, "active_mask"), per_slot


def moe_permute(x, expert_ids, T, H, K, num_experts, permuted, sorted_slot, row_of_slot,
                expert_counts, expert_offsets, ws, stream=None, *, active_mask=None):
    mp, per_slot = _mask(active_mask, T, K)
    _check(load().moe_permute(
        _ptr(x, _BF16, "x"), _ptr(expert_ids, _I32, "expert_ids"), mp, per_slot, T, H, K,
        num_experts,
        _ptr(permuted, _BF16, "permuted"), _ptr(sorted_slot, _I32, "sorted_slot"),
        _ptr(row_of_slot, _I32, "row_of_slot"), _ptr(expert_counts, _I32, "expert_counts"),
        _ptr(expert_offsets, _I32, "expert_offsets"), _ptr(ws, None, "workspace"),
        ws.numel() if ws is not None else 0, _stream(stream)), "moe_permute")


def moe_permute_rows(x, row_of_slot, T, H, K, N, permuted, stream=None):
    """The permute's row move alone: permuted[row_of_slot[t, k]] = x[t]."""
    _check(load().moe_permute_rows(
        _ptr(x, _BF16, "x"), _ptr(row_of_slot, _I32, "row_of_slot"), T, H, K, N,
        _ptr(permuted, _BF16, "permuted"), _stream(stream)), "moe_permute_rows")


def moe_permute_noalloc(x, expert_ids, T, H, K, num_experts, permuted, sorted_slot, row_of_slot,
                        expert_counts, expert_offsets, stream=None, *, active_mask=None):
    """moe_permute without a workspace: the library's own per-GPU array holds the
    count table (calls overlapping in time on one GPU must not be issued)."""
    mp, per_slot = _mask(active_mask, T, K)
    _check(load().moe_permute_noalloc(
        _ptr(x, _BF16, "x"), _ptr(expert_ids, _I32, "expert_ids"), mp, per_slot, T, H, K,
        num_experts,
        _ptr(permuted, _BF16, "permuted"), _ptr(sorted_slot, _I32, "sorted_slot"),
        _ptr(row_of_slot, _I32, "row_of_slot"), _ptr(expert_counts, _I32, "expert_counts"),
        _ptr(expert_offsets, _I32, "expert_offsets"), _stream(stream)), "moe_permute_noalloc")


def moe_rank_to_expert_reorder(x_rank_major, counts, R, E_local, N, H, y_expert_major, perm,
                               inv_perm, tokens_per_expert, expert_offsets, ws, stream=None):
    _check(load().moe_rank_to_expert_reorder(
        _ptr(x_rank_major, _BF16, "x_rank_major"), _ptr(counts, _I32, "counts"), R, E_local, N, H,
        _ptr(y_expert_major, _BF16, "y_expert_major"), _ptr(perm, _I32, "perm"),
        _ptr(inv_perm, _I32, "inv_perm"), _ptr(tokens_per_expert, _I32, "tokens_per_expert"),
        _ptr(expert_offsets, _I32, "expert_offsets"), _ptr(ws, None, "workspace"),
        ws.numel() if ws is not None else 0, _stream(stream)), "moe_rank_to_expert_reorder")


def moe_grouped_gemm_swiglu(x, expert_offsets, E, N_cap, H, I, w_gate, w_up, w_down, h, y, ws,
                            stream=None, preact=None):
    _check(load().moe_grouped_gemm_swiglu(
        _ptr(x, _BF16, "x"), _ptr(expert_offsets, _I32, "expert_offsets"), E, N_cap, H, I,
        _ptr(w_gate, _BF16, "w_gate"), _ptr(w_up, _BF16, "w_up"), _ptr(w_down, _BF16, "w_down"),
        _ptr(h, _BF16, "h"), _ptr(y, _BF16, "y"), _ptr(preact, _F32, "preact"),
        _ptr(ws, None, "workspace"), ws.numel() if ws is not None else 0, _stream(stream)),
        "moe_grouped_gemm_swiglu")


def make_special(num_zero=0, num_copy=0, num_const=0, ori_x=None, alpha1=None, alpha2=None,
                 alpha_strides=(0, 0, 0), const_v=None):
    """Build the moe_special_experts_t struct; keep the tensors alive meanwhile."""
    st, sc, sh = (int(v) for v in alpha_strides)
    return MoeSpecialExperts(num_zero, num_copy, num_const, _ptr(ori_x, _BF16, "ori_x"),
                             _ptr(alpha1, _F32, "alpha1"), _ptr(alpha2, _F32, "alpha2"), st, sc,
                             sh, _ptr(const_v, _BF16, "const_v"))


def moe_unpermute_combine(expert_out, N, row_of_slot, row_map, expert_ids, probs, T, K, H,
                          num_experts, special, shared_x, out, stream=None, *, active_mask=None):
    sp = ctypes.byref(special) if special is not None else None
    mp, per_slot = _mask(active_mask, T, K)
    _check(load().moe_unpermute_combine(
        _ptr(expert_out, _BF16, "expert_out"), N, _ptr(row_of_slot, _I32, "row_of_slot"),
        _ptr(row_map, _I32, "row_map"), _ptr(expert_ids, _I32, "expert_ids"),
        _ptr(probs, _F32, "probs"), mp, per_slot, T, K, H, num_experts, sp, _ptr(shared_x, _BF16, "shared_x"),
        _ptr(out, _BF16, "out"), _stream(stream)), "moe_unpermute_combine")


def moe_unpermute_grad(grad_out, permuted, N, row_of_slot, probs, T, K, H, d_permuted, d_probs,
                       stream=None):
    _check(load().moe_unpermute_grad(
        _ptr(grad_out, _BF16, "grad_out"), _ptr(permuted, _BF16, "permuted"), N,
        _ptr(row_of_slot, _I32, "row_of_slot"), _ptr(probs, _F32, "probs"), T, K, H,
        _ptr(d_permuted, _BF16, "d_permuted"), _ptr(d_probs, _F32, "d_probs"), _stream(stream)),
        "moe_unpermute_grad")


def moe_permute_grad(d_permuted, N, row_of_slot, T, K, H, d_x, stream=None):
    _check(load().moe_permute_grad(
        _ptr(d_permuted, _BF16, "d_permuted"), N, _ptr(row_of_slot, _I32, "row_of_slot"), T, K, H,
        _ptr(d_x, _BF16, "d_x"), _stream(stream)), "moe_permute_grad")


def moe_unpermute_combine_grad(grad_out, expert_out, N, row_of_slot, row_map, expert_ids, probs, T,
                               K, H, num_experts, special, d_expert_out, d_probs, d_ori_x,
                               d_alpha1, d_alpha2, d_const_v, ws, stream=None, *, active_mask=None):
    sp = ctypes.byref(special) if special is not None else None
    mp, per_slot = _mask(active_mask, T, K)
    _check(load().moe_unpermute_combine_grad(
        _ptr(grad_out, _BF16, "grad_out"), _ptr(expert_out, _BF16, "expert_out"), N,
        _ptr(row_of_slot, _I32, "row_of_slot"), _ptr(row_map, _I32, "row_map"),
        _ptr(expert_ids, _I32, "expert_ids"), _ptr(probs, _F32, "probs"), mp, per_slot, T, K, H,
        num_experts, sp,
        _ptr(d_expert_out, _BF16, "d_expert_out"), _ptr(d_probs, _F32, "d_probs"),
        _ptr(d_ori_x, _BF16, "d_ori_x"), _ptr(d_alpha1, _F32, "d_alpha1"),
        _ptr(d_alpha2, _F32, "d_alpha2"), _ptr(d_const_v, _BF16, "d_const_v"),
        _ptr(ws, None, "workspace"), ws.numel() if ws is not None else 0, _stream(stream)),
        "moe_unpermute_combine_grad")


def moe_deredundency_dispatch_indices_workspace_size(oep_size, num_experts, iep_size,
                                                     num_local_experts) -> int:
    n = ctypes.c_size_t(0)
    _check(load().moe_deredundency_dispatch_indices_workspace_size(
        oep_size, num_experts, iep_size, num_local_experts, ctypes.byref(n)),
        "moe_deredundency_dispatch_indices_workspace_size")
    return n.value


def moe_deredundency_dispatch_indices(tokens_per_expert_by_source, oep_size, num_experts,
                                      expert_start, iep_size, num_local_experts, capacity, indices,
                                      counts_by_dest, total, ws, stream=None):
    _check(load().moe_deredundency_dispatch_indices(
        _ptr(tokens_per_expert_by_source, _I32, "tokens_per_expert_by_source"), oep_size,
        num_experts, expert_start, iep_size, num_local_experts, capacity,
        _ptr(indices, _I32, "indices"), _ptr(counts_by_dest, _I32, "counts_by_dest"),
        _ptr(total, _I32, "total"), _ptr(ws, None, "workspace"),
        ws.numel() if ws is not None else 0, _stream(stream)), "moe_deredundency_dispatch_indices")


def moe_deredundency_combine_workspace_size(n, G) -> int:
    b = ctypes.c_size_t(0)
    _check(load().moe_deredundency_combine_workspace_size(n, G, ctypes.byref(b)),
           "moe_deredundency_combine_workspace_size")
    return b.value


def moe_deredundency_combine(outer_output, router_coeff, dispatch_indices, n, H, G, whiteboard, ws,
                             stream=None):
    _check(load().moe_deredundency_combine(
        _ptr(outer_output, _BF16, "outer_output"), _ptr(router_coeff, _F32, "router_coeff"),
        _ptr(dispatch_indices, _I32, "dispatch_indices"), n, H, G,
        _ptr(whiteboard, _BF16, "whiteboard"), _ptr(ws, None, "workspace"),
        ws.numel() if ws is not None else 0, _stream(stream)), "moe_deredundency_combine")


def moe_grouped_gemm_swiglu_grad_workspace_size(E, N_cap, H, I) -> int:
    n = ctypes.c_size_t(0)
    _check(load().moe_grouped_gemm_swiglu_grad_workspace_size(E, N_cap, H, I, ctypes.byref(n)),
           "moe_grouped_gemm_swiglu_grad_workspace_size")
    return n.value


def moe_grouped_gemm_swiglu_grad(x, expert_offsets, E, N_cap, H, I, w_gate, w_up, w_down, h, dy,
                                 dx, dw_gate, dw_up, dw_down, ws, stream=None, preact=None):
    _check(load().moe_grouped_gemm_swiglu_grad(
        _ptr(x, _BF16, "x"), _ptr(expert_offsets, _I32, "expert_offsets"), E, N_cap, H, I,
        _ptr(w_gate, _BF16, "w_gate"), _ptr(w_up, _BF16, "w_up"), _ptr(w_down, _BF16, "w_down"),
        _ptr(h, _BF16, "h"), _ptr(dy, _BF16, "dy"), _ptr(dx, _BF16, "dx"),
        _ptr(dw_gate, _BF16, "dw_gate"), _ptr(dw_up, _BF16, "dw_up"),
        _ptr(dw_down, _BF16, "dw_down"), _ptr(preact, _F32, "preact"),
        _ptr(ws, None, "workspace"), ws.numel() if ws is not None else 0, _stream(stream)),
        "moe_grouped_gemm_swiglu_grad")


# --------------------------------------------------------------------------- allocating helpers

def permute_alloc(x, expert_ids, num_experts, *, rows: bool = True, active_mask=None, stream=None):
    T, K = expert_ids.shape
    dev = expert_ids.device
    H = x.shape[1] if rows else 0
    S = T * K
    out = dict(
        permuted=torch.empty((S, H), dtype=_BF16, device=dev) if rows else None,
        sorted_slot=torch.empty(S, dtype=_I32, device=dev),
        row_of_slot=torch.empty((T, K), dtype=_I32, device=dev),
        expert_counts=torch.empty(num_experts, dtype=_I32, device=dev),
        expert_offsets=torch.empty(num_experts + 1, dtype=_I32, device=dev),
    )
    ws = workspace(moe_permute_workspace_size(T, K, num_experts), dev)
    moe_permute(x if rows else None, expert_ids, T, H, K, num_experts, out["permuted"],
                out["sorted_slot"], out["row_of_slot"], out["expert_counts"],
                out["expert_offsets"], ws, stream, active_mask=active_mask)
    return out


def reorder_alloc(x_rank_major, counts, R, E_local, N=None, *, rows: bool = True, stream=None):
    dev = counts.device
    if N is None:
        N = x_rank_major.shape[0]
    H = x_rank_major.shape[1] if rows else 0
    out = dict(
        y=torch.empty((N, H), dtype=_BF16, device=dev) if rows else None,
        perm=torch.empty(N, dtype=_I32, device=dev),
        inv_perm=torch.empty(N, dtype=_I32, device=dev),
        tokens_per_expert=torch.empty(E_local, dtype=_I32, device=dev),
        expert_offsets=torch.empty(E_local + 1, dtype=_I32, device=dev),
    )
    ws = workspace(moe_rank_to_expert_reorder_workspace_size(R, E_local), dev)
    moe_rank_to_expert_reorder(x_rank_major if rows else None, counts, R, E_local, N, H, out["y"],
                               out["perm"], out["inv_perm"], out["tokens_per_expert"],
                               out["expert_offsets"], ws, stream)
    return out


def grouped_gemm_alloc(x, expert_offsets, w_gate, w_up, w_down, *, stream=None,
                       keep_preact=False):
    """Returns (h, y), or (h, y, preact) with keep_preact (fp32 [N_cap, 2I], g | u)."""
    E, H, I = w_gate.shape
    N_cap = x.shape[0]
    dev = x.device
    h = torch.empty((N_cap, I), dtype=_BF16, device=dev)
    y = torch.empty((N_cap, H), dtype=_BF16, device=dev)
    preact = torch.empty((N_cap, 2 * I), dtype=_F32, device=dev) if keep_preact else None
    ws = workspace(moe_grouped_gemm_swiglu_workspace_size(E, N_cap, H, I), dev)
    moe_grouped_gemm_swiglu(x, expert_offsets, E, N_cap, H, I, w_gate, w_up, w_down, h, y, ws,
                            stream, preact=preact)
    return (h, y, preact) if keep_preact else (h, y)


def combine_alloc(expert_out, row_of_slot, expert_ids, probs, num_experts, *, row_map=None,
                  special=None, shared_x=None, H=None, active_mask=None, stream=None):
    T, K = expert_ids.shape
    if H is None:
        H = expert_out.shape[1]
    N = expert_out.shape[0] if expert_out is not None else 0
    out = torch.empty((T, H), dtype=_BF16, device=expert_ids.device)
    moe_unpermute_combine(expert_out, N, row_of_slot, row_map, expert_ids, probs, T, K, H,
                          num_experts, special, shared_x, out, stream, active_mask=active_mask)
    return out


def unpermute_grad_alloc(grad_out, permuted, row_of_slot, probs, *, d_permuted=None, stream=None):
    T, K = probs.shape
    N, H = permuted.shape
    if d_permuted is None:
        d_permuted = torch.zeros((N, H), dtype=_BF16, device=permuted.device)
    d_probs = torch.empty((T, K), dtype=_F32, device=permuted.device)
    moe_unpermute_grad(grad_out, permuted, N, row_of_slot, probs, T, K, H, d_permuted, d_probs,
                       stream)
    return d_permuted, d_probs


def permute_grad_alloc(d_permuted, row_of_slot, *, stream=None):
    T, K = row_of_slot.shape
    N, H = d_permuted.shape
    d_x = torch.empty((T, H), dtype=_BF16, device=d_permuted.device)
    moe_permute_grad(d_permuted, N, row_of_slot, T, K, H, d_x, stream)
    return d_x


def combine_grad_alloc(grad_out, expert_out, row_of_slot, expert_ids, probs, num_experts, *,
                       row_map=None, special=None, alpha_numel=0, d_expert_out=None,
                       want=("d_expert_out", "d_probs", "d_ori_x", "d_alpha", "d_const_v"),
                       active_mask=None, stream=None):
    """Backward of the combine. Returns a dict with the requested outputs
    (d_alpha1 / d_alpha2 as flat fp32 tensors of alpha_numel elements,
    zero-filled before the call)."""
    T, K = expert_ids.shape
    H = grad_out.shape[1]
    N = expert_out.shape[0] if expert_out is not None else 0
    dev = grad_out.device
    nc = special.num_const if special is not None else 0
    r = {"d_probs": torch.empty((T, K), dtype=_F32, device=dev)}
    if "d_expert_out" in want:
        r["d_expert_out"] = (d_expert_out if d_expert_out is not None
                             else torch.zeros((N, H), dtype=_BF16, device=dev))
    if "d_ori_x" in want:
        r["d_ori_x"] = torch.empty((T, H), dtype=_BF16, device=dev)
    if "d_alpha" in want and nc > 0:
        r["d_alpha1"] = torch.zeros(alpha_numel, dtype=_F32, device=dev)
        r["d_alpha2"] = torch.zeros(alpha_numel, dtype=_F32, device=dev)
    if "d_const_v" in want:
        r["d_const_v"] = torch.empty((nc, H), dtype=_BF16, device=dev)
    ws = workspace(moe_unpermute_combine_grad_workspace_size(T, H, nc), dev)
    moe_unpermute_combine_grad(grad_out, expert_out, N, row_of_slot, row_map, expert_ids, probs, T,
                               K, H, num_experts, special, r.get("d_expert_out"), r["d_probs"],
                               r.get("d_ori_x"), r.get("d_alpha1"), r.get("d_alpha2"),
                               r.get("d_const_v"), ws, stream, active_mask=active_mask)
    return r


def dered_indices_alloc(tokens_per_expert_by_source, expert_start, iep_size, num_local_experts, *,
                        capacity=None, stream=None):
    """Returns dict(indices [capacity], counts_by_dest, total [1]); capacity
    defaults to the number of gathered rows (no host read of the counts)."""
    oep, E = tokens_per_expert_by_source.shape
    dev = tokens_per_expert_by_source.device
    if capacity is None:
        raise ValueError("capacity: give the row capacity of the indices buffer")
    out = dict(indices=torch.empty(capacity, dtype=_I32, device=dev),
               counts_by_dest=torch.empty(iep_size * num_local_experts, dtype=_I32, device=dev),
               total=torch.empty(1, dtype=_I32, device=dev))
    ws = workspace(moe_deredundency_dispatch_indices_workspace_size(oep, E, iep_size,
                                                                    num_local_experts), dev)
    moe_deredundency_dispatch_indices(tokens_per_expert_by_source, oep, E, expert_start, iep_size,
                                      num_local_experts, capacity, out["indices"],
                                      out["counts_by_dest"], out["total"], ws, stream)
    return out


def dered_combine_alloc(outer_output, router_coeff, dispatch_indices, G, *, stream=None):
    n, H = outer_output.shape
    wb = torch.empty((G, H), dtype=_BF16, device=outer_output.device)
    ws = workspace(moe_deredundency_combine_workspace_size(n, G), outer_output.device)
    moe_deredundency_combine(outer_output, router_coeff, dispatch_indices, n, H, G, wb, ws, stream)
    return wb


def grouped_gemm_grad_alloc(x, expert_offsets, w_gate, w_up, w_down, h, dy, *, stream=None,
                            preact=None):
    """Backward of the grouped SwiGLU FFN. Returns dict(dx, dw_gate, dw_up, dw_down).
    preact: the forward's pre-activations (grouped_gemm_alloc(keep_preact=True)), or None
    to recompute them."""
    E, H, I = w_gate.shape
    N_cap = x.shape[0]
    dev = x.device
    out = dict(dx=torch.zeros((N_cap, H), dtype=_BF16, device=dev),
               dw_gate=torch.empty((E, H, I), dtype=_BF16, device=dev),
               dw_up=torch.empty((E, H, I), dtype=_BF16, device=dev),
               dw_down=torch.empty((E, I, H), dtype=_BF16, device=dev))
    ws = workspace(moe_grouped_gemm_swiglu_grad_workspace_size(E, N_cap, H, I), dev)
    moe_grouped_gemm_swiglu_grad(x, expert_offsets, E, N_cap, H, I, w_gate, w_up, w_down, h, dy,
                                 out["dx"], out["dw_gate"], out["dw_up"], out["dw_down"], ws,
                                 stream, preact=preact)
    return out
