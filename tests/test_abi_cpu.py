"""Host-side checks of libmoeperm (no GPU needed): the library loads, exports
every entry point include/libmoeperm.h declares, and every argument check
returns its status before anything is enqueued.

The argument checks are driven with fake, never-dereferenced pointers; they run
only where no GPU is visible, so that a check that wrongly passed could not
launch a kernel on such pointers."""
import ctypes
import os
import re
import subprocess

import pytest
import torch

import __graft_entry__ as ge

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "libmoeperm.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
no_gpu = pytest.mark.skipif(torch.cuda.is_available(),
                            reason="fake-pointer argument checks run only without a GPU")


@pytest.fixture(scope="module")
def lib():
    ge._ensure_built()
    from unpermute_combine_moe_amd import binding

    return binding.load()


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_\w+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    from unpermute_combine_moe_amd import binding

    names = _declared()
    assert set(names) == set(binding.EXPORTS), names
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r" T (\w+)$", out, flags=re.M))
    for n in names:
        assert n in exported, n
        assert hasattr(lib, n)
    # nothing else of ours leaks out of the library
    assert {s for s in exported if s.startswith("moe_")} == set(names)


def test_status_strings_and_version(lib):
    from unpermute_combine_moe_amd import binding

    assert binding.status_str(0) == "MOE_OK"
    assert binding.status_str(3) == "MOE_ERR_WORKSPACE"
    assert binding.status_str(99) == "MOE_ERR_UNKNOWN"
    assert lib.moe_abi_version() == 3


def test_workspace_sizes(lib):
    from unpermute_combine_moe_amd import binding as b

    assert b.moe_permute_workspace_size(8192, 8, 256) >= 4 * 256
    assert b.moe_permute_workspace_size(0, 8, 256) > 0
    assert b.moe_rank_to_expert_reorder_workspace_size(8, 32) >= 4 * 8 * 32 * 4
    assert b.moe_grouped_gemm_swiglu_workspace_size(256, 65536, 2048, 512) >= 8 * 257
    with pytest.raises(b.MoeError):
        b.moe_permute_workspace_size(10, 17, 4)
    with pytest.raises(b.MoeError):
        b.moe_permute_workspace_size(10, 2, 1025)
    with pytest.raises(b.MoeError):
        b.moe_rank_to_expert_reorder_workspace_size(512, 256)
    with pytest.raises(b.MoeError) as e:
        b.moe_grouped_gemm_swiglu_workspace_size(8, 100, 96, 64)
    assert e.value.status == UNSUPPORTED
    # H and I above 2^20 (the epilogue's 32-bit tile offsets) are refused,
    # for the forward and the backward alike
    for H, I in ((1 << 20, 64), (64, 1 << 20)):
        assert b.moe_grouped_gemm_swiglu_workspace_size(8, 100, H, I) > 0
        assert b.moe_grouped_gemm_swiglu_grad_workspace_size(8, 100, H, I) > 0
    for H, I in (((1 << 20) + 64, 64), (64, (1 << 20) + 64)):
        for f in (b.moe_grouped_gemm_swiglu_workspace_size,
                  b.moe_grouped_gemm_swiglu_grad_workspace_size):
            with pytest.raises(b.MoeError) as e:
                f(8, 100, H, I)
            assert e.value.status == UNSUPPORTED


P = 0x10000        # fake 16-byte aligned device address, never dereferenced
PM = P + 2         # misaligned


def _permute(lib, x=P, ids=P, T=16, H=64, K=2, E=4, perm=P, ss=P, ros=P, cnt=P, off=P, ws=P,
             wsb=1 << 20, mask=None, per_slot=0):
    return lib.moe_permute(x, ids, mask, per_slot, T, H, K, E, perm, ss, ros, cnt, off, ws, wsb,
                           None)


@no_gpu
def test_permute_checks(lib):
    assert _permute(lib, T=-1) == INVALID
    assert _permute(lib, K=0) == INVALID
    assert _permute(lib, K=17) == INVALID
    assert _permute(lib, E=0) == INVALID
    assert _permute(lib, E=1025) == INVALID
    assert _permute(lib, T=2**30, K=4) == INVALID       # T*K past int32
    assert _permute(lib, H=12) == UNSUPPORTED
    assert _permute(lib, H=0) == INVALID
    assert _permute(lib, ids=None) == INVALID
    assert _permute(lib, ros=PM) == INVALID
    assert _permute(lib, x=P + 8) == INVALID            # rows need 16-byte alignment
    assert _permute(lib, x=None) == INVALID             # rows requested without x
    assert _permute(lib, cnt=None) == INVALID
    assert _permute(lib, ws=None) == WORKSPACE
    assert _permute(lib, wsb=4) == WORKSPACE
    assert _permute(lib, mask=P, per_slot=2) == INVALID


def test_permute_table_fits_the_noalloc_array(lib):
    """moe_permute_noalloc keeps the permute's count table in a 64 KiB array:
    every legal (T*K, E) must need at most that."""
    from unpermute_combine_moe_amd import binding as b

    Es = sorted({1, 2, 3, 5, 7, 8, 63, 64, 65, 100, 127, 128, 255, 256, 257, 500, 511, 512, 513,
                 1000, 1023, 1024})
    Ss = sorted({0, 1, 2, 255, 256, 257, 511, 512, 513, 4095, 4096, 24576, 65536, 65537, 131072,
                 10**6, 2**24 + 3, 2**28, 2**31 - 1})
    worst = max(b.moe_permute_workspace_size(S, 1, E) for S in Ss for E in Es)
    assert worst <= 64 * 1024


@no_gpu
def test_permute_rows_checks(lib):
    f = lambda x=P, ros=P, T=16, H=64, K=2, N=32, out=P: lib.moe_permute_rows(x, ros, T, H, K, N,
                                                                             out, None)
    assert f(T=-1) == INVALID
    assert f(K=0) == INVALID
    assert f(K=17) == INVALID
    assert f(H=12) == UNSUPPORTED
    assert f(N=-1) == INVALID
    assert f(x=P + 8) == INVALID
    assert f(ros=None) == INVALID
    assert f(out=None) == INVALID


@no_gpu
def test_permute_noalloc_checks(lib):
    # size checks come first, before any device lookup
    f = lambda T=16, K=2, E=4: lib.moe_permute_noalloc(P, P, None, 0, T, 64, K, E, P, P, P, P, P,
                                                       None)
    assert f(T=-1) == INVALID
    assert f(K=0) == INVALID
    assert f(K=17) == INVALID
    assert f(E=0) == INVALID
    assert f(E=1025) == INVALID
    assert f(T=2**30, K=4) == INVALID


def _reorder(lib, x=P, cnt=P, R=8, El=32, N=1000, H=64, y=P, perm=P, inv=P, tpe=P, off=P, ws=P,
             wsb=1 << 20):
    return lib.moe_rank_to_expert_reorder(x, cnt, R, El, N, H, y, perm, inv, tpe, off, ws, wsb,
                                          None)


@no_gpu
def test_reorder_checks(lib):
    assert _reorder(lib, R=0) == INVALID
    assert _reorder(lib, El=0) == INVALID
    assert _reorder(lib, R=300, El=300) == INVALID
    assert _reorder(lib, N=-1) == INVALID
    assert _reorder(lib, N=2**31) == INVALID
    assert _reorder(lib, y=None) == INVALID             # x given without y
    assert _reorder(lib, H=4) == UNSUPPORTED
    assert _reorder(lib, cnt=None) == INVALID
    assert _reorder(lib, perm=None) == INVALID
    assert _reorder(lib, inv=PM) == INVALID
    assert _reorder(lib, ws=None) == WORKSPACE
    assert _reorder(lib, wsb=8) == WORKSPACE


def _gemm(lib, x=P, off=P, E=8, N=1000, H=256, I=128, wg=P, wu=P, wd=P, h=P, y=P, pre=None,
          ws=P, wsb=1 << 20):
    return lib.moe_grouped_gemm_swiglu(x, off, E, N, H, I, wg, wu, wd, h, y, pre, ws, wsb, None)


@no_gpu
def test_gemm_checks(lib):
    assert _gemm(lib, E=0) == INVALID
    assert _gemm(lib, E=1025) == INVALID
    assert _gemm(lib, N=-5) == INVALID
    assert _gemm(lib, H=0) == INVALID
    assert _gemm(lib, H=96) == UNSUPPORTED
    assert _gemm(lib, I=100) == UNSUPPORTED
    assert _gemm(lib, H=(1 << 20) + 64) == UNSUPPORTED
    assert _gemm(lib, I=(1 << 20) + 64) == UNSUPPORTED
    assert _gemm(lib, off=None) == INVALID
    assert _gemm(lib, wd=P + 4) == INVALID
    assert _gemm(lib, y=None) == INVALID
    assert _gemm(lib, pre=P + 8) == INVALID             # preact must be 16-byte aligned
    assert _gemm(lib, ws=None) == WORKSPACE
    assert _gemm(lib, wsb=4) == WORKSPACE


def _ggrad(lib, x=P, off=P, E=8, N=1000, H=256, I=128, wg=P, wu=P, wd=P, h=P, dy=P, dx=P,
           dwg=P, dwu=P, dwd=P, pre=None, ws=P, wsb=1 << 30):
    return lib.moe_grouped_gemm_swiglu_grad(x, off, E, N, H, I, wg, wu, wd, h, dy, dx, dwg, dwu,
                                            dwd, pre, ws, wsb, None)


@no_gpu
def test_gemm_grad_checks(lib):
    assert _ggrad(lib, E=0) == INVALID
    assert _ggrad(lib, N=-1) == INVALID
    assert _ggrad(lib, H=96) == UNSUPPORTED
    assert _ggrad(lib, I=(1 << 20) + 64) == UNSUPPORTED
    assert _ggrad(lib, dx=None) == INVALID
    assert _ggrad(lib, dwd=P + 4) == INVALID
    assert _ggrad(lib, pre=P + 8) == INVALID             # preact must be 16-byte aligned
    assert _ggrad(lib, ws=None) == WORKSPACE
    assert _ggrad(lib, ws=P + 16) == WORKSPACE           # 256-byte aligned
    assert _ggrad(lib, wsb=4) == WORKSPACE


def _combine(lib, eo=P, N=100, ros=P, rmap=None, ids=P, probs=P, T=50, K=2, H=64, E=8, sp=None,
             shared=None, out=P, mask=None, per_slot=0):
    from unpermute_combine_moe_amd.binding import MoeSpecialExperts

    spp = ctypes.byref(sp) if isinstance(sp, MoeSpecialExperts) else None
    return lib.moe_unpermute_combine(eo, N, ros, rmap, ids, probs, mask, per_slot, T, K, H, E, spp,
                                     shared, out, None)


@no_gpu
def test_combine_checks(lib):
    from unpermute_combine_moe_amd.binding import MoeSpecialExperts as S

    assert _combine(lib, T=-1) == INVALID
    assert _combine(lib, K=17) == INVALID
    assert _combine(lib, H=10) == UNSUPPORTED
    assert _combine(lib, E=0) == INVALID
    assert _combine(lib, N=-1) == INVALID
    assert _combine(lib, eo=None) == INVALID
    assert _combine(lib, out=P + 2) == INVALID
    assert _combine(lib, rmap=PM) == INVALID
    assert _combine(lib, mask=P, per_slot=-1) == INVALID
    assert _combine(lib, shared=P + 8) == INVALID
    # the combine_v2 page: ori_x is required by copy / const experts, alpha and v by const ones
    assert _combine(lib, sp=S(0, 1, 0, None, None, None, 0, 0, 0, None)) == INVALID
    assert _combine(lib, sp=S(0, 0, 1, P, None, P, 1, 0, 0, P)) == INVALID
    assert _combine(lib, sp=S(0, 0, 1, P, P, P, 1, 0, 0, None)) == INVALID
    assert _combine(lib, sp=S(-1, 0, 0, None, None, None, 0, 0, 0, None)) == INVALID
    # moe_expert_num + zero + copy + const must stay below 2^31 - 1
    assert _combine(lib, E=8, sp=S(2**31 - 10, 1, 1, P, P, P, 1, 0, 0, P)) == INVALID


def _grad(lib, g=P, perm=P, N=100, ros=P, probs=P, T=50, K=2, H=64, dperm=P, dprobs=P):
    return lib.moe_unpermute_grad(g, perm, N, ros, probs, T, K, H, dperm, dprobs, None)


@no_gpu
def test_grad_checks(lib):
    assert _grad(lib, T=-3) == INVALID
    assert _grad(lib, K=0) == INVALID
    assert _grad(lib, H=6) == UNSUPPORTED
    assert _grad(lib, N=-1) == INVALID
    assert _grad(lib, g=None) == INVALID
    assert _grad(lib, dperm=P + 8) == INVALID
    assert _grad(lib, dprobs=None) == INVALID
    assert _grad(lib, probs=PM) == INVALID


def _pgrad(lib, dperm=P, N=100, ros=P, T=50, K=2, H=64, dx=P):
    return lib.moe_permute_grad(dperm, N, ros, T, K, H, dx, None)


@no_gpu
def test_permute_grad_checks(lib):
    assert _pgrad(lib, T=-1) == INVALID
    assert _pgrad(lib, K=17) == INVALID
    assert _pgrad(lib, H=12) == UNSUPPORTED
    assert _pgrad(lib, N=-1) == INVALID
    assert _pgrad(lib, N=2**31) == INVALID
    assert _pgrad(lib, dperm=None) == INVALID
    assert _pgrad(lib, ros=PM) == INVALID
    assert _pgrad(lib, dx=P + 8) == INVALID


def _cgrad(lib, g=P, eo=P, N=100, ros=P, rmap=None, ids=P, probs=P, T=50, K=2, H=64, E=8,
           sp=None, deo=P, dpr=P, dori=P, da1=None, da2=None, dcv=None, ws=P, wsb=1 << 24,
           mask=None, per_slot=0):
    spp = ctypes.byref(sp) if sp is not None else None
    return lib.moe_unpermute_combine_grad(g, eo, N, ros, rmap, ids, probs, mask, per_slot, T, K,
                                          H, E, spp, deo, dpr, dori, da1, da2, dcv, ws, wsb, None)


@no_gpu
def test_combine_grad_checks(lib):
    from unpermute_combine_moe_amd.binding import MoeSpecialExperts as S
    from unpermute_combine_moe_amd import binding as b

    tok = S(0, 1, 2, P, P, P, 1, 0, 0, P)           # per-token alpha
    other = S(0, 1, 2, P, P, P, 64, 0, 1, P)        # [T, H] alpha: no d_alpha kernel
    assert _cgrad(lib, T=-1) == INVALID
    assert _cgrad(lib, K=17) == INVALID
    assert _cgrad(lib, H=12) == UNSUPPORTED
    assert _cgrad(lib, mask=P, per_slot=3) == INVALID
    assert _cgrad(lib, g=None) == INVALID
    assert _cgrad(lib, dpr=None) == INVALID
    assert _cgrad(lib, deo=P + 2) == INVALID
    assert _cgrad(lib, dori=P + 8) == INVALID
    assert _cgrad(lib, sp=tok, da1=P + 2) == INVALID
    assert _cgrad(lib, sp=S(0, 0, 1, P, None, P, 1, 0, 0, P)) == INVALID     # alpha1 missing
    assert _cgrad(lib, sp=other, da1=P) == UNSUPPORTED
    assert _cgrad(lib, sp=tok, dcv=P, ws=None) == WORKSPACE
    need = b.moe_unpermute_combine_grad_workspace_size(50, 64, 2)
    assert _cgrad(lib, sp=tok, dcv=P, wsb=need - 1) == WORKSPACE
    assert _cgrad(lib, sp=tok, dcv=P, ws=P + 4) == WORKSPACE
    assert b.moe_unpermute_combine_grad_workspace_size(50, 64, 0) > 0
    assert b.moe_unpermute_combine_grad_workspace_size(8192, 4096, 4) >= 3 * 4 * 4096 * 4
    with pytest.raises(b.MoeError):
        b.moe_unpermute_combine_grad_workspace_size(-1, 64, 2)


@no_gpu
def test_dered_checks(lib):
    def idx(c=P, oep=4, E=16, start=0, iep=2, El=4, cap=100, ind=P, cbd=P, tot=None, ws=P,
            wsb=1 << 20):
        return lib.moe_deredundency_dispatch_indices(c, oep, E, start, iep, El, cap, ind, cbd, tot,
                                                     ws, wsb, None)

    assert idx(oep=0) == INVALID
    assert idx(start=-1) == INVALID
    assert idx(start=9) == INVALID                     # 9 + 2*4 > 16
    assert idx(iep=5) == INVALID                       # 5*4 > 16
    assert idx(oep=1 << 20, E=16) == INVALID           # count table too large
    assert idx(cap=-1) == INVALID
    assert idx(c=None) == INVALID
    assert idx(ind=PM) == INVALID
    assert idx(tot=PM) == INVALID
    assert idx(ws=None) == WORKSPACE
    assert idx(wsb=8) == WORKSPACE

    def comb(src=P, cf=None, ind=P, n=10, H=64, G=20, wb=P, ws=P, wsb=1 << 20):
        return lib.moe_deredundency_combine(src, cf, ind, n, H, G, wb, ws, wsb, None)

    assert comb(n=-1) == INVALID
    assert comb(G=-1) == INVALID
    assert comb(H=12) == UNSUPPORTED
    assert comb(src=P + 8) == INVALID
    assert comb(cf=PM) == INVALID
    assert comb(wb=None) == INVALID
    assert comb(ws=None) == WORKSPACE
    assert comb(wsb=4) == WORKSPACE
    # the workspace holds the per-row counts and segment starts and the source list
    from unpermute_combine_moe_amd import binding as b
    small = b.moe_deredundency_combine_workspace_size(10, 20)
    assert small >= 4 * (20 + 21 + 10)
    assert b.moe_deredundency_combine_workspace_size(1000, 20) > small
    assert comb(wsb=small - 4) == WORKSPACE
    for n, G in ((-1, 5), (5, -1), (2**31, 5)):
        with pytest.raises(b.MoeError):
            b.moe_deredundency_combine_workspace_size(n, G)


def test_binding_rejects_wrong_tensors(lib):
    from unpermute_combine_moe_amd import binding as b

    with pytest.raises(TypeError):
        b._ptr(torch.zeros(4, dtype=torch.float32), torch.int32, "ids")
    with pytest.raises(ValueError):
        b._ptr(torch.zeros(4, dtype=torch.int32), torch.int32, "ids")   # host tensor
