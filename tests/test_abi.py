"""Host-side contract of libft.so (no GPU needed).

Checks that the library loads, exports every entry point include/ft.h declares,
and refuses bad arguments on the host before any HIP call: unsupported
(weight, activation) pairs, shapes that are not block multiples, NULL pointers,
misaligned pointers.  The capability table is checked against the dispatcher's
refusals (an op reported unsupported must refuse; a supported one must get past
the format check).
"""
import ctypes
import os
import re

import pytest

from block_quantized_matvec_amd import ft

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

W = ["Q4_0", "Q8_0", "Q4_K", "Q5_K", "Q6_K", "MXFP4", "Q2_K", "Q3_K", "Q4_1", "Q5_0", "Q5_1"]
A = ["Q8_1", "Q8_K", "Q8_0"]
ST = {v: k for k, v in ft.STATUS.items()}


def _declared():
    src = open(os.path.join(ROOT, "include", "ft.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ft_[a-z0-9_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported():
    L = ft.lib()
    names = _declared()
    assert len(names) >= 15
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(ft.EXPORTS), set(names) ^ set(ft.EXPORTS)


def test_block_sizes():
    sizes = {"Q4_0": (32, 18), "Q8_0": (32, 34), "Q4_K": (256, 144), "Q5_K": (256, 176),
             "Q6_K": (256, 210), "MXFP4": (32, 17), "Q8_1": (32, 36), "Q8_K": (256, 292),
             "Q2_K": (256, 84), "Q3_K": (256, 110), "Q4_1": (32, 20), "Q5_0": (32, 22), "Q5_1": (32, 24)}
    for t, (e, b) in sizes.items():
        assert ft.block_elems(t) == e and ft.block_bytes(t) == b
    assert ft.lib().ft_block_elems(99) == 0 and ft.lib().ft_block_bytes(-1) == 0


def test_capability_table():
    expect_mmvq = ({(w, "Q8_1") for w in W} | {(w, "Q8_0") for w in W} |
                   {(w, "Q8_K") for w in ("Q4_K", "Q5_K", "Q6_K", "MXFP4")})
    expect_moe = {("Q4_K", "Q8_1"), ("MXFP4", "Q8_K"), ("Q4_K", "Q8_K"), ("Q5_K", "Q8_K"), ("Q6_K", "Q8_K")}
    expect_grp = {("Q4_K", "Q8_K"), ("Q5_K", "Q8_K"), ("Q6_K", "Q8_K"), ("MXFP4", "Q8_K")}
    for w in W:
        for a in A:
            assert ft.supported("mmvq", w, a) == ((w, a) in expect_mmvq)
            assert ft.supported("moe_vec", w, a) == ((w, a) in expect_moe)
            assert ft.supported("grouped", w, a) == ((w, a) in expect_grp)
            assert ft.supported("block_dots", w, a)
        assert ft.supported("dequant", w, "Q8_1")
    assert ft.supported("quantize", "Q4_0", "Q8_1") and ft.supported("quantize", "Q4_0", "Q8_K")
    assert ft.supported("quantize", "Q4_0", "Q8_0")
    assert not ft.supported("quantize", "Q4_0", "Q4_0")
    assert not ft.supported("dequant", "Q8_1", "Q8_1")


def test_unsupported_pairs_refused_before_launch():
    L = ft.lib()
    T = ft.TYPES
    for w in W:
        for a in A:
            st = L.ft_mul_mat_vec_q(T[w], None, 16, 256, T[a], None, 1, None, 16, None)
            if ft.supported("mmvq", w, a):
                assert st == ST["FT_ERR_INVALID_ARG"]   # got past the format check to the NULLs
            else:
                assert st == ST["FT_ERR_UNSUPPORTED"]
            st = L.ft_grouped_gemm_q(T[w], None, 4, 16, 256, T[a], None, 0, None, 2, 2, None, None)
            assert st == (ST["FT_ERR_INVALID_ARG"] if ft.supported("grouped", w, a) else ST["FT_ERR_UNSUPPORTED"])
            st = L.ft_moe_q_vec(T[w], None, None, None, 4, 256, 256, T[a], None, 1, None, None, 2, None, None, None)
            assert st == (ST["FT_ERR_INVALID_ARG"] if ft.supported("moe_vec", w, a) else ST["FT_ERR_UNSUPPORTED"])


def test_shape_and_pointer_checks():
    L = ft.lib()
    T = ft.TYPES
    fake = ctypes.c_void_p(0x10000)       # never dereferenced: refused first
    odd = ctypes.c_void_p(0x10008)
    # k not a multiple of the block
    assert L.ft_quantize_act(T["Q8_1"], fake, 1, 48, 48, fake, None) == ST["FT_ERR_SHAPE"]
    assert L.ft_quantize_act(T["Q8_K"], fake, 1, 128, 128, fake, None) == ST["FT_ERR_SHAPE"]
    assert L.ft_dequant(T["Q4_K"], fake, 1, 100, fake, None) == ST["FT_ERR_SHAPE"]
    assert L.ft_mul_mat_vec_q(T["Q4_K"], fake, 4, 320, T["Q8_1"], fake, 1, fake, 4, None) == ST["FT_ERR_SHAPE"]
    # ldy < n, negative sizes
    assert L.ft_mul_mat_vec_q(T["Q4_0"], fake, 4, 64, T["Q8_1"], fake, 1, fake, 3, None) == ST["FT_ERR_INVALID_ARG"]
    assert L.ft_dequant(T["Q4_0"], fake, -1, 32, fake, None) == ST["FT_ERR_INVALID_ARG"]
    # NULL and misaligned pointers
    assert L.ft_dequant(T["Q4_0"], None, 1, 32, fake, None) == ST["FT_ERR_INVALID_ARG"]
    assert L.ft_dequant(T["Q4_0"], odd, 1, 32, fake, None) == ST["FT_ERR_ALIGNMENT"]
    assert L.ft_mul_mat_vec_q(T["Q8_0"], fake, 4, 64, T["Q8_1"], odd, 1, fake, 4, None) == ST["FT_ERR_ALIGNMENT"]
    # routing / sort limits
    assert L.ft_moe_route(fake, 1, 128, 9, fake, fake, None) == ST["FT_ERR_SHAPE"]
    assert L.ft_moe_route(fake, 1, 4, 5, fake, fake, None) == ST["FT_ERR_SHAPE"]
    assert L.ft_moe_route(fake, 1, 2048, 8, fake, fake, None) == ST["FT_ERR_SHAPE"]
    assert L.ft_moe_sort(fake, 1, 0, 8, fake, fake, fake, None) == ST["FT_ERR_SHAPE"]
    # empty problems are no-ops that need no pointers
    assert L.ft_mul_mat_vec_q(T["Q4_K"], None, 0, 256, T["Q8_1"], None, 1, None, 0, None) == 0
    assert L.ft_mul_mat_vec_q(T["Q4_K"], None, 8, 256, T["Q8_1"], None, 0, None, 8, None) == 0
    assert L.ft_quantize_act(T["Q8_1"], None, 0, 64, 64, None, None) == 0
    # topk out of range for the MoE path
    assert L.ft_moe_q_vec(T["Q4_K"], fake, fake, fake, 4, 256, 256, T["Q8_1"], fake, 1, fake, fake, 9,
                          fake, None, None) == ST["FT_ERR_SHAPE"]
    # measurement microkernels: unknown kind, NULL output, misaligned or ragged read
    assert L.ft_debug_ceiling(4, None, 0, 1, fake, None) == ST["FT_ERR_INVALID_ARG"]
    assert L.ft_debug_ceiling(1, None, 0, 1, None, None) == ST["FT_ERR_INVALID_ARG"]
    assert L.ft_debug_ceiling(0, odd, 64, 0, fake, None) == ST["FT_ERR_ALIGNMENT"]
    assert L.ft_debug_ceiling(0, fake, 40, 0, fake, None) == ST["FT_ERR_INVALID_ARG"]
    assert L.ft_debug_ceiling(0, fake, 0, 0, fake, None) == 0   # empty read: no launch


def test_moe_route_options_refused_on_host():
    """Forced sorted tiles need Q8_K activations; bad options are refused before
    anything is launched (no GPU needed)."""
    L = ft.lib()
    T = ft.TYPES
    fake = ctypes.c_void_p(1 << 20)

    def call(w, a, route, dmax=0, n_expert=4, t=1):
        o = ft._MoeOpts(route, dmax, None, None, None, None, None, None, None, None, None)
        return L.ft_moe_q_vec(T[w], fake, fake, fake, n_expert, 256, 256, T[a], fake, t, fake, fake, 2, fake,
                              ctypes.byref(o), None)

    assert call("Q4_K", "Q8_1", 2) == ST["FT_ERR_UNSUPPORTED"]
    assert call("Q4_K", "Q8_1", 3) == ST["FT_ERR_INVALID_ARG"]
    assert call("MXFP4", "Q8_K", -1) == ST["FT_ERR_INVALID_ARG"]
    assert call("MXFP4", "Q8_K", 0, dmax=-2) == ST["FT_ERR_INVALID_ARG"]
    # K-quant experts x Q8_K have no direct kernels: the direct route is refused
    for w in ("Q4_K", "Q5_K", "Q6_K"):
        assert call(w, "Q8_K", 1) == ST["FT_ERR_UNSUPPORTED"]
    # the sorted tiles take at most 8192 experts (forced, or chosen by the auto
    # route above direct_max_t, or for a pair without direct kernels); the direct
    # route has no such limit
    assert call("MXFP4", "Q8_K", 2, n_expert=9000) == ST["FT_ERR_SHAPE"]
    assert call("MXFP4", "Q8_K", 0, n_expert=9000, t=9) == ST["FT_ERR_SHAPE"]
    assert call("Q5_K", "Q8_K", 0, n_expert=9000) == ST["FT_ERR_SHAPE"]


def test_status_strings():
    for code in range(7):
        assert ft.lib().ft_status_str(code)
    assert ft.lib().ft_status_str(1234) == b"unknown status"


def test_scratch_sizes_are_monotone():
    a = ft.moe_scratch_bytes("Q4_K", "Q8_1", 128, 2048, 768, 1, 8)
    b = ft.moe_scratch_bytes("Q4_K", "Q8_1", 128, 2048, 768, 4, 8)
    assert 0 < a < b


def test_moe_noalloc_refusals_on_host():
    """ft_moe_q_vec_noalloc validates as ft_moe_q_vec and refuses a problem whose
    scratch exceeds its fixed array before anything is enqueued (no GPU needed)."""
    L = ft.lib()
    T = ft.TYPES
    fake = ctypes.c_void_p(1 << 20)
    assert L.ft_moe_q_vec_noalloc(T["Q5_0"], fake, fake, fake, 4, 256, 256, T["Q8_1"], fake, 1, fake, fake, 2,
                                  fake, None, None) == ST["FT_ERR_UNSUPPORTED"]
    assert L.ft_moe_q_vec_noalloc(T["Q4_K"], fake, fake, fake, 4, 256, 256, T["Q8_1"], fake, 1, fake, fake, 9,
                                  fake, None, None) == ST["FT_ERR_SHAPE"]
    H, I, E, K, t = 4096, 256, 8, 8, 1024
    assert ft.moe_scratch_bytes("Q4_K", "Q8_1", E, H, I, t, K) > 32 << 20
    assert L.ft_moe_q_vec_noalloc(T["Q4_K"], fake, fake, fake, E, H, I, T["Q8_1"], fake, t, fake, fake, K,
                                  fake, None, None) == ST["FT_ERR_SHAPE"]
