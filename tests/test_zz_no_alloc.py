"""GPU: ft_moe_q_vec_noalloc (the routed-MoE layer on the library's fixed per-GPU
scratch, for callers that cannot allocate) against ft_moe_q_vec (the stream's
pool) on the same inputs, called through the C ABI: two calls in a row, the
second with fewer tokens, on the direct route and on the sorted tiles.  Both run
the same kernels in the same order, so the outputs must agree bit for bit; the
oracle checks the combine as well."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from block_quantized_matvec_amd import ft, synth
from tests.gpu_util import check_fp32, dev, host, log, need_gpu

pytestmark = pytest.mark.gpu

CASES = [
    # name, weight, act, hidden, inter, experts, topk, route, first t, second t
    ("q4k_direct", "Q4_K", "Q8_1", 2048, 768, 16, 8, 0, 4, 1),
    ("mxfp4_direct", "MXFP4", "Q8_K", 1024, 512, 12, 4, 0, 8, 3),
    ("mxfp4_tiles", "MXFP4", "Q8_K", 1024, 512, 12, 4, 0, 40, 9),
    ("q5k_tiles", "Q5_K", "Q8_K", 1024, 768, 10, 8, 0, 24, 2),
]


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def _call(entry, c, banks, x, ids, ew, y, hq_tap):
    name, w, a, H, I, E, K, route = c[:8]
    opts = ft._MoeOpts(route, 0, None, None, None, ft._ptr(hq_tap), None, None, None, None, None)
    st = getattr(ft.lib(), entry)(ft.TYPES[w], *(ft._ptr(b) for b in banks), E, H, I, ft.TYPES[a], ft._ptr(x),
                                  x.shape[0], ft._ptr(ids), ft._ptr(ew), K, ft._ptr(y), ctypes.byref(opts),
                                  ft._stream())
    assert st == 0, f"{entry}: {ft.STATUS.get(st, st)}"


@pytest.mark.parametrize("c", CASES, ids=[c[0] for c in CASES])
def test_noalloc_matches_pool_entry(c):
    name, w, a, H, I, E, K, route, t1, t2 = c
    g = synth.rng(700, CASES.index(c))
    hb = [synth.expert_bank(w, E, I, H, g), synth.expert_bank(w, E, I, H, g), synth.expert_bank(w, E, H, I, g)]
    banks = [dev(b) for b in hb]
    for t in (t1, t2):
        log(f"noalloc {name} t={t}")
        x = dev(synth.activations(t, H, g))
        idh = synth.expert_ids(t, E, K, g)
        ewh = synth.expert_weights(t, K, g)
        ids, ew = dev(idh), dev(ewh)
        y_pool = torch.full((t, H), 3.0, device="cuda")
        y_fixed = torch.full((t, H), -3.0, device="cuda")
        hq_pool = torch.empty((t * K, ft.row_bytes(a, I)), dtype=torch.uint8, device="cuda")
        hq_fixed = torch.empty_like(hq_pool)
        _call("ft_moe_q_vec", c, banks, x, ids, ew, y_pool, hq_pool)
        _call("ft_moe_q_vec_noalloc", c, banks, x, ids, ew, y_fixed, hq_fixed)
        yp, yf = host(y_pool), host(y_fixed)
        assert np.array_equal(yp, yf), f"t={t}: outputs differ"
        assert np.array_equal(host(hq_pool), host(hq_fixed)), f"t={t}: quantized h differs"
        d = oracle.moe_down(w, hb[2], E, H, I, a, host(hq_fixed), idh)
        check_fp32(yf, oracle.moe_combine(d, ewh), f"{name} t={t} combine")


def test_noalloc_refuses_oversized_problem():
    # 1024 tokens x top-8 x hidden 4096: the per-pair down rows alone are 128 MiB
    H, I, E, K, t = 4096, 256, 8, 8, 1024
    need = ft.lib().ft_moe_scratch_bytes(ft.TYPES["Q4_K"], ft.TYPES["Q8_1"], E, H, I, t, K)
    # the refusal happens on the host before anything is enqueued; never call with
    # the placeholder pointers unless the size is certain to be refused
    assert need > 32 << 20
    fake = ctypes.c_void_p(1 << 20)
    st = ft.lib().ft_moe_q_vec_noalloc(ft.TYPES["Q4_K"], fake, fake, fake, E, H, I, ft.TYPES["Q8_1"], fake, t, fake,
                                       fake, K, fake, None, ft._stream())
    assert ft.STATUS[st] == "FT_ERR_SHAPE"
