"""Pins for the oracle's routing, token->expert sort, routed-MoE stages and
grouped GEMM.

Readings adopted (the pages describe the routed-expert path -- ds4 PR #656
"Add ROCm MXFP4 routed expert kernels", Summary: gate/up, SwiGLU, down; vllm.cpp
PR #523, What changed: grouped over expert_ids -- without its arithmetic):
top-k of the router logits with ties toward the lower expert index, weights the
softmax over the selected logits; SwiGLU as silu(gate) * up; the combine a
weighted sum in slot order.
Pins: numpy's stable argsort; softmax over all experts restricted to the chosen
ones and renormalised; numpy dequantize-then-matmul per stage; closed forms of
silu; top-1 MoE with one expert equal to a dense FFN; grouped GEMM with one
expert equal to the matvec; token permutations permute the outputs.
"""
import numpy as np
import pytest

import oracle
from block_quantized_matvec_amd import synth
from tests import brute


def test_route_matches_stable_argsort_and_softmax():
    l = synth.logits(64, 128, synth.rng(30))
    ids, w = oracle.route(l, 8)
    ref_ids = np.argsort(-l, axis=1, kind="stable")[:, :8]
    assert np.array_equal(ids, ref_ids)
    l64 = l.astype(np.float64)
    full = np.exp(l64 - l64.max(1, keepdims=True))
    full /= full.sum(1, keepdims=True)
    sel = np.take_along_axis(full, ref_ids, 1)
    ref_w = sel / sel.sum(1, keepdims=True)
    assert np.allclose(w, ref_w, rtol=2 ** -23, atol=0)
    assert np.all(np.abs(w.astype(np.float64).sum(1) - 1.0) <= 8 * 2 ** -24)
    assert np.all(np.diff(w, axis=1) <= 0)     # slot 0 holds the largest


def test_route_ties_go_to_lower_index():
    l = np.zeros((2, 16), np.float32)
    l[0, [3, 5, 9]] = 1.0
    l[1, :] = 0.5
    ids, w = oracle.route(l, 4)
    assert list(ids[0]) == [3, 5, 9, 0]
    assert list(ids[1]) == [0, 1, 2, 3]
    assert np.allclose(w[1], 0.25, rtol=0, atol=0)


def test_sort_pairs_matches_stable_argsort():
    ids = synth.expert_ids(512, 128, 8, synth.rng(31))
    counts, offsets, pairs = oracle.sort_pairs(ids, 128)
    flat = ids.ravel()
    assert np.array_equal(pairs, np.argsort(flat, kind="stable"))
    assert np.array_equal(counts, np.bincount(flat, minlength=128))
    assert np.array_equal(offsets, np.concatenate([[0], np.cumsum(counts)]))


def _moe_small(wfmt, afmt, hidden, inter, E, t, topk, seed):
    g = synth.rng(32, seed)
    wg = synth.expert_bank(wfmt, E, inter, hidden, g)
    wu = synth.expert_bank(wfmt, E, inter, hidden, g)
    wd = synth.expert_bank(wfmt, E, hidden, inter, g)
    x = synth.activations(t, hidden, g)
    ids = synth.expert_ids(t, E, topk, g)
    w = synth.expert_weights(t, topk, g)
    return wg, wu, wd, x, ids, w


@pytest.mark.parametrize("wfmt,afmt", [("Q4_K", "Q8_1"), ("MXFP4", "Q8_K")])
def test_moe_stages_match_brute(wfmt, afmt):
    hidden, inter, E, t, topk = 512, 256, 6, 3, 2
    wg, wu, wd, x, ids, w = _moe_small(wfmt, afmt, hidden, inter, E, t, topk, 0)
    out = oracle.moe_forward(wfmt, wg, wu, wd, E, hidden, inter, afmt, x, ids, w)
    xd = brute.dequant(afmt, out["xq"], t, hidden)
    for p in range(t * topk):
        e = ids.ravel()[p]
        G = brute.dequant(wfmt, wg[e], inter, hidden)
        U = brute.dequant(wfmt, wu[e], inter, hidden)
        g_ref = G @ xd[p // topk]
        u_ref = U @ xd[p // topk]
        assert np.allclose(out["g"][p], g_ref, rtol=2 ** -23, atol=1e-12)
        assert np.allclose(out["u"][p], u_ref, rtol=2 ** -23, atol=1e-12)
        h_ref = g_ref / (1 + np.exp(-g_ref)) * u_ref
        assert np.allclose(out["h"][p], h_ref, rtol=2 ** -22, atol=1e-12)
        D = brute.dequant(wfmt, wd[e], hidden, inter)
        hd = brute.dequant(afmt, out["hq"][p], 1, inter)[0]
        assert np.allclose(out["d"][p], D @ hd, rtol=2 ** -23, atol=1e-12)
    y_ref = (w.astype(np.float64)[:, :, None] * out["d"].reshape(t, topk, hidden)).sum(1)
    assert np.allclose(out["y"], y_ref, rtol=2 ** -23, atol=1e-12)


def test_silu_closed_forms():
    # one expert, Q8_0 rows with a single code: g and u are picked activations
    hidden, inter = 256, 32
    blk0 = np.zeros((inter, hidden // 32, 34), np.uint8)
    blk0[:, :, 0:2] = np.array([1.0], np.float16).view(np.uint8)
    wg, wu = blk0.copy(), blk0.copy()
    for r in range(inter):
        wg[r, 0, 2 + r % 32] = 1
        wu[r, 1, 2 + r % 32] = 1
    x = np.zeros((1, hidden), np.float32)
    x[0, :32] = np.linspace(-30, 30, 32, dtype=np.float32)   # gate inputs
    x[0, 32:64] = 2.0                                         # up inputs
    x[0, 255] = 127.0
    xq = oracle.quantize("Q8_1", x)
    g, u, h = oracle.moe_gate_up("Q8_0", wg[None], wu[None], 1, hidden, inter, "Q8_1", xq,
                                 np.zeros((1, 1), np.int32))
    xd = brute.dequant("Q8_1", xq, 1, hidden)[0]
    gv = xd[:32]
    assert np.array_equal(g[0], gv.astype(np.float32))
    # silu(0) = 0, silu(g) -> g for large g, silu(g) -> 0 for very negative g
    hv = gv / (1 + np.exp(-gv)) * xd[32:64]
    assert np.allclose(h[0], hv, rtol=2 ** -22)
    assert abs(h[0][np.argmax(gv)] - gv.max() * xd[32]) <= 1e-6 * gv.max() * xd[32]


def test_top1_single_expert_is_dense_ffn():
    hidden, inter = 512, 256
    wg, wu, wd, x, _, _ = _moe_small("Q4_K", "Q8_1", hidden, inter, 1, 2, 1, 1)
    ids = np.zeros((2, 1), np.int32)
    w = np.ones((2, 1), np.float32)
    out = oracle.moe_forward("Q4_K", wg, wu, wd, 1, hidden, inter, "Q8_1", x, ids, w)
    xq = oracle.quantize("Q8_1", x)
    g = oracle.matvec("Q4_K", wg[0], inter, hidden, "Q8_1", xq, 2).astype(np.float64)
    u = oracle.matvec("Q4_K", wu[0], inter, hidden, "Q8_1", xq, 2).astype(np.float64)
    assert np.array_equal(out["g"], g.astype(np.float32))
    hq = oracle.quantize("Q8_1", out["h"])
    y = oracle.matvec("Q4_K", wd[0], hidden, inter, "Q8_1", hq, 2)
    assert np.array_equal(out["y"], y)


def test_token_permutation_permutes_outputs():
    hidden, inter, E, t, topk = 512, 256, 5, 4, 2
    wg, wu, wd, x, ids, w = _moe_small("MXFP4", "Q8_K", hidden, inter, E, t, topk, 2)
    a = oracle.moe_forward("MXFP4", wg, wu, wd, E, hidden, inter, "Q8_K", x, ids, w)
    perm = np.array([2, 0, 3, 1])
    b = oracle.moe_forward("MXFP4", wg, wu, wd, E, hidden, inter, "Q8_K", x[perm], ids[perm], w[perm])
    assert np.array_equal(a["y"][perm], b["y"])


@pytest.mark.parametrize("wfmt", ["Q5_K", "Q6_K", "MXFP4"])
def test_grouped_single_expert_equals_matvec(wfmt):
    g = synth.rng(33)
    n, k, t, topk = 24, 512, 5, 1
    W = synth.expert_bank(wfmt, 1, n, k, g)
    xq = oracle.quantize("Q8_K", synth.activations(t, k, g))
    y = oracle.grouped(wfmt, W, 1, n, k, "Q8_K", xq, False, np.zeros((t, topk), np.int32))
    assert np.array_equal(y, oracle.matvec(wfmt, W[0], n, k, "Q8_K", xq, t))


@pytest.mark.parametrize("x_per_pair", [False, True])
def test_grouped_matches_brute(x_per_pair):
    g = synth.rng(34)
    E, n, k, t, topk = 6, 16, 512, 5, 3
    W = synth.expert_bank("Q6_K", E, n, k, g)
    ids = synth.expert_ids(t, E, topk, g)
    rows = t * topk if x_per_pair else t
    xq = oracle.quantize("Q8_K", synth.activations(rows, k, g))
    y = oracle.grouped("Q6_K", W, E, n, k, "Q8_K", xq, x_per_pair, ids)
    xd = brute.dequant("Q8_K", xq, rows, k)
    for p in range(t * topk):
        ref = brute.dequant("Q6_K", W[ids.ravel()[p]], n, k) @ xd[p if x_per_pair else p // topk]
        assert np.allclose(y[p], ref, rtol=2 ** -23, atol=1e-12)
