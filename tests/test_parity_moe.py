"""GPU parity: routing (ids bit-exact, weights fp32), token->expert sort
(bit-exact), and the routed-MoE vector path checked stage by stage against the
oracle: g, u, h (fp32), quantized h bit-exact against the oracle's quantizer
applied to the GPU's h, down and the weighted combine from the GPU's quantized h."""
import numpy as np
import pytest
import torch

import oracle
from block_quantized_matvec_amd import ft, synth
from tests.gpu_util import check_fp32, dev, host, log, need_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


@pytest.mark.parametrize("t,e,topk", [(1, 128, 8), (4, 128, 8), (37, 256, 8), (512, 128, 8), (3, 16, 1), (5, 1024, 4)])
def test_route(t, e, topk):
    l = synth.logits(t, e, synth.rng(300, t, e))
    ids, w = ft.moe_route(dev(l), topk)
    rid, rw = oracle.route(l, topk)
    assert np.array_equal(host(ids), rid)
    check_fp32(host(w), rw, "route weights", rel=1e-6, nmse=1e-12)


def test_route_ties():
    l = np.zeros((3, 64), np.float32)
    l[0, [5, 9, 40, 63]] = 2.0
    l[2] = np.repeat(np.arange(8, dtype=np.float32), 8)
    ids, w = ft.moe_route(dev(l), 8)
    rid, rw = oracle.route(l, 8)
    assert np.array_equal(host(ids), rid)
    check_fp32(host(w), rw, rel=1e-6, nmse=1e-12)


def _edge_logits(e):
    """Rows that stress the key order and the tie rule: signed zeros, infinities,
    the largest and smallest magnitudes, all-equal rows and winners in the last
    64-expert slice."""
    rows = []
    r = np.full(e, -1.0, np.float32)
    r[np.arange(0, e, 7)] = -0.0
    r[np.arange(3, e, 11)] = 0.0
    rows.append(r)                                          # -0 and +0 tie: index order
    r = np.full(e, -np.inf, np.float32)
    r[[e - 1, e // 2, 1]] = [np.float32(3e38), -np.float32(3e38), np.float32(1e-45)]
    rows.append(r)                                          # infinities, extreme magnitudes
    rows.append(np.full(e, 0.25, np.float32))               # all equal: the first k indices
    r = np.linspace(-1.0, 1.0, e).astype(np.float32)
    rows.append(r)                                          # winners at the highest indices
    r = np.zeros(e, np.float32)
    r[e - 9:] = 5.0
    r[2] = 5.0
    rows.append(r)                                          # a tie spanning the last slice
    return np.stack(rows)


@pytest.mark.parametrize("e,topk", [(8, 8), (64, 8), (100, 8), (128, 8), (200, 6), (256, 8), (1000, 4)])
def test_route_edge_values(e, topk):
    l = _edge_logits(e)
    ids, w = ft.moe_route(dev(l), topk)
    rid, rw = oracle.route(l, topk)
    assert np.array_equal(host(ids), rid)
    check_fp32(host(w), rw, "route weights", rel=1e-6, nmse=1e-12)


@pytest.mark.parametrize("t,e,topk", [(1, 128, 8), (5, 256, 8), (512, 128, 8), (700, 64, 3), (4096, 256, 8),
                                      (1, 1, 1), (3000, 8, 8), (2048, 8192, 8), (2048, 512, 8), (2049, 512, 8),
                                      (33, 2, 2), (2048, 513, 8)])
def test_sort(t, e, topk):
    ids = synth.expert_ids(t, e, topk, synth.rng(301, t))
    c, o, p = ft.moe_sort(dev(ids), e)
    rc, ro, rp = oracle.sort_pairs(ids, e)
    assert np.array_equal(host(c), rc) and np.array_equal(host(o), ro) and np.array_equal(host(p), rp)


@pytest.mark.parametrize("t,e,topk", [(512, 128, 8), (2048, 512, 8), (64, 3, 2), (1, 256, 8)])
def test_sort_skewed(t, e, topk):
    """Slot 0 of every token names expert e - 1 and slot 1 expert 0, so two
    experts hold a third or more of the pairs (long runs of equal keys in every
    64-pair round) and most experts few or none; the order within each expert's
    segment must still be pair order."""
    ids = synth.expert_ids(t, e, topk, synth.rng(302, t))
    ids[:, 0] = e - 1
    ids[:, 1] = 0
    c, o, p = ft.moe_sort(dev(ids), e)
    rc, ro, rp = oracle.sort_pairs(ids, e)
    assert np.array_equal(host(c), rc) and np.array_equal(host(o), ro) and np.array_equal(host(p), rp)


CASES = {
    "q4k": dict(w="Q4_K", a="Q8_1", hidden=2048, inter=768, E=128, topk=8),
    "mxfp4": dict(w="MXFP4", a="Q8_K", hidden=4096, inter=2048, E=256, topk=8),
    "q4k_small": dict(w="Q4_K", a="Q8_1", hidden=512, inter=256, E=6, topk=2),
    # rows of 68 units: both stages take the workgroup-tile kernels, not the rings
    "q4k_wide": dict(w="Q4_K", a="Q8_1", hidden=4352, inter=4352, E=3, topk=2),
    # the two-launch layer's largest gate/up rows (64 lanes per row, one row per
    # ring stage) and 32 lanes per down row
    "q4k_h4096": dict(w="Q4_K", a="Q8_1", hidden=4096, inter=1536, E=16, topk=8),
    "mxfp4_small": dict(w="MXFP4", a="Q8_K", hidden=512, inter=512, E=5, topk=3),
    # K-quant experts x Q8_K on the sorted tiles (grouped gate/up + SwiGLU, h
    # quantize, grouped down, combine)
    "q4k8k_small": dict(w="Q4_K", a="Q8_K", hidden=512, inter=768, E=6, topk=2),
    "q5k_small": dict(w="Q5_K", a="Q8_K", hidden=768, inter=512, E=5, topk=3),
    "q6k_small": dict(w="Q6_K", a="Q8_K", hidden=512, inter=256, E=7, topk=4),
    # the grouped-GEMM workload's layer: hidden 4096, 128 experts of 1536, top-8
    "q5k_c4": dict(w="Q5_K", a="Q8_K", hidden=4096, inter=1536, E=128, topk=8),
    "q6k_c4": dict(w="Q6_K", a="Q8_K", hidden=4096, inter=1536, E=128, topk=8),
    # one superblock per row: K parts with no superblock, four experts on one router lane
    "mxfp4_tiny": dict(w="MXFP4", a="Q8_K", hidden=256, inter=256, E=4, topk=2),
    # 6 superblocks per row: the LDS-ring walks' K parts hold 3 (the upper part starts
    # at an odd superblock and walks down through both parities)
    "mxfp4_mid": dict(w="MXFP4", a="Q8_K", hidden=1536, inter=1536, E=16, topk=4),
}

_banks = {}


def _bank(name):
    if name not in _banks:
        c = CASES[name]
        g = synth.rng(302, list(CASES).index(name))
        wg = synth.expert_bank(c["w"], c["E"], c["inter"], c["hidden"], g)
        wu = synth.expert_bank(c["w"], c["E"], c["inter"], c["hidden"], g)
        wd = synth.expert_bank(c["w"], c["E"], c["hidden"], c["inter"], g)
        _banks[name] = (wg, wu, wd, dev(wg), dev(wu), dev(wd))
    return _banks[name]


def _run_stages(name, t, route, seed=0, dup=False, rep=False, from_logits=False):
    c = CASES[name]
    wg, wu, wd, dwg, dwu, dwd = _bank(name)
    g = synth.rng(303, t, seed)
    x = synth.activations(t, c["hidden"], g)
    ids = synth.expert_ids(t, c["E"], c["topk"], g)
    if from_logits:
        logits = synth.logits(t, c["E"], g)
        ids, rw = oracle.route(logits, c["topk"])
    if rep:
        # slot 1 repeats slot 0's expert in every token: both pairs get the same
        # h and d, each with its own weight in the combine
        ids[:, 1] = ids[:, 0]
    if dup and t > 1:
        # every token picks expert ids[0, 0] at slot 0 (still distinct within a token)
        e0 = ids[0, 0]
        for i in range(1, t):
            hit = np.nonzero(ids[i] == e0)[0]
            if len(hit):
                ids[i, hit[0]] = ids[i, 0]
            ids[i, 0] = e0
    ew = synth.expert_weights(t, c["topk"], g)
    np_, I, H = t * c["topk"], c["inter"], c["hidden"]
    taps = {"g": torch.empty(np_, I, device="cuda"), "u": torch.empty(np_, I, device="cuda"),
            "h": torch.empty(np_, I, device="cuda"),
            "hq": torch.empty(np_, ft.row_bytes(c["a"], I), dtype=torch.uint8, device="cuda"),
            "down": torch.empty(np_, H, device="cuda")}
    if from_logits:
        ids_out = torch.empty((t, c["topk"]), dtype=torch.int32, device="cuda")
        w_out = torch.empty((t, c["topk"]), device="cuda")
        y = ft.moe_q_vec(c["w"], dwg, dwu, dwd, c["E"], H, I, c["a"], dev(x), None, None, route=route, taps=taps,
                         logits=dev(logits), topk=c["topk"], ids_out=ids_out, w_out=w_out)
        assert np.array_equal(host(ids_out), ids), "routing ids differ from the oracle's"
        check_fp32(host(w_out), rw, "routing weights", rel=1e-6, nmse=1e-12)
        ew = host(w_out)
    else:
        y = ft.moe_q_vec(c["w"], dwg, dwu, dwd, c["E"], H, I, c["a"], dev(x), dev(ids), dev(ew),
                         route=route, taps=taps)
    xq = oracle.quantize(c["a"], x)
    rg, ru, rh = oracle.moe_gate_up(c["w"], wg, wu, c["E"], H, I, c["a"], xq, ids)
    check_fp32(host(taps["g"]), rg, "g")
    check_fp32(host(taps["u"]), ru, "u")
    h = host(taps["h"])
    check_fp32(h, rh, "h")
    hq = host(taps["hq"])
    assert np.array_equal(hq, oracle.quantize(c["a"], h)), "quantized h differs from the oracle quantizer"
    rd = oracle.moe_down(c["w"], wd, c["E"], H, I, c["a"], hq, ids)
    d = host(taps["down"])
    check_fp32(d, rd, "down")
    ry = oracle.moe_combine(d, ew)
    check_fp32(host(y), ry, "combine")
    return host(y), x, ids, ew


@pytest.mark.parametrize("name", ["q4k_small", "mxfp4_small"])
@pytest.mark.parametrize("t", [1, 2, 3, 4, 5, 9])
def test_moe_stages_small(name, t):
    log(f"moe {name} t={t}")
    _run_stages(name, t, route=1)


@pytest.mark.parametrize("name", ["q4k_small", "mxfp4_small"])
def test_moe_shared_experts(name):
    _run_stages(name, 4, route=1, dup=True)


@pytest.mark.parametrize("name,t,route", [("q4k_small", 3, 1), ("mxfp4_small", 2, 1), ("mxfp4_small", 5, 2),
                                          ("q4k", 1, 1), ("mxfp4", 2, 1), ("mxfp4_small", 1, 1), ("mxfp4", 1, 1)])
def test_moe_repeated_expert_in_token(name, t, route):
    log(f"moe {name} repeated expert t={t} route={route}")
    _run_stages(name, t, route=route, rep=True)


@pytest.mark.parametrize("name,t,route", [("q4k", 1, 1), ("q4k", 4, 1), ("mxfp4", 3, 1), ("mxfp4", 5, 2),
                                          ("mxfp4_small", 6, 2), ("mxfp4", 1, 1), ("mxfp4_small", 1, 1),
                                          ("mxfp4", 2, 1), ("mxfp4_small", 2, 1)])
def test_moe_down_from_given_hq(name, t, route):
    """The down stage and the combine alone: the quantized h rows come from the
    oracle (in_hq), so the check does not depend on the GPU's gate/up."""
    c = CASES[name]
    wg, wu, wd, dwg, dwu, dwd = _bank(name)
    g = synth.rng(306, t, route)
    H, I, E, K = c["hidden"], c["inter"], c["E"], c["topk"]
    x = synth.activations(t, H, g)
    ids = synth.expert_ids(t, E, K, g)
    ew = synth.expert_weights(t, K, g)
    _, _, rh = oracle.moe_gate_up(c["w"], wg, wu, E, H, I, c["a"], oracle.quantize(c["a"], x), ids)
    hq = oracle.quantize(c["a"], rh.astype(np.float32))
    taps = {"hq": torch.empty(t * K, ft.row_bytes(c["a"], I), dtype=torch.uint8, device="cuda"),
            "down": torch.empty(t * K, H, device="cuda")}
    log(f"moe {name} down from given hq t={t} route={route}")
    y = host(ft.moe_q_vec(c["w"], dwg, dwu, dwd, E, H, I, c["a"], dev(x), dev(ids), dev(ew), route=route, taps=taps,
                          in_hq=dev(hq)))
    assert np.array_equal(host(taps["hq"]), hq), "hq tap differs from the given blocks"
    rd = oracle.moe_down(c["w"], wd, E, H, I, c["a"], hq, ids)
    check_fp32(host(taps["down"]), rd, "down")
    check_fp32(y, oracle.moe_combine(rd, ew), "combine")


@pytest.mark.parametrize("t", [1, 3])
def test_moe_q4k_wide_rows(t):
    log(f"moe q4k_wide t={t}")
    _run_stages("q4k_wide", t, route=1)


@pytest.mark.parametrize("t", [1, 2, 3, 4])
def test_moe_q4k_layer(t):
    log(f"moe q4k layer t={t}")
    _run_stages("q4k", t, route=0)


@pytest.mark.parametrize("t", [1, 2, 3, 4, 6, 8, 11])
def test_moe_mxfp4_direct(t):
    log(f"moe mxfp4 t={t}")
    _run_stages("mxfp4", t, route=1)


@pytest.mark.parametrize("t,from_logits", [(1, True), (2, True), (3, False), (5, False), (8, False)])
def test_moe_mxfp4_direct_odd_parts(t, from_logits):
    """The direct route's LDS-ring K walks with 3 superblocks per K part (hidden and
    inter 1536): odd parts start on an odd superblock; 1-2 tokens routed inside the
    gate/up launch with down and combine in one launch, 3-5 tokens on the per-expert
    down ring, 8 without it."""
    log(f"moe mxfp4_mid t={t} logits={from_logits}")
    _run_stages("mxfp4_mid", t, route=1, from_logits=from_logits)


@pytest.mark.parametrize("t", [1, 3, 5, 9, 40])
def test_moe_mxfp4_small_tiles(t):
    """Sorted-tile route forced at every t (stage taps against the oracle)."""
    log(f"moe mxfp4_small tiles t={t}")
    _run_stages("mxfp4_small", t, route=2)


def test_moe_mxfp4_small_tiles_shared_experts():
    _run_stages("mxfp4_small", 6, route=2, dup=True)


@pytest.mark.parametrize("t", [200, 64])
def test_moe_mxfp4_small_tiles_hot_expert(t):
    """Skewed routing on the sorted tiles: every token picks one expert (t pairs on
    it, several passes of the grouped kernels over its weights: at t = 200 the
    kernel holds 64 pairs per pass, at t = 64 32); every pair is compared."""
    log(f"moe mxfp4_small tiles hot expert t={t}")
    _run_stages("mxfp4_small", t, route=2, dup=True)


@pytest.mark.parametrize("t,route", [(1, 2), (4, 2), (5, 0), (9, 0), (12, 0)])
def test_moe_mxfp4_tiles(t, route):
    """Full-size MXFP4 bank (hidden 4096, 256 experts of 2048): route 0 takes the
    direct route up to 8 tokens and the tiles above."""
    log(f"moe mxfp4 tiles t={t} route={route}")
    _run_stages("mxfp4", t, route=route)


@pytest.mark.parametrize("t", [32, 128, 512])
def test_moe_mxfp4_tiles_sampled(t):
    """Sorted tiles at 32-512 tokens on the full bank; the oracle checks a sample of
    pairs stage by stage (g, u, h, quantized h, down) and the whole combine."""
    c = CASES["mxfp4"]
    wg, wu, wd, dwg, dwu, dwd = _bank("mxfp4")
    g = synth.rng(305, t)
    H, I, E, K = c["hidden"], c["inter"], c["E"], c["topk"]
    x = synth.activations(t, H, g)
    ids = synth.expert_ids(t, E, K, g)
    ew = synth.expert_weights(t, K, g)
    np_ = t * K
    taps = {"g": torch.empty(np_, I, device="cuda"), "u": torch.empty(np_, I, device="cuda"),
            "h": torch.empty(np_, I, device="cuda"),
            "hq": torch.empty(np_, ft.row_bytes(c["a"], I), dtype=torch.uint8, device="cuda"),
            "down": torch.empty(np_, H, device="cuda")}
    log(f"moe mxfp4 tiles sampled t={t}")
    y = host(ft.moe_q_vec(c["w"], dwg, dwu, dwd, E, H, I, c["a"], dev(x), dev(ids), dev(ew), route=0, taps=taps))
    gg, uu, hh, hq, dd = (host(taps[k]) for k in ("g", "u", "h", "hq", "down"))
    xq = oracle.quantize(c["a"], x)
    flat = ids.reshape(-1)
    pairs = np.unique(np.concatenate([np.arange(4), np.arange(np_ - 4, np_), g.choice(np_, 12, replace=False)]))
    # the oracle's gate/up stage on the sampled pairs alone: one token per pair
    # (its token's quantized x), top-1 routing to the pair's expert
    rg_all, ru_all, rh_all = oracle.moe_gate_up(c["w"], wg, wu, E, H, I, c["a"],
                                                np.ascontiguousarray(xq[pairs // K]),
                                                np.ascontiguousarray(flat[pairs][:, None]))
    for j, p in enumerate(pairs):
        e = flat[p]
        check_fp32(gg[p], rg_all[j], f"g pair {p}")
        check_fp32(uu[p], ru_all[j], f"u pair {p}")
        check_fp32(hh[p], rh_all[j], f"h pair {p}")
        assert np.array_equal(hq[p], oracle.quantize(c["a"], hh[p][None])[0]), f"hq pair {p}"
        rd = oracle.matvec(c["w"], np.ascontiguousarray(wd[e]), H, I, c["a"], hq[p][None], 1)[0]
        check_fp32(dd[p], rd, f"down pair {p}")
    check_fp32(y, oracle.moe_combine(dd, ew), "combine")


@pytest.mark.parametrize("name", ["q4k8k_small", "q5k_small", "q6k_small"])
@pytest.mark.parametrize("t", [1, 2, 3, 4, 5, 9, 32])
def test_moe_kq_tiles_small(name, t):
    """K-quant experts on the sorted tiles at every t (the auto route takes them:
    these pairs have no direct kernels); stage taps against the oracle."""
    log(f"moe {name} tiles t={t}")
    _run_stages(name, t, route=2 if t % 2 else 0)


@pytest.mark.parametrize("name", ["q4k8k_small", "q5k_small", "q6k_small"])
def test_moe_kq_tiles_hot_expert(name):
    """Skewed routing: every token picks one expert (several passes of the grouped
    kernels over its weights); every pair is compared stage by stage."""
    log(f"moe {name} tiles hot expert t=160")
    _run_stages(name, 160, route=2, dup=True)


@pytest.mark.parametrize("name", ["q4k8k_small", "q6k_small"])
def test_moe_kq_tiles_repeated_expert(name):
    _run_stages(name, 6, route=2, rep=True)


def test_moe_kq_no_direct_route():
    c = CASES["q5k_small"]
    wg, wu, wd, dwg, dwu, dwd = _bank("q5k_small")
    x = dev(synth.activations(2, c["hidden"], synth.rng(307)))
    ids = dev(synth.expert_ids(2, c["E"], c["topk"], synth.rng(308)))
    ew = dev(synth.expert_weights(2, c["topk"], synth.rng(309)))
    with pytest.raises(ft.FtError, match="FT_ERR_UNSUPPORTED"):
        ft.moe_q_vec(c["w"], dwg, dwu, dwd, c["E"], c["hidden"], c["inter"], c["a"], x, ids, ew, route=1)


@pytest.mark.parametrize("name,t,hot", [("q5k_c4", 32, False), ("q5k_c4", 512, False), ("q6k_c4", 128, False),
                                        ("q6k_c4", 512, True)])
def test_moe_kq_tiles_sampled(name, t, hot):
    """The grouped-GEMM workload as a whole layer (hidden 4096, 128 experts of 1536,
    top-8) at 32-512 tokens; the oracle checks a sample of pairs stage by stage (g,
    u, h, quantized h, down) and the whole combine.  hot: every token's slot 0 on
    one expert, whose pairs are all in the sample."""
    c = CASES[name]
    wg, wu, wd, dwg, dwu, dwd = _bank(name)
    g = synth.rng(310, t, hot)
    H, I, E, K = c["hidden"], c["inter"], c["E"], c["topk"]
    x = synth.activations(t, H, g)
    ids = synth.expert_ids(t, E, K, g)
    if hot:
        e0 = 3
        for i in range(t):
            hit = np.nonzero(ids[i] == e0)[0]
            if len(hit):
                ids[i, hit[0]] = ids[i, 0]
            ids[i, 0] = e0
    ew = synth.expert_weights(t, K, g)
    np_ = t * K
    taps = {"g": torch.empty(np_, I, device="cuda"), "u": torch.empty(np_, I, device="cuda"),
            "h": torch.empty(np_, I, device="cuda"),
            "hq": torch.empty(np_, ft.row_bytes(c["a"], I), dtype=torch.uint8, device="cuda"),
            "down": torch.empty(np_, H, device="cuda")}
    log(f"moe {name} tiles sampled t={t} hot={hot}")
    y = host(ft.moe_q_vec(c["w"], dwg, dwu, dwd, E, H, I, c["a"], dev(x), dev(ids), dev(ew), route=0, taps=taps))
    gg, uu, hh, hq, dd = (host(taps[k]) for k in ("g", "u", "h", "hq", "down"))
    xq = oracle.quantize(c["a"], x)
    flat = ids.reshape(-1)
    pick = [np.arange(4), np.arange(np_ - 4, np_), g.choice(np_, 12, replace=False)]
    if hot:
        pick.append(np.nonzero(flat == 3)[0][:: max(1, t // 48)])
    pairs = np.unique(np.concatenate(pick))
    rg_all, ru_all, rh_all = oracle.moe_gate_up(c["w"], wg, wu, E, H, I, c["a"],
                                                np.ascontiguousarray(xq[pairs // K]),
                                                np.ascontiguousarray(flat[pairs][:, None]))
    rd_all = oracle.moe_down(c["w"], wd, E, H, I, c["a"], np.ascontiguousarray(hq[pairs]),
                             np.ascontiguousarray(flat[pairs][:, None]))
    for j, p in enumerate(pairs):
        check_fp32(gg[p], rg_all[j], f"g pair {p}")
        check_fp32(uu[p], ru_all[j], f"u pair {p}")
        check_fp32(hh[p], rh_all[j], f"h pair {p}")
        assert np.array_equal(hq[p], oracle.quantize(c["a"], hh[p][None])[0]), f"hq pair {p}"
        check_fp32(dd[p], rd_all[j], f"down pair {p}")
    check_fp32(y, oracle.moe_combine(dd, ew), "combine")


@pytest.mark.parametrize("name,t,route", [("q4k", 1, 0), ("q4k", 4, 0), ("q4k", 6, 1), ("q4k_small", 3, 1),
                                          ("q4k_wide", 2, 1), ("mxfp4_small", 5, 0), ("mxfp4_small", 12, 0),
                                          ("q5k_small", 9, 0), ("mxfp4_small", 1, 0), ("mxfp4_small", 3, 1),
                                          ("mxfp4_small", 4, 1), ("mxfp4", 1, 1), ("mxfp4", 4, 1),
                                          ("mxfp4_small", 2, 1), ("mxfp4", 2, 1), ("mxfp4_tiny", 1, 1),
                                          ("mxfp4_tiny", 2, 1), ("mxfp4_tiny", 3, 1)])
def test_moe_routes_from_logits(name, t, route):
    """The layer routes each token itself from router logits (inside the first
    launch of the Q4_K layer and of the MXFP4 direct route at 1-2 tokens, else
    through the router first): its ids equal the oracle's routing bit for bit, its
    weights within 1e-6, and every stage matches the oracle."""
    log(f"moe {name} from logits t={t} route={route}")
    _run_stages(name, t, route=route, from_logits=True)


@pytest.mark.parametrize("t,from_logits", [(1, True), (3, False), (4, True), (6, True)])
def test_moe_q4k_two_launch_shapes(t, from_logits):
    """The two-launch Q4_K layer at hidden 4096 (gate/up rows of 64 units) and
    intermediate 1536 (down rows of 24 units), one and several 4-token chunks."""
    log(f"moe q4k_h4096 t={t} logits={from_logits}")
    _run_stages("q4k_h4096", t, route=1, from_logits=from_logits)


def test_moe_end_to_end_reported():
    """End to end from fp32 x (not gated on exact h codes): the GPU output stays
    close to the oracle's own end-to-end result."""
    c = CASES["q4k"]
    wg, wu, wd, dwg, dwu, dwd = _bank("q4k")
    g = synth.rng(304)
    t = 2
    x = synth.activations(t, c["hidden"], g)
    ids = synth.expert_ids(t, c["E"], c["topk"], g)
    ew = synth.expert_weights(t, c["topk"], g)
    y = host(ft.moe_q_vec(c["w"], dwg, dwu, dwd, c["E"], c["hidden"], c["inter"], c["a"], dev(x), dev(ids), dev(ew)))
    ref = oracle.moe_forward(c["w"], wg, wu, wd, c["E"], c["hidden"], c["inter"], c["a"], x, ids, ew)["y"]
    rel = np.max(np.abs(y - ref)) / np.max(np.abs(ref))
    log(f"end-to-end normwise rel {rel:.2e}")
    assert rel < 1e-2
