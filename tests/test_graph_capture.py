"""GPU: a decode step captured in a HIP graph and replayed (vllm.cpp PR #523, review
and rework: no per-call allocation or synchronisation, so the path can be
captured; a grow-only pool sized before capture).

The step is the library's own calls on one stream: quantize x (Q8_1), a dense
Q4_K matvec, the router, and the routed-MoE layer on the matvec's output
(direct route: Q4_K x Q8_1; sorted tiles: MXFP4 x Q8_K).  Between replays the
test changes the inputs with eager work and synchronises; every replay must
equal the same calls run eagerly, byte for byte, and match the oracle.  A
stream whose pool is too small is refused with FT_ERR_NO_SCRATCH while it is
being captured, instead of allocating."""
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


STEPS = {
    "q4k_direct": dict(w="Q4_K", a="Q8_1", hidden=2048, inter=768, E=16, topk=8, t=3),
    "mxfp4_tiles": dict(w="MXFP4", a="Q8_K", hidden=1024, inter=512, E=12, topk=4, t=20),
}


@pytest.mark.parametrize("name", list(STEPS))
def test_captured_decode_step(name):
    c = STEPS[name]
    H, I, E, K, t, w, a = c["hidden"], c["inter"], c["E"], c["topk"], c["t"], c["w"], c["a"]
    g = synth.rng(800, list(STEPS).index(name))
    Wd = synth.weights("Q4_K", H, H, g)                 # dense H x H projection
    banks = [synth.expert_bank(w, E, I, H, g), synth.expert_bank(w, E, I, H, g), synth.expert_bank(w, E, H, I, g)]
    dWd = dev(Wd)
    dbanks = [dev(b) for b in banks]
    s = torch.cuda.Stream()
    x = torch.zeros((t, H), device="cuda")
    logits = torch.zeros((t, E), device="cuda")
    xq = torch.empty((t, ft.row_bytes("Q8_1", H)), dtype=torch.uint8, device="cuda")
    y1 = torch.empty((t, H), device="cuda")
    ids = torch.empty((t, K), dtype=torch.int32, device="cuda")
    ew = torch.empty((t, K), device="cuda")
    y = torch.empty((t, H), device="cuda")

    def step():
        ft.quantize_act("Q8_1", x, out=xq, stream=s)
        ft.mul_mat_vec_q("Q4_K", dWd, H, H, "Q8_1", xq, t, out=y1, stream=s)
        ft.moe_route(logits, K, ids=ids, w=ew, stream=s)
        ft.moe_q_vec(w, *dbanks, E, H, I, a, y1, ids, ew, out=y, stream=s)

    def draw(seed):
        # x at 1/1000 of N(0, 1): the dense output then feeds the layer at a scale
        # whose intermediate h stays inside Q8_1's fp16 scale range
        gg = synth.rng(801, seed)
        xn = synth.activations(t, H, gg) * np.float32(0.001)
        return xn, synth.logits(t, E, gg)

    def load(seed):
        xn, ln = draw(seed)
        x.copy_(torch.from_numpy(xn))
        logits.copy_(torch.from_numpy(ln))
        torch.cuda.synchronize()

    # size the pool on the capture stream, then capture
    assert ft.lib().ft_scratch_reserve(ft._stream(s), ft.moe_scratch_bytes(w, a, E, H, I, t, K)) == 0
    load(0)
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        step()
    torch.cuda.synchronize()

    outs = []
    for rep in range(4):
        load(rep % 2)                                       # inputs alternate between two draws
        graph.replay()
        torch.cuda.synchronize()
        got = [host(v).copy() for v in (xq, y1, ids, ew, y)]
        with torch.cuda.stream(s):                          # the same calls, eagerly
            step()
        torch.cuda.synchronize()
        eager = [host(v).copy() for v in (xq, y1, ids, ew, y)]
        for a_, b_ in zip(got, eager):
            assert np.all(np.isfinite(a_)), f"replay {rep}: non-finite output"
            assert np.array_equal(a_, b_), f"replay {rep} differs from the eager step"
        outs.append(got)
        log(f"graph {name} replay {rep} ok")
    for rep in (2, 3):
        for a_, b_ in zip(outs[rep], outs[rep - 2]):
            assert np.array_equal(a_, b_), "replays of the same inputs differ"

    # the replay against the oracle (last inputs: draw 1)
    xn, ln = draw(1)
    got_xq, got_y1, got_ids, got_ew, got_y = outs[3]
    rxq = oracle.quantize("Q8_1", xn)
    assert np.array_equal(got_xq, rxq)
    check_fp32(got_y1, oracle.matvec("Q4_K", Wd, H, H, "Q8_1", rxq, t), "dense")
    rid, rw = oracle.route(ln, K)
    assert np.array_equal(got_ids, rid)
    check_fp32(got_ew, rw, "route weights", rel=1e-6, nmse=1e-12)
    # the MoE layer from the replay's own y1 (end to end from fp32, as the layer runs)
    ref = oracle.moe_forward(w, *banks, E, H, I, a, got_y1, got_ids, got_ew)["y"]
    rel = np.max(np.abs(got_y - ref)) / np.max(np.abs(ref))
    assert rel < 1e-2, rel


def test_capture_with_small_pool_refused():
    c = STEPS["q4k_direct"]
    H, I, E, K, t = c["hidden"], c["inter"], c["E"], c["topk"], 2
    g = synth.rng(802)
    banks = [dev(synth.expert_bank("Q4_K", E, I, H, g)), dev(synth.expert_bank("Q4_K", E, I, H, g)),
             dev(synth.expert_bank("Q4_K", E, H, I, g))]
    x = dev(synth.activations(t, H, g))
    ids = dev(synth.expert_ids(t, E, K, g))
    ew = dev(synth.expert_weights(t, K, g))
    y = torch.empty((t, H), device="cuda")
    s = torch.cuda.Stream()                                 # a new stream: its pool is empty
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    status = None
    with torch.cuda.graph(graph, stream=s):
        status = ft.lib().ft_moe_q_vec(ft.TYPES["Q4_K"], *(ft._ptr(b) for b in banks), E, H, I, ft.TYPES["Q8_1"],
                                       ft._ptr(x), t, ft._ptr(ids), ft._ptr(ew), K, ft._ptr(y), None, ft._stream(s))
    torch.cuda.synchronize()
    assert ft.STATUS[status] == "FT_ERR_NO_SCRATCH"
    # outside capture the same call grows the pool and runs
    ft.moe_q_vec("Q4_K", *banks, E, H, I, "Q8_1", x, ids, ew, out=y, stream=s)
    torch.cuda.synchronize()
    assert np.all(np.isfinite(host(y)))
