"""GPU parity: grouped keep-quant expert GEMM over expert_ids (fp32, normwise
1e-5 / NMSE 1e-9) against the oracle."""
import numpy as np
import pytest

import oracle
from block_quantized_matvec_amd import ft, synth
from tests.gpu_util import check_fp32, dev, host, log, need_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


@pytest.mark.parametrize("w", ["Q4_K", "Q5_K", "Q6_K", "MXFP4"])
@pytest.mark.parametrize("x_per_pair", [False, True])
@pytest.mark.parametrize("t,E,n,k,topk", [(5, 6, 40, 512, 3), (33, 16, 100, 1536, 8), (1, 4, 24, 256, 2)])
def test_grouped_small(w, x_per_pair, t, E, n, k, topk):
    log(f"grouped {w} t={t} E={E} n={n} k={k} per_pair={x_per_pair}")
    g = synth.rng(400, t, n, k)
    W = synth.expert_bank(w, E, n, k, g)
    ids = synth.expert_ids(t, E, topk, g)
    rows = t * topk if x_per_pair else t
    xq = oracle.quantize("Q8_K", synth.activations(rows, k, g))
    y = host(ft.grouped_gemm_q(w, dev(W), E, n, k, "Q8_K", dev(xq), x_per_pair, dev(ids)))
    check_fp32(y, oracle.grouped(w, W, E, n, k, "Q8_K", xq, x_per_pair, ids), w)


@pytest.mark.parametrize("w", ["Q5_K", "Q6_K"])
@pytest.mark.parametrize("proj", ["gate_up", "down"])
def test_grouped_full_size_sampled(w, proj):
    """512 tokens, 128 experts, top-8 at full size; the oracle checks a sample of
    pairs (all outputs of those pairs)."""
    t, E, topk, H, I = 512, 128, 8, 4096, 1536
    n, k = (I, H) if proj == "gate_up" else (H, I)
    log(f"grouped full {w} {proj}")
    g = synth.rng(401, proj == "down")
    W = synth.expert_bank(w, E, n, k, g)
    ids = synth.expert_ids(t, E, topk, g)
    per_pair = proj == "down"
    xq = oracle.quantize("Q8_K", synth.activations(t * topk if per_pair else t, k, g))
    y = host(ft.grouped_gemm_q(w, dev(W), E, n, k, "Q8_K", dev(xq), per_pair, dev(ids)))
    pairs = np.unique(np.concatenate([np.arange(16), g.choice(t * topk, 48, replace=False)]))
    flat = ids.reshape(-1)
    for p in pairs:
        xrow = xq[p] if per_pair else xq[p // topk]
        ref = oracle.matvec(w, np.ascontiguousarray(W[flat[p]]), n, k, "Q8_K", xrow[None], 1)[0]
        check_fp32(y[p], ref, f"pair {p}")


@pytest.mark.parametrize("w", ["Q5_K", "Q6_K"])
@pytest.mark.parametrize("proj", ["gate_up", "down"])
def test_grouped_full_size_hot_expert(w, proj):
    """512 tokens, 128 experts, top-8 with every token's slot 0 on one expert: that
    expert has 512 pairs and the kernel (48 pairs per pass at this batch) walks its
    weights 11 times.  Every pair of the hot expert is compared on a sample of
    rows (the first row tile, the ragged last rows), and a sample of other pairs on
    all rows."""
    t, E, topk, H, I = 512, 128, 8, 4096, 1536
    n, k = (I, H) if proj == "gate_up" else (H, I)
    log(f"grouped full hot expert {w} {proj}")
    g = synth.rng(402, proj == "down", w == "Q6_K")
    W = synth.expert_bank(w, E, n, k, g)
    ids = synth.expert_ids(t, E, topk, g)
    e0 = 7
    for i in range(t):   # move e0 to slot 0 of every token, keeping the ids distinct
        hit = np.nonzero(ids[i] == e0)[0]
        if len(hit):
            ids[i, hit[0]] = ids[i, 0]
        ids[i, 0] = e0
    assert np.count_nonzero(ids == e0) == t
    per_pair = proj == "down"
    xq = oracle.quantize("Q8_K", synth.activations(t * topk if per_pair else t, k, g))
    y = host(ft.grouped_gemm_q(w, dev(W), E, n, k, "Q8_K", dev(xq), per_pair, dev(ids)))
    flat = ids.reshape(-1)
    hot = np.nonzero(flat == e0)[0]
    rows = np.unique(np.concatenate([np.arange(144), np.arange(n - 40, n)]))
    xh = xq[hot] if per_pair else xq[hot // topk]
    ref = oracle.matvec(w, np.ascontiguousarray(W[e0][rows]), len(rows), k, "Q8_K", np.ascontiguousarray(xh),
                        len(hot))
    check_fp32(y[hot][:, rows], ref, f"hot expert {e0}")
    others = g.choice(np.nonzero(flat != e0)[0], 24, replace=False)
    for p in others:
        xrow = xq[p] if per_pair else xq[p // topk]
        r = oracle.matvec(w, np.ascontiguousarray(W[flat[p]]), n, k, "Q8_K", xrow[None], 1)[0]
        check_fp32(y[p], r, f"pair {p}")
