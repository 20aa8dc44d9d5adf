"""GPU: the measurement microkernels run and the bench's ceiling figures are in a
plausible range for this part (they are reference points for the rooflines, not
part of the method)."""
import pytest
import torch

from block_quantized_matvec_amd import ft
from tests.gpu_util import log, need_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _gpu():
    need_gpu()


def test_microkernels_run():
    log("ceiling microkernels")
    buf = torch.empty(64 << 20, dtype=torch.uint8, device="cuda")
    out = torch.zeros(1, dtype=torch.int32, device="cuda")
    for which, kw in (("stream_read", {"buf": buf}), ("mfma_i8", {"iters": 16}), ("mfma_i8_k64", {"iters": 16}),
                      ("dot4", {"iters": 64})):
        ft.debug_ceiling(which, out=out, **kw)
    torch.cuda.synchronize()
    assert int(out.item()) == 0   # the results never match the value that would be stored


def test_measured_ceilings_plausible():
    import bench
    c = bench.measure_ceilings(torch, ft)
    log(f"ceilings {c}")
    assert 2000 < c["stream_read_GBps"] < 8000 * 1.05
    assert 500 < c["mfma_i8_TOPS"] <= c["mfma_i8_k64_TOPS"] < 5000 * 1.05
    assert 50 < c["dot4_TOPS"] < 1000
