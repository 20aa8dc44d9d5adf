"""Helpers for the GPU parity tests (compare the HIP path with the oracle)."""
import numpy as np
import pytest
import torch

# Acceptance for fp32 outputs, normwise over the compared set:
#   max|y - r| / max|r| <= 1e-5   and   sum (y - r)^2 / sum r^2 <= 1e-9
REL = 1e-5
NMSE = 1e-9


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def dev(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def check_fp32(y, r, what="", rel=REL, nmse=NMSE):
    y = np.asarray(y, np.float64)
    r = np.asarray(r, np.float64)
    assert y.shape == r.shape, (y.shape, r.shape)
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    den = np.max(np.abs(r))
    err = np.max(np.abs(y - r)) / den if den > 0 else np.max(np.abs(y))
    nm = np.sum((y - r) ** 2) / max(np.sum(r ** 2), 1e-300)
    assert err <= rel and nm <= nmse, f"{what}: normwise max rel {err:.3e}, NMSE {nm:.3e}"
    return err, nm


def log(msg):
    print(msg, flush=True)


def abs_terms(wfmt, W, n, k, afmt, xq, t):
    """[t][n] sum over k of |w * xhat| (fp64, from the oracle's exact values): the
    scale of the rounding an fp32 sum of the products may carry."""
    import oracle
    w = oracle.dequant(wfmt, W, n, k).astype(np.float64)
    x = oracle.dequant(afmt, xq, t, k).astype(np.float64)
    return np.abs(x) @ np.abs(w).T


def check_fp32_small(y, r, terms, what="", rel=REL):
    """The per-output form of the fp32 bar for a compared set too small for a
    normwise maximum to mean anything (a single output is its own maximum, and
    heavy cancellation leaves it far below its terms): |y - r| <= rel * sum|terms|."""
    y = np.asarray(y, np.float64)
    r = np.asarray(r, np.float64)
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    bad = np.abs(y - r) > rel * np.asarray(terms)
    assert not bad.any(), f"{what}: {int(bad.sum())} outputs beyond {rel} of their term sums"
