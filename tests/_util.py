"""Shared helpers of the test suite (comparison bars, device plumbing)."""

import zlib

import numpy as np
import pytest
import torch

# Numeric bars for the HIP path against the fp64 oracle.
OUT_MAX_ABS = 1e-2
OUT_MEAN_ABS = 1e-3
LSE_MAX_ABS = 1e-3
GRAD_REL_L2 = 1e-2


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    return torch.device("cuda:0")


def f64(t):
    """Exact upcast of a (CPU or GPU) tensor to a float64 numpy array."""
    return t.detach().to("cpu", torch.float64).numpy()


def check_out_lse(out, lse, ref_out, ref_lse, what=""):
    """out/ref_out [..., D] and lse/ref_lse arrays; NaN entries of the
    reference (rows the oracle did not compute) are ignored."""
    out, lse = np.asarray(out), np.asarray(lse)
    sel = ~np.isnan(ref_lse)
    assert sel.any(), "nothing to compare"
    osel = ~np.isnan(ref_out)
    d_out = np.abs(out[osel] - ref_out[osel])
    d_lse = np.abs(lse[sel] - ref_lse[sel])
    bar = out_bar(ref_out[osel])
    msg = (f"{what}: out max {d_out.max():.3e} mean {d_out.mean():.3e} (worst vs its bar "
           f"{(d_out / bar).max():.3f}); lse max {d_lse.max():.3e}")
    assert np.isfinite(out[osel]).all() and np.isfinite(lse[sel]).all(), msg
    assert (d_out <= bar).all(), msg
    assert d_out.mean() <= OUT_MEAN_ABS, msg
    assert d_lse.max() <= LSE_MAX_ABS, msg
    return d_out.max(), d_out.mean(), d_lse.max()


def bf16_ulp(x):
    """Spacing of bf16 numbers (8 significant bits) at |x|."""
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -126)))
    return np.exp2(e - 7)


def out_bar(ref):
    """Per-element bar of the bf16 output: OUT_MAX_ABS, or one bf16 ulp of the
    exact value where that is larger (|out| >= 2, e.g. a window-1 row whose
    output is one value row; rounding the exact value to bf16 alone costs
    half an ulp, 0.0156 at |out| >= 4, above the 1e-2 bar)."""
    return np.maximum(OUT_MAX_ABS, bf16_ulp(ref))


def rel_l2(x, ref):
    x, ref = np.asarray(x, dtype=np.float64), np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(x - ref) / max(np.linalg.norm(ref), 1e-300))


def seed_of(*parts):
    """Deterministic seed for a test case (Python's hash() of a str is salted
    per process)."""
    return zlib.crc32(repr(parts).encode()) % 100000
