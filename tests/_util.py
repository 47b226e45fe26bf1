"""Shared helpers of the test suite (comparison bars, device plumbing)."""

import os
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


def check_out_lse(out, lse, ref_out, ref_lse, what="", ref_abs=None):
    """out/ref_out [..., D] and lse/ref_lse arrays; NaN entries of the
    reference (rows the oracle did not compute) are ignored.  ref_abs, when
    given, is sum_j P_ij |v_j| per output element (the oracle's forward of
    |v|), which bounds what the rounding of P to bf16 can cost (out_bar);
    without it |ref_out| stands in, a smaller and so stricter bound."""
    out, lse = np.asarray(out), np.asarray(lse)
    sel = ~np.isnan(ref_lse)
    assert sel.any(), "nothing to compare"
    osel = ~np.isnan(ref_out)
    d_out = np.abs(out[osel] - ref_out[osel])
    d_lse = np.abs(lse[sel] - ref_lse[sel])
    bar = out_bar(ref_out[osel], None if ref_abs is None else np.asarray(ref_abs)[osel])
    wide = int((bar > OUT_MAX_ABS).sum())
    msg = (f"{what}: out max {d_out.max():.3e} mean {d_out.mean():.3e} (worst vs its bar "
           f"{(d_out / bar).max():.3f}; {wide} of {bar.size} elements carry the rounding-derived bar above "
           f"1e-2); lse max {d_lse.max():.3e}")
    print(msg, flush=True)
    assert np.isfinite(out[osel]).all() and np.isfinite(lse[sel]).all(), msg
    assert (d_out <= bar).all(), msg
    assert d_out.mean() <= OUT_MEAN_ABS, msg
    assert d_lse.max() <= LSE_MAX_ABS, msg
    return d_out.max(), d_out.mean(), d_lse.max()


def bf16_ulp(x):
    """Spacing of bf16 numbers (8 significant bits) at |x|."""
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -126)))
    return np.exp2(e - 7)


def out_bar(ref, ref_abs=None):
    """Per-element bar of the bf16 output: OUT_MAX_ABS wherever a bf16 MFMA
    path can attain it, else the error its arithmetic admits.  The P.V
    product consumes probabilities rounded to bf16 (8 significant bits), each
    off by up to 2^-8 of itself, which moves out_i by at most
    2^-8 sum_j P_ij |v_j| (ref_abs; |ref| when not given); the result is
    rounded to bf16 (half an ulp of |out| <= |ref| (1 + 2^-7)); 1e-3 covers
    the fp32 accumulation.  This exceeds 1e-2 only where sum_j P_ij |v_j| is
    above about 1.3 (a row dominated by one key with a large value, e.g. a
    window-1 row)."""
    ref = np.abs(ref)
    a = ref if ref_abs is None else np.maximum(np.abs(ref_abs), ref)
    return np.maximum(OUT_MAX_ABS, 2.0 ** -8 * a + 0.5 * bf16_ulp(ref * (1 + 2.0 ** -7)) + 1e-3)


def rel_l2(x, ref):
    x, ref = np.asarray(x, dtype=np.float64), np.asarray(ref, dtype=np.float64)
    return float(np.linalg.norm(x - ref) / max(np.linalg.norm(ref), 1e-300))


def seed_of(*parts):
    """Deterministic seed for a test case (Python's hash() of a str is salted
    per process)."""
    return zlib.crc32(repr(parts).encode()) % 100000


def oracle_map(fn, tasks):
    """fn over tasks on host threads (numpy leaves the interpreter lock in its
    array loops), BLAS held to one thread per task; results in task order."""
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    workers = max(1, min(16, len(os.sched_getaffinity(0)), len(tasks)))
    with threadpool_limits(1):
        with ThreadPoolExecutor(workers) as ex:
            return list(ex.map(fn, tasks))


def nan_like(shape, dtype, dev):
    """An output buffer filled with NaN, so an element the kernel never
    writes cannot pass for a finite result."""
    import torch
    return torch.full(tuple(shape), float("nan"), dtype=dtype, device=dev)


def nan_grads(q, k, v, Hq):
    import torch
    return (nan_like(q.shape, torch.bfloat16, q.device), nan_like(k.shape, torch.bfloat16, q.device),
            nan_like(v.shape, torch.bfloat16, q.device), nan_like((Hq,), torch.float32, q.device))


def ref_fwd_groups(q, k, v, sinks, window, scale, rows=None):
    """The oracle forward (fp64 arrays in, ref_fwd per batch and KV group on
    host threads).  With ``rows`` given, returns only those rows:
    out [B, len(rows), Hq, D] and lse [B, Hq, len(rows)]."""
    from oracle import ref_fwd
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    sel = np.arange(S) if rows is None else np.asarray(rows)
    tasks = [(b, c) for b in range(B) for c in range(Hkv)]

    def one(t):
        b, c = t
        hs = slice(c * G, (c + 1) * G)
        o, l = ref_fwd(q[b:b + 1, :, hs], k[b:b + 1, :, c:c + 1], v[b:b + 1, :, c:c + 1], sinks[hs], window,
                       scale, rows=rows)
        return o[0, sel], l[0][:, sel]

    out = np.full((B, len(sel), Hq, D), np.nan)
    lse = np.full((B, Hq, len(sel)), np.nan)
    for (b, c), (o, l) in zip(tasks, oracle_map(one, tasks)):
        out[b, :, c * G:(c + 1) * G] = o
        lse[b, c * G:(c + 1) * G] = l
    return out, lse


def ref_bwd_groups(q, k, v, sinks, dout, window, scale):
    """The oracle backward (ref_bwd per batch and KV group on host threads):
    (dq, dk, dv, dsinks) of the whole problem."""
    from oracle import ref_bwd
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    tasks = [(b, c) for b in range(B) for c in range(Hkv)]

    def one(t):
        b, c = t
        hs = slice(c * G, (c + 1) * G)
        return ref_bwd(q[b:b + 1, :, hs], k[b:b + 1, :, c:c + 1], v[b:b + 1, :, c:c + 1], sinks[hs],
                       dout[b:b + 1, :, hs], window, scale)

    dq, dk, dv = np.zeros(q.shape), np.zeros(k.shape), np.zeros(v.shape)
    ds = np.zeros(Hq)
    for (b, c), (gq, gk, gv, gs) in zip(tasks, oracle_map(one, tasks)):
        hs = slice(c * G, (c + 1) * G)
        dq[b, :, hs] = gq[0]
        dk[b, :, c] = gk[0, :, 0]
        dv[b, :, c] = gv[0, :, 0]
        ds[hs] += gs
    return dq, dk, dv, ds


def check_grads_by_group(grads, ref, Hkv, what, bar=GRAD_REL_L2):
    """Relative L2 of each gradient over the whole tensor and over each KV
    group on its own (its G query heads' dq, its dk and dv, and with G >= 8
    its heads' dsinks: a group of one or two heads has as many dsink values,
    each one possibly cancelling sum, too few for a relative L2)."""
    dq, dk, dv, ds = grads
    rdq, rdk, rdv, rds = ref
    Hq = dq.shape[2]
    G = Hq // Hkv
    errs = {n: rel_l2(a, r) for n, a, r in (("dq", dq, rdq), ("dk", dk, rdk), ("dv", dv, rdv), ("dsinks", ds, rds))}
    worst = {}
    for c in range(Hkv):
        hs = slice(c * G, (c + 1) * G)
        parts = [("dq", dq[:, :, hs], rdq[:, :, hs]), ("dk", dk[:, :, c], rdk[:, :, c]),
                 ("dv", dv[:, :, c], rdv[:, :, c])]
        if G >= 8:
            parts.append(("dsinks", ds[hs], rds[hs]))
        for n, a, r in parts:
            e = rel_l2(a, r)
            if e > worst.get(n, (-1.0, None))[0]:
                worst[n] = (e, c)
    msg = (f"{what}: " + ", ".join(f"{n} {e:.2e}" for n, e in errs.items()) + "; worst group: " +
           ", ".join(f"{n} {e:.2e} (group {c})" for n, (e, c) in worst.items()))
    print(msg, flush=True)
    assert all(e <= bar for e in errs.values()), msg
    assert all(e <= bar for e, _ in worst.values()), msg
    return errs
