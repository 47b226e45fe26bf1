"""Forward parity of the HIP path against the fp64 oracle (GPU)."""

import numpy as np
import pytest
import torch

import attention_attn_fwd_amd as attn
from attention_attn_fwd_amd import synth
from oracle import ref_fwd

from _util import check_out_lse, f64, nan_like, need_gpu, out_bar, ref_fwd_groups, seed_of

pytestmark = pytest.mark.gpu


def _run(case, window, dev):
    q, k, v, s = (t.to(dev) for t in (case.q, case.k, case.v, case.sinks))
    out, lse = attn.fwd(q, k, v, s, window, case.scale)
    torch.cuda.synchronize()
    return out, lse


def _oracle(case, window, **kw):
    return ref_fwd(f64(case.q), f64(case.k), f64(case.v), f64(case.sinks), window, case.scale, **kw)


SMALL = [  # B, S, Hq, Hkv
    (1, 1, 8, 1), (1, 17, 8, 1), (2, 129, 8, 1), (1, 300, 8, 8), (1, 1000, 8, 1), (2, 77, 16, 2),
    (1, 200, 6, 2), (1, 333, 1, 1), (1, 260, 4, 4),
    (2, 200, 16, 8), (3, 150, 24, 8),  # B * Hkv = 16, 24: the XCD-aware order with 2, 3 groups per XCD
]


@pytest.mark.parametrize("shape", SMALL, ids=lambda s: "B%dS%dH%dx%d" % s)
@pytest.mark.parametrize("window", [0, 1, 127, 128, 129])
def test_fwd_small_shapes(shape, window):
    dev = need_gpu()
    B, S, Hq, Hkv = shape
    case = synth.make_prefill(B, S, Hq, Hkv, seed=seed_of(shape, window))
    print(f"fwd shape={shape} window={window}", flush=True)
    out, lse = _run(case, window, dev)
    ro, rl = _oracle(case, window)
    check_out_lse(f64(out), f64(lse), ro, rl, f"{shape} W={window}")


# group sizes G = Hq / Hkv up to the supported 128: a workgroup's 256
# columns hold 256 / G positions (16 .. 2), and G = 12 and 40 divide neither
# 256 nor the backward's 64-column steps
LARGE_GROUPS = [(16, 1), (32, 1), (64, 1), (128, 1), (12, 1), (80, 2)]


@pytest.mark.parametrize("heads", LARGE_GROUPS, ids=lambda h: "H%dx%d" % h)
@pytest.mark.parametrize("window", [0, 128])
def test_fwd_large_groups(heads, window):
    dev = need_gpu()
    Hq, Hkv = heads
    case = synth.make_prefill(1, 190, Hq, Hkv, seed=seed_of(heads, window, "fwdG"))
    print(f"fwd heads={heads} window={window}", flush=True)
    out, lse = _run(case, window, dev)
    ro, rl = _oracle(case, window)
    check_out_lse(f64(out), f64(lse), ro, rl, f"heads={heads} W={window}")


@pytest.mark.parametrize("sink", [-np.inf, 20.0, -20.0])
@pytest.mark.parametrize("window", [0, 128])
def test_fwd_extreme_sinks(sink, window):
    dev = need_gpu()
    case = synth.make_prefill(1, 300, 8, 1, seed=7)
    case.sinks[:] = sink
    out, lse = _run(case, window, dev)
    ro, rl = _oracle(case, window)
    check_out_lse(f64(out), f64(lse), ro, rl, f"sink={sink} W={window}")


def test_fwd_window_at_least_S_is_full_causal():
    dev = need_gpu()
    case = synth.make_prefill(1, 200, 8, 1, seed=8)
    o0, l0 = _run(case, 0, dev)
    for w in (200, 205, 100000):
        o, l = _run(case, w, dev)
        assert torch.equal(o, o0) and torch.equal(l, l0)


def test_fwd_is_deterministic():
    dev = need_gpu()
    case = synth.make_prefill(2, 700, 16, 2, seed=9)
    a = _run(case, 0, dev)
    b = _run(case, 0, dev)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_fwd_row0_closed_form_on_gpu_output():
    """Row 0 sees one key: out_0 = sigmoid(s00 - sink) v_0, lse_0 = logaddexp(s00, sink)."""
    dev = need_gpu()
    case = synth.make_prefill(1, 64, 8, 1, seed=10)
    out, lse = _run(case, 128, dev)
    q, k, v, s = f64(case.q), f64(case.k), f64(case.v), f64(case.sinks)
    for h in range(8):
        s00 = case.scale * q[0, 0, h] @ k[0, 0, 0]
        ref = 1 / (1 + np.exp(s[h] - s00)) * v[0, 0, 0]
        assert (np.abs(f64(out)[0, 0, h] - ref) <= out_bar(ref)).all()
        assert abs(f64(lse)[0, h, 0] - np.logaddexp(s00, s[h])) <= 1e-3


def test_fwd_small_workload_both_layers():
    dev = need_gpu()
    case = synth.config_inputs("small_b1_s512_h8x1")
    for window in (128, 0):
        out, lse = _run(case, window, dev)
        ro, rl = _oracle(case, window)
        check_out_lse(f64(out), f64(lse), ro, rl, f"small workload W={window}")


def _run_poisoned(case, window, dev):
    """The forward into NaN-filled out and lse buffers."""
    q, k, v, s = (t.to(dev) for t in (case.q, case.k, case.v, case.sinks))
    B, S, Hq, D = q.shape
    out = nan_like((B, S, Hq, D), torch.bfloat16, dev)
    lse = nan_like((B, Hq, S), torch.float32, dev)
    attn.fwd(q, k, v, s, window, case.scale, out=out, lse=lse)
    torch.cuda.synchronize()
    # every element written: finite, and every lse at least the sink (it is in the sum)
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    assert (lse >= s.view(1, -1, 1) - 1e-4).all()
    return out, lse


@pytest.mark.parametrize("window", [128, 0])
def test_fwd_prefill_workload_whole(window):
    """B=4, S=4096, 64q/8kv in the launch configuration bench.py times:
    every output and lse element against the oracle (run per batch and KV
    group on the host's cores)."""
    dev = need_gpu()
    case = synth.config_inputs("prefill_b4_s4096_h64x8")
    print(f"fwd B4 S4096 W={window}", flush=True)
    out, lse = _run_poisoned(case, window, dev)
    ro, rl = ref_fwd_groups(f64(case.q), f64(case.k), f64(case.v), f64(case.sinks), window, case.scale)
    check_out_lse(f64(out), f64(lse), ro, rl, f"B4 S4096 W={window}")


def _long_context_rows(S, W, rng):
    """512 query rows: the first 128, W - 1 .. W + 1, the last 64, and random
    rows to make up 512."""
    rows = set(range(128)) | {W - 1, W, W + 1} | set(range(S - 64, S))
    while len(rows) < 512:
        rows.add(int(rng.integers(0, S)))
    return np.array(sorted(rows))


@pytest.mark.parametrize("window", [128, 0])
def test_fwd_long_context_sampled_rows(window):
    """B=1, S=65536, 64q/8kv in the launch configuration bench.py times:
    all 64 heads at 512 query rows (each row exact over all its keys), and
    every element of the output written and finite."""
    dev = need_gpu()
    case = synth.config_inputs("long_b1_s65536_h64x8")
    print(f"fwd B1 S65536 W={window}", flush=True)
    out, lse = _run_poisoned(case, window, dev)
    S = case.q.shape[1]
    rows = _long_context_rows(S, 128, np.random.default_rng(S + window))
    ro, rl = ref_fwd_groups(f64(case.q), f64(case.k), f64(case.v), f64(case.sinks), window, case.scale, rows=rows)
    ri = torch.from_numpy(rows).to(dev)
    check_out_lse(f64(out[:, ri]), f64(lse[:, :, ri]), ro, rl, f"B1 S65536 W={window}")
