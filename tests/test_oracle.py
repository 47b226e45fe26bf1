"""Pins of the fp64 oracle against things other than itself (CPU only).

* hand-derived exact cases (tests/golden/hand_cases.json)
* a scalar brute force written independently (oracle/brute.py)
* torch's fp64 scaled_dot_product_attention through an augmented-key
  reduction (an all-zero key/value row whose additive bias is the sink)
* invariants: sink -inf is standard attention; the sink scales rows by
  sum(e)/(sum(e)+e^sink); window >= S equals full causal
* closed forms: row 0, window 1, q = 0
* GQA equals MHA with repeated K/V; decode equals the prefill row L-1
* backward: central finite differences on every input element incl. sinks
"""

import ast
import json
import math
import os
import operator
import zlib

import numpy as np
import pytest
import torch

from oracle import brute_fwd, ref_bwd, ref_decode, ref_fwd, unmasked_pairs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")


# --------------------------------------------------------------------------
# helpers

_OPS = {ast.Add: operator.add, ast.Sub: operator.sub, ast.Mult: operator.mul,
        ast.Div: operator.truediv, ast.USub: operator.neg, ast.UAdd: operator.pos}


def _eval_expr(text):
    """Evaluate an arithmetic expression over numbers, log() and inf."""
    def ev(node):
        if isinstance(node, ast.Expression):
            return ev(node.body)
        if isinstance(node, ast.Constant) and isinstance(node.value, (int, float)):
            return float(node.value)
        if isinstance(node, ast.Name) and node.id == "inf":
            return math.inf
        if isinstance(node, ast.BinOp) and type(node.op) in _OPS:
            return _OPS[type(node.op)](ev(node.left), ev(node.right))
        if isinstance(node, ast.UnaryOp) and type(node.op) in _OPS:
            return _OPS[type(node.op)](ev(node.operand))
        if (isinstance(node, ast.Call) and isinstance(node.func, ast.Name)
                and node.func.id == "log" and len(node.args) == 1):
            return math.log(ev(node.args[0]))
        raise ValueError(f"unsupported expression {ast.dump(node)}")
    return ev(ast.parse(text, mode="eval"))


def _arr(nested):
    if isinstance(nested, str):
        return _eval_expr(nested)
    return np.array([_arr(x) for x in nested], dtype=np.float64)


def _rand(rng, shape, std=1.0):
    return rng.standard_normal(shape) * std


def _case(rng, B, S, Hq, Hkv, D, std=1.0):
    q = _rand(rng, (B, S, Hq, D), std)
    k = _rand(rng, (B, S, Hkv, D), std)
    v = _rand(rng, (B, S, Hkv, D))
    sinks = rng.standard_normal(Hq)
    return q, k, v, sinks


def _sdpa_augmented(q, k, v, sinks, window, scale):
    """torch fp64 SDPA over keys + one zero key/value whose bias is the sink."""
    B, S, Hq, D = q.shape
    G = Hq // k.shape[2]
    Q = torch.from_numpy(q).permute(0, 2, 1, 3)                       # B,H,S,D
    K = torch.from_numpy(k).permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    V = torch.from_numpy(v).permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    zero = torch.zeros(B, Hq, 1, D, dtype=torch.float64)
    Ka, Va = torch.cat([K, zero], 2), torch.cat([V, zero], 2)
    i = torch.arange(S)[:, None]
    j = torch.arange(S)[None, :]
    ok = j <= i
    if window > 0:
        ok = ok & (i - j < window)
    band = torch.where(ok, 0.0, -math.inf).to(torch.float64)         # S,S
    sink_col = torch.from_numpy(np.asarray(sinks, dtype=np.float64))  # H
    mask = torch.cat([band.expand(B, Hq, S, S),
                      sink_col.view(1, Hq, 1, 1).expand(B, Hq, S, 1)], dim=3)
    out = torch.nn.functional.scaled_dot_product_attention(Q, Ka, Va, attn_mask=mask,
                                                           scale=scale)
    logits = scale * (Q @ Ka.transpose(-1, -2)) + mask
    lse = torch.logsumexp(logits, dim=-1)                             # B,H,S
    return out.permute(0, 2, 1, 3).numpy(), lse.numpy()


# --------------------------------------------------------------------------
# hand-derived exact cases

def _golden_cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_hand_cases(case):
    q, k, v = _arr(case["q"]), _arr(case["k"]), _arr(case["v"])
    sinks = _arr(case["sinks"])
    scale, window = _eval_expr(case["scale"]), case["window"]
    out, lse = ref_fwd(q, k, v, sinks, window, scale)
    np.testing.assert_allclose(out, _arr(case["out"]), rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, _arr(case["lse"]), rtol=0, atol=1e-14)
    if "dout" in case:
        dq, dk, dv, ds = ref_bwd(q, k, v, sinks, _arr(case["dout"]), window, scale)
        np.testing.assert_allclose(dq, _arr(case["dq"]), rtol=0, atol=1e-14)
        np.testing.assert_allclose(dk, _arr(case["dk"]), rtol=0, atol=1e-14)
        np.testing.assert_allclose(dv, _arr(case["dv"]), rtol=0, atol=1e-14)
        np.testing.assert_allclose(ds, _arr(case["dsinks"]), rtol=0, atol=1e-14)


# --------------------------------------------------------------------------
# brute force

BRUTE_SHAPES = [  # B, S, Hq, Hkv, D
    (1, 1, 1, 1, 1), (1, 7, 1, 1, 4), (2, 9, 2, 1, 3), (1, 16, 4, 2, 8), (1, 12, 4, 1, 5),
]


@pytest.mark.parametrize("shape", BRUTE_SHAPES)
@pytest.mark.parametrize("window", [0, 1, 2, 3, 7, 100])
@pytest.mark.parametrize("sink_kind", ["normal", "neg_inf", "large"])
def test_matches_brute_force(shape, window, sink_kind):
    B, S, Hq, Hkv, D = shape
    rng = np.random.default_rng(zlib.crc32(repr((shape, window, sink_kind)).encode()))
    q, k, v, sinks = _case(rng, B, S, Hq, Hkv, D, std=0.7)
    if sink_kind == "neg_inf":
        sinks[:] = -np.inf
    elif sink_kind == "large":
        sinks[:] = 6.0
    scale = 1.0 / math.sqrt(D)
    out, lse = ref_fwd(q, k, v, sinks, window, scale)
    bo, bl = brute_fwd(q.tolist(), k.tolist(), v.tolist(), sinks.tolist(), window, scale)
    np.testing.assert_allclose(out, np.array(bo), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, np.array(bl), rtol=1e-12, atol=1e-12)


def test_row_subsets_are_exact():
    rng = np.random.default_rng(5)
    q, k, v, sinks = _case(rng, 2, 40, 4, 2, 8)
    full_o, full_l = ref_fwd(q, k, v, sinks, 6, 0.3)
    rows = np.array([0, 5, 6, 7, 39])
    o, l = ref_fwd(q, k, v, sinks, 6, 0.3, rows=rows, heads=[1, 3], batches=[1], row_block=2)
    # a different row block changes only the BLAS summation order
    np.testing.assert_allclose(o[1][rows][:, [1, 3]], full_o[1][rows][:, [1, 3]], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(l[1][[1, 3]][:, rows], full_l[1][[1, 3]][:, rows], rtol=1e-14, atol=1e-14)
    assert np.isnan(o[0]).all() and np.isnan(l[1][0]).all()


# --------------------------------------------------------------------------
# library reduction and invariants

@pytest.mark.parametrize("window", [0, 1, 5, 13, 64])
@pytest.mark.parametrize("heads", [(1, 1), (4, 1), (4, 2), (8, 8)])
def test_augmented_sdpa(window, heads):
    Hq, Hkv = heads
    rng = np.random.default_rng(window * 31 + Hq * 7 + Hkv)
    q, k, v, sinks = _case(rng, 2, 33, Hq, Hkv, 16)
    out, lse = ref_fwd(q, k, v, sinks, window, 0.25)
    so, sl = _sdpa_augmented(q, k, v, sinks, window, 0.25)
    np.testing.assert_allclose(out, so, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(lse, sl, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("window", [0, 4])
def test_invariant_neg_inf_sink_is_standard_attention(window):
    rng = np.random.default_rng(11)
    B, S, Hq, D = 1, 30, 2, 8
    q, k, v, _ = _case(rng, B, S, Hq, Hq, D)
    sinks = np.full(Hq, -np.inf)
    out, _ = ref_fwd(q, k, v, sinks, window, 0.35)
    Q, K, V = (torch.from_numpy(x).permute(0, 2, 1, 3) for x in (q, k, v))
    if window == 0:
        ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, is_causal=True, scale=0.35)
    else:
        i, j = torch.arange(S)[:, None], torch.arange(S)[None, :]
        band = (j <= i) & (i - j < window)
        ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, attn_mask=band, scale=0.35)
    np.testing.assert_allclose(out, ref.permute(0, 2, 1, 3).numpy(), rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("window", [0, 3])
def test_invariant_sink_scales_rows(window):
    rng = np.random.default_rng(12)
    q, k, v, sinks = _case(rng, 2, 25, 4, 2, 8)
    o_s, l_s = ref_fwd(q, k, v, sinks, window, 0.4)
    o_n, l_n = ref_fwd(q, k, v, np.full(4, -np.inf), window, 0.4)
    # sum(e) / (sum(e) + e^sink) per row, in terms of the no-sink lse
    sink_b = sinks[None, :, None]
    factor = np.exp(l_n) / (np.exp(l_n) + np.exp(sink_b))       # [B, H, S]
    np.testing.assert_allclose(o_s, o_n * factor.transpose(0, 2, 1)[..., None],
                               rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l_s, np.logaddexp(l_n, sink_b), rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("S", [1, 9, 40])
def test_invariant_window_at_least_S_is_full(S):
    rng = np.random.default_rng(S)
    q, k, v, sinks = _case(rng, 1, S, 4, 1, 8)
    o0, l0 = ref_fwd(q, k, v, sinks, 0, 0.3)
    for w in (S, S + 1, 10 * S):
        o, l = ref_fwd(q, k, v, sinks, w, 0.3)
        np.testing.assert_array_equal(o, o0)
        np.testing.assert_array_equal(l, l0)


def test_gqa_equals_repeated_mha():
    rng = np.random.default_rng(13)
    q, k, v, sinks = _case(rng, 2, 20, 6, 2, 8)
    o, l = ref_fwd(q, k, v, sinks, 5, 0.3)
    kr, vr = np.repeat(k, 3, axis=2), np.repeat(v, 3, axis=2)
    o2, l2 = ref_fwd(q, kr, vr, sinks, 5, 0.3)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(l, l2)


# --------------------------------------------------------------------------
# closed forms

def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def test_closed_form_row0_and_window1():
    rng = np.random.default_rng(14)
    q, k, v, sinks = _case(rng, 2, 17, 4, 2, 8)
    scale = 0.3
    G = 2
    for window in (0, 1):
        out, lse = ref_fwd(q, k, v, sinks, window, scale)
        rows = [0] if window == 0 else range(17)
        for b in range(2):
            for h in range(4):
                for i in rows:
                    s = scale * q[b, i, h] @ k[b, i, h // G]
                    np.testing.assert_allclose(out[b, i, h], _sigmoid(s - sinks[h]) * v[b, i, h // G],
                                               rtol=1e-13, atol=1e-14)
                    np.testing.assert_allclose(lse[b, h, i], np.logaddexp(s, sinks[h]), rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("window", [0, 4])
def test_closed_form_zero_query(window):
    rng = np.random.default_rng(15)
    _, k, v, sinks = _case(rng, 1, 11, 2, 1, 8)
    q = np.zeros((1, 11, 2, 8))
    out, lse = ref_fwd(q, k, v, sinks, window, 0.5)
    for h in range(2):
        for i in range(11):
            lo = 0 if window == 0 else max(0, i - window + 1)
            n = i - lo + 1
            mean_v = v[0, lo:i + 1, 0].mean(axis=0)
            np.testing.assert_allclose(out[0, i, h], n / (n + np.exp(sinks[h])) * mean_v,
                                       rtol=1e-13, atol=1e-14)
            np.testing.assert_allclose(lse[0, h, i], np.log(n + np.exp(sinks[h])), rtol=1e-14, atol=1e-14)


def test_unmasked_pair_counts():
    for S in (1, 5, 128, 300):
        assert unmasked_pairs(S, 0) == S * (S + 1) // 2
        for W in (1, 7, 128):
            if W <= S:
                assert unmasked_pairs(S, W) == W * (W + 1) // 2 + (S - W) * W
            else:
                assert unmasked_pairs(S, W) == S * (S + 1) // 2


# --------------------------------------------------------------------------
# decode

@pytest.mark.parametrize("window", [0, 1, 3, 8])
def test_decode_equals_prefill_last_row(window):
    rng = np.random.default_rng(16 + window)
    Hq, Hkv, D = 4, 2, 8
    lengths = [1, 2, 5, 8, 13]
    cu = np.concatenate([[0], np.cumsum(lengths)])
    T = cu[-1]
    q = rng.standard_normal((len(lengths), Hq, D))
    kc = rng.standard_normal((T, Hkv, D))
    vc = rng.standard_normal((T, Hkv, D))
    sinks = rng.standard_normal(Hq)
    out, lse = ref_decode(q, kc, vc, cu, sinks, window, 0.35)
    for n, L in enumerate(lengths):
        qp = np.zeros((1, L, Hq, D))
        qp[0, L - 1] = q[n]
        kp, vp = kc[cu[n]:cu[n + 1]][None], vc[cu[n]:cu[n + 1]][None]
        o, l = ref_fwd(qp, kp, vp, sinks, window, 0.35, rows=[L - 1])
        np.testing.assert_allclose(out[n], o[0, L - 1], rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(lse[n], l[0, :, L - 1], rtol=1e-13, atol=1e-14)


def test_decode_empty_sequence_sees_only_sink():
    rng = np.random.default_rng(17)
    cu = np.array([0, 0, 3, 3])
    q = rng.standard_normal((3, 2, 4))
    kc = rng.standard_normal((3, 1, 4))
    vc = rng.standard_normal((3, 1, 4))
    sinks = np.array([0.5, -np.inf])
    out, lse = ref_decode(q, kc, vc, cu, sinks, 0, 0.5)
    for n in (0, 2):
        assert (out[n] == 0).all()
        np.testing.assert_array_equal(lse[n], sinks)
    assert np.isfinite(out[1]).all()


# --------------------------------------------------------------------------
# backward: finite differences on every element

def _loss(q, k, v, sinks, dout, window, scale):
    out, _ = ref_fwd(q, k, v, sinks, window, scale)
    return float(np.sum(out * dout))


@pytest.mark.parametrize("window", [0, 2])
def test_bwd_finite_differences(window):
    rng = np.random.default_rng(18 + window)
    B, S, Hq, Hkv, D = 2, 5, 4, 2, 3
    q, k, v, sinks = _case(rng, B, S, Hq, Hkv, D)
    dout = rng.standard_normal((B, S, Hq, D))
    scale = 0.45
    dq, dk, dv, ds = ref_bwd(q, k, v, sinks, dout, window, scale)
    args = [q, k, v, sinks]
    h = 1e-6
    for idx, grad in enumerate((dq, dk, dv, ds)):
        x = args[idx]
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            mi = it.multi_index
            old = x[mi]
            x[mi] = old + h
            lp = _loss(*args, dout, window, scale)
            x[mi] = old - h
            lm = _loss(*args, dout, window, scale)
            x[mi] = old
            num[mi] = (lp - lm) / (2 * h)
        rel = np.linalg.norm(num - grad) / np.linalg.norm(grad)
        assert rel <= 1e-6, (idx, rel)


def test_bwd_head_and_batch_subsets():
    rng = np.random.default_rng(19)
    q, k, v, sinks = _case(rng, 2, 9, 4, 2, 4)
    dout = rng.standard_normal(q.shape)
    dq, dk, dv, ds = ref_bwd(q, k, v, sinks, dout, 3, 0.5)
    dq2, dk2, dv2, ds2 = ref_bwd(q, k, v, sinks, dout, 3, 0.5, heads=[2, 3], batches=[0, 1])
    np.testing.assert_array_equal(dq2[:, :, 2:], dq[:, :, 2:])
    np.testing.assert_array_equal(dk2[:, :, 1], dk[:, :, 1])
    np.testing.assert_array_equal(dv2[:, :, 1], dv[:, :, 1])
    np.testing.assert_array_equal(ds2[2:], ds[2:])
    assert (dq2[:, :, :2] == 0).all() and (dk2[:, :, 0] == 0).all()
