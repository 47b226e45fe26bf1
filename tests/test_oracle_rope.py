"""Pins of the RoPE / YaRN oracle (oracle/rope.py), CPU only.

* the rotation against a scalar complex-multiplication restatement
  (oracle/brute.py, brute_rope) for random vectors, positions and YaRN
  settings
* YaRN's two limits reduce to textbook cases: every pair interpolated
  (all turns below alpha) is position interpolation, the rotation at position
  p equals plain RoPE at position p / s; every pair extrapolated (all turns
  above beta) is plain RoPE; s = 1 is plain RoPE with temperature 1
* hand values of the ramp on a two-pair head (D = 4)
* norm: each pair's length is multiplied by the temperature; position 0 is
  the temperature times the identity
* relative position: <R(p) q, R(p') k> depends only on p - p'
* the bf16 rotation is the exact rational value rounded once to bf16
  (checked element by element by integer arithmetic), including a hand case
  where two fp32 roundings would land on the other side of a bf16 midpoint;
  the rounding's ties and its two-term input on hand values
* the temperature m = 0.1 ln(s) + 1 at s = e and s = e^10 (1.1 and 2.0)
* attention with the identity table is attention without RoPE; decode with
  RoPE is the last row of prefill with RoPE
* backward: the adjoint satisfies <R x, y> = <x, R^T y>; gradients with
  respect to the unrotated q and k (and v, sinks) against central finite
  differences of the fp64 loss through the rotation
"""

import math
from fractions import Fraction

import numpy as np
import pytest

from oracle import (apply_rope_adjoint, apply_rope_bf16, apply_rope_exact, brute_rope, ref_bwd_rope, ref_decode,
                    ref_decode_rope, ref_fwd, ref_fwd_rope, rope_table, round_bf16, yarn_inv_freq, yarn_mscale)

GPTOSS_LIKE = dict(base=150000.0, factor=32.0, orig_ctx=4096, alpha=1.0, beta=32.0)


def _bf16(a):
    import torch
    return torch.tensor(a, dtype=torch.float32).to(torch.bfloat16).to(torch.float64).numpy()


@pytest.mark.parametrize("params", [GPTOSS_LIKE, dict(base=10000.0, factor=1.0, orig_ctx=2048, alpha=1.0, beta=32.0),
                                    dict(base=500000.0, factor=8.0, orig_ctx=8192, alpha=2.0, beta=16.0)])
def test_rotation_matches_complex_brute_force(params):
    rng = np.random.default_rng(3)
    D, P = 64, 300
    cos, sin = rope_table(P, D, dtype=np.float64, **params)
    freqs = yarn_inv_freq(D, **params)
    m = yarn_mscale(params["factor"])
    x = rng.standard_normal((5, 2, D))
    pos = np.array([0, 1, 17, 255, 299])
    y = apply_rope_exact(x, pos, cos, sin)
    for t in range(5):
        for h in range(2):
            ref = brute_rope(x[t, h].tolist(), int(pos[t]), freqs.tolist(), m)
            np.testing.assert_allclose(y[t, h], ref, rtol=1e-12, atol=1e-12)


def test_all_interpolated_is_position_interpolation():
    # alpha, beta above every pair's turn count: h_i = theta_i / s
    D, s = 64, 8.0
    h = yarn_inv_freq(D, 10000.0, s, 4096, 1e9, 2e9)
    theta = 10000.0 ** (-np.arange(32) * 2.0 / 64)
    np.testing.assert_allclose(h, theta / s, rtol=1e-15)
    rng = np.random.default_rng(4)
    x = rng.standard_normal(D)
    p = 1000
    ref = brute_rope(x.tolist(), p / s, theta.tolist(), yarn_mscale(s))  # plain RoPE at p / s
    cos, sin = rope_table(p + 1, D, 10000.0, s, 4096, 1e9, 2e9, dtype=np.float64)
    y = apply_rope_exact(x[None, None], np.array([p]), cos, sin)[0, 0]
    np.testing.assert_allclose(y, ref, rtol=1e-10, atol=1e-12)


def test_all_extrapolated_is_plain_rope():
    # alpha, beta below every pair's turn count: h_i = theta_i
    h = yarn_inv_freq(64, 10000.0, 8.0, 4096, 1e-9, 2e-9)
    np.testing.assert_allclose(h, 10000.0 ** (-np.arange(32) * 2.0 / 64), rtol=1e-15)
    assert yarn_inv_freq(64, 10000.0, 1.0, 4096, 1.0, 32.0).tolist() == \
        (10000.0 ** (-np.arange(32) * 2.0 / 64)).tolist()
    assert yarn_mscale(1.0) == 1.0
    assert abs(yarn_mscale(32.0) - (1 + 0.1 * math.log(32))) < 1e-15


def test_ramp_hand_values():
    # D = 4: theta = (1, base^-1/2) with base = (200 pi)^2, so theta_1 =
    # 1 / (200 pi); over L = 100 tokens the pairs turn L theta / (2 pi) =
    # 100 / (2 pi) ~ 15.92 and 1 / (4 pi^2) ~ 0.025 times
    base = (2 * math.pi * 100) ** 2
    L = 100
    th = np.array([1.0, 1.0 / (200 * math.pi)])
    h = yarn_inv_freq(4, base, 4.0, L, 1.0, 32.0)
    # pair 0: r = 15.92 inside [1, 32]: gamma = (15.92 - 1) / 31
    g0 = (L / (2 * math.pi) - 1.0) / 31.0
    assert abs(h[0] - ((1 - g0) * 1.0 / 4.0 + g0 * 1.0)) < 1e-15
    # pair 1: r = 1 / (4 pi^2) < 1: fully interpolated
    assert abs(h[1] - th[1] / 4.0) < 1e-18


def test_norm_and_position_zero():
    rng = np.random.default_rng(5)
    cos, sin = rope_table(50, 64, dtype=np.float64, **GPTOSS_LIKE)
    m = yarn_mscale(GPTOSS_LIKE["factor"])
    x = rng.standard_normal((50, 3, 64))
    y = apply_rope_exact(x, np.arange(50), cos, sin)
    pair = lambda a: np.hypot(a[..., :32], a[..., 32:])
    np.testing.assert_allclose(pair(y), m * pair(x), rtol=1e-13)
    np.testing.assert_allclose(y[0], m * x[0], rtol=1e-15)


def test_relative_position():
    rng = np.random.default_rng(6)
    cos, sin = rope_table(400, 64, dtype=np.float64, **GPTOSS_LIKE)
    q = rng.standard_normal((1, 1, 64))
    k = rng.standard_normal((1, 1, 64))
    for p, pk, t in ((10, 3, 100), (200, 200, 37), (5, 90, 250)):
        a = apply_rope_exact(q, np.array([p]), cos, sin)[0, 0] @ apply_rope_exact(k, np.array([pk]), cos, sin)[0, 0]
        b = (apply_rope_exact(q, np.array([p + t]), cos, sin)[0, 0]
             @ apply_rope_exact(k, np.array([pk + t]), cos, sin)[0, 0])
        assert abs(a - b) <= 1e-10 * max(1.0, abs(a))


def _exact_bf16(fr):
    """Nearest bf16 (ties to even) of an exact rational, by integer
    arithmetic on the rational itself (no floating point on the value)."""
    if fr == 0:
        return 0.0
    sign, a = (1 if fr > 0 else -1), abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    ulp = Fraction(2) ** (e - 7)  # 8 significant bits
    n, rem = divmod(a, ulp)
    n = int(n)
    if rem * 2 > ulp or (rem * 2 == ulp and n % 2 == 1):
        n += 1
    return sign * float(n * ulp)


def test_bf16_rotation_is_the_exact_value_rounded_once():
    """Every element against the exact rational value of the rotation with
    the fp32 table entries, rounded to bf16 by integer arithmetic."""
    rng = np.random.default_rng(7)
    c32, s32 = rope_table(4096, 64, **GPTOSS_LIKE)
    x = _bf16(rng.standard_normal((40, 2, 64)))
    pos = rng.integers(0, 4096, 40)
    y = apply_rope_bf16(x, pos, c32, s32)
    for t in range(40):
        for h in range(2):
            for i in range(32):
                c, s = Fraction(float(c32[pos[t], i])), Fraction(float(s32[pos[t], i]))
                a, b = Fraction(float(x[t, h, i])), Fraction(float(x[t, h, i + 32]))
                assert y[t, h, i] == _exact_bf16(a * c - b * s)
                assert y[t, h, i + 32] == _exact_bf16(b * c + a * s)
    # and so within half a bf16 ulp of the fp64 rotation (no second rounding)
    ex = apply_rope_exact(x, pos, c32.astype(np.float64), s32.astype(np.float64))
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(y), 1e-30))) - 7)
    assert (np.abs(y - ex) <= 0.5 * ulp * (1 + 1e-12)).all()
    # a unit pair (1, 0) rotates to (c, s) rounded once to bf16
    e = np.zeros((1, 1, 64))
    e[0, 0, 5] = 1.0
    y = apply_rope_bf16(e, np.array([77]), c32, s32)
    assert y[0, 0, 5] == _bf16(c32[77, 5]) and y[0, 0, 37] == _bf16(s32[77, 5])


def test_bf16_rotation_where_two_fp32_roundings_would_differ():
    """x_i = 0x1.66p-6, x_(i+32) = -0x1.4ap+0, c = 0x1.58b9p+0,
    s = 0x1.670b4cp-10: the exact value x_i c - x_(i+32) s lies just below the
    bf16 midpoint 0x1.ffp-6, so it rounds to 0x1.fep-6; rounding x_i c to fp32
    first carries it past the midpoint (to 0x1.00p-5).  The oracle must give
    the single rounding."""
    x1, x2 = float.fromhex("0x1.66p-6"), float.fromhex("-0x1.4ap+0")
    c, s = float.fromhex("0x1.58b9p+0"), float.fromhex("0x1.670b4cp-10")
    exact = Fraction(x1) * Fraction(c) - Fraction(x2) * Fraction(s)
    mid = Fraction(float.fromhex("0x1.ffp-6"))
    assert exact < mid and mid - exact < Fraction(1, 2 ** 29)
    x = np.zeros((1, 1, 64))
    x[0, 0, 0], x[0, 0, 32] = x1, x2
    c32 = np.ones((1, 32), np.float32)
    s32 = np.zeros((1, 32), np.float32)
    c32[0, 0], s32[0, 0] = c, s
    y = apply_rope_bf16(x, np.array([0]), c32, s32)
    assert y[0, 0, 0] == float.fromhex("0x1.fep-6")
    assert float(np.float32(np.float32(x1 * c) - np.float32(x2 * s))) >= float(mid)


def test_round_bf16_ties_and_pairs():
    one, step = 1.0, 2.0 ** -7            # bf16 neighbours 1 and 1 + 2^-7
    midpoint = one + step / 2
    assert round_bf16(np.array([midpoint]))[0] == one                    # tie: even (1.0000000)
    assert round_bf16(np.array([midpoint + step]))[0] == one + 2 * step  # tie: even (1.0000010)
    assert round_bf16(np.array([midpoint]), np.array([2.0 ** -60]))[0] == one + step   # just above
    assert round_bf16(np.array([midpoint]), np.array([-2.0 ** -60]))[0] == one         # just below
    assert round_bf16(np.array([-midpoint]), np.array([-2.0 ** -60]))[0] == -(one + step)
    assert round_bf16(np.array([-midpoint]), np.array([2.0 ** -60]))[0] == -one
    assert round_bf16(np.array([0.0, 3.0, 255.0, 511.0])).tolist() == [0.0, 3.0, 255.0, 512.0]  # 8 bits exact; 9 bits a tie
    assert round_bf16(np.array([257.0]))[0] == 256.0                     # 257 = 256 + half a step: even
    assert round_bf16(np.array([259.0]))[0] == 260.0
    with pytest.raises(ValueError):
        round_bf16(np.array([1e-40]))


def test_yarn_mscale_hand_values():
    """The temperature 0.1 ln(s) + 1 at points where the logarithm is known
    exactly: s = e gives 1.1, s = e^10 gives 2.0; no scaling (s <= 1) gives 1."""
    assert abs(yarn_mscale(math.e) - 1.1) < 1e-15
    assert abs(yarn_mscale(math.exp(10.0)) - 2.0) < 1e-15
    assert yarn_mscale(0.5) == 1.0
    assert yarn_mscale(1.0) == 1.0
    assert abs(yarn_mscale(32.0) - 1.3465735902799727) < 1e-15   # 0.1 * 5 ln 2 + 1


def test_identity_table_is_attention_without_rope():
    rng = np.random.default_rng(8)
    q = _bf16(rng.standard_normal((2, 40, 4, 64)))
    k = _bf16(rng.standard_normal((2, 40, 2, 64)))
    v = _bf16(rng.standard_normal((2, 40, 2, 64)))
    sinks = rng.standard_normal(4)
    one = np.ones((40, 32), np.float32)
    zero = np.zeros((40, 32), np.float32)
    out, lse, kr = ref_fwd_rope(q, k, v, sinks, 7, 0.125, one, zero)
    o2, l2 = ref_fwd(q, k, v, sinks, 7, 0.125)
    np.testing.assert_array_equal(out, o2)
    np.testing.assert_array_equal(lse, l2)
    np.testing.assert_array_equal(kr, k)


@pytest.mark.parametrize("window", [0, 5])
def test_decode_with_rope_is_last_prefill_row(window):
    rng = np.random.default_rng(9 + window)
    c32, s32 = rope_table(64, 64, **GPTOSS_LIKE)
    lens = [1, 9, 23]
    for L in lens:
        q = _bf16(rng.standard_normal((1, L, 8, 64)))
        k = _bf16(rng.standard_normal((1, L, 1, 64)))
        v = _bf16(rng.standard_normal((1, L, 1, 64)))
        sinks = rng.standard_normal(8)
        out, lse, kr = ref_fwd_rope(q, k, v, sinks, window, 0.125, c32, s32)
        o, l = ref_decode_rope(q[0, L - 1:L], kr[0], v[0], np.array([0, L]), sinks, window, 0.125, c32, s32)
        np.testing.assert_allclose(o[0], out[0, L - 1], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(l[0], lse[0, :, L - 1], rtol=1e-12, atol=1e-13)


def test_adjoint_identity():
    rng = np.random.default_rng(20)
    cos, sin = rope_table(30, 64, dtype=np.float64, **GPTOSS_LIKE)
    pos = rng.integers(0, 30, 12)
    x = rng.standard_normal((12, 3, 64))
    y = rng.standard_normal((12, 3, 64))
    a = np.sum(apply_rope_exact(x, pos, cos, sin) * y)
    b = np.sum(x * apply_rope_adjoint(y, pos, cos, sin))
    assert abs(a - b) <= 1e-12 * max(1.0, abs(a))


@pytest.mark.parametrize("window", [0, 2])
def test_bwd_rope_finite_differences(window):
    rng = np.random.default_rng(21 + window)
    B, S, Hq, Hkv, D = 1, 5, 2, 1, 8
    params = dict(base=100.0, factor=4.0, orig_ctx=6, alpha=0.5, beta=3.0)
    cos, sin = rope_table(S, D, dtype=np.float64, **params)
    q = rng.standard_normal((B, S, Hq, D)) * 0.7
    k = rng.standard_normal((B, S, Hkv, D)) * 0.7
    v = rng.standard_normal((B, S, Hkv, D))
    sinks = rng.standard_normal(Hq)
    dout = rng.standard_normal((B, S, Hq, D))
    scale = 0.4
    pos = np.arange(S)

    def loss(q_, k_, v_, s_):
        qr = np.stack([apply_rope_exact(q_[b], pos, cos, sin) for b in range(B)])
        kr = np.stack([apply_rope_exact(k_[b], pos, cos, sin) for b in range(B)])
        out, _ = ref_fwd(qr, kr, v_, s_, window, scale)
        return float(np.sum(out * dout))

    grads = ref_bwd_rope(q, k, v, sinks, dout, window, scale, cos, sin, exact=True)
    args = [q, k, v, sinks]
    h = 1e-6
    for idx, grad in enumerate(grads):
        x = args[idx]
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            mi = it.multi_index
            old = x[mi]
            x[mi] = old + h
            lp = loss(*args)
            x[mi] = old - h
            lm = loss(*args)
            x[mi] = old
            num[mi] = (lp - lm) / (2 * h)
        rel = np.linalg.norm(num - grad) / np.linalg.norm(grad)
        assert rel <= 1e-6, (idx, rel)
