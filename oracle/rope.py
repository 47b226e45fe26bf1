"""Rotary position embedding with YaRN frequency scaling, for the oracle.
TEST INFRASTRUCTURE ONLY (imported by tests/, __graft_entry__.smoke() and
bench.py's cpu_baseline leg; the HIP library never imports it).

Megatron-LM issue "gpt-oss implementation", section "Positional Encodings /
YaRN RoPE Scaling", names YaRN scaling of rotary embeddings (to 128k+
context) and cites the YaRN paper, arXiv:2309.00071; the pages give no
formula and no parameters.  The reading used here restates the paper:

* base frequencies theta_i = base^(-2 i / D), i = 0 .. D/2 - 1;
* wavelength lambda_i = 2 pi / theta_i and r_i = L / lambda_i, the number of
  turns of pair i over the original context length L;
* ramp gamma(r) = 0 for r < alpha, 1 for r > beta, (r - alpha) / (beta -
  alpha) between; the scaled frequency is
  h_i = (1 - gamma(r_i)) theta_i / s + gamma(r_i) theta_i  (s = the factor);
* the attention temperature sqrt(1/t) = 0.1 ln(s) + 1 multiplies both q and k
  (so it is folded into cos and sin); s = 1 is plain RoPE.
* pairing (the pages do not fix it): element i is rotated with element
  i + D/2 ("half-split"), the angle of position p being p h_i:
  y_i = x_i cos - x_{i+D/2} sin,  y_{i+D/2} = x_{i+D/2} cos + x_i sin.
* precision (a reading: the attention consumes bf16 q and k, as any bf16
  pipeline that applies RoPE before attention does): the table holds
  fp32(m cos(p h_i)) and fp32(m sin(p h_i)) computed in fp64; a rotated
  element is the exact value x_i c - x_j s (resp. x_j c + x_i s) of those
  fp32 entries and the bf16 inputs, rounded once to bf16 (nearest, ties to
  even) -- the plain definition of "the rotation, in bf16".  The products
  are exact in fp64 (8 x 24 significant bits); the sum is carried as an
  unevaluated fp64 pair (Knuth's two-sum) so that the one rounding sees the
  exact value.  The fp64 rotation without the final rounding
  (`apply_rope_exact`) is kept for the pins.
"""

import math

import numpy as np

__all__ = ["yarn_inv_freq", "yarn_mscale", "rope_table", "apply_rope_exact", "apply_rope_bf16", "round_bf16",
           "apply_rope_adjoint", "ref_fwd_rope", "ref_decode_rope", "ref_bwd_rope"]


def yarn_inv_freq(D, base, factor, orig_ctx, alpha, beta):
    """Scaled frequencies h_i (fp64, length D/2)."""
    i = np.arange(D // 2, dtype=np.float64)
    theta = base ** (-2.0 * i / D)
    if factor == 1.0:
        return theta
    r = orig_ctx * theta / (2.0 * math.pi)
    gamma = np.clip((r - alpha) / (beta - alpha), 0.0, 1.0)
    return (1.0 - gamma) * theta / factor + gamma * theta


def yarn_mscale(factor):
    return 1.0 if factor <= 1.0 else 0.1 * math.log(factor) + 1.0


def rope_table(P, D, base, factor, orig_ctx, alpha, beta, dtype=np.float32):
    """(cos, sin) tables [P, D/2] of m cos(p h_i), m sin(p h_i), computed in
    fp64 and rounded to `dtype` (fp32 by default; fp64 for exact pins)."""
    h = yarn_inv_freq(D, base, factor, orig_ctx, alpha, beta)
    ang = np.arange(P, dtype=np.float64)[:, None] * h[None, :]
    m = yarn_mscale(factor)
    return (m * np.cos(ang)).astype(dtype), (m * np.sin(ang)).astype(dtype)


def apply_rope_exact(x, positions, cos, sin):
    """fp64 rotation of x [..., T, H, D] (positions [T]) with fp64 tables."""
    half = x.shape[-1] // 2
    c = cos[positions][:, None, :]
    s = sin[positions][:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def apply_rope_adjoint(g, positions, cos, sin):
    """The adjoint R^T of the rotation (fp64): carries a gradient with
    respect to rotated rows back to the unrotated ones."""
    half = g.shape[-1] // 2
    c = cos[positions][:, None, :]
    s = sin[positions][:, None, :]
    g1, g2 = g[..., :half], g[..., half:]
    return np.concatenate([g1 * c + g2 * s, g2 * c - g1 * s], axis=-1)


def _two_sum(a, b):
    """Knuth's error-free sum: a + b == s + e exactly, s = fl(a + b)."""
    s = a + b
    bb = s - a
    e = (a - (s - bb)) + (b - bb)
    return s, e


def round_bf16(hi, lo=None):
    """Round the exact value hi + lo (an unevaluated fp64 pair, |lo| at most
    half an fp64 ulp of hi; lo = 0 when omitted) to the nearest bf16 (8
    significant bits), ties to even; returns fp64.  Only hi can sit exactly
    on a midpoint between two bf16 numbers (a midpoint strictly between
    hi + lo and hi would be closer to hi + lo than hi is); there the sign of
    lo decides.  Values must be 0 or of magnitude >= 2^-126 (bf16 normals)
    and below the bf16 overflow threshold."""
    hi = np.asarray(hi, dtype=np.float64)
    lo = np.zeros_like(hi) if lo is None else np.asarray(lo, dtype=np.float64)
    a = np.abs(hi[hi != 0])
    if a.size and (a.min() < 2.0 ** -126 or a.max() >= 2.0 ** 128 * (1 - 2.0 ** -9)):
        raise ValueError("round_bf16: value outside the bf16 normal range")
    m, e = np.frexp(hi)                 # hi = m 2^e, 0.5 <= |m| < 1
    t = np.ldexp(m, 8)                  # 8 significant bits above the point
    r = np.rint(t)                      # nearest, ties to even
    mid = (t - np.floor(t)) == 0.5
    r = np.where(mid & (lo > 0), np.ceil(t), r)
    r = np.where(mid & (lo < 0), np.floor(t), r)
    return np.ldexp(r, e - 8)


def apply_rope_bf16(x, positions, cos32, sin32):
    """The rotation in bf16 (see the header): the exact value of the
    rotation of x (bf16 values, any float dtype) with the fp32 table entries
    cos32/sin32, rounded once to bf16, nearest even."""
    half = x.shape[-1] // 2
    xd = np.asarray(x, dtype=np.float64)
    c = np.asarray(cos32[positions], dtype=np.float64)[:, None, :]
    s = np.asarray(sin32[positions], dtype=np.float64)[:, None, :]
    x1, x2 = xd[..., :half], xd[..., half:]
    y1 = round_bf16(*_two_sum(x1 * c, -(x2 * s)))
    y2 = round_bf16(*_two_sum(x2 * c, x1 * s))
    return np.concatenate([y1, y2], axis=-1)


def ref_fwd_rope(q, k, v, sinks, window, scale, cos32, sin32, **kw):
    """Prefill with RoPE on q and k at positions 0..S-1 of each batch:
    returns (out, lse, k_rot) where k_rot is the rotated, bf16-rounded k
    [B, S, Hkv, D] and out/lse are ref_fwd over the rotated q and k."""
    from .attn import ref_fwd
    S = q.shape[1]
    pos = np.arange(S)
    qr = np.stack([apply_rope_bf16(q[b], pos, cos32, sin32) for b in range(q.shape[0])])
    kr = np.stack([apply_rope_bf16(k[b], pos, cos32, sin32) for b in range(k.shape[0])])
    out, lse = ref_fwd(qr, kr, v, sinks, window, scale, **kw)
    return out, lse, kr


def ref_decode_rope(q, k_cache, v_cache, cu_seqlens, sinks, window, scale, cos32, sin32):
    """Decode with the query rotated at its position L_n - 1 (the cache holds
    rotated keys); an empty sequence sees only the sink."""
    from .attn import ref_decode
    L = np.diff(np.asarray(cu_seqlens))
    pos = np.maximum(L - 1, 0)
    qr = apply_rope_bf16(q, pos, cos32, sin32) if q.shape[0] else q
    return ref_decode(qr, k_cache, v_cache, cu_seqlens, sinks, window, scale)


def ref_bwd_rope(q, k, v, sinks, dout, window, scale, cos, sin, exact=False, **kw):
    """Backward of sum(dout * out) for prefill with RoPE on q and k, with
    respect to the unrotated q and k: the rotated q, k enter ref_bwd and
    dq, dk come back through the adjoint.  exact=False follows the bf16 path
    (rotated q, k rounded as in ref_fwd_rope; cos/sin the fp32 tables; the
    rounding's derivative taken as 1); exact=True rotates in fp64 (cos/sin
    fp64 tables), the plain derivative for finite-difference pins."""
    from .attn import ref_bwd
    S = q.shape[1]
    pos = np.arange(S)
    if exact:
        rot = lambda x: apply_rope_exact(x, pos, cos, sin)
    else:
        rot = lambda x: apply_rope_bf16(x, pos, cos, sin)
    qr = np.stack([rot(q[b]) for b in range(q.shape[0])])
    kr = np.stack([rot(k[b]) for b in range(k.shape[0])])
    dqr, dkr, dv, ds = ref_bwd(qr, kr, v, sinks, dout, window, scale, **kw)
    c64, s64 = cos.astype(np.float64), sin.astype(np.float64)
    dq = np.stack([apply_rope_adjoint(dqr[b], pos, c64, s64) for b in range(q.shape[0])])
    dk = np.stack([apply_rope_adjoint(dkr[b], pos, c64, s64) for b in range(k.shape[0])])
    return dq, dk, dv, ds
