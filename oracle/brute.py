"""Scalar brute force of sink attention.  TEST INFRASTRUCTURE ONLY.

An independent, deliberately naive restatement of the forward definition in
``oracle/attn.py`` (pure Python loops, ``math.exp``/``math.fsum``, no numpy
arithmetic, no max subtraction), for tiny shapes only.  It exists to pin the
vectorised oracle: a dropped term, a wrong sign or a transposed operand in one
of the two shows up as a mismatch.

Sinks: Megatron-LM issue "gpt-oss implementation", "Attention Sinks"; sliding
window: same issue, "Alternating Sliding-Window Attention Pattern".
"""

import math

__all__ = ["brute_fwd"]


def brute_fwd(q, k, v, sinks, window, scale):
    """q [B][S][Hq][D], k/v [B][S][Hkv][D] nested sequences of floats.

    Returns (out as nested lists [B][S][Hq][D], lse as nested lists [B][Hq][S]).
    Scores are exponentiated directly (inputs must be small enough not to
    overflow), which is a different route from the oracle's max-shifted one.
    """
    B, S, Hq, D = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    Hkv = len(k[0][0])
    G = Hq // Hkv
    out = [[[[0.0] * D for _ in range(Hq)] for _ in range(S)] for _ in range(B)]
    lse = [[[0.0] * S for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        for h in range(Hq):
            c = h // G
            sink = float(sinks[h])
            for i in range(S):
                weights = []
                for j in range(S):
                    if j > i:
                        continue
                    if window > 0 and i - j >= window:
                        continue
                    dot = math.fsum(q[b][i][h][d] * k[b][j][c][d] for d in range(D))
                    weights.append((j, math.exp(scale * dot)))
                sink_w = 0.0 if sink == -math.inf else math.exp(sink)
                Z = math.fsum([w for _, w in weights] + [sink_w])
                for d in range(D):
                    out[b][i][h][d] = math.fsum(w * v[b][j][c][d] for j, w in weights) / Z
                lse[b][h][i] = math.log(Z)
    return out, lse
