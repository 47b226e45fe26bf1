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

__all__ = ["brute_fwd", "brute_fwd_docs", "brute_rope"]


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


def brute_fwd_docs(q, k, v, doc_of_row, sinks, window, scale):
    """Packed documents as one block-diagonal mask over the token rows.

    q [T][Hq][D], k/v [T][Hkv][D] nested floats; doc_of_row[t] is the document
    id of row t (None for a row in no document).  Key row j is visible from
    query row i when both carry the same document id, j <= i and, for a
    window W >= 1, i - j < W.  (Megatron-LM issue "gpt-oss implementation",
    discussion thread: attention confined to each document of a packed
    sequence.)  Returns (out [T][Hq][D], lse [Hq][T]) with None for rows in no
    document.
    """
    T, Hq, D = len(q), len(q[0]), len(q[0][0])
    Hkv = len(k[0])
    G = Hq // Hkv
    out = [[None] * Hq for _ in range(T)]
    lse = [[None] * T for _ in range(Hq)]
    for i in range(T):
        if doc_of_row[i] is None:
            continue
        for h in range(Hq):
            c = h // G
            weights = []
            for j in range(T):
                if doc_of_row[j] != doc_of_row[i] or j > i:
                    continue
                if window > 0 and i - j >= window:
                    continue
                dot = math.fsum(q[i][h][d] * k[j][c][d] for d in range(D))
                weights.append((j, math.exp(scale * dot)))
            sink = float(sinks[h])
            sink_w = 0.0 if sink == -math.inf else math.exp(sink)
            Z = math.fsum([w for _, w in weights] + [sink_w])
            out[i][h] = [math.fsum(w * v[j][c][d] for j, w in weights) / Z for d in range(D)]
            lse[h][i] = math.log(Z)
    return out, lse


def brute_rope(x, position, freqs, mscale):
    """Rotary embedding of one vector x (length D, nested floats) as complex
    multiplication: z_i = (x_i + 1j x_{i+D/2}) * mscale * exp(1j position f_i),
    y_i = Re z_i, y_{i+D/2} = Im z_i (the half-split pairing).  A restatement
    of the rotation in oracle/rope.py by a different route, for pins."""
    import cmath
    half = len(x) // 2
    out = [0.0] * len(x)
    for i in range(half):
        z = complex(x[i], x[i + half]) * mscale * cmath.exp(1j * position * freqs[i])
        out[i], out[i + half] = z.real, z.imag
    return out
