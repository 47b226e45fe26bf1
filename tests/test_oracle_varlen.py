"""Pins of the packed-document oracle (ref_fwd_varlen / ref_bwd_varlen), CPU only.

The reading pinned here (Megatron-LM issue "gpt-oss implementation",
discussion thread on intra-document masking): documents packed along the
token dimension, attention confined to each document, positions restarting at
0 in each, the sink joining every row.

* a scalar brute force that states the same thing differently: one
  block-diagonal causal/window mask over all token rows from per-row document
  ids (oracle/brute.py, brute_fwd_docs), including empty documents and rows
  that belong to no document
* closed form: the first row of every document sees only its own key, so
  out = sigmoid(s - sink) v and lse = log(e^s + e^sink)
* documents of equal length are a dense batch (lse [Hq, T] against [B, Hq, S])
* editing one document leaves every other document's outputs bit-identical
* backward: central finite differences of the brute-force loss on every input
  element, the sinks included; rows outside every document get no gradient
"""

import math

import numpy as np
import pytest

from oracle import brute_fwd_docs, ref_bwd_varlen, ref_fwd, ref_fwd_varlen


def _case(rng, lengths, Hq, Hkv, D, lead=0, tail=0, std=1.0):
    cu = [lead]
    for L in lengths:
        cu.append(cu[-1] + L)
    T = cu[-1] + tail
    q = rng.standard_normal((T, Hq, D)) * std
    k = rng.standard_normal((T, Hkv, D)) * std
    v = rng.standard_normal((T, Hkv, D))
    sinks = rng.standard_normal(Hq)
    return q, k, v, sinks, np.array(cu)


def _doc_ids(cu, T):
    ids = [None] * T
    for b in range(len(cu) - 1):
        for t in range(int(cu[b]), int(cu[b + 1])):
            ids[t] = b
    return ids


LAYOUTS = [
    dict(lengths=[5], lead=0, tail=0),
    dict(lengths=[3, 1, 4], lead=0, tail=0),
    dict(lengths=[2, 0, 6, 0], lead=0, tail=0),
    dict(lengths=[4, 3], lead=2, tail=3),
    dict(lengths=[0, 0], lead=1, tail=1),
    dict(lengths=[1, 1, 1, 7], lead=0, tail=1),
]


@pytest.mark.parametrize("layout", LAYOUTS, ids=lambda l: f"{l['lengths']}-{l['lead']}-{l['tail']}")
@pytest.mark.parametrize("window", [0, 1, 2, 5])
@pytest.mark.parametrize("heads", [(2, 1), (4, 2)])
def test_matches_block_diagonal_brute_force(layout, window, heads):
    rng = np.random.default_rng(len(layout["lengths"]) * 31 + window * 7 + heads[0])
    Hq, Hkv = heads
    q, k, v, sinks, cu = _case(rng, layout["lengths"], Hq, Hkv, 3, layout["lead"], layout["tail"])
    if window == 2:
        sinks[0] = -math.inf  # a head without a sink
    scale = 0.6
    out, lse = ref_fwd_varlen(q, k, v, cu, sinks, window, scale)
    ids = _doc_ids(cu, q.shape[0])
    bout, blse = brute_fwd_docs(q.tolist(), k.tolist(), v.tolist(), ids, sinks.tolist(), window, scale)
    for t in range(q.shape[0]):
        for h in range(Hq):
            if ids[t] is None:
                assert np.isnan(out[t, h]).all() and np.isnan(lse[h, t])
                assert bout[t][h] is None and blse[h][t] is None
            else:
                np.testing.assert_allclose(out[t, h], bout[t][h], rtol=1e-12, atol=1e-12)
                assert abs(lse[h, t] - blse[h][t]) <= 1e-12


def test_first_row_of_each_document_closed_form():
    rng = np.random.default_rng(5)
    q, k, v, sinks, cu = _case(rng, [3, 5, 1, 4], 4, 2, 6, lead=1, tail=2)
    scale = 0.3
    out, lse = ref_fwd_varlen(q, k, v, cu, sinks, 0, scale)
    for b in range(len(cu) - 1):
        a = int(cu[b])
        for h in range(4):
            c = h // 2
            s = scale * float(q[a, h] @ k[a, c])
            w = 1.0 / (1.0 + math.exp(sinks[h] - s))
            np.testing.assert_allclose(out[a, h], w * v[a, c], rtol=1e-13, atol=1e-14)
            assert abs(lse[h, a] - math.log(math.exp(s) + math.exp(sinks[h]))) <= 1e-13


@pytest.mark.parametrize("window", [0, 3])
def test_equal_lengths_are_a_dense_batch(window):
    rng = np.random.default_rng(11 + window)
    N, S, Hq, Hkv, D = 3, 7, 4, 2, 5
    q, k, v, sinks, cu = _case(rng, [S] * N, Hq, Hkv, D)
    out, lse = ref_fwd_varlen(q, k, v, cu, sinks, window, 0.4)
    dout_, dlse = ref_fwd(q.reshape(N, S, Hq, D), k.reshape(N, S, Hkv, D), v.reshape(N, S, Hkv, D), sinks,
                          window, 0.4)
    np.testing.assert_array_equal(out, dout_.reshape(N * S, Hq, D))
    np.testing.assert_array_equal(lse, dlse.transpose(1, 0, 2).reshape(Hq, N * S))


def test_documents_are_independent():
    rng = np.random.default_rng(12)
    q, k, v, sinks, cu = _case(rng, [4, 6, 3], 4, 1, 4)
    out, lse = ref_fwd_varlen(q, k, v, cu, sinks, 0, 0.5)
    a, e = int(cu[1]), int(cu[2])
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    q2[a:e] += 1.0
    k2[a:e] *= -2.0
    v2[a:e] += 3.0
    out2, lse2 = ref_fwd_varlen(q2, k2, v2, cu, sinks, 0, 0.5)
    keep = np.r_[0:a, e:q.shape[0]]
    np.testing.assert_array_equal(out2[keep], out[keep])
    np.testing.assert_array_equal(lse2[:, keep], lse[:, keep])
    assert not np.allclose(out2[a:e], out[a:e])


def _brute_loss(q, k, v, sinks, dout, ids, window, scale):
    out, _ = brute_fwd_docs(q.tolist(), k.tolist(), v.tolist(), ids, sinks.tolist(), window, scale)
    tot = []
    for t, row in enumerate(out):
        for h, o in enumerate(row):
            if o is not None:
                tot.extend(o[d] * dout[t, h, d] for d in range(len(o)))
    return math.fsum(tot)


@pytest.mark.parametrize("window", [0, 2])
def test_bwd_finite_differences(window):
    rng = np.random.default_rng(23 + window)
    q, k, v, sinks, cu = _case(rng, [3, 0, 4], 2, 1, 3, lead=1, tail=1, std=0.7)
    dout = rng.standard_normal(q.shape)
    scale = 0.5
    ids = _doc_ids(cu, q.shape[0])
    inside = np.array([i is not None for i in ids])
    dq, dk, dv, ds = ref_bwd_varlen(q, k, v, cu, sinks, dout, window, scale)
    assert np.isnan(dq[~inside]).all() and np.isnan(dk[~inside]).all() and np.isnan(dv[~inside]).all()
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
            lp = _brute_loss(*args, dout, ids, window, scale)
            x[mi] = old - h
            lm = _brute_loss(*args, dout, ids, window, scale)
            x[mi] = old
            num[mi] = (lp - lm) / (2 * h)
        if idx < 3:
            assert (num[~inside] == 0).all()  # rows in no document do not reach the loss
            num, grad = num[inside], grad[inside]
        rel = np.linalg.norm(num - grad) / np.linalg.norm(grad)
        assert rel <= 1e-6, (idx, rel)
