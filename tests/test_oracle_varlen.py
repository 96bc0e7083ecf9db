"""Pins of the oracle's packed variable-length forward (``oracle.fwd_varlen``).

It is checked against computations it does not share:
  * the pure-Python loops of ``tests/brute.py`` on tiny packed inputs, with
    equal and unequal query/key lengths, empty sequences, GQA, windows and
    the soft cap;
  * the C oracle: equal query and key offsets make the sequences exactly
    the documents of a one-row batch (``oracle.fwd`` with doc_offsets);
  * closed forms: one query per sequence under the causal mask sees every
    key of its sequence (the C decode oracle with lens = the key counts),
    and q = 0 gives the mean of the visible V rows with LSE = ln(count).
"""
import math

import numpy as np
import pytest

import attn_inputs as gen
import oracle
from tests import brute

pytestmark = pytest.mark.filterwarnings("ignore")


def _draw(seed, tq, tk, Hq, Hkv, d, factor=1.0):
    rng = np.random.Generator(np.random.PCG64(seed))
    q = gen.draw_bf16(rng, (tq, Hq, d), factor)
    k = gen.draw_bf16(rng, (tk, Hkv, d), factor)
    v = gen.draw_bf16(rng, (tk, Hkv, d), factor)
    return q, k, v


def _f(bits):
    return gen.f32_from_bf16_bits(bits).astype(np.float64)


CASES = [
    dict(lq=[3, 5, 2], lk=[3, 5, 2], causal=True),          # the pages' example
    dict(lq=[3, 5, 2], lk=[3, 5, 2]),
    dict(lq=[2, 0, 4], lk=[5, 3, 4], causal=True),          # fewer queries than keys
    dict(lq=[4, 3], lk=[2, 3], causal=True),                # more queries than keys
    dict(lq=[6, 1], lk=[7, 4], window=(2, 1)),
    dict(lq=[5, 3], lk=[5, 6], causal=True, window=(2, 0), softcap=0.8),
    dict(lq=[0, 4, 0], lk=[3, 0, 2]),                       # empty sequences both ways
]


@pytest.mark.parametrize("group", [1, 2])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_matches_brute_force(case, group):
    c = dict(CASES[case])
    lq, lk = c.pop("lq"), c.pop("lk")
    cu_q = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    Hkv, d = 2, 4
    q, k, v = _draw(700 + case, int(cu_q[-1]), int(cu_k[-1]), Hkv * group, Hkv, d, 1.5)
    o, lse = oracle.fwd_varlen(q, k, v, cu_q, cu_k, scale=0.7, **c)
    bo, bl = brute.attention_varlen(_f(q).tolist(), _f(k).tolist(), _f(v).tolist(),
                                    cu_q.tolist(), cu_k.tolist(), 0.7, **c)
    if q.shape[0]:
        assert np.allclose(o, np.array(bo), rtol=1e-12, atol=1e-13)
        bl = np.array(bl)
        assert np.array_equal(np.isneginf(lse), np.isneginf(bl))
        fin = np.isfinite(bl)
        assert np.allclose(lse[fin], bl[fin], rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("window", [None, 40])
def test_equal_offsets_are_documents(window):
    # sequences with equal query and key offsets = documents of one batch row
    lens = [130, 1, 77, 300, 12]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    N, Hq, Hkv, d = int(cu[-1]), 4, 2, 16
    q, k, v = _draw(720, N, N, Hq, Hkv, d)
    o, lse = oracle.fwd_varlen(q, k, v, cu, cu, scale=0.25, causal=True, window=window)
    q4, k4, v4 = (np.ascontiguousarray(np.swapaxes(x, 0, 1))[None] for x in (q, k, v))
    ro, rl = oracle.fwd(q4, k4, v4, scale=0.25, causal=True, window=window,
                        doc_offsets=cu[None, :])
    assert np.allclose(o, np.swapaxes(ro[0], 0, 1), rtol=1e-11, atol=1e-12)
    assert np.allclose(lse, rl[0], rtol=1e-11, atol=1e-12)


def test_single_query_per_sequence_is_decode():
    # causal with Lq = 1: the query lines up with the last key and sees all
    lk = [5, 64, 1, 200]
    B, Hq, Hkv, d, T = len(lk), 4, 2, 8, max(lk)
    cu_q = np.arange(B + 1, dtype=np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    q, k, v = _draw(730, B, int(cu_k[-1]), Hq, Hkv, d)
    o, lse = oracle.fwd_varlen(q, k, v, cu_q, cu_k, scale=0.3, causal=True)
    kc = np.zeros((B, Hkv, T, d), np.uint16)
    vc = np.zeros((B, Hkv, T, d), np.uint16)
    for b in range(B):
        kc[b, :, :lk[b]] = np.swapaxes(k[cu_k[b]:cu_k[b + 1]], 0, 1)
        vc[b, :, :lk[b]] = np.swapaxes(v[cu_k[b]:cu_k[b + 1]], 0, 1)
    do, dl = oracle.decode(q, kc, vc, np.array(lk, np.int32), scale=0.3)
    assert np.allclose(o, do, rtol=1e-12, atol=1e-13)
    assert np.allclose(lse.T, dl, rtol=1e-12, atol=1e-13)


def test_zero_queries_average_visible_values():
    lq, lk = [3, 4], [6, 4]
    cu_q = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    _, k, v = _draw(740, 7, 10, 2, 2, 8)
    q = np.zeros((7, 2, 8), np.uint16)
    o, lse = oracle.fwd_varlen(q, k, v, cu_q, cu_k, scale=1.0, causal=True)
    vf = _f(v)
    for s in range(2):
        for il in range(lq[s]):
            i = cu_q[s] + il
            n = il + lk[s] - lq[s] + 1  # visible keys 0 .. il + Lk - Lq
            want = vf[cu_k[s]:cu_k[s] + n].mean(axis=0)
            assert np.allclose(o[i], want, rtol=1e-13, atol=1e-14)
            assert np.allclose(lse[:, i], math.log(n), rtol=1e-13)


def test_selected_rows_match_all_rows():
    lq, lk = [9, 17], [12, 17]
    cu_q = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    q, k, v = _draw(750, 26, 29, 4, 1, 8)
    o, lse = oracle.fwd_varlen(q, k, v, cu_q, cu_k, scale=0.4, causal=True, window=(3, 0))
    rows = np.array([[0, 0], [3, 8], [1, 9], [2, 25]])
    so, sl = oracle.fwd_varlen(q, k, v, cu_q, cu_k, scale=0.4, causal=True, window=(3, 0), rows=rows)
    assert np.array_equal(so, o[rows[:, 1], rows[:, 0]])
    assert np.array_equal(sl, lse[rows[:, 0], rows[:, 1]])
