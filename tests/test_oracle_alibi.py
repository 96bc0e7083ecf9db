"""Pins of the oracle's ALiBi distance bias (score -= slope_h * |i - j|).

  * brute force: the pure-Python loops of ``tests/brute.py`` on tiny inputs,
    for every mask kind, with the soft cap and GQA;
  * closed form: with q = 0 under the causal mask, row i weighs key j by
    exp(-slope * (i - j)), so LSE_i = ln((1 - r^(i+1)) / (1 - r)) with
    r = exp(-slope) and O_i is the r-geometric average of v_0 .. v_i;
  * reductions: zero slopes are the unbiased oracle; a slope shared by all
    heads with one visible key changes nothing but the LSE by -slope * |i-j|.
"""
import math

import numpy as np
import pytest

import attn_inputs as gen
import oracle
from tests import brute

pytestmark = pytest.mark.filterwarnings("ignore")


def _f(bits):
    return gen.f32_from_bf16_bits(bits).astype(np.float64)


CASES = [dict(causal=True), dict(), dict(window=2), dict(causal=True, softcap=0.9),
         dict(causal=True, docs=True)]


@pytest.mark.parametrize("group", [1, 2])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_matches_brute_force(case, group):
    kw = dict(CASES[case])
    B, Hkv, N, d = 2, 2, 9, 4
    Hq = Hkv * group
    q, k, v, _ = gen.fwd_inputs(900 + case, B, Hq, Hkv, N, d, factor=1.5)
    if kw.pop("docs", False):
        kw["doc_offsets"] = np.array([[0, 4, 9], [0, 2, 9]], dtype=np.int32)
    slopes = [0.5 * 2.0 ** -h for h in range(Hq)]
    o, lse = oracle.fwd(q, k, v, scale=0.6, alibi_slopes=slopes, **kw)
    bo, bl = brute.attention(_f(q).tolist(), _f(k).tolist(), _f(v).tolist(), 0.6,
                             alibi_slopes=slopes, **kw)
    assert np.allclose(o, np.array(bo), rtol=1e-12, atol=1e-13)
    assert np.allclose(lse, np.array(bl), rtol=1e-12, atol=1e-13)


def test_zero_queries_give_geometric_weights():
    B, H, N, d = 1, 3, 40, 8
    _, k, v, _ = gen.fwd_inputs(910, B, H, H, N, d)
    q = np.zeros((B, H, N, d), np.uint16)
    slopes = np.array([0.05, 0.5, 2.0])
    o, lse = oracle.fwd(q, k, v, scale=1.0, causal=True, alibi_slopes=slopes)
    vf = _f(v)
    for h, sl in enumerate(slopes):
        r = math.exp(-sl)
        for i in (0, 1, 17, N - 1):
            want_lse = math.log((1.0 - r ** (i + 1)) / (1.0 - r))
            assert lse[0, h, i] == pytest.approx(want_lse, rel=1e-12, abs=1e-13)
            w = np.array([r ** (i - j) for j in range(i + 1)])
            want_o = (w[:, None] * vf[0, h, : i + 1]).sum(axis=0) / w.sum()
            assert np.allclose(o[0, h, i], want_o, rtol=1e-12, atol=1e-13)


def test_zero_slopes_are_unbiased():
    q, k, v, _ = gen.fwd_inputs(911, 2, 4, 2, 50, 16)
    a = oracle.fwd(q, k, v, scale=0.3, causal=True, window=(7, 3), alibi_slopes=np.zeros(4))
    b = oracle.fwd(q, k, v, scale=0.3, causal=True, window=(7, 3))
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_single_visible_key_shifts_lse_only():
    # window (-3, 3): query i sees key i + 3 only (rows past N - 4 see nothing)
    q, k, v, _ = gen.fwd_inputs(912, 1, 2, 2, 20, 8)
    sl = np.array([0.25, 1.5])
    a_o, a_l = oracle.fwd(q, k, v, scale=0.4, window=(-3, 3), alibi_slopes=sl)
    b_o, b_l = oracle.fwd(q, k, v, scale=0.4, window=(-3, 3))
    fin = np.isfinite(b_l)
    assert np.array_equal(a_o, b_o)
    assert np.allclose(a_l[fin], (b_l - 3.0 * sl[None, :, None])[fin], rtol=1e-13, atol=1e-13)
