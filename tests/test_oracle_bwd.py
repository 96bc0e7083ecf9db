"""Pins of the oracle's backward (gradients of exact attention).

The analytic gradients of ``oracle.bwd`` are checked against quantities it
does not compute itself:
  * central finite differences of the independent pure-Python forward
    (``tests/brute.py``) of the loss L = sum(O * dO), for every mask kind,
    the soft cap and GQA;
  * closed forms: a single visible key (O = that value row), keys that no
    query sees (zero gradient), the column sums of dV (sum_j P_ij = 1) and
    of dK (softmax is invariant to a shift of a row's scores);
  * the GQA reduction: dK, dV of a KV head are the sums of the MHA gradients
    of the query heads sharing it.
"""
import numpy as np
import pytest

import attn_inputs as gen
import oracle
from tests import brute

pytestmark = pytest.mark.filterwarnings("ignore")


def _f64(bits):
    return gen.f32_from_bf16_bits(bits).astype(np.float64)


def _loss(qf, kf, vf, G, scale, **kw):
    O, _ = brute.attention(qf.tolist(), kf.tolist(), vf.tolist(), scale, **kw)
    return float(np.sum(np.array(O) * G))


def _fd_grad(x, f, eps=1e-5):
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        idx = it.multi_index
        old = x[idx]
        x[idx] = old + eps
        fp = f()
        x[idx] = old - eps
        fm = f()
        x[idx] = old
        g[idx] = (fp - fm) / (2 * eps)
    return g


CASES = [
    dict(causal=True),
    dict(),
    dict(window=2),
    dict(window=(3, 0), causal=True),
    dict(softcap=0.7),
    dict(window=2, softcap=1.5),
    dict(causal=True, docs=True),
]


@pytest.mark.parametrize("group", [1, 2])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_gradients_match_finite_differences(case, group):
    kw = dict(CASES[case])
    B, Hkv, N, d = 2, 1, 7, 4
    Hq = Hkv * group
    q, k, v, _ = gen.fwd_inputs(300 + case, B, Hq, Hkv, N, d, factor=1.5)
    rng = np.random.Generator(np.random.PCG64(400 + case))
    do = gen.draw_bf16(rng, (B, Hq, N, d), 1.0)
    if kw.pop("docs", False):
        kw["doc_offsets"] = np.array([[0, 3, 7], [0, 5, 7]], dtype=np.int32)
    scale = 0.6
    dq, dk, dv = oracle.bwd(q, k, v, do, scale=scale, **kw)
    qf, kf, vf, G = _f64(q), _f64(k), _f64(v), _f64(do)
    bkw = dict(kw)
    f = lambda: _loss(qf, kf, vf, G, scale, **bkw)
    for name, x, g in (("dq", qf, dq), ("dk", kf, dk), ("dv", vf, dv)):
        fd = _fd_grad(x, f)
        assert np.allclose(g, fd, rtol=1e-6, atol=1e-7), (name, float(np.abs(g - fd).max()))


def test_single_key_gives_value_gradient_only():
    # N = 1: O = v, so dv = dO and q, k get no gradient
    q, k, v, _ = gen.fwd_inputs(310, 1, 2, 2, 1, 8)
    rng = np.random.Generator(np.random.PCG64(311))
    do = gen.draw_bf16(rng, (1, 2, 1, 8), 1.0)
    dq, dk, dv = oracle.bwd(q, k, v, do, scale=0.3)
    assert np.array_equal(dv, _f64(do))
    assert not dq.any() and not dk.any()


def test_unseen_keys_and_empty_rows_get_zero_gradient():
    # keys i+1..i+2 only: key 0 is never visible, the last row sees nothing
    N = 9
    q, k, v, _ = gen.fwd_inputs(312, 1, 2, 2, N, 8)
    rng = np.random.Generator(np.random.PCG64(313))
    do = gen.draw_bf16(rng, (1, 2, N, 8), 1.0)
    dq, dk, dv = oracle.bwd(q, k, v, do, scale=0.3, window=(-1, 2))
    assert not dk[:, :, 0].any() and not dv[:, :, 0].any()
    assert not dq[:, :, N - 1].any()


def test_column_sums():
    # sum_j dv_j = sum_i dO_i (rows with a visible key), and without a cap
    # sum_j dk_j = 0 (each row's dS sums to zero)
    N, d = 40, 16
    q, k, v, _ = gen.fwd_inputs(314, 2, 4, 2, N, d)
    rng = np.random.Generator(np.random.PCG64(315))
    do = gen.draw_bf16(rng, (2, 4, N, d), 1.0)
    dq, dk, dv = oracle.bwd(q, k, v, do, scale=0.25, causal=True)
    G = _f64(do).reshape(2, 2, 2, N, d).sum(axis=2)  # per KV head: its query heads
    assert np.allclose(dv.sum(axis=2), G.sum(axis=2), rtol=1e-12, atol=1e-12)
    assert np.allclose(dk.sum(axis=2), 0.0, atol=1e-12)


def test_gqa_gradients_are_sums_of_mha_gradients():
    B, Hq, Hkv, N, d = 1, 4, 2, 30, 8
    q, k, v, _ = gen.fwd_inputs(316, B, Hq, Hkv, N, d)
    rng = np.random.Generator(np.random.PCG64(317))
    do = gen.draw_bf16(rng, (B, Hq, N, d), 1.0)
    dq, dk, dv = oracle.bwd(q, k, v, do, scale=0.3, causal=True, window=(5, 0))
    kr = np.repeat(k, Hq // Hkv, axis=1)
    vr = np.repeat(v, Hq // Hkv, axis=1)
    dq2, dk2, dv2 = oracle.bwd(q, kr, vr, do, scale=0.3, causal=True, window=(5, 0))
    assert np.allclose(dq, dq2, rtol=1e-12, atol=1e-13)
    assert np.allclose(dk, dk2.reshape(B, Hkv, Hq // Hkv, N, d).sum(axis=2), rtol=1e-12, atol=1e-13)
    assert np.allclose(dv, dv2.reshape(B, Hkv, Hq // Hkv, N, d).sum(axis=2), rtol=1e-12, atol=1e-13)
