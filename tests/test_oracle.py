"""Pins for the fp64 oracle (CPU only).

Each test ties the oracle to something other than itself: values printed on
the pages, closed forms, invariants, reductions to simpler cases, a second
algorithm, or an independent pure-Python brute force.
"""
import math
import os

import numpy as np
import pytest

import attn_inputs as gen
import oracle
from tests import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bits(x):
    return gen.bf16_bits_from_f32(np.asarray(x, dtype=np.float32))


def widen(b):
    return gen.f32_from_bf16_bits(b).astype(np.float64)


def rand_qkv(rng, B, Hq, Hkv, N, d, factor=1.0):
    q = gen.draw_bf16(rng, (B, Hq, N, d), factor)
    k = gen.draw_bf16(rng, (B, Hkv, N, d), factor)
    v = gen.draw_bf16(rng, (B, Hkv, N, d), factor)
    return q, k, v


def one_doc_offsets(B, N):
    return np.tile(np.array([0, N], dtype=np.int32), (B, 1))


# --------------------------------------------------------------------------
# Printed values: the worked softmax example (llm-systems-engineering,
# "Attention 최적화가 어려운 이유", Figure 4).
# --------------------------------------------------------------------------
def _read_worked_example():
    rows, tile_local = [], None
    with open(os.path.join(GOLDEN, "softmax_worked_example.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            parts = [p.strip() for p in line.split("|")]
            if parts[0] == "tile_local_p0":
                tile_local = float(parts[1])
                continue
            scores = [float(x) for x in parts[0].split()]
            rows.append((scores, float(parts[1]), float(parts[2]),
                         float(parts[3]), float(parts[4])))
    return rows, tile_local


def _worked_example_through_oracle(scores):
    # q = e0, K row j = s_j * e0, scale 1, V = identity: O row == P row.
    d = 8
    n = len(scores)
    q = np.zeros((1, 1, n, d), np.float32)
    q[0, 0, :, 0] = 1.0
    k = np.zeros((1, 1, n, d), np.float32)
    k[0, 0, :, 0] = scores
    v = np.zeros((1, 1, n, d), np.float32)
    for j in range(n):
        v[0, 0, j, j] = 1.0
    o, lse, p = oracle.fwd(bits(q), bits(k), bits(v), scale=1.0, want_probs=True)
    return o[0, 0, 0, :n], lse[0, 0, 0], p[0, 0, 0]


def test_worked_example_printed_values():
    rows, _ = _read_worked_example()
    assert len(rows) == 2
    for scores, p0, p0_tol, expsum, expsum_tol in rows:
        o, lse, p = _worked_example_through_oracle(scores)
        assert abs(p[0] - p0) <= p0_tol + 1e-12
        assert abs(o[0] - p0) <= p0_tol + 1e-12       # O row is the P row
        assert abs(math.exp(lse) - expsum) <= expsum_tol + 1e-12


def test_worked_example_is_not_tile_local():
    rows, tile_local = _read_worked_example()
    for scores, *_ in rows:
        _, _, p = _worked_example_through_oracle(scores)
        assert abs(p[0] - tile_local) > 0.2
        assert abs(p[0:2].sum() - 1.0) > 0.4   # the first two keys alone do not sum to 1


# --------------------------------------------------------------------------
# Invariants: rows of P sum to 1; masked keys get weight exactly 0.
# --------------------------------------------------------------------------
MASKS = [
    dict(causal=True),
    dict(window=3),
    dict(window=(2, 0)),
    dict(window=2, softcap=5.0),
    dict(doc=True, causal=True),
    dict(doc=True),
    dict(),
]


def _mask_kwargs(m, B, N, rng):
    kw = {}
    if m.get("causal"):
        kw["causal"] = True
    if "window" in m:
        kw["window"] = m["window"]
    if "softcap" in m:
        kw["softcap"] = m["softcap"]
    if m.get("doc"):
        rows = gen.draw_doc_offsets(rng, B, N, 2, 6)
        kw["doc_offsets"] = gen.pad_offsets(rows, N)[0]
    return kw


def _visible_matrix(kw, b, N):
    vis = np.ones((N, N), bool)
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    if kw.get("causal"):
        vis &= j <= i
    if "window" in kw:
        w = kw["window"]
        wl, wr = (w, w) if np.isscalar(w) else w
        vis &= (j >= i - wl) & (j <= i + wr)
    if "doc_offsets" in kw:
        ids = np.array(brute.doc_ids_from_offsets(kw["doc_offsets"][b], N))
        vis &= ids[:, None] == ids[None, :]
    return vis


@pytest.mark.parametrize("m", MASKS)
def test_probability_rows_sum_to_one_and_masked_are_zero(m, rng):
    B, H, N, d = 2, 2, 13, 8
    q, k, v = rand_qkv(rng, B, H, H, N, d)
    kw = _mask_kwargs(m, B, N, rng)
    _, _, p = oracle.fwd(q, k, v, scale=0.35, want_probs=True, **kw)
    for b in range(B):
        vis = _visible_matrix(kw, b, N)
        for h in range(H):
            assert np.all(p[b, h][~vis] == 0.0)
            sums = p[b, h].sum(-1)
            has = vis.any(-1)
            assert np.allclose(sums[has], 1.0, atol=1e-12, rtol=0)


# --------------------------------------------------------------------------
# Closed forms: one visible key; equal scores.
# --------------------------------------------------------------------------
def test_single_visible_key_gives_that_value_row(rng):
    B, H, N, d = 1, 2, 9, 8
    q, k, v = rand_qkv(rng, B, H, H, N, d)
    scale = 0.3
    # causal row 0
    o, lse = oracle.fwd(q, k, v, scale=scale, causal=True)
    assert np.array_equal(o[0, :, 0], widen(v[0, :, 0]))
    s00 = scale * (widen(q[0, :, 0]) * widen(k[0, :, 0])).sum(-1)
    assert np.allclose(lse[0, :, 0], s00, rtol=0, atol=1e-12)
    # window 0: each row sees only itself
    o, lse = oracle.fwd(q, k, v, scale=scale, window=0)
    assert np.array_equal(o[0], widen(v[0]))
    # first token of each document (documents + causal)
    offs = np.array([[0, 3, 7, N]], np.int32)
    o, _ = oracle.fwd(q, k, v, scale=scale, causal=True, doc_offsets=offs)
    for start in (0, 3, 7):
        assert np.array_equal(o[0, :, start], widen(v[0, :, start]))


def _equal_score_case(N, d, rng):
    q = np.zeros((1, 1, N, d), np.uint16)      # Q = 0: every visible score is 0
    k = gen.draw_bf16(rng, (1, 1, N, d))
    v = gen.draw_bf16(rng, (1, 1, N, d))
    return q, k, v


def test_equal_scores_mean_and_log_count(rng):
    N, d = 37, 8
    q, k, v = _equal_score_case(N, d, rng)
    V = widen(v[0, 0])
    W = 5
    offs = np.array([[0, 10, 11, 30, N]], np.int32)
    starts = [0, 10, 11, 30]
    cases = {
        "causal": (dict(causal=True), lambda i: (0, i)),
        "window": (dict(window=W), lambda i: (max(0, i - W), min(N - 1, i + W))),
        "left_window": (dict(window=(W, 0)), lambda i: (max(0, i - W), i)),
        "docs_causal": (dict(causal=True, doc_offsets=offs),
                        lambda i: (max(s for s in starts if s <= i), i)),
        "full": (dict(), lambda i: (0, N - 1)),
    }
    for name, (kw, interval) in cases.items():
        o, lse = oracle.fwd(q, k, v, scale=0.7, **kw)
        for i in range(N):
            lo, hi = interval(i)
            n = hi - lo + 1
            assert lse[0, 0, i] == pytest.approx(math.log(n), abs=1e-12), name
            assert np.allclose(o[0, 0, i], V[lo:hi + 1].mean(0), atol=1e-12, rtol=0), name
    # the window count closed form min(i,W) + min(N-1-i,W) + 1
    o, lse = oracle.fwd(q, k, v, scale=1.0, window=W)
    for i in range(N):
        assert lse[0, 0, i] == pytest.approx(math.log(min(i, W) + min(N - 1 - i, W) + 1), abs=1e-12)


def test_equal_scores_decode_log_len(rng):
    B, Hq, Hkv, T, d = 3, 4, 2, 50, 8
    q = np.zeros((B, Hq, d), np.uint16)
    kc = gen.draw_bf16(rng, (B, Hkv, T, d))
    vc = gen.draw_bf16(rng, (B, Hkv, T, d))
    lens = np.array([1, 17, 50], np.int32)
    o, lse = oracle.decode(q, kc, vc, lens, scale=0.1)
    for b in range(B):
        for h in range(Hq):
            assert lse[b, h] == pytest.approx(math.log(lens[b]), abs=1e-12)
            assert np.allclose(o[b, h], widen(vc[b, h // 2, : lens[b]]).mean(0), atol=1e-12)


# --------------------------------------------------------------------------
# Independent brute force on tiny shapes, every mask kind, GQA 1 and 2.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("m", MASKS)
@pytest.mark.parametrize("group", [1, 2])
def test_brute_force_tiny(m, group, rng):
    B, Hkv, N, d = 2, 2, 11, 5
    Hq = Hkv * group
    q, k, v = rand_qkv(rng, B, Hq, Hkv, N, d)
    kw = _mask_kwargs(m, B, N, rng)
    scale = 0.41
    o, lse = oracle.fwd(q, k, v, scale=scale, **kw)
    bkw = dict(causal=kw.get("causal", False), window=kw.get("window"),
               doc_offsets=kw.get("doc_offsets"), softcap=kw.get("softcap"))
    bo, bl = brute.attention(widen(q).tolist(), widen(k).tolist(), widen(v).tolist(),
                             scale, **bkw)
    assert np.allclose(o, np.array(bo), atol=1e-12, rtol=0)
    assert np.allclose(lse, np.array(bl), atol=1e-12, rtol=0)


# --------------------------------------------------------------------------
# Reductions to simpler cases.
# --------------------------------------------------------------------------
def test_gqa_equals_mha_on_repeated_kv(rng):
    B, Hkv, group, N, d = 2, 2, 3, 19, 8
    q, k, v = rand_qkv(rng, B, Hkv * group, Hkv, N, d)
    kr = np.repeat(k, group, axis=1)
    vr = np.repeat(v, group, axis=1)
    o1, l1 = oracle.fwd(q, k, v, scale=0.2, causal=True)
    o2, l2 = oracle.fwd(q, kr, vr, scale=0.2, causal=True)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_single_document_equals_causal(rng):
    B, H, N, d = 2, 2, 23, 8
    q, k, v = rand_qkv(rng, B, H, H, N, d)
    o1, l1 = oracle.fwd(q, k, v, scale=0.3, causal=True, doc_offsets=one_doc_offsets(B, N))
    o2, l2 = oracle.fwd(q, k, v, scale=0.3, causal=True)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_documents_equal_separate_sequences(rng):
    B, H, N, d = 1, 2, 20, 8
    q, k, v = rand_qkv(rng, B, H, H, N, d)
    offs = np.array([[0, 7, 20]], np.int32)
    o, l = oracle.fwd(q, k, v, scale=0.3, causal=True, doc_offsets=offs)
    for a, b in ((0, 7), (7, 20)):
        os_, ls_ = oracle.fwd(q[:, :, a:b].copy(), k[:, :, a:b].copy(), v[:, :, a:b].copy(),
                              scale=0.3, causal=True)
        assert np.allclose(o[:, :, a:b], os_, atol=1e-13)
        assert np.allclose(l[:, :, a:b], ls_, atol=1e-13)


def test_wide_window_equals_full(rng):
    B, H, N, d = 1, 2, 17, 8
    q, k, v = rand_qkv(rng, B, H, H, N, d)
    o1, l1 = oracle.fwd(q, k, v, scale=0.3, window=N - 1)
    o2, l2 = oracle.fwd(q, k, v, scale=0.3)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    o3, l3 = oracle.fwd(q, k, v, scale=0.3, window=(N - 1, 0))
    o4, l4 = oracle.fwd(q, k, v, scale=0.3, causal=True)
    assert np.array_equal(o3, o4) and np.array_equal(l3, l4)


def test_softcap_huge_is_identity(rng):
    B, H, N, d = 1, 2, 15, 8
    q, k, v = rand_qkv(rng, B, H, H, N, d)
    o1, l1 = oracle.fwd(q, k, v, scale=0.3, window=4, softcap=1e30)
    o2, l2 = oracle.fwd(q, k, v, scale=0.3, window=4)
    assert np.allclose(o1, o2, atol=1e-14) and np.allclose(l1, l2, atol=1e-14)


def _single_key_lse(dot, scale, softcap):
    """LSE of a row whose only visible key has q.k == dot (exact in bf16)."""
    d = 8
    q = np.zeros((1, 1, 1, d), np.float32)
    k = np.zeros((1, 1, 1, d), np.float32)
    q[..., 0] = 1.0
    k[..., 0] = dot
    v = np.ones((1, 1, 1, d), np.float32)
    _, lse = oracle.fwd(bits(q), bits(k), bits(v), scale=scale, softcap=softcap)
    return lse[0, 0, 0]


def test_softcap_small_score_taylor():
    # c*tanh(s/c) = s - s^3/(3c^2) + 2 s^5/(15 c^4) - ...
    s, c = 2.0, 50.0
    taylor = s - s ** 3 / (3 * c * c)
    assert _single_key_lse(2.0, 1.0, c) == pytest.approx(taylor, abs=2 * s ** 5 / (15 * c ** 4) + 1e-12)


def test_softcap_applies_after_scaling():
    # dot = 800, scale 1/8: scaled score 100 -> 50*tanh(2) = 48.20137900379...
    # (capping the raw 800 first would give 50*tanh(16)/8 = 6.25).
    tanh2 = 0.9640275800758169  # tanh(2), table value
    got = _single_key_lse(800.0, 0.125, 50.0)
    assert got == pytest.approx(50.0 * tanh2, abs=1e-9)
    assert abs(got - 6.25) > 1.0


def test_scale_is_applied():
    # A single key scores q.k*scale; with scale 0.5 and q.k = 3 the LSE is 1.5.
    assert _single_key_lse(3.0, 0.5, None) == pytest.approx(1.5, abs=1e-15)


def test_decode_equals_last_row_of_unmasked_forward(rng):
    B, Hq, Hkv, T, d = 2, 4, 2, 40, 8
    q = gen.draw_bf16(rng, (B, Hq, d))
    kc = gen.draw_bf16(rng, (B, Hkv, T, d))
    vc = gen.draw_bf16(rng, (B, Hkv, T, d))
    lens = np.array([13, 40], np.int32)
    o, lse = oracle.decode(q, kc, vc, lens, scale=0.25)
    for b in range(B):
        L = int(lens[b])
        qq = np.zeros((1, Hq, L, d), np.uint16)
        qq[0, :, L - 1] = q[b]
        fo, fl = oracle.fwd(qq, kc[b:b + 1, :, :L].copy(), vc[b:b + 1, :, :L].copy(), scale=0.25)
        assert np.allclose(o[b], fo[0, :, L - 1], atol=1e-13)
        assert np.allclose(lse[b], fl[0, :, L - 1], atol=1e-13)


def test_decode_ignores_cache_past_lens(rng):
    B, Hq, Hkv, T, d = 1, 2, 1, 30, 8
    q = gen.draw_bf16(rng, (B, Hq, d))
    kc = gen.draw_bf16(rng, (B, Hkv, T, d))
    vc = gen.draw_bf16(rng, (B, Hkv, T, d))
    lens = np.array([11], np.int32)
    o1, l1 = oracle.decode(q, kc, vc, lens, scale=0.25)
    kc2, vc2 = kc.copy(), vc.copy()
    kc2[:, :, 11:] = 0x7FC0   # NaN
    vc2[:, :, 11:] = 0x7FC0
    o2, l2 = oracle.decode(q, kc2, vc2, lens, scale=0.25)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


# --------------------------------------------------------------------------
# Second algorithms: the blockwise online recurrence and the split-KV merge.
# --------------------------------------------------------------------------
def blockwise_forward(Q, K, V, scale, bq, bk, visible):
    """Tile-by-tile exact attention in fp64 (youngju.dev "FlashAttention 논문
    분석", section "알고리즘 의사코드"): per query block, sweep key blocks and
    keep a running max m, running sum l and a normalised output; each block
    rescales the old state by exp(m_old - m_new) and the new block by
    exp(m_blk - m_new)."""
    N, d = Q.shape
    O = np.zeros((N, d))
    m = np.full(N, -np.inf)
    l = np.zeros(N)
    for i0 in range(0, N, bq):
        i1 = min(N, i0 + bq)
        for j0 in range(0, N, bk):
            j1 = min(N, j0 + bk)
            S = scale * Q[i0:i1] @ K[j0:j1].T
            S = np.where(visible[i0:i1, j0:j1], S, -np.inf)
            m_blk = S.max(axis=1)
            with np.errstate(invalid="ignore"):
                P = np.exp(S - np.where(np.isinf(m_blk), 0.0, m_blk)[:, None])
            l_blk = P.sum(axis=1)
            m_old = m[i0:i1]
            m_new = np.maximum(m_old, m_blk)
            safe = np.where(np.isinf(m_new), 0.0, m_new)
            alpha = np.exp(m_old - safe)
            beta = np.exp(m_blk - safe)
            l_new = alpha * l[i0:i1] + beta * l_blk
            num = (alpha * l[i0:i1])[:, None] * O[i0:i1] + beta[:, None] * (P @ V[j0:j1])
            with np.errstate(invalid="ignore", divide="ignore"):
                O[i0:i1] = np.where(l_new[:, None] > 0, num / l_new[:, None], 0.0)
            m[i0:i1] = m_new
            l[i0:i1] = l_new
    with np.errstate(divide="ignore"):
        lse = m + np.log(l)
    return O, lse


@pytest.mark.parametrize("bq,bk", [(1, 1), (4, 3), (8, 16), (37, 37)])
def test_blockwise_recurrence_equals_direct(bq, bk, rng):
    N, d = 37, 8
    q, k, v = rand_qkv(rng, 1, 1, 1, N, d)
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    for kw, vis in ((dict(causal=True), j <= i),
                    (dict(window=4), np.abs(i - j) <= 4),
                    (dict(), np.ones((N, N), bool))):
        o, lse = oracle.fwd(q, k, v, scale=0.3, **kw)
        bo, bl = blockwise_forward(widen(q[0, 0]), widen(k[0, 0]), widen(v[0, 0]), 0.3, bq, bk, vis)
        assert np.allclose(o[0, 0], bo, atol=1e-12, rtol=0)
        assert np.allclose(lse[0, 0], bl, atol=1e-12, rtol=0)


@pytest.mark.parametrize("chunk", [1, 7, 16, 64])
def test_split_kv_merge_equals_unsplit(chunk, rng):
    """Per-chunk (O_c, LSE_c) merged by rescaling with the chunk maxima
    (aegloslab "3.7 어텐션 II", section 3.7.4) equals the unsplit decode."""
    B, Hq, Hkv, T, d = 2, 4, 2, 64, 8
    q = gen.draw_bf16(rng, (B, Hq, d))
    kc = gen.draw_bf16(rng, (B, Hkv, T, d))
    vc = gen.draw_bf16(rng, (B, Hkv, T, d))
    lens = np.array([29, 64], np.int32)
    o, lse = oracle.decode(q, kc, vc, lens, scale=0.3)
    for b in range(B):
        L = int(lens[b])
        parts = []
        for c0 in range(0, L, chunk):
            c1 = min(L, c0 + chunk)
            po, pl = oracle.decode(q[b:b + 1], kc[b:b + 1, :, c0:c1].copy(),
                                   vc[b:b + 1, :, c0:c1].copy(),
                                   np.array([c1 - c0], np.int32), scale=0.3)
            parts.append((po[0], pl[0]))
        M = np.max([pl for _, pl in parts], axis=0)
        w = [np.exp(pl - M) for _, pl in parts]
        Lsum = np.sum(w, axis=0)
        merged = np.sum([wc[:, None] * po for wc, (po, _) in zip(w, parts)], axis=0) / Lsum[:, None]
        assert np.allclose(merged, o[b], atol=1e-12, rtol=0)
        assert np.allclose(M + np.log(Lsum), lse[b], atol=1e-12, rtol=0)


# --------------------------------------------------------------------------
# Input-generator structure.
# --------------------------------------------------------------------------
def test_cu_seqlens_example():
    # aegloslab "3.7 어텐션 II" section 3.7.6: lengths [3, 5, 2] -> [0, 3, 8, 10]
    assert gen.lengths_to_offsets([3, 5, 2]).tolist() == [0, 3, 8, 10]


def test_document_draws_cover_n():
    rng = np.random.Generator(np.random.PCG64(7))
    rows = gen.draw_doc_offsets(rng, 4, 8192)
    for r in rows:
        assert r[0] == 0 and r[-1] == 8192
        lens = np.diff(r)
        assert np.all(lens[:-1] >= 256) and np.all(lens <= 4096) and np.all(lens >= 1)


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20, -2.0 - 2 ** -8], np.float32)
    y = gen.f32_from_bf16_bits(gen.bf16_bits_from_f32(x))
    assert y.tolist() == [1.0, 1.0 + 4 * 2 ** -8, 1.0 + 2 * 2 ** -8, -2.0]
