"""GPU parity of the forward path (block-mask builder + forward kernel)
against the fp64 oracle, element by element, through the C ABI."""
import math

import numpy as np
import pytest

import attn_inputs as gen
import oracle
from tests.helpers import bf16_to_f64, compare, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def ea():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_attention_15_amd as ea
    ea.library()
    return ea


def _docs_dev(offs_rows, N):
    padded, _ = gen.pad_offsets(offs_rows, N)
    return padded, torch.from_numpy(padded).cuda()


def run_case(ea, *, B, Hq, Hkv, N, d, seed, factor=1.0, causal=False, window=None,
             softcap=None, docs=None, scale=None, label=""):
    q, k, v, _ = gen.fwd_inputs(seed, B, Hq, Hkv, N, d, factor)
    scale = scale if scale is not None else 1.0 / math.sqrt(d)
    kw_dev, kw_ref = {}, {}
    if docs is not None:
        padded, dev = _docs_dev(docs, N)
        kw_dev["doc_offsets"] = dev
        kw_ref["doc_offsets"] = padded
    print(f"[case] {label} B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} causal={causal} "
          f"window={window} softcap={softcap} docs={docs is not None}", flush=True)
    o, lse = ea.fwd(to_dev(q), to_dev(k), to_dev(v), causal=causal, window=window,
                    softcap=softcap, scale=scale, **kw_dev)
    torch.cuda.synchronize()
    ro, rl = oracle.fwd(q, k, v, scale=scale, causal=causal, window=window,
                        softcap=softcap, **kw_ref)
    return compare(bf16_to_f64(o), lse.cpu().numpy(), ro, rl, label)


def test_small_causal_config(ea):
    # the small causal workload: B=1, H=2, N=256, d=64, scale 1/8
    c = gen.CONFIGS[1]
    run_case(ea, B=1, Hq=2, Hkv=2, N=256, d=64, seed=c["seed"], causal=True, label="cfg1")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 65, 1000])
def test_causal_ragged(ea, d, N):
    run_case(ea, B=2, Hq=3, Hkv=3, N=N, d=d, seed=11 + N, causal=True, factor=0.5,
             label=f"causal N={N} d={d}")


@pytest.mark.parametrize("d", [64, 128])
def test_full_bidirectional(ea, d):
    run_case(ea, B=1, Hq=2, Hkv=1, N=777, d=d, seed=21, label="no mask")


def test_window_softcap(ea):
    run_case(ea, B=1, Hq=2, Hkv=2, N=3000, d=128, seed=31, window=300, softcap=50.0,
             label="window300+cap50")


def test_window_1024_softcap_rows(ea):
    run_case(ea, B=1, Hq=1, Hkv=1, N=4100, d=128, seed=32, window=1024, softcap=50.0,
             label="window1024+cap50")


def test_left_window_and_causal(ea):
    run_case(ea, B=1, Hq=2, Hkv=2, N=1500, d=64, seed=33, window=(200, 0), label="left window")
    run_case(ea, B=1, Hq=2, Hkv=2, N=1500, d=128, seed=34, window=(129, 0), causal=True,
             label="left window+causal")


def test_window_zero_is_identity(ea):
    q, k, v, _ = gen.fwd_inputs(35, 1, 2, 2, 300, 128)
    o, lse = ea.fwd(to_dev(q), to_dev(k), to_dev(v), window=0)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_to_f64(o), gen.f32_from_bf16_bits(v).astype(np.float64))


def test_empty_rows(ea):
    # keys i+1..i+2 only: the last row sees nothing -> O = 0, LSE = -inf
    run_case(ea, B=1, Hq=2, Hkv=2, N=200, d=128, seed=36, window=(-1, 2), label="future-only")


def test_softcap_large_scores(ea):
    # scale 1 and factor 2: scaled scores reach hundreds, so the cap (c=20) dominates
    run_case(ea, B=1, Hq=2, Hkv=2, N=700, d=128, seed=37, factor=2.0, scale=1.0,
             softcap=20.0, causal=True, label="cap20 scale1")


@pytest.mark.parametrize("group", [1, 4, 8])
def test_gqa_docs_causal(ea, group):
    rng = np.random.Generator(np.random.PCG64(41 + group))
    N = 2048
    docs = gen.draw_doc_offsets(rng, 2, N, 64, 700)
    run_case(ea, B=2, Hq=8, Hkv=8 // group, N=N, d=128, seed=42 + group, causal=True,
             docs=docs, label=f"gqa{group} docs")


def test_single_document_equals_causal(ea):
    q, k, v, _ = gen.fwd_inputs(51, 2, 4, 2, 1100, 128)
    Q, K, V = to_dev(q), to_dev(k), to_dev(v)
    offs = torch.tensor([[0, 1100], [0, 1100]], dtype=torch.int32, device="cuda")
    o1, l1 = ea.fwd(Q, K, V, causal=True, doc_offsets=offs)
    o2, l2 = ea.fwd(Q, K, V, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_docs_without_causal(ea):
    rng = np.random.Generator(np.random.PCG64(52))
    docs = gen.draw_doc_offsets(rng, 1, 1500, 100, 600)
    run_case(ea, B=1, Hq=2, Hkv=2, N=1500, d=64, seed=53, docs=docs, label="docs bidirectional")


@pytest.mark.parametrize("kind", ["causal", "window", "docs"])
def test_block_skipping_is_bitwise_neutral(ea, kind):
    N = 1500
    q, k, v, _ = gen.fwd_inputs(61, 1, 4, 2, N, 128)
    Q, K, V = to_dev(q), to_dev(k), to_dev(v)
    kw = {}
    if kind == "causal":
        kw = dict(causal=True)
    elif kind == "window":
        kw = dict(window=200, softcap=50.0)
    else:
        rng = np.random.Generator(np.random.PCG64(62))
        _, dev = _docs_dev(gen.draw_doc_offsets(rng, 1, N, 100, 500), N)
        kw = dict(causal=True, doc_offsets=dev)
    o1, l1 = ea.fwd(Q, K, V, **kw)
    o2, l2 = ea.fwd(Q, K, V, no_skip=True, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert torch.equal(l1, l2)


def test_strided_layout_bnhd(ea):
    # [B, N, H, d] storage viewed as [B, H, N, d]: no copies, same result
    q, k, v, _ = gen.fwd_inputs(71, 2, 4, 4, 600, 128)
    Q, K, V = to_dev(q), to_dev(k), to_dev(v)
    Qt = Q.transpose(1, 2).contiguous().transpose(1, 2)
    Kt = K.transpose(1, 2).contiguous().transpose(1, 2)
    Vt = V.transpose(1, 2).contiguous().transpose(1, 2)
    assert Qt.stride(1) == 128 and not Qt.is_contiguous()
    o1, l1 = ea.fwd(Q, K, V, causal=True)
    out = torch.empty(2, 600, 4, 128, dtype=torch.bfloat16, device="cuda").transpose(1, 2)
    o2, l2 = ea.fwd(Qt, Kt, Vt, causal=True, out=out)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_prebuilt_block_mask_is_reusable(ea):
    q, k, v, _ = gen.fwd_inputs(81, 1, 2, 2, 900, 128)
    Q, K, V = to_dev(q), to_dev(k), to_dev(v)
    spec = ea.MaskSpec(causal=True)
    bm = ea.mask_build(spec, 1, 900)
    o1, l1 = ea.fwd(Q, K, V, spec=spec, block_mask=bm)
    o2, l2 = ea.fwd(Q, K, V, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


# --------------------------------------------------------------------------
# Block-mask builder vs a host classification of the same intervals.
# --------------------------------------------------------------------------
def _host_intervals(kind, B, N, docs):
    i = np.arange(N)
    lo = np.zeros((B, N), np.int64)
    hi = np.tile(np.arange(N) * 0 + N - 1, (B, 1)).astype(np.int64)
    if kind in ("causal", "docs"):
        hi = np.minimum(hi, i)
    if kind == "window":
        lo = np.maximum(lo, i - 300)
        hi = np.minimum(hi, i + 300)
    if kind == "ahead":  # window (-40, 100): keys i+40 .. i+100, the last 40 rows see none
        lo = np.maximum(lo, i + 40)
        hi = np.minimum(hi, i + 100)
    if kind == "docs":
        for b in range(B):
            offs = docs[b]
            idx = np.searchsorted(offs, i, side="right") - 1
            lo[b] = np.maximum(lo[b], offs[idx])
            hi[b] = np.minimum(hi[b], offs[idx + 1] - 1)
    empty = lo > hi  # rows with no visible key are stored as lo = 1, hi = 0
    lo[empty], hi[empty] = 1, 0
    return lo, hi


@pytest.mark.parametrize("kind", ["causal", "window", "docs", "ahead"])
@pytest.mark.parametrize("N", [256, 1000, 4096, 20000])
def test_mask_builder_matches_host(ea, kind, N):
    # N = 20000 has 313 key tiles: the builder classifies them in two rounds
    B = 2
    docs_dev = None
    docs = None
    if kind == "docs":
        rng = np.random.Generator(np.random.PCG64(N))
        docs = gen.draw_doc_offsets(rng, B, N, 64, 900)
        _, docs_dev = _docs_dev(docs, N)
    window = 300 if kind == "window" else ((-40, 100) if kind == "ahead" else None)
    spec = ea.MaskSpec(causal=kind in ("causal", "docs"), window=window, doc_offsets=docs_dev)
    bm = ea.mask_build(spec, B, N)
    torch.cuda.synchronize()
    m = ea.mask_unpack(bm, B, N)
    lo, hi = _host_intervals(kind, B, N, docs)
    assert np.array_equal(m["lo"].numpy(), lo) and np.array_equal(m["hi"].numpy(), hi)
    nqt, nkt = m["nqt"], m["nkt"]
    BM, BN = ea.BLOCK_M, ea.BLOCK_N
    counts = np.zeros((B, nqt), np.int64)
    c0 = np.arange(nkt) * BN
    c1 = c0 + BN - 1
    for b in range(B):
        for qt in range(nqt):
            rows = np.arange(qt * BM, min(N, qt * BM + BM))
            lr, hr = lo[b, rows][:, None], hi[b, rows][:, None]
            any_vis = np.any(np.maximum(lr, c0) <= np.minimum(hr, c1), axis=0)
            full = np.all((lr <= c0) & (hr >= c1), axis=0)
            expect = [kt * 2 + (0 if full[kt] else 1) for kt in range(nkt) if any_vis[kt]]
            counts[b, qt] = len(expect)
            got = m["list"][b, qt, : len(expect)].numpy().tolist()
            assert m["count"][b, qt].item() == len(expect)
            assert got == expect, (b, qt)
    # heavy-first order per batch row: a permutation, counts non-increasing,
    # ties by tile index; with documents, grouped first by the interval start
    # of each tile's first row (its document), documents in order
    order = m["order"].numpy().reshape(B, nqt)
    for b in range(B):
        assert sorted(order[b].tolist()) == list(range(nqt))
        doc = (lambda x: int(lo[b, x * BM])) if kind == "docs" else (lambda x: 0)
        expect_order = sorted(range(nqt), key=lambda x: (doc(x), -counts[b, x], x))
        assert order[b].tolist() == expect_order


@pytest.mark.parametrize("N", [1000, 20000])
def test_mask_builder_no_skip(ea, N):
    # ATTN_MASK_NO_SKIP lists every key tile of every query tile as PARTIAL
    # (element masks everywhere), whatever the mask
    B = 2
    bm = ea.mask_build(ea.MaskSpec(causal=True, no_skip=True), B, N)
    torch.cuda.synchronize()
    m = ea.mask_unpack(bm, B, N)
    nqt, nkt = m["nqt"], m["nkt"]
    expect = [2 * kt + 1 for kt in range(nkt)]
    assert np.all(m["count"].numpy() == nkt)
    for b in range(B):
        for qt in range(nqt):
            assert m["list"][b, qt, :nkt].numpy().tolist() == expect, (b, qt)
    assert np.array_equal(m["order"].numpy().reshape(B, nqt), np.tile(np.arange(nqt), (B, 1)))


@pytest.mark.parametrize("d", [64, 128])
def test_softcap_both_forms_in_one_call(ea, d):
    # Scores of most tiles stay within the range where the kernel uses the
    # polynomial form of the cap (|scale * s / c| <= 0.15); the query rows
    # 300..339 are scaled by 12 so that their tiles take the exact form.
    # Both must match the oracle's libm tanh, including the rows at the
    # boundary between the two.
    N, c = 700, 50.0
    q, k, v, _ = gen.fwd_inputs(40 + d, 1, 2, 2, N, d)
    qf = gen.f32_from_bf16_bits(q)
    qf[:, :, 300:340] *= 12.0
    q = gen.bf16_bits_from_f32(qf)
    scale = 1.0 / math.sqrt(d)
    s_big = float(np.abs(np.einsum("hid,hjd->hij", gen.f32_from_bf16_bits(q)[0, :, 300:340].astype(np.float64),
                                   gen.f32_from_bf16_bits(k)[0].astype(np.float64))).max()) * scale / c
    assert s_big > 0.15  # the scaled rows leave the polynomial's range
    print(f"[case] cap50 both forms d={d}, max |scale*s/c| of the scaled rows {s_big:.2f}", flush=True)
    o, lse = ea.fwd(to_dev(q), to_dev(k), to_dev(v), window=200, softcap=c, scale=scale)
    torch.cuda.synchronize()
    ro, rl = oracle.fwd(q, k, v, scale=scale, window=200, softcap=c)
    compare(bf16_to_f64(o), lse.cpu().numpy(), ro, rl, f"cap50 both forms d={d}")


def test_long_sequence_sampled(ea):
    # 65536 tokens (512 query tiles, tile lists of up to 1024 key tiles),
    # causal with GQA 2:1, checked on sampled rows including both ends and
    # the rows around the middle
    from tests.helpers import sample_rows
    N = 65536
    q, k, v, _ = gen.fwd_inputs(45, 1, 2, 1, N, 128)
    rng = np.random.Generator(np.random.PCG64(46))
    rows = sample_rows(rng, 1, 2, N, 24, must=[(0, 0, 0), (0, 1, N - 1), (0, 0, 32767), (0, 1, 32768),
                                               (0, 0, N - 64), (0, 1, 127)])
    scale = 1.0 / math.sqrt(128)
    print("[case] causal N=65536 GQA 2:1, sampled rows", flush=True)
    o, lse = ea.fwd(to_dev(q), to_dev(k), to_dev(v), causal=True, scale=scale)
    torch.cuda.synchronize()
    ro, rl = oracle.fwd(q, k, v, scale=scale, causal=True, rows=rows)
    og = bf16_to_f64(o)[rows[:, 0], rows[:, 1], rows[:, 2]]
    lg = lse.cpu().numpy()[rows[:, 0], rows[:, 1], rows[:, 2]]
    compare(og, lg, ro, rl, "causal N=65536")


# --------------------------------------------------------------------------
# The running-max rescale of the plain kernels (no cap, no bias).  The
# kernels keep a reference max per row and rescale O and l by
# alpha = 2^(m_old - m_new) only when a row's max grows by more than 8
# base-2 units over it; with N(0,1) inputs that almost never happens after
# the first tile, so these inputs force it.
# --------------------------------------------------------------------------
def _ramp_inputs(seed, H, N, d):
    """K rows scaled by 1 + j/16: a tile's largest score grows by about
    ten base-2 units per 64-key tile, so the running max moves past the
    threshold at almost every tile of a row."""
    q, k, v, _ = gen.fwd_inputs(seed, 1, H, H, N, d)
    kf = gen.f32_from_bf16_bits(k) * (1.0 + np.arange(N, dtype=np.float32) / 16.0)[None, None, :, None]
    return q, gen.bf16_bits_from_f32(kf), v


def _plateau_spike_inputs(seed, H, N, d):
    """Every row sees a plateau of keys with scores near 0, then a few
    'spike' keys (two at 250-251, three at 600-602, one at 900) whose
    scores sit J nats higher, J = 7, 10.5 or 14 by row (i mod 3).  The
    first spike a row meets lifts its max by J (10-20 base-2 units) while
    the plateau keeps a sizeable share of the weight (about (i+1) : 2 e^J),
    so a wrong alpha moves O by far more than the tolerance.  V carries 1
    on the spike keys and 0 on the plateau (plus small noise), so O is the
    spikes' share of the mass."""
    rng = np.random.Generator(np.random.PCG64(seed))
    u = np.ones(d, np.float32) / np.float32(np.sqrt(d))  # unit vector
    amp = (1.0 + 0.5 * (np.arange(N) % 3)).astype(np.float32)
    q = amp[None, None, :, None] * u * np.float32(np.sqrt(d)) \
        + 0.05 * rng.standard_normal((1, H, N, d), dtype=np.float32)
    level = np.zeros(N, np.float32)
    spikes = [250, 251, 600, 601, 602, 900]
    level[spikes] = 7.0
    # score = scale * q.k = (amp * sqrt(d) u + e).(level u + e') / sqrt(d) ~ amp * level
    k = level[None, None, :, None] * u + 0.05 * rng.standard_normal((1, H, N, d), dtype=np.float32)
    vv = np.zeros((1, H, N, d), np.float32)
    vv[:, :, spikes, :] = 1.0
    vv += 0.1 * rng.standard_normal((1, H, N, d), dtype=np.float32)
    return gen.bf16_bits_from_f32(q), gen.bf16_bits_from_f32(k), gen.bf16_bits_from_f32(vv)


def _max_rises(q, k, scale, causal, thresh_log2=8.0):
    """Per row, how many times the running max over ascending 64-key tiles
    rises by more than thresh_log2 base-2 units over the reference max a
    lazily rescaling kernel would keep (fp64, from the input scores)."""
    qf = gen.f32_from_bf16_bits(q)[0].astype(np.float64)
    kf = gen.f32_from_bf16_bits(k)[0].astype(np.float64)
    s = np.einsum("hid,hjd->hij", qf, kf) * scale / np.log(2.0)
    N = s.shape[-1]
    if causal:
        s = np.where(np.tril(np.ones((N, N), bool)), s, -np.inf)
    H = s.shape[0]
    ref = np.full((H, N), -np.inf)
    rises = np.zeros((H, N), np.int64)
    for t in range(0, N, 64):
        mt = s[:, :, t:t + 64].max(axis=-1)
        up = np.isfinite(ref) & (mt > ref + thresh_log2)
        rises += up
        ref = np.where(up | ~np.isfinite(ref), np.maximum(ref, mt), ref)
    return rises


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("kind", ["ramp", "plateau_spikes"])
def test_running_max_rescale(ea, kind, causal, d):
    H, N = 2, 1000
    scale = 1.0 / math.sqrt(d)
    if kind == "ramp":
        q, k, v = _ramp_inputs(70 + d, H, N, d)
    else:
        q, k, v = _plateau_spike_inputs(80 + d, H, N, d)
    rises = _max_rises(q, k, scale, causal)
    # the inputs do what they are for: most rows past the first spike or
    # tile rescale mid-row, the ramp rows several times
    late = rises[:, 700:]
    assert (late >= 1).mean() > 0.9, kind
    if kind == "ramp":
        assert np.median(late) >= 5
    print(f"[case] running-max rescale {kind} causal={causal} d={d}: "
          f"rises per row median {np.median(rises):.0f}, max {rises.max()}", flush=True)
    o, lse = ea.fwd(to_dev(q), to_dev(k), to_dev(v), causal=causal, scale=scale)
    torch.cuda.synchronize()
    ro, rl = oracle.fwd(q, k, v, scale=scale, causal=causal)
    eo, el = compare(bf16_to_f64(o), lse.cpu().numpy(), ro, rl, f"rescale {kind}")
    print(f"[case] rescale {kind}: max|dO|={eo:.3e} max|dLSE|={el:.3e}", flush=True)
    if kind == "plateau_spikes":
        # the plateau's share of the weight is what a wrong alpha would get
        # wrong: it must be substantial on the rows checked
        share = ro[0, 0, 300:599, :].mean(axis=-1)
        assert share.min() < 0.97 and share.max() > 0.5
