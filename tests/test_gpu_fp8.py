"""GPU checks of the FP8 path through the C ABI.

Quantizer: the E4M3 codes and the power-of-two scales must equal the
oracle's bit for bit (both divide exactly by a power of two and round to
nearest even; the rotation's butterflies are the same fp32 operations).

Forward: compared with the fp64 oracle run on the dequantized inputs (codes
times scales, which are exact bf16 values), so the only difference left is
the kernel's rounding of the probabilities to E4M3 and fp32 accumulation.
The kernel encodes p * 2^6 with p taken against a reference max that trails
the row max by at most a factor 4, so p * 2^6 <= 256.  In E4M3 (3 mantissa
bits, round to nearest) that is off by at most 2^-4 relative, or 2^-10
absolute below the normal range, i.e. 2^-16 in units of p; with the oracle's
normalized probabilities P and the dequantized V, per output element
    |O - O_ref| <= 2^-4 * sum_j P_ij |v_jt| + 2^-16 * sum_j |v_jt|
                   + 2^-8 |O_ref| + 1e-5
(the last two terms: the bf16 output and fp32 sums).  The LSE uses the
unrounded probabilities: 1e-3, as the bf16 path.
"""
import math

import numpy as np
import pytest

import attn_inputs as gen
import oracle
from tests.helpers import bf16_to_f64, sample_rows, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def ea():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_attention_15_amd as ea
    ea.library()
    return ea


def _signs(seed, d=128):
    return gen.hadamard_signs(seed, d)


@pytest.mark.parametrize("per_head", [False, True])
@pytest.mark.parametrize("rotate", [False, True])
def test_quantizer_bitexact(ea, rotate, per_head):
    B, H, N = 2, 3, 150
    x = gen.draw_bf16(np.random.Generator(np.random.PCG64(1300)), (B, H, N, 128), 1.0)
    x[1, 2, 100] = gen.bf16_bits_from_f32(np.linspace(-60, 60, 128).astype(np.float32))
    signs = _signs(1301) if rotate else None
    print(f"[case] quantizer rotate={rotate} per_head={per_head}", flush=True)
    codes, scales = ea.quantize_fp8(to_dev(x), per_head=per_head,
                                    signs=None if signs is None else torch.from_numpy(signs).cuda())
    torch.cuda.synchronize()
    rc, rs = oracle.quantize_fp8(x, signs=signs, per_head=per_head)
    assert np.array_equal(scales.cpu().numpy(), rs)
    got = codes.cpu().numpy()
    assert np.array_equal(got, rc), f"{int((got != rc).sum())} codes differ"


def _quantized_inputs(ea, seed, B, Hq, Hkv, N, rotate):
    q, k, v, docs = gen.fwd_inputs(seed, B, Hq, Hkv, N, 128)
    sg = _signs(seed + 1) if rotate else None
    sgd = None if sg is None else torch.from_numpy(sg).cuda()
    Q8, QS = ea.quantize_fp8(to_dev(q), signs=sgd)
    K8, KS = ea.quantize_fp8(to_dev(k), signs=sgd)
    V8, VS = ea.quantize_fp8(to_dev(v), per_head=True)
    rq = oracle.dequantize_fp8(*oracle.quantize_fp8(q, signs=sg))
    rk = oracle.dequantize_fp8(*oracle.quantize_fp8(k, signs=sg))
    rv = oracle.dequantize_fp8(*oracle.quantize_fp8(v, per_head=True))
    return (Q8, K8, V8, QS, KS, VS), (rq, rk, rv)


def _check(o, lse, ro, rl, pv, vsum, label):
    """o, ro [n, d]; lse, rl [n]; pv [n, d] = sum_j P_ij |v_jt| with the
    oracle's probabilities; vsum [n, d] = sum_j |v_jt| over the row's KV head."""
    bound = 2.0 ** -4 * pv + 2.0 ** -16 * vsum + 2.0 ** -8 * np.abs(ro) + 1e-5
    err = np.abs(o - ro)
    assert np.all(np.isfinite(o)), f"{label}: non-finite output"
    worst = float((err / bound).max())
    assert np.all(err <= bound), f"{label}: error/bound = {worst:.3f}"
    fin = np.isfinite(rl)
    assert np.array_equal(np.isneginf(lse), ~fin)
    el = float(np.abs(lse[fin] - rl[fin]).max()) if fin.any() else 0.0
    assert el <= 1e-3, f"{label}: max|dLSE| = {el:.3e}"
    print(f"[ok] {label}: max error/bound {worst:.3f}, max|dLSE| {el:.2e}, "
          f"max|dO| {float(err.max()):.2e}", flush=True)


def run_case(ea, *, B, Hq, Hkv, N, seed, rotate=True, causal=False, window=None, softcap=None,
             docs=None, label=""):
    print(f"[case] {label} B={B} Hq={Hq} Hkv={Hkv} N={N} causal={causal} window={window} "
          f"softcap={softcap} docs={docs is not None} rotate={rotate}", flush=True)
    dev, ref = _quantized_inputs(ea, seed, B, Hq, Hkv, N, rotate)
    kw_dev, kw_ref = {}, {}
    if docs is not None:
        padded, _ = gen.pad_offsets(docs, N)
        kw_dev["doc_offsets"] = torch.from_numpy(padded).cuda()
        kw_ref["doc_offsets"] = padded
    scale = 1.0 / math.sqrt(128)
    o, lse = ea.fwd_fp8(*dev, causal=causal, window=window, softcap=softcap, scale=scale, **kw_dev)
    torch.cuda.synchronize()
    rq, rk, rv = ref
    ro, rl, P = oracle.fwd(rq, rk, rv, scale=scale, causal=causal, window=window, softcap=softcap,
                           want_probs=True, **kw_ref)
    G = Hq // Hkv
    va = np.abs(gen.f32_from_bf16_bits(rv).astype(np.float64))  # [B, Hkv, N, d]
    pv = np.empty((B, Hq, N, 128))
    vsum = np.empty((B, Hq, N, 128))
    for b in range(B):
        for h in range(Hq):
            pv[b, h] = P[b, h] @ va[b, h // G]
            vsum[b, h] = va[b, h // G].sum(axis=0)
    _check(bf16_to_f64(o).reshape(-1, 128), lse.cpu().numpy().reshape(-1), ro.reshape(-1, 128),
           rl.reshape(-1), pv.reshape(-1, 128), vsum.reshape(-1, 128), label)


def test_causal_gqa_rotated(ea):
    run_case(ea, B=2, Hq=4, Hkv=2, N=300, seed=1310, causal=True, label="fp8 causal GQA")


def test_bidirectional_ragged(ea):
    run_case(ea, B=1, Hq=2, Hkv=2, N=333, seed=1311, rotate=False, label="fp8 bidirectional")


def test_window_softcap(ea):
    run_case(ea, B=1, Hq=2, Hkv=1, N=400, seed=1312, window=100, softcap=2.0,
             label="fp8 window+cap")


def test_documents(ea):
    rng = np.random.Generator(np.random.PCG64(1313))
    docs = gen.draw_doc_offsets(rng, 2, 350, 60, 200)
    run_case(ea, B=2, Hq=2, Hkv=2, N=350, seed=1314, causal=True, docs=docs, label="fp8 docs")


def test_full_size_headline_slices(ea):
    # the causal MHA workload (B8 H32 N4096 d128), rotated and quantized:
    # every row of sixteen (batch row, head) slices, two per batch row with
    # the heads spread over the range (each slice spans every query and key
    # tile of its head)
    c = gen.CONFIGS[2]
    B, H, N = c["B"], c["Hq"], c["N"]
    q, k, v, _ = gen.fwd_inputs(c["seed"], B, H, H, N, 128, c["factor"])
    sg = _signs(1320)
    sgd = torch.from_numpy(sg).cuda()
    print("[case] full-size fp8 causal MHA", flush=True)
    Q8, QS = ea.quantize_fp8(to_dev(q), signs=sgd)
    K8, KS = ea.quantize_fp8(to_dev(k), signs=sgd)
    V8, VS = ea.quantize_fp8(to_dev(v), per_head=True)
    o, lse = ea.fwd_fp8(Q8, K8, V8, QS, KS, VS, causal=True)
    torch.cuda.synchronize()
    slices = [(b, (5 * b + 16 * j) % H) for b in range(B) for j in range(2)]
    o_np, l_np = bf16_to_f64(o), lse.cpu().numpy()
    scale = 1.0 / math.sqrt(128)
    loc = np.stack([np.zeros(N, np.int32), np.zeros(N, np.int32), np.arange(N, dtype=np.int32)], axis=1)
    for b, h in slices:
        qh = oracle.dequantize_fp8(*oracle.quantize_fp8(q[b:b + 1, h:h + 1], signs=sg))
        kh = oracle.dequantize_fp8(*oracle.quantize_fp8(k[b:b + 1, h:h + 1], signs=sg))
        vh = oracle.dequantize_fp8(*oracle.quantize_fp8(v[b:b + 1, h:h + 1], per_head=True))
        ro, rl, P = oracle.fwd(qh, kh, vh, scale=scale, causal=True, rows=loc, want_probs=True)
        va = np.abs(gen.f32_from_bf16_bits(vh[0, 0]).astype(np.float64))
        _check(o_np[b, h], l_np[b, h], ro, rl, P @ va, np.broadcast_to(va.sum(axis=0), (N, 128)),
               f"full-size b={b} h={h}")
        del P


def test_rotation_lowers_end_to_end_error_with_outliers(ea):
    # against the unquantized bf16 attention: with outlier channels in Q and
    # K the rotated path is closer (the pages' reason for incoherent
    # processing)
    B, H, N = 1, 4, 512
    rng = np.random.Generator(np.random.PCG64(1330))
    qf = rng.standard_normal((B, H, N, 128)).astype(np.float32)
    kf = rng.standard_normal((B, H, N, 128)).astype(np.float32)
    qf[..., :4] *= 20.0
    kf[..., :4] *= 20.0
    q, k = gen.bf16_bits_from_f32(qf), gen.bf16_bits_from_f32(kf)
    v = gen.draw_bf16(rng, (B, H, N, 128), 1.0)
    scale = 1.0 / math.sqrt(128)
    ref, _ = oracle.fwd(q, k, v, scale=scale * 0.25, causal=True)
    errs = []
    for sg in (None, _signs(1331)):
        sgd = None if sg is None else torch.from_numpy(sg).cuda()
        Q8, QS = ea.quantize_fp8(to_dev(q), signs=sgd)
        K8, KS = ea.quantize_fp8(to_dev(k), signs=sgd)
        V8, VS = ea.quantize_fp8(to_dev(v), per_head=True)
        o, _ = ea.fwd_fp8(Q8, K8, V8, QS, KS, VS, causal=True, scale=scale * 0.25)
        torch.cuda.synchronize()
        errs.append(float(np.sqrt(np.mean((bf16_to_f64(o) - ref) ** 2))))
    print(f"[ok] rms error vs bf16 attention: plain {errs[0]:.4f}, rotated {errs[1]:.4f}", flush=True)
    assert errs[1] < errs[0]


@pytest.mark.parametrize("N", [1, 65])
def test_ragged_small_gqa8(ea, N):
    run_case(ea, B=2, Hq=8, Hkv=1, N=N, seed=1340 + N, causal=True, label=f"fp8 N={N} GQA 8")


def test_empty_rows(ea):
    # keys i+1 .. i+2 only: the last row sees nothing -> O = 0, LSE = -inf
    run_case(ea, B=1, Hq=2, Hkv=2, N=200, seed=1343, window=(-1, 2), label="fp8 future-only")


def test_left_window_documents(ea):
    rng = np.random.Generator(np.random.PCG64(1344))
    docs = gen.draw_doc_offsets(rng, 1, 500, 40, 300)
    run_case(ea, B=1, Hq=4, Hkv=2, N=500, seed=1345, window=(100, 0), docs=docs, label="fp8 left window docs")


def _codes(ea, seed, B, Hq, Hkv, N):
    q, k, v, _ = gen.fwd_inputs(seed, B, Hq, Hkv, N, 128)
    sg = torch.from_numpy(_signs(seed + 1)).cuda()
    return (*ea.quantize_fp8(to_dev(q), signs=sg), *ea.quantize_fp8(to_dev(k), signs=sg),
            *ea.quantize_fp8(to_dev(v), per_head=True))


@pytest.mark.parametrize("kind", ["causal", "window", "docs"])
def test_block_skipping_is_bitwise_neutral(ea, kind):
    N = 1500
    Q8, QS, K8, KS, V8, VS = _codes(ea, 1350, 1, 4, 2, N)
    if kind == "causal":
        kw = dict(causal=True)
    elif kind == "window":
        kw = dict(window=200, softcap=50.0)
    else:
        rng = np.random.Generator(np.random.PCG64(1351))
        padded, _ = gen.pad_offsets(gen.draw_doc_offsets(rng, 1, N, 100, 500), N)
        kw = dict(causal=True, doc_offsets=torch.from_numpy(padded).cuda())
    print(f"[case] fp8 skipping neutral {kind}", flush=True)
    o1, l1 = ea.fwd_fp8(Q8, K8, V8, QS, KS, VS, **kw)
    o2, l2 = ea.fwd_fp8(Q8, K8, V8, QS, KS, VS, no_skip=True, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_strided_layout_bnhd(ea):
    # codes stored [B, N, H, 128] and viewed as [B, H, N, 128]: same result
    Q8, QS, K8, KS, V8, VS = _codes(ea, 1352, 2, 4, 2, 600)
    t = lambda x: x.transpose(1, 2).contiguous().transpose(1, 2)
    Q8t, K8t, V8t = t(Q8), t(K8), t(V8)
    assert Q8t.stride(2) == 4 * 128 and not Q8t.is_contiguous()
    print("[case] fp8 strided codes", flush=True)
    o1, l1 = ea.fwd_fp8(Q8, K8, V8, QS, KS, VS, causal=True)
    out = torch.empty(2, 600, 4, 128, dtype=torch.bfloat16, device="cuda").transpose(1, 2)
    o2, l2 = ea.fwd_fp8(Q8t, K8t, V8t, QS, KS, VS, causal=True, out=out)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_empty_inputs(ea):
    # B = 0 and N = 0 are valid calls that do nothing
    for B, N in ((0, 64), (2, 0)):
        x = torch.empty(B, 2, N, 128, dtype=torch.bfloat16, device="cuda")
        codes, scales = ea.quantize_fp8(x)
        o, lse = ea.fwd_fp8(codes, codes, codes, scales, scales, scales, causal=True)
        torch.cuda.synchronize()
        assert o.shape == (B, 2, N, 128) and lse.shape == (B, 2, N)


def test_binding_rejects_bad_shapes(ea):
    # scale tensors and code tensors are checked before anything is launched
    Q8, QS, K8, KS, V8, VS = _codes(ea, 1360, 1, 2, 1, 100)
    with pytest.raises(ValueError):
        ea.fwd_fp8(Q8, K8, V8, QS[:, :, :1], KS, VS, causal=True)
    with pytest.raises(ValueError):
        ea.fwd_fp8(Q8, K8[:, :, :64], V8, QS, KS, VS, causal=True)
    with pytest.raises(ValueError):
        ea.quantize_fp8(torch.zeros(1, 2, 100, 128, dtype=torch.bfloat16, device="cuda"),
                        scales=torch.empty(1, 2, 1, device="cuda"))


def test_long_sequence_sampled(ea):
    # 65536 tokens in FP8 (1024 quantization blocks per head), causal,
    # rotated, on sampled rows
    from tests.helpers import sample_rows
    N = 65536
    q, k, v, _ = gen.fwd_inputs(1370, 1, 2, 2, N, 128)
    sg = _signs(1371)
    sgd = torch.from_numpy(sg).cuda()
    print("[case] fp8 causal N=65536", flush=True)
    Q8, QS = ea.quantize_fp8(to_dev(q), signs=sgd)
    K8, KS = ea.quantize_fp8(to_dev(k), signs=sgd)
    V8, VS = ea.quantize_fp8(to_dev(v), per_head=True)
    o, lse = ea.fwd_fp8(Q8, K8, V8, QS, KS, VS, causal=True)
    torch.cuda.synchronize()
    rng = np.random.Generator(np.random.PCG64(1372))
    rows = sample_rows(rng, 1, 2, N, 12, must=[(0, 0, 0), (0, 1, N - 1), (0, 0, 32768)])
    rq = oracle.dequantize_fp8(*oracle.quantize_fp8(q, signs=sg))
    rk = oracle.dequantize_fp8(*oracle.quantize_fp8(k, signs=sg))
    rv = oracle.dequantize_fp8(*oracle.quantize_fp8(v, per_head=True))
    scale = 1.0 / math.sqrt(128)
    o_np, l_np = bf16_to_f64(o), lse.cpu().numpy()
    for h in range(2):
        sel = rows[rows[:, 1] == h]
        loc = np.stack([np.zeros(len(sel), np.int32), np.zeros(len(sel), np.int32), sel[:, 2]], axis=1)
        ro, rl, P = oracle.fwd(rq[:, h:h + 1], rk[:, h:h + 1], rv[:, h:h + 1], scale=scale, causal=True,
                               rows=loc, want_probs=True)
        va = np.abs(gen.f32_from_bf16_bits(rv[0, h]).astype(np.float64))
        _check(o_np[0, h, sel[:, 2]], l_np[0, h, sel[:, 2]], ro, rl, P @ va,
               np.broadcast_to(va.sum(axis=0), (len(sel), 128)), f"fp8 N=65536 h={h}")
