"""GPU parity of the backward path (dQ, dK, dV) against the fp64 oracle,
element by element, through the C ABI.

The GPU side runs its own forward (bf16 O, fp32 LSE) and then the backward
on those outputs, as a training step would; the oracle computes the exact
gradients of the same bf16 inputs in fp64.

Tolerance.  Each gradient entry is a sum over up to N keys (dQ) or N rows
(dK, dV) of products in which the kernel rounds P and dS to bf16 (relative
error 2^-9 each) before the fp32-accumulated MFMA, uses the bf16-rounded O
in D = rowsum(dO * O) (2^-9), and rounds the result to bf16 (2^-9): four
roundings of 2^-9, 7.8e-3 in all.  The error is therefore a few units of
2^-9 relative to the magnitude of the entries, not of their (possibly
cancelling) sum, so it is measured against the largest entry of each
tensor: max|g - g_ref| <= GRAD_TOL * max|g_ref| with GRAD_TOL = 1e-2, just
above those four roundings (measured: at most 5.5e-3 over every case
here).  Where the exact gradient cancels to zero (a row with a
single visible key has dS = 0) the fp32 residue of D - dP is left; GRAD_ABS
= 1e-4 covers it (fp32 rounding, 2^-24, of sums of up to d unit-scale
products).  Rows with no visible key and keys that no row sees get exactly
zero.
"""
import math

import numpy as np
import pytest

import attn_inputs as gen
import oracle
from tests.helpers import bf16_to_f64, compare_grads, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

@pytest.fixture(scope="module")
def ea():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_attention_15_amd as ea
    ea.library()
    return ea


def _grad_inputs(seed, B, Hq, Hkv, N, d, factor):
    q, k, v, _ = gen.fwd_inputs(seed, B, Hq, Hkv, N, d, factor)
    return q, k, v, gen.dout_input(seed + 7919, B, Hq, N, d)


def run_case(ea, *, B, Hq, Hkv, N, d, seed, factor=1.0, causal=False, window=None,
             softcap=None, docs=None, scale=None, label=""):
    q, k, v, dout = _grad_inputs(seed, B, Hq, Hkv, N, d, factor)
    scale = scale if scale is not None else 1.0 / math.sqrt(d)
    kw_dev, kw_ref = {}, {}
    if docs is not None:
        padded, _ = gen.pad_offsets(docs, N)
        kw_dev["doc_offsets"] = torch.from_numpy(padded).cuda()
        kw_ref["doc_offsets"] = padded
    print(f"[case] {label} B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} causal={causal} "
          f"window={window} softcap={softcap} docs={docs is not None}", flush=True)
    Q, K, V, G = to_dev(q), to_dev(k), to_dev(v), to_dev(dout)
    o, lse = ea.fwd(Q, K, V, causal=causal, window=window, softcap=softcap, scale=scale, **kw_dev)
    dq, dk, dv = ea.bwd(Q, K, V, o, lse, G, causal=causal, window=window, softcap=softcap,
                        scale=scale, **kw_dev)
    torch.cuda.synchronize()
    ref = oracle.bwd(q, k, v, dout, scale=scale, causal=causal, window=window,
                     softcap=softcap, **kw_ref)
    errs = compare_grads((bf16_to_f64(dq), bf16_to_f64(dk), bf16_to_f64(dv)), ref,
                         lse.cpu().numpy(), label)
    print(f"[case] {label}: max error / max|ref| dq {errs[0]:.2e} dk {errs[1]:.2e} dv {errs[2]:.2e}",
          flush=True)
    return errs


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N", [1, 65, 1000])
def test_causal_ragged(ea, d, N):
    run_case(ea, B=2, Hq=3, Hkv=3, N=N, d=d, seed=501 + N, causal=True, factor=0.5,
             label=f"causal N={N} d={d}")


@pytest.mark.parametrize("d", [64, 128])
def test_bidirectional_gqa(ea, d):
    run_case(ea, B=1, Hq=4, Hkv=2, N=777, d=d, seed=511, label=f"no mask GQA d={d}")


@pytest.mark.parametrize("d", [64, 128])
def test_window_softcap(ea, d):
    # window 300 either side plus a tanh cap that bites (large scores)
    run_case(ea, B=1, Hq=2, Hkv=2, N=1500, d=d, seed=521, factor=2.0, window=300,
             softcap=5.0, label=f"window300+cap5 d={d}")


def test_window_1024_softcap_50(ea):
    run_case(ea, B=1, Hq=1, Hkv=1, N=2500, d=128, seed=522, window=1024, softcap=50.0,
             label="window1024+cap50")


def test_left_window_causal(ea):
    run_case(ea, B=1, Hq=2, Hkv=1, N=1300, d=128, seed=531, window=(129, 0), causal=True,
             label="left window 129 + causal")


def test_documents_gqa_causal(ea):
    rng = np.random.Generator(np.random.PCG64(541))
    N = 2000
    docs = gen.draw_doc_offsets(rng, 2, N, 100, 700)
    run_case(ea, B=2, Hq=4, Hkv=2, N=N, d=128, seed=542, causal=True, docs=docs,
             label="docs GQA causal")


def test_rows_without_keys(ea):
    # keys i+1 .. i+2 only: key 0 is never seen and the last row sees nothing
    run_case(ea, B=1, Hq=2, Hkv=2, N=300, d=64, seed=551, window=(-1, 2),
             label="right-only window")


def test_no_skip_is_bitwise_equal(ea):
    B, Hq, Hkv, N, d = 1, 4, 2, 1100, 128
    q, k, v, dout = _grad_inputs(561, B, Hq, Hkv, N, d, 1.0)
    Q, K, V, G = to_dev(q), to_dev(k), to_dev(v), to_dev(dout)
    print(f"[case] no-skip bitwise B={B} Hq={Hq} Hkv={Hkv} N={N} d={d}", flush=True)
    o, lse = ea.fwd(Q, K, V, causal=True, window=(300, 0))
    a = ea.bwd(Q, K, V, o, lse, G, causal=True, window=(300, 0))
    b = ea.bwd(Q, K, V, o, lse, G, causal=True, window=(300, 0), no_skip=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_strided_layout_bshd(ea):
    # [B, N, H, d] storage for every tensor, outputs included
    B, Hq, Hkv, N, d = 1, 4, 2, 600, 128
    q, k, v, dout = _grad_inputs(571, B, Hq, Hkv, N, d, 1.0)
    print(f"[case] bshd layout B={B} Hq={Hq} Hkv={Hkv} N={N} d={d}", flush=True)

    def bshd(x):
        return to_dev(np.ascontiguousarray(np.swapaxes(x, 1, 2))).transpose(1, 2)
    Q, K, V, G = bshd(q), bshd(k), bshd(v), bshd(dout)
    o = torch.empty((B, N, Hq, d), dtype=torch.bfloat16, device="cuda").transpose(1, 2)
    o, lse = ea.fwd(Q, K, V, causal=True, out=o)
    dq = torch.empty((B, N, Hq, d), dtype=torch.bfloat16, device="cuda").transpose(1, 2)
    dk = torch.empty((B, N, Hkv, d), dtype=torch.bfloat16, device="cuda").transpose(1, 2)
    dv = torch.empty((B, N, Hkv, d), dtype=torch.bfloat16, device="cuda").transpose(1, 2)
    ea.bwd(Q, K, V, o, lse, G, causal=True, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    ref = oracle.bwd(q, k, v, dout, scale=1.0 / math.sqrt(d), causal=True)
    compare_grads((bf16_to_f64(dq), bf16_to_f64(dk), bf16_to_f64(dv)), ref, lse.cpu().numpy(), "bshd")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("softcap", [None, 5.0])
def test_unequal_kv_token_strides(ea, d, softcap):
    # K stored [B, N, Hkv, d] (token stride Hkv*d) and V contiguous
    # [B, Hkv, N, d] (token stride d): the dQ kernels that stream K and V
    # tiles with separate offsets (the others share one set when the two
    # token strides are equal)
    B, Hq, Hkv, N = 2, 4, 2, 700
    factor = 2.0 if softcap else 1.0
    q, k, v, dout = _grad_inputs(581 + d, B, Hq, Hkv, N, d, factor)
    print(f"[case] unequal K/V token strides B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} "
          f"softcap={softcap}", flush=True)
    Q, V, G = to_dev(q), to_dev(v), to_dev(dout)
    K = to_dev(np.ascontiguousarray(np.swapaxes(k, 1, 2))).transpose(1, 2)
    assert K.stride(2) == Hkv * d and V.stride(2) == d
    o, lse = ea.fwd(Q, K, V, causal=True, window=(400, 0), softcap=softcap)
    dq, dk, dv = ea.bwd(Q, K, V, o, lse, G, causal=True, window=(400, 0), softcap=softcap)
    torch.cuda.synchronize()
    ref = oracle.bwd(q, k, v, dout, scale=1.0 / math.sqrt(d), causal=True, window=(400, 0),
                     softcap=softcap)
    errs = compare_grads((bf16_to_f64(dq), bf16_to_f64(dk), bf16_to_f64(dv)), ref,
                         lse.cpu().numpy(), f"unequal strides d={d} cap={softcap}")
    print(f"[case] relative errors dq/dk/dv {errs}", flush=True)
