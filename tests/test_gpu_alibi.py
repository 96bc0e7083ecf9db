"""GPU parity of the forward with the ALiBi distance bias against the fp64
oracle, element by element, through the C ABI (max-abs 2e-2 on O, 1e-3 on
LSE).  Slopes follow a geometric sequence over the heads, as ALiBi is
usually configured; the library takes them as an input."""
import math

import numpy as np
import pytest

import attn_inputs as gen
import oracle
from tests.helpers import bf16_to_f64, compare, sample_rows, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def ea():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_attention_15_amd as ea
    ea.library()
    return ea


def geometric_slopes(H, top=8.0):
    return np.array([2.0 ** (-top * (h + 1) / H) for h in range(H)], dtype=np.float32)


def run_case(ea, *, B, Hq, Hkv, N, d, seed, slopes, causal=False, window=None, softcap=None,
             docs=None, rows=None, label=""):
    q, k, v, _ = gen.fwd_inputs(seed, B, Hq, Hkv, N, d)
    scale = 1.0 / math.sqrt(d)
    kw_dev, kw_ref = {}, {}
    if docs is not None:
        padded, _ = gen.pad_offsets(docs, N)
        kw_dev["doc_offsets"] = torch.from_numpy(padded).cuda()
        kw_ref["doc_offsets"] = padded
    print(f"[case] {label} B={B} Hq={Hq} Hkv={Hkv} N={N} d={d} causal={causal} window={window} "
          f"softcap={softcap} docs={docs is not None}", flush=True)
    o, lse = ea.fwd(to_dev(q), to_dev(k), to_dev(v), causal=causal, window=window, softcap=softcap,
                    scale=scale, alibi_slopes=torch.from_numpy(slopes).cuda(), **kw_dev)
    torch.cuda.synchronize()
    sl = slopes.astype(np.float64)
    if rows is None:
        ro, rl = oracle.fwd(q, k, v, scale=scale, causal=causal, window=window, softcap=softcap,
                            alibi_slopes=sl, **kw_ref)
        return compare(bf16_to_f64(o), lse.cpu().numpy(), ro, rl, label)
    ro, rl = oracle.fwd(q, k, v, scale=scale, causal=causal, window=window, softcap=softcap,
                        alibi_slopes=sl, rows=rows, **kw_ref)
    og = bf16_to_f64(o)[rows[:, 0], rows[:, 1], rows[:, 2]]
    lg = lse.cpu().numpy()[rows[:, 0], rows[:, 1], rows[:, 2]]
    return compare(og, lg, ro, rl, label)


@pytest.mark.parametrize("d", [64, 128])
def test_causal_gqa(ea, d):
    run_case(ea, B=2, Hq=8, Hkv=2, N=1000, d=d, seed=901, slopes=geometric_slopes(8), causal=True,
             label=f"alibi causal d={d}")


def test_bidirectional(ea):
    run_case(ea, B=1, Hq=4, Hkv=4, N=777, d=64, seed=902, slopes=geometric_slopes(4),
             label="alibi bidirectional")


@pytest.mark.parametrize("d", [64, 128])
def test_window_softcap(ea, d):
    # a cap small enough to bite on the biased scores
    run_case(ea, B=1, Hq=4, Hkv=2, N=1500, d=d, seed=903 if d == 128 else 913,
             slopes=geometric_slopes(4, 4.0), window=300, softcap=2.0, label=f"alibi window+cap d={d}")


def test_documents(ea):
    rng = np.random.Generator(np.random.PCG64(904))
    docs = gen.draw_doc_offsets(rng, 2, 2000, 100, 700)
    run_case(ea, B=2, Hq=4, Hkv=2, N=2000, d=128, seed=905, slopes=geometric_slopes(4),
             causal=True, docs=docs, label="alibi docs")


def test_steep_zero_and_negative_slopes(ea):
    # slope 4 leaves almost only the diagonal; slope 0 is no bias; a negative
    # slope favours distant keys (the bias is -slope * |i - j| as given)
    run_case(ea, B=1, Hq=4, Hkv=4, N=600, d=128, seed=906,
             slopes=np.array([4.0, 0.0, 1e-3, -0.01], np.float32), causal=True,
             label="alibi steep/zero/negative")


def test_full_size_headline_every_row(ea):
    # the causal MHA workload (B8 H32 N4096 d128) with ALiBi: every output
    # row, one batch row at a time
    c = gen.CONFIGS[2]
    B, H, N, d = c["B"], c["Hq"], c["N"], c["d"]
    q, k, v, _ = gen.fwd_inputs(c["seed"], B, H, c["Hkv"], N, d, c["factor"])
    slopes = geometric_slopes(H)
    scale = 1.0 / math.sqrt(d)
    print("[case] full-size causal MHA with ALiBi, every row", flush=True)
    o, lse = ea.fwd(to_dev(q), to_dev(k), to_dev(v), causal=True, scale=scale,
                    alibi_slopes=torch.from_numpy(slopes).cuda())
    torch.cuda.synchronize()
    hh, ii = np.meshgrid(np.arange(H, dtype=np.int32), np.arange(N, dtype=np.int32), indexing="ij")
    worst_o = worst_l = 0.0
    for b in range(B):
        rows = np.stack([np.full(H * N, b, np.int32), hh.ravel(), ii.ravel()], axis=1)
        ro, rl = oracle.fwd(q, k, v, scale=scale, causal=True, alibi_slopes=slopes.astype(np.float64),
                            rows=rows)
        eo, el = compare(bf16_to_f64(o[b]).reshape(H * N, d), lse[b].cpu().numpy().reshape(H * N), ro, rl,
                         f"full-size alibi batch row {b}")
        worst_o, worst_l = max(worst_o, eo), max(worst_l, el)
        del ro, rl
    print(f"[case] full-size alibi every row: max|dO|={worst_o:.3e} max|dLSE|={worst_l:.3e}", flush=True)
