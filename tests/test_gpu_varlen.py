"""GPU parity of the packed variable-length forward (attn_fwd_varlen) against
the fp64 oracle, element by element, through the C ABI.  Tolerances are the
forward's: max-abs 2e-2 on O, 1e-3 on LSE."""
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


def _cu(lens):
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)


def _draw(seed, tq, tk, Hq, Hkv, d, factor=1.0):
    rng = np.random.Generator(np.random.PCG64(seed))
    return (gen.draw_bf16(rng, (tq, Hq, d), factor), gen.draw_bf16(rng, (tk, Hkv, d), factor),
            gen.draw_bf16(rng, (tk, Hkv, d), factor))


def run_case(ea, lq, lk, *, Hq, Hkv, d, seed, causal=False, window=None, softcap=None,
             factor=1.0, label=""):
    cu_q, cu_k = _cu(lq), _cu(lk)
    tq, tk = int(cu_q[-1]), int(cu_k[-1])
    q, k, v = _draw(seed, tq, tk, Hq, Hkv, d, factor)
    scale = 1.0 / math.sqrt(d)
    print(f"[case] {label} nseq={len(lq)} tq={tq} tk={tk} Hq={Hq} Hkv={Hkv} d={d} causal={causal} "
          f"window={window} softcap={softcap}", flush=True)
    o, lse = ea.fwd_varlen(to_dev(q), to_dev(k), to_dev(v), torch.from_numpy(cu_q).cuda(),
                           torch.from_numpy(cu_k).cuda(), causal=causal, window=window,
                           softcap=softcap, scale=scale)
    torch.cuda.synchronize()
    ro, rl = oracle.fwd_varlen(q, k, v, cu_q, cu_k, scale=scale, causal=causal, window=window,
                               softcap=softcap)
    return compare(bf16_to_f64(o), lse.cpu().numpy(), ro, rl, label)


def test_pages_example(ea):
    # lengths [3, 5, 2] -> cu_seqlens [0, 3, 8, 10], causal
    run_case(ea, [3, 5, 2], [3, 5, 2], Hq=2, Hkv=2, d=64, seed=801, causal=True, label="3,5,2")


@pytest.mark.parametrize("d", [64, 128])
def test_random_lengths_causal_gqa(ea, d):
    rng = np.random.Generator(np.random.PCG64(802))
    lens = [int(x) for x in rng.integers(0, 700, size=9)] + [1, 128, 129]
    run_case(ea, lens, lens, Hq=4, Hkv=2, d=d, seed=803, causal=True, label=f"random causal d={d}")


def test_bidirectional(ea):
    lens = [300, 64, 65, 1000]
    run_case(ea, lens, lens, Hq=2, Hkv=1, d=128, seed=804, label="bidirectional")


def test_unequal_lengths_causal(ea):
    # fewer queries than keys (a prefix of cached keys) and more queries than keys
    run_case(ea, [200, 1, 700, 300], [900, 513, 700, 100], Hq=4, Hkv=4, d=128, seed=805,
             causal=True, label="unequal causal")


def test_unequal_lengths_window_softcap(ea):
    # unit-scale inputs (the O bound is absolute) with a cap small enough to bite
    run_case(ea, [500, 33, 800], [650, 33, 1200], Hq=2, Hkv=2, d=128, seed=806, causal=True,
             window=(150, 0), softcap=1.5, label="unequal window+cap")


def test_empty_sequences_and_keys(ea):
    # sequences with no queries, with no keys, and nothing at all
    run_case(ea, [0, 70, 10, 0, 90], [40, 0, 10, 0, 200], Hq=2, Hkv=2, d=64, seed=807,
             causal=True, label="empty")


def test_no_keys_at_all(ea):
    run_case(ea, [5, 7], [0, 0], Hq=2, Hkv=2, d=64, seed=808, label="no keys")


def test_packed_documents_match_docs_mask(ea):
    # equal query and key offsets: the same result as the documents mask on
    # a one-row batch (both compared with the oracle; their tile
    # decompositions are identical, so also bitwise)
    rng = np.random.Generator(np.random.PCG64(809))
    N = 3000
    offs = gen.draw_doc_offsets(rng, 1, N, 100, 900)[0]
    q, k, v = _draw(810, N, N, 8, 2, 128)
    cu = torch.from_numpy(offs.astype(np.int32)).cuda()
    o1, l1 = ea.fwd_varlen(to_dev(q), to_dev(k), to_dev(v), cu, cu, causal=True)
    padded, _ = gen.pad_offsets([offs], N)
    q4, k4, v4 = (to_dev(np.ascontiguousarray(np.swapaxes(x, 0, 1))[None]) for x in (q, k, v))
    o2, l2 = ea.fwd(q4, k4, v4, causal=True, doc_offsets=torch.from_numpy(padded).cuda())
    torch.cuda.synchronize()
    assert torch.equal(o1, o2[0].transpose(0, 1))
    assert torch.equal(l1, l2[0])


def test_full_size_packed_documents(ea):
    # the GQA document workload (2 x 8192 tokens, documents U[256, 4096], 32
    # query heads over 8 KV heads, d 128) packed into one varlen call:
    # every output equal, bit for bit, to the documents-mask forward of the
    # same inputs (which the full-size forward test checks on every row
    # against the oracle), and sampled rows against the varlen oracle
    c = gen.CONFIGS[4]
    q4, k4, v4, docs = gen.fwd_inputs(c["seed"], c["B"], c["Hq"], c["Hkv"], c["N"], c["d"],
                                      c["factor"], docs=True)
    N = c["N"]
    q = np.concatenate([np.swapaxes(q4[b], 0, 1) for b in range(c["B"])])
    k = np.concatenate([np.swapaxes(k4[b], 0, 1) for b in range(c["B"])])
    v = np.concatenate([np.swapaxes(v4[b], 0, 1) for b in range(c["B"])])
    cu = np.concatenate([docs[0][:-1], docs[1] + N]).astype(np.int32)
    print(f"[case] full-size packed documents tq={q.shape[0]} nseq={len(cu) - 1}", flush=True)
    scale = 1.0 / math.sqrt(c["d"])
    cud = torch.from_numpy(cu).cuda()
    o, lse = ea.fwd_varlen(to_dev(q), to_dev(k), to_dev(v), cud, cud, causal=True, scale=scale)
    torch.cuda.synchronize()
    rng = np.random.Generator(np.random.PCG64(811))
    rows = np.stack([rng.integers(0, c["Hq"], 48), rng.integers(0, q.shape[0], 48)], axis=1)
    rows = np.concatenate([rows, [[0, 0], [31, q.shape[0] - 1], [5, N - 1], [6, N]]])
    ro, rl = oracle.fwd_varlen(q, k, v, cu, cu, scale=scale, causal=True, rows=rows)
    og = bf16_to_f64(o)[rows[:, 1], rows[:, 0]]
    lg = lse.cpu().numpy()[rows[:, 0], rows[:, 1]]
    compare(og, lg, ro, rl, "full-size packed documents")
    padded, _ = gen.pad_offsets(docs, N)
    o2, l2 = ea.fwd(to_dev(q4), to_dev(k4), to_dev(v4), causal=True, scale=scale,
                    doc_offsets=torch.from_numpy(padded).cuda())
    torch.cuda.synchronize()
    B = c["B"]
    assert torch.equal(o, o2.transpose(1, 2).reshape(B * N, c["Hq"], c["d"])), "packed O differs from the docs mask"
    assert torch.equal(lse, l2.transpose(0, 1).reshape(c["Hq"], B * N)), "packed LSE differs from the docs mask"
