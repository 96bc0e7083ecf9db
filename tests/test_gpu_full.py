"""Parity at the full workload sizes, in the launch configuration the
benchmark times (same C-ABI calls, same seeded inputs, prebuilt block mask).
Every output row of the causal MHA, window + cap and GQA-document forward
workloads and every decode output is compared with the fp64 oracle; the
backward of the causal MHA workload is compared on eight whole (batch row,
head) slices."""
import numpy as np
import pytest

import attn_inputs as gen
import bench
import oracle
from tests.helpers import bf16_to_f64, compare, compare_grads, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def ea():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_attention_15_amd as ea
    ea.library()
    return ea


@pytest.mark.parametrize("cid", [2, 3, 4])
def test_full_size_forward_every_row(ea, cid):
    dev = torch.device("cuda", 0)
    w = bench.fwd_workload(cid, dev)
    c = w["cfg"]
    B, H, N, d = c["B"], c["Hq"], c["N"], c["d"]
    print(f"[case] full-size config {cid} {c['name']}", flush=True)
    spec = ea.MaskSpec(**w["kw_dev"])
    bm = ea.mask_build(spec, B, N)
    o, lse = ea.fwd(w["q"], w["k"], w["v"], spec=spec, scale=w["scale"], block_mask=bm)
    torch.cuda.synchronize()
    # every row, one batch row at a time (the oracle's fp64 output of one
    # batch row is Hq * N * d * 8 bytes)
    hh, ii = np.meshgrid(np.arange(H, dtype=np.int32), np.arange(N, dtype=np.int32), indexing="ij")
    worst_o = worst_l = 0.0
    for b in range(B):
        rows = np.stack([np.full(H * N, b, np.int32), hh.ravel(), ii.ravel()], axis=1)
        ro, rl = oracle.fwd(w["q_bits"], w["k_bits"], w["v_bits"], scale=w["scale"], rows=rows,
                            **w["kw_ref"])
        og = bf16_to_f64(o[b]).reshape(H * N, d)
        lg = lse[b].cpu().numpy().reshape(H * N)
        eo, el = compare(og, lg, ro, rl, f"{c['name']} batch row {b}")
        worst_o, worst_l = max(worst_o, eo), max(worst_l, el)
        print(f"[case] {c['name']} batch row {b}: max|dO|={eo:.3e} max|dLSE|={el:.3e}", flush=True)
        del ro, rl, og
    print(f"[case] {c['name']} every row: max|dO|={worst_o:.3e} max|dLSE|={worst_l:.3e}", flush=True)


def test_full_size_decode_all_outputs(ea):
    dev = torch.device("cuda", 0)
    w = bench.decode_workload(dev)
    c = w["cfg"]
    print(f"[case] full-size decode {c['name']} lens={w['lens'].tolist()}", flush=True)
    o, lse = ea.decode(w["q"], w["k"], w["v"], w["lens_dev"], scale=w["scale"], chunk=c["chunk"])
    torch.cuda.synchronize()
    ro, rl = oracle.decode(w["q_bits"], w["k_bits"], w["v_bits"], w["lens"], scale=w["scale"])
    eo, el = compare(bf16_to_f64(o), lse.cpu().numpy(), ro, rl, c["name"])
    print(f"[case] {c['name']}: max|dO|={eo:.3e} max|dLSE|={el:.3e}", flush=True)


# (batch row, head) slices of the backward check: every batch row once, the
# heads spread over the range.  Each slice covers all 32 key blocks of its
# head in the dK/dV kernel and all 32 query tiles in the dQ kernel.
BWD_SLICES = [(0, 0), (1, 9), (2, 18), (3, 27), (4, 4), (5, 13), (6, 22), (7, 31)]


def test_full_size_backward_slices(ea):
    """The backward as the benchmark runs it: the causal MHA workload
    (B 8, H 32, N 4096, d 128), its own forward O and LSE, the seeded dO and
    one attn_bwd call on the whole batch.  With one query head per KV head a
    slice's dQ, dK and dV depend on that slice's Q, K, V and dO alone, so
    the oracle's exact gradients of the eight slices, taken as the heads of
    one batch row, are compared with those slices of the GPU gradients,
    every element, to the backward bound of the smaller cases."""
    dev = torch.device("cuda", 0)
    w = bench.fwd_workload(6, dev)
    c = w["cfg"]
    B, Hq, Hkv, N, d = c["B"], c["Hq"], c["Hkv"], c["N"], c["d"]
    assert Hq == Hkv
    print(f"[case] full-size backward {c['name']} slices {BWD_SLICES}", flush=True)
    spec = ea.MaskSpec(**w["kw_dev"])
    g_bits = gen.dout_input(c["dout_seed"], B, Hq, N, d)
    g = to_dev(g_bits, dev)
    o, lse = ea.fwd(w["q"], w["k"], w["v"], spec=spec, scale=w["scale"])
    dq, dk, dv = ea.bwd(w["q"], w["k"], w["v"], o, lse, g, spec=spec, scale=w["scale"])
    torch.cuda.synchronize()
    bs = [b for b, _ in BWD_SLICES]
    hs = [h for _, h in BWD_SLICES]

    def pick(a):
        return np.ascontiguousarray(a[bs, hs][None])

    ref = oracle.bwd(pick(w["q_bits"]), pick(w["k_bits"]), pick(w["v_bits"]), pick(g_bits),
                     scale=w["scale"], **w["kw_ref"])
    got = tuple(bf16_to_f64(t[bs, hs])[None] for t in (dq, dk, dv))
    errs = compare_grads(got, ref, lse[bs, hs].cpu().numpy()[None], f"full-size backward {c['name']}")
    print(f"[case] full-size backward: max err / max|ref| dq {errs[0]:.2e} dk {errs[1]:.2e} "
          f"dv {errs[2]:.2e}", flush=True)
