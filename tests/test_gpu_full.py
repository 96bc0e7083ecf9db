"""Parity at the full workload sizes, in the launch configuration the
benchmark times (same C-ABI calls, same seeded inputs, prebuilt block mask).
Every output row of the causal MHA, window + cap and GQA-document forward
workloads and every decode output is compared with the fp64 oracle."""
import numpy as np
import pytest

import bench
import oracle
from tests.helpers import bf16_to_f64, compare

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
