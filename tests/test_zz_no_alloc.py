"""attn_decode_noalloc (the decode entry point that allocates nothing, its
chunk partials in the library's static per-GPU scratch) against attn_decode
with a caller workspace, through the C ABI: the same kernels, so the outputs
must be bitwise equal, and both within the oracle bar.  Two calls in a row,
the second smaller, so the second runs over the first call's leftover
partials in the shared scratch."""
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


def _case(ea, seed, B, Hq, Hkv, T, d, chunk, lens_lo, lens_hi):
    q, kc, vc, lens = gen.decode_inputs(seed, B, Hq, Hkv, T, d, lens_lo=lens_lo, lens_hi=lens_hi)
    print(f"[case] noalloc decode seed={seed} B={B} Hq={Hq} Hkv={Hkv} T={T} d={d} chunk={chunk} "
          f"lens={lens.tolist()}", flush=True)
    Q, K, V = to_dev(q), to_dev(kc), to_dev(vc)
    L = torch.from_numpy(lens).cuda()
    scale = 1.0 / math.sqrt(d)
    o_ref, l_ref = ea.decode(Q, K, V, L, scale=scale, chunk=chunk)
    o = torch.empty((B, Hq, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    ea.decode_noalloc(Q, K, V, L, out=o, lse=lse, scale=scale, chunk=chunk)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref), "O differs from attn_decode"
    assert torch.equal(lse, l_ref), "LSE differs from attn_decode"
    ro, rl = oracle.decode(q, kc, vc, lens, scale=scale)
    eo, el = compare(bf16_to_f64(o), lse.cpu().numpy(), ro, rl, "noalloc decode")
    print(f"[case] noalloc decode: max|dO|={eo:.3e} max|dLSE|={el:.3e}", flush=True)


def test_noalloc_decode_matches_workspace_decode_twice(ea):
    # first a large call (8 query heads per KV head, 20 chunks per row),
    # then a smaller one (fewer rows, heads and chunks) over its leftovers
    _case(ea, 1301, B=4, Hq=16, Hkv=2, T=20480, d=128, chunk=1024, lens_lo=15000, lens_hi=20480)
    _case(ea, 1302, B=2, Hq=4, Hkv=2, T=3000, d=64, chunk=256, lens_lo=1, lens_hi=3000)


def test_noalloc_decode_workload_size(ea):
    # the decode workload's shape (B16, 32 over 8 heads, T 32768, chunk 1024)
    # fits the scratch; a cache twice as long is refused before any launch
    c = gen.CONFIGS[5]
    _case(ea, c["seed"], B=c["B"], Hq=c["Hq"], Hkv=c["Hkv"], T=c["T"], d=c["d"], chunk=c["chunk"],
          lens_lo=1024, lens_hi=c["T"])
    q = torch.zeros((16, 32, 128), dtype=torch.bfloat16, device="cuda")
    # a zero-stride view: the call is refused before anything is read
    kc = torch.zeros((1, 1, 1, 128), dtype=torch.bfloat16, device="cuda").expand(16, 8, 65536, 128)
    lens = torch.full((16,), 65536, dtype=torch.int32, device="cuda")
    o = torch.empty((16, 32, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((16, 32), dtype=torch.float32, device="cuda")
    with pytest.raises(ea.AttnError) as ei:
        ea.decode_noalloc(q, kc, kc, lens, out=o, lse=lse)
    assert ei.value.status == 3  # ATTN_ERR_WORKSPACE
    assert "static" in str(ei.value)
