"""The C-ABI calls enqueue work only: no allocation, no synchronisation and
no memset inside, so they can be captured into a HIP graph.  Every replay of
the captured graph must reproduce the eager results bitwise."""
import math

import numpy as np
import pytest

import attn_inputs as gen
from tests.helpers import to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def ea():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import exact_attention_15_amd as ea
    ea.library()
    return ea


def test_graph_capture_replays_match_eager(ea):
    dev = torch.device("cuda", 0)
    # forward: causal GQA with documents, mask built inside the call
    B, Hq, Hkv, N, d = 2, 8, 2, 1500, 128
    q, k, v, _ = gen.fwd_inputs(91, B, Hq, Hkv, N, d)
    Q, K, V = to_dev(q), to_dev(k), to_dev(v)
    rng = np.random.Generator(np.random.PCG64(92))
    padded, _ = gen.pad_offsets(gen.draw_doc_offsets(rng, B, N, 100, 600), N)
    spec = ea.MaskSpec(causal=True, doc_offsets=torch.from_numpy(padded).to(dev))
    # decode
    dq, dk, dv, lens = gen.decode_inputs(93, 3, 8, 2, 3000, 128, lens_lo=1, lens_hi=3000)
    DQ, DK, DV = to_dev(dq), to_dev(dk), to_dev(dv)
    L = torch.from_numpy(lens).to(dev)
    scale = 1.0 / math.sqrt(d)

    o_ref, l_ref = ea.fwd(Q, K, V, spec=spec, scale=scale)
    do_ref, dl_ref = ea.decode(DQ, DK, DV, L, scale=scale, chunk=256)
    torch.cuda.synchronize()

    o = torch.empty_like(o_ref)
    lse = torch.empty_like(l_ref)
    do = torch.empty_like(do_ref)
    dl = torch.empty_like(dl_ref)
    ws_dec = torch.empty(ea.decode_workspace_bytes(3, 8, 3000, 128, 256), dtype=torch.uint8,
                         device=dev)

    def body():
        # the forward workspace is allocated by the binding (inside the
        # capture it comes from the graph's private pool)
        ea.fwd(Q, K, V, spec=spec, scale=scale, out=o, lse=lse)
        ea.decode(DQ, DK, DV, L, scale=scale, chunk=256, out=do, lse=dl, workspace=ws_dec)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        body()  # warm-up on a side stream, as graph capture requires
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        body()

    for rep in range(3):
        # eager work between replays: clobber the outputs
        o.zero_()
        lse.fill_(1.0)
        do.zero_()
        dl.fill_(1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), f"replay {rep}: forward output differs"
        assert torch.equal(lse, l_ref), f"replay {rep}: forward LSE differs"
        assert torch.equal(do, do_ref), f"replay {rep}: decode output differs"
        assert torch.equal(dl, dl_ref), f"replay {rep}: decode LSE differs"
