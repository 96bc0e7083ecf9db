"""GPU parity of split-KV decode (split + combine kernels) against the fp64
oracle, element by element, through the C ABI."""
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


def run_decode(ea, *, B, Hq, Hkv, T, d, seed, lens, chunk=1024, label=""):
    q, kc, vc, _ = gen.decode_inputs(seed, B, Hq, Hkv, T, d)
    lens = np.asarray(lens, np.int32)
    scale = 1.0 / math.sqrt(d)
    print(f"[case] {label} B={B} Hq={Hq} Hkv={Hkv} T={T} d={d} chunk={chunk} "
          f"lens={lens.tolist()}", flush=True)
    o, lse = ea.decode(to_dev(q), to_dev(kc), to_dev(vc), torch.from_numpy(lens).cuda(),
                       scale=scale, chunk=chunk)
    torch.cuda.synchronize()
    ro, rl = oracle.decode(q, kc, vc, lens, scale=scale)
    return compare(bf16_to_f64(o), lse.cpu().numpy(), ro, rl, label)


def test_decode_gqa4_edges(ea):
    run_decode(ea, B=6, Hq=8, Hkv=2, T=3000, d=128, seed=101,
               lens=[1, 1023, 1024, 1025, 2049, 3000], label="gqa4 lens edges")


@pytest.mark.parametrize("chunk", [64, 256, 2048])
def test_decode_chunk_sizes(ea, chunk):
    run_decode(ea, B=3, Hq=8, Hkv=2, T=4100, d=128, seed=102, lens=[4100, 77, 2500],
               chunk=chunk, label=f"chunk {chunk}")


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (8, 4), (8, 1), (16, 2), (12, 1), (6, 2)])
def test_decode_group_sizes(ea, Hq, Hkv):
    run_decode(ea, B=2, Hq=Hq, Hkv=Hkv, T=1500, d=128, seed=103 + Hq, lens=[1500, 333],
               label=f"Hq={Hq} Hkv={Hkv}")


def test_decode_d64(ea):
    run_decode(ea, B=3, Hq=8, Hkv=2, T=2100, d=64, seed=104, lens=[2100, 1, 1500], label="d64")


def test_decode_zero_length(ea):
    q, kc, vc, _ = gen.decode_inputs(105, 2, 4, 1, 500, 128)
    lens = torch.tensor([0, 300], dtype=torch.int32, device="cuda")
    o, lse = ea.decode(to_dev(q), to_dev(kc), to_dev(vc), lens)
    torch.cuda.synchronize()
    assert torch.all(o[0] == 0) and torch.all(torch.isneginf(lse[0]))
    ro, rl = oracle.decode(q, kc, vc, lens.cpu().numpy(), scale=1 / math.sqrt(128))
    compare(bf16_to_f64(o)[1:], lse.cpu().numpy()[1:], ro[1:], rl[1:], "len 0 neighbour")


def test_decode_never_reads_past_lens(ea):
    # NaN in every cache slot at or beyond lens[b]: output must be bitwise the same.
    B, Hq, Hkv, T, d = 4, 8, 2, 2600, 128
    q, kc, vc, _ = gen.decode_inputs(106, B, Hq, Hkv, T, d)
    lens = np.array([1, 1025, 2048, 2599], np.int32)
    kc2, vc2 = kc.copy(), vc.copy()
    for b in range(B):
        kc2[b, :, lens[b]:] = 0x7FC0
        vc2[b, :, lens[b]:] = 0x7FC0
    L = torch.from_numpy(lens).cuda()
    o1, l1 = ea.decode(to_dev(q), to_dev(kc), to_dev(vc), L)
    o2, l2 = ea.decode(to_dev(q), to_dev(kc2), to_dev(vc2), L)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.all(torch.isfinite(o2.float()))


def test_decode_strided_cache(ea):
    # cache stored [B, T, Hkv, d] and viewed as [B, Hkv, T, d]
    B, Hq, Hkv, T, d = 2, 8, 2, 1800, 128
    q, kc, vc, _ = gen.decode_inputs(107, B, Hq, Hkv, T, d)
    lens = torch.tensor([1800, 999], dtype=torch.int32, device="cuda")
    K, V = to_dev(kc), to_dev(vc)
    Kt = K.transpose(1, 2).contiguous().transpose(1, 2)
    Vt = V.transpose(1, 2).contiguous().transpose(1, 2)
    o1, l1 = ea.decode(to_dev(q), K, V, lens)
    o2, l2 = ea.decode(to_dev(q), Kt, Vt, lens)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_decode_workspace_reuse(ea):
    # One workspace serves consecutive calls with different lengths (every
    # chunk partial a call reads is written by that call): each result equals
    # the one computed with a fresh workspace.
    B, Hq, Hkv, T, d, chunk = 5, 8, 2, 5000, 128, 512
    q, kc, vc, _ = gen.decode_inputs(131, B, Hq, Hkv, T, d)
    Q, K, V = to_dev(q), to_dev(kc), to_dev(vc)
    ws = torch.full((ea.decode_workspace_bytes(B, Hq, T, d, chunk),), 0x7F, dtype=torch.uint8, device="cuda")
    for lens in ([5000, 1, 0, 2049, 777], [512, 4999, 3000, 0, 1], [0, 0, 0, 0, 0], [64] * 5):
        L = torch.tensor(lens, dtype=torch.int32, device="cuda")
        print(f"[case] reuse lens={lens}", flush=True)
        o1, l1 = ea.decode(Q, K, V, L, chunk=chunk, workspace=ws)
        o2, l2 = ea.decode(Q, K, V, L, chunk=chunk)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2), lens
    run_decode(ea, B=B, Hq=Hq, Hkv=Hkv, T=T, d=d, seed=131, lens=[512, 4999, 3000, 0, 1], chunk=chunk,
               label="reuse oracle")


def test_decode_long_cache(ea):
    # 131072 cached keys: 128 chunk partials per row, so the merge runs over
    # several batches of chunks; every output is checked
    run_decode(ea, B=2, Hq=8, Hkv=2, T=131072, d=128, seed=120, lens=[131072, 70001],
               label="T=131072")
