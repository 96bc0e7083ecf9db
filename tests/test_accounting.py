"""Closed forms of the benchmark's work accounting (CPU only).

The byte and FLOP formulas the benchmark divides by are pinned to sizes the
pages print and to textbook sums."""
import numpy as np

import attn_inputs as gen
import bench


def test_score_matrix_sizes_printed_on_the_pages():
    # youngju.dev "FlashAttention 논문 분석", standard-attention benchmark:
    # 4 x 32 x 4096 x 4096 x 2 bytes = 4.29 GB
    assert bench.score_matrix_bytes(4, 32, 4096) == 4 * 32 * 4096 * 4096 * 2
    assert round(bench.score_matrix_bytes(4, 32, 4096) / 1e9, 2) == 4.29
    # same page, memory analysis: batch 4, 32 heads, N = 16384 -> about 68 GB
    assert 68e9 <= bench.score_matrix_bytes(4, 32, 16384) < 69e9
    # llm-systems-engineering "Attention 최적화가 어려운 이유": one T x T 2-byte
    # matrix is 32 MiB at T = 4096 and 128 MiB at T = 8192
    assert bench.score_matrix_bytes(1, 1, 4096) == 32 * 2 ** 20
    assert bench.score_matrix_bytes(1, 1, 8192) == 128 * 2 ** 20


def test_kv_cache_exercise_sizes():
    # aegloslab "3.7 어텐션 II", exercise 3: 32 query heads, d = 128, fp16,
    # T = 16384, batch 1, K and V, with 32 / 8 / 1 KV heads
    assert bench.kv_cache_bytes(1, 32, 16384, 128) == 256 * 2 ** 20
    assert bench.kv_cache_bytes(1, 8, 16384, 128) == 64 * 2 ** 20
    assert bench.kv_cache_bytes(1, 1, 16384, 128) == 8 * 2 ** 20


def test_causal_pairs_closed_form():
    for N in (1, 7, 256, 4096):
        assert bench.visible_pairs("causal", 1, N) == N * (N + 1) // 2
    # the causal headline: 8 x 32 heads of N = 4096 at d = 128
    flops = bench.fwd_flops(bench.visible_pairs("causal", 8, 4096), 32, 128)
    assert flops == 4 * 128 * 32 * 8 * (4096 * 4097 // 2)


def test_window_pairs_closed_form():
    N, W = 16384, 1024
    expect = sum(min(i, W) + min(N - 1 - i, W) + 1 for i in range(N))
    assert bench.visible_pairs("window_softcap", 1, N, window=W) == expect
    assert expect == 32521216


def test_document_pairs_closed_form():
    rows = [gen.lengths_to_offsets([3, 5, 2]), gen.lengths_to_offsets([10])]
    assert bench.visible_pairs("docs_causal", 2, 10, doc_rows=rows) == (6 + 15 + 3) + 55


def test_decode_bytes():
    lens = np.array([1024, 32768])
    b = bench.decode_bytes(lens, 8, 32, 128)
    assert b == (1024 + 32768) * 8 * 128 * 2 * 2 + 2 * 32 * 128 * 2 * 2 + 2 * 32 * 4 + 2 * 4


def test_bench_refuses_more_than_one_gpu(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err
