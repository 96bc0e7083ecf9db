"""Seeded synthetic inputs for exact attention.

This module is shared by the oracle side (tests, ``bench.py``'s CPU baseline)
and the HIP side (the binding's tests, ``bench.py``'s timed path).  It holds
no attention arithmetic: it only draws random numbers, rounds them to bf16
and builds the integer structure (document offsets, decode lengths) that the
workloads need.

Recipe (the same for every caller):

* ``numpy.random.Generator(PCG64(seed))``; tensors are drawn in the order
  Q, K, V (decode: q, K-cache, V-cache), then document lengths or decode
  lengths.
* Each value is ``standard_normal(dtype=float32)``, optionally multiplied by
  an exact power-of-two factor, then rounded to bf16 with round-to-nearest-
  even.  The bf16 bit patterns (uint16) are what both sides receive.
* Document lengths are integers uniform on [256, 4096] (inclusive), drawn one
  after another per batch row until they cover N; the last one is cut at N.
  Offsets follow the packed-sequence convention of cumulative boundaries
  (the ``cu_seqlens`` walkthrough in the aegloslab textbook chapter
  "3.7 어텐션 II", section 3.7.6: lengths [3, 5, 2] give [0, 3, 8, 10]).
* Decode lengths are integers uniform on [1024, 32768] (inclusive).
* The output gradient dO of a backward workload comes from a generator of
  its own, ``PCG64(seed)``, drawn N(0,1) after the same rounding.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_bits_from_f32",
    "f32_from_bf16_bits",
    "draw_bf16",
    "lengths_to_offsets",
    "draw_doc_offsets",
    "pad_offsets",
    "draw_decode_lens",
    "fwd_inputs",
    "decode_inputs",
    "dout_input",
    "CONFIGS",
]


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round-to-nearest-even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    nan = np.isnan(x)
    u = x.view(np.uint32)
    if nan.any():
        u = np.where(nan, np.uint32(0x7FC00000), u)
    # For every non-NaN pattern u + 0x8000 stays below 2**32, so uint32 is exact.
    out = ((u + np.uint32(0x7FFF) + ((u >> 16) & np.uint32(1))) >> 16).astype(np.uint16)
    return out


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def draw_bf16(rng: np.random.Generator, shape, factor: float = 1.0) -> np.ndarray:
    """Draw N(0,1) float32, multiply by ``factor``, round to bf16 bits."""
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if factor != 1.0:
        x = x * np.float32(factor)
    return bf16_bits_from_f32(x)


def lengths_to_offsets(lengths) -> np.ndarray:
    """Cumulative boundaries of packed segments: [3,5,2] -> [0,3,8,10]."""
    lengths = np.asarray(lengths, dtype=np.int64)
    out = np.zeros(len(lengths) + 1, dtype=np.int32)
    out[1:] = np.cumsum(lengths)
    return out


def draw_doc_offsets(rng: np.random.Generator, B: int, N: int,
                     lo: int = 256, hi: int = 4096) -> list[np.ndarray]:
    """Per batch row, document boundaries covering [0, N)."""
    rows = []
    for _ in range(B):
        lengths = []
        total = 0
        while total < N:
            n = int(rng.integers(lo, hi + 1))
            n = min(n, N - total)
            lengths.append(n)
            total += n
        rows.append(lengths_to_offsets(lengths))
    return rows


def pad_offsets(rows: list[np.ndarray], N: int) -> tuple[np.ndarray, int]:
    """Stack per-row offsets into int32 [B][max_docs+1], padding with N."""
    max_docs = max(len(r) - 1 for r in rows)
    out = np.full((len(rows), max_docs + 1), N, dtype=np.int32)
    for b, r in enumerate(rows):
        out[b, : len(r)] = r
    return out, max_docs


def draw_decode_lens(rng: np.random.Generator, B: int, lo: int = 1024,
                     hi: int = 32768) -> np.ndarray:
    return rng.integers(lo, hi + 1, size=B).astype(np.int32)


# The workloads.  ``kind`` selects the mask; sizes are the full ones.
CONFIGS = {
    1: dict(name="causal_b1_h2_n256_d64", kind="causal", B=1, Hq=2, Hkv=2,
            N=256, d=64, factor=1.0, seed=1001),
    2: dict(name="causal_b8_h32_n4096_d128", kind="causal", B=8, Hq=32, Hkv=32,
            N=4096, d=128, factor=0.5, seed=1002),
    3: dict(name="window1024_softcap50_b4_h32_n16384_d128", kind="window_softcap",
            B=4, Hq=32, Hkv=32, N=16384, d=128, factor=1.0, seed=1003,
            window=1024, softcap=50.0),
    4: dict(name="gqa32x8_docs_causal_b2_n8192_d128", kind="docs_causal",
            B=2, Hq=32, Hkv=8, N=8192, d=128, factor=1.0, seed=1004),
    5: dict(name="decode_b16_gqa32x8_t32768_d128_chunk1024", kind="decode",
            B=16, Hq=32, Hkv=8, T=32768, d=128, factor=1.0, seed=1005,
            chunk=1024),
    # backward of workload 2: its Q, K, V and a seeded output gradient dO
    6: dict(name="bwd_causal_b8_h32_n4096_d128", kind="causal", B=8, Hq=32, Hkv=32,
            N=4096, d=128, factor=0.5, seed=1002, dout_seed=1006),
    # workload 2 in FP8: Q and K rotated by the same random-sign Hadamard
    # matrix, all three block-quantized to E4M3 (V with one scale per head)
    9: dict(name="fp8_causal_b8_h32_n4096_d128", kind="causal", B=8, Hq=32, Hkv=32,
            N=4096, d=128, factor=0.5, seed=1002, signs_seed=1009),
}


def fwd_inputs(seed: int, B: int, Hq: int, Hkv: int, N: int, d: int,
               factor: float = 1.0, docs: bool = False,
               doc_lo: int = 256, doc_hi: int = 4096):
    """Q [B,Hq,N,d], K/V [B,Hkv,N,d] as bf16 bits, plus document offsets."""
    rng = np.random.Generator(np.random.PCG64(seed))
    q = draw_bf16(rng, (B, Hq, N, d), factor)
    k = draw_bf16(rng, (B, Hkv, N, d), factor)
    v = draw_bf16(rng, (B, Hkv, N, d), factor)
    offs = None
    if docs:
        offs = draw_doc_offsets(rng, B, N, doc_lo, doc_hi)
    return q, k, v, offs


def decode_inputs(seed: int, B: int, Hq: int, Hkv: int, T: int, d: int,
                  factor: float = 1.0, lens_lo: int = 1024,
                  lens_hi: int = 32768):
    """q [B,Hq,d], K/V caches [B,Hkv,T,d] as bf16 bits, lens [B] int32."""
    rng = np.random.Generator(np.random.PCG64(seed))
    q = draw_bf16(rng, (B, Hq, d), factor)
    kc = draw_bf16(rng, (B, Hkv, T, d), factor)
    vc = draw_bf16(rng, (B, Hkv, T, d), factor)
    lens = draw_decode_lens(rng, B, lens_lo, lens_hi)
    return q, kc, vc, lens


def hadamard_signs(seed: int, d: int = 128) -> np.ndarray:
    """Random +-1 signs (int8 [d]) of the rotation used before FP8
    quantization."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.choice([-1, 1], size=d).astype(np.int8)


def dout_input(seed: int, B: int, Hq: int, N: int, d: int) -> np.ndarray:
    """Output gradient dO [B,Hq,N,d] as bf16 bits, N(0,1)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return draw_bf16(rng, (B, Hq, N, d), 1.0)
