"""Pins of the oracle's FP8 pieces: the E4M3 codec, the randomized
Hadamard rotation and block quantization.

  * E4M3 values fixed by the format's definition (bias 7, 3 mantissa bits,
    largest finite 448, smallest subnormal 2^-9, S.1111.111 = NaN), and
    round-to-nearest-even checked by brute force against the decoded table;
  * the butterfly rotation equals the dense matrix diag(signs) H / sqrt(d)
    with H from scipy.linalg.hadamard, is orthogonal, and leaves Q K^T
    unchanged when applied to both;
  * quantization: scales are powers of two putting each block's maximum in
    (224, 448], every code is the nearest E4M3 value of x / scale, and
    dequantized values are bf16 values;
  * the pages' claim for incoherent processing: with an outlier channel the
    rotation lowers the quantization error of Q K^T.
"""
import numpy as np
import pytest
import scipy.linalg

import attn_inputs as gen
import oracle


def test_e4m3_defining_values():
    dec = oracle.e4m3_decode
    assert dec(0x38) == 1.0 and dec(0x40) == 2.0 and dec(0xB8) == -1.0
    assert dec(0x7E) == 448.0 and dec(0xFE) == -448.0
    assert dec(0x01) == 2.0 ** -9 and dec(0x07) == 7 * 2.0 ** -9 and dec(0x08) == 2.0 ** -6
    assert dec(0x00) == 0.0 and np.isnan(dec(0x7F)) and np.isnan(dec(0xFF))
    vals = dec(np.arange(0, 0x7F, dtype=np.uint8))
    assert np.all(np.diff(vals) > 0)  # positive codes are ordered


def test_e4m3_encode_is_nearest_even():
    table = oracle.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))
    rng = np.random.Generator(np.random.PCG64(1200))
    x = np.concatenate([rng.uniform(-448, 448, 4000), rng.uniform(-0.02, 0.02, 4000),
                        (table[:-1] + table[1:]) / 2])  # exact midpoints
    codes = oracle.e4m3_encode(x)
    got = oracle.e4m3_decode(codes)
    a = np.abs(x)
    dist = np.abs(table[None, :] - a[:, None])
    best = dist.min(axis=1)
    assert np.all(np.abs(np.abs(got) - a) == best)  # a nearest value, never a farther one
    ties = (dist == best[:, None]).sum(axis=1) == 2
    assert ties.sum() > 100
    assert np.all((codes[ties] & 1) == 0)  # ties go to the even mantissa
    assert np.array_equal((codes & 0x80) != 0, np.signbit(x))


@pytest.mark.parametrize("d", [64, 128])
def test_rotation_matches_dense_hadamard(d):
    rng = np.random.Generator(np.random.PCG64(1201))
    signs = rng.choice([-1, 1], size=d).astype(np.int8)
    y = rng.standard_normal((5, d)).astype(np.float32)
    got = oracle.hadamard_rotate(y, signs).astype(np.float64)
    R = np.diag(signs.astype(np.float64)) @ scipy.linalg.hadamard(d) / np.sqrt(d)
    assert np.allclose(R @ R.T, np.eye(d), atol=1e-14)
    assert np.allclose(got, y.astype(np.float64) @ R, rtol=1e-5, atol=1e-5)


def test_rotation_keeps_qk():
    rng = np.random.Generator(np.random.PCG64(1202))
    signs = rng.choice([-1, 1], size=128).astype(np.int8)
    q = rng.standard_normal((7, 128)).astype(np.float32)
    k = rng.standard_normal((9, 128)).astype(np.float32)
    qr = oracle.hadamard_rotate(q, signs).astype(np.float64)
    kr = oracle.hadamard_rotate(k, signs).astype(np.float64)
    assert np.allclose(qr @ kr.T, q.astype(np.float64) @ k.astype(np.float64).T, rtol=1e-5, atol=1e-4)


@pytest.mark.parametrize("per_head", [False, True])
@pytest.mark.parametrize("rotate", [False, True])
def test_quantize_blocks(per_head, rotate):
    rng = np.random.Generator(np.random.PCG64(1203))
    B, H, N, d = 2, 3, 150, 128
    x = gen.draw_bf16(rng, (B, H, N, d), 1.0)
    x[0, 1, 70] = gen.bf16_bits_from_f32(np.full(d, 30.0, np.float32))  # a large row in block 1
    signs = rng.choice([-1, 1], size=d).astype(np.int8) if rotate else None
    codes, scales = oracle.quantize_fp8(x, signs=signs, per_head=per_head)
    assert codes.shape == x.shape and scales.shape == (B, H, 3)
    e = np.log2(scales.astype(np.float64))
    assert np.array_equal(e, np.round(e))  # powers of two
    xf = gen.f32_from_bf16_bits(x)
    y = oracle.hadamard_rotate(xf, signs) if rotate else xf
    for b in range(B):
        for h in range(H):
            for i in range(3):
                blk = np.abs(y[b, h, 64 * i:64 * (i + 1)]).max()
                s = scales[b, h, i]
                if per_head:
                    blk = np.abs(y[b, h]).max()
                    assert s == scales[b, h, 0]
                assert 224.0 < blk / s <= 448.0
    deq = oracle.e4m3_decode(codes) * np.repeat(scales, 64, axis=2)[:, :, :N, None]
    # each value is within half a code step of the exact one
    step = np.maximum(np.exp2(np.floor(np.log2(np.maximum(np.abs(y / np.repeat(scales, 64, axis=2)[:, :, :N, None]),
                                                                   2.0 ** -6)))) / 8, 2.0 ** -9)
    assert np.all(np.abs(deq - y) <= 0.5 * step * np.repeat(scales, 64, axis=2)[:, :, :N, None] * (1 + 1e-12))
    bits = oracle.dequantize_fp8(codes, scales)
    assert np.array_equal(gen.f32_from_bf16_bits(bits).astype(np.float64), deq)


def test_incoherent_processing_reduces_error_with_outliers():
    # Q and K with a few large channels: rotating spreads them over all
    # dimensions, so the block scales fit the bulk better
    rng = np.random.Generator(np.random.PCG64(1204))
    B, H, N, d = 1, 2, 256, 128
    qf = rng.standard_normal((B, H, N, d)).astype(np.float32)
    kf = rng.standard_normal((B, H, N, d)).astype(np.float32)
    qf[..., :3] *= 40.0
    kf[..., :3] *= 40.0
    q, k = gen.bf16_bits_from_f32(qf), gen.bf16_bits_from_f32(kf)
    signs = rng.choice([-1, 1], size=d).astype(np.int8)
    exact = np.einsum("bhid,bhjd->bhij", gen.f32_from_bf16_bits(q).astype(np.float64),
                      gen.f32_from_bf16_bits(k).astype(np.float64))
    errs = []
    for s in (None, signs):
        cq, sq = oracle.quantize_fp8(q, signs=s)
        ck, sk = oracle.quantize_fp8(k, signs=s)
        dq = gen.f32_from_bf16_bits(oracle.dequantize_fp8(cq, sq)).astype(np.float64)
        dk = gen.f32_from_bf16_bits(oracle.dequantize_fp8(ck, sk)).astype(np.float64)
        errs.append(np.sqrt(np.mean((np.einsum("bhid,bhjd->bhij", dq, dk) - exact) ** 2)))
    assert errs[1] < 0.7 * errs[0], errs
