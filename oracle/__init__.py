"""fp64 CPU oracle for exact attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The library under test never does.

The arithmetic lives in ``oracle.c`` (plain fp64 C, OpenMP over rows); this
module compiles it with gcc when no build is present and marshals numpy
arrays of bf16 bit patterns (uint16) into it.  The packed variable-length
forward (``fwd_varlen``) is written here in numpy fp64, from the definition.
Nothing here is shared with the HIP library.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

CAUSAL, WINDOW, DOCS, SOFTCAP, ALIBI = 1, 2, 4, 8, 16

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so (gcc, -O2, OpenMP, IEEE math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared",
                               "-std=c99", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32, i64, f64 = ctypes.c_int, ctypes.c_int64, ctypes.c_double
        lib.oracle_fwd.restype = i32
        lib.oracle_fwd.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32, i32,
                                   i32, i64, i64, f64, P, i32, f64, i64, P, P,
                                   P, P, P]
        lib.oracle_decode.restype = i32
        lib.oracle_decode.argtypes = [P, P, P, P, P, P, i32, i32, i32, i32,
                                      i32, f64, P, P]
        lib.oracle_bwd.restype = i32
        lib.oracle_bwd.argtypes = [P, P, P, P, P, P, P, i32, i32, i32, i32, i32,
                                   i32, i64, i64, f64, P, i32, f64, P, P, P]
        lib.oracle_threads.restype = i32
        lib.oracle_threads.argtypes = []
        _lib = lib
    return _lib


def threads() -> int:
    return _load().oracle_threads()


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _strides(a: np.ndarray) -> np.ndarray:
    """(b, h, n) element strides of a 4-D array with unit last stride."""
    if a.ndim != 4 or a.strides[3] != a.itemsize:
        raise ValueError("expected a 4-D array with contiguous last axis")
    return np.array([s // a.itemsize for s in a.strides[:3]], dtype=np.int64)


def fwd(q, k, v, *, scale, causal=False, window=None, doc_offsets=None,
        softcap=None, alibi_slopes=None, rows=None, want_probs=False):
    """Exact attention, fp64.

    q [B,Hq,N,d], k/v [B,Hkv,N,d]: uint16 bf16 bit patterns.
    window: None, an int w (|i-j| <= w) or a pair (left, right).
    doc_offsets: int32 [B][max_docs+1] padded with N, or None.
    alibi_slopes: None or [Hq] floats: score -= slope[h] * |i - j|.
    rows: None for every row, else int array [n,3] of (b, h, i).
    Returns (O [..., d] float64, LSE float64[, P]) shaped [B,Hq,N,...] for
    all rows, or [n, ...] for selected rows.
    """
    lib = _load()
    for a in (q, k, v):
        if a.dtype != np.uint16:
            raise TypeError("oracle inputs are bf16 bit patterns (uint16)")
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    flags = 0
    wl = wr = 0
    if causal:
        flags |= CAUSAL
    if window is not None:
        flags |= WINDOW
        wl, wr = (window, window) if np.isscalar(window) else window
    offs = None
    doc_stride = 0
    if doc_offsets is not None:
        flags |= DOCS
        offs = np.ascontiguousarray(doc_offsets, dtype=np.int32)
        doc_stride = offs.shape[1]
    cap = 0.0
    if softcap is not None:
        flags |= SOFTCAP
        cap = float(softcap)
    slopes = None
    if alibi_slopes is not None:
        flags |= ALIBI
        slopes = np.ascontiguousarray(alibi_slopes, dtype=np.float64)
        if slopes.shape != (Hq,):
            raise ValueError("alibi_slopes must hold one slope per query head")
    if rows is None:
        nrows = B * Hq * N
        rows_arr = None
    else:
        rows_arr = np.ascontiguousarray(rows, dtype=np.int32).reshape(-1, 3)
        nrows = rows_arr.shape[0]
    o = np.empty((nrows, d), dtype=np.float64)
    lse = np.empty(nrows, dtype=np.float64)
    p = np.empty((nrows, N), dtype=np.float64) if want_probs else None
    qs, ks, vs = _strides(q), _strides(k), _strides(v)
    rc = lib.oracle_fwd(_ptr(q), _ptr(qs), _ptr(k), _ptr(ks), _ptr(v), _ptr(vs),
                        B, Hq, Hkv, N, d, flags, int(wl), int(wr), cap,
                        _ptr(offs), doc_stride, float(scale), nrows,
                        _ptr(rows_arr), _ptr(o), _ptr(lse), _ptr(p), _ptr(slopes))
    if rc != 0:
        raise ValueError("oracle_fwd rejected its arguments")
    if rows is None:
        o = o.reshape(B, Hq, N, d)
        lse = lse.reshape(B, Hq, N)
        if p is not None:
            p = p.reshape(B, Hq, N, N)
    return (o, lse, p) if want_probs else (o, lse)


def bwd(q, k, v, dout, *, scale, causal=False, window=None, doc_offsets=None,
        softcap=None):
    """Gradients of exact attention, fp64: (dq [B,Hq,N,d], dk, dv [B,Hkv,N,d]).

    q, k, v as for fwd(); dout [B,Hq,N,d] bf16 bits is the gradient of the
    loss with respect to O.
    """
    lib = _load()
    for a in (q, k, v, dout):
        if a.dtype != np.uint16:
            raise TypeError("oracle inputs are bf16 bit patterns (uint16)")
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    if dout.shape != q.shape:
        raise ValueError("dout must have the shape of q")
    flags = 0
    wl = wr = 0
    if causal:
        flags |= CAUSAL
    if window is not None:
        flags |= WINDOW
        wl, wr = (window, window) if np.isscalar(window) else window
    offs = None
    doc_stride = 0
    if doc_offsets is not None:
        flags |= DOCS
        offs = np.ascontiguousarray(doc_offsets, dtype=np.int32)
        doc_stride = offs.shape[1]
    cap = 0.0
    if softcap is not None:
        flags |= SOFTCAP
        cap = float(softcap)
    dout = np.ascontiguousarray(dout)
    dq = np.empty((B, Hq, N, d), dtype=np.float64)
    dk = np.empty((B, Hkv, N, d), dtype=np.float64)
    dv = np.empty((B, Hkv, N, d), dtype=np.float64)
    qs, ks, vs = _strides(q), _strides(k), _strides(v)
    rc = lib.oracle_bwd(_ptr(q), _ptr(qs), _ptr(k), _ptr(ks), _ptr(v), _ptr(vs), _ptr(dout),
                        B, Hq, Hkv, N, d, flags, int(wl), int(wr), cap, _ptr(offs), doc_stride,
                        float(scale), _ptr(dq), _ptr(dk), _ptr(dv))
    if rc != 0:
        raise ValueError("oracle_bwd rejected its arguments")
    return dq, dk, dv


def decode(q, kc, vc, lens, *, scale):
    """One query per (b, hq) against cache keys j < lens[b]; fp64.

    q [B,Hq,d], kc/vc [B,Hkv,T,d] uint16 bf16 bits, lens int32 [B].
    Returns (O [B,Hq,d], LSE [B,Hq]).
    """
    lib = _load()
    B, Hq, d = q.shape
    Hkv, T = kc.shape[1], kc.shape[2]
    q = np.ascontiguousarray(q)
    lens = np.ascontiguousarray(lens, dtype=np.int32)
    o = np.empty((B, Hq, d), dtype=np.float64)
    lse = np.empty((B, Hq), dtype=np.float64)
    ks, vs = _strides(kc), _strides(vc)
    rc = lib.oracle_decode(_ptr(q), _ptr(kc), _ptr(ks), _ptr(vc), _ptr(vs),
                           _ptr(lens), B, Hq, Hkv, T, d, float(scale), _ptr(o),
                           _ptr(lse))
    if rc != 0:
        raise ValueError("oracle_decode rejected its arguments")
    return o, lse


def _bf16_to_f64(bits):
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def fwd_varlen(q, k, v, cu_q, cu_k, *, scale, causal=False, window=None, softcap=None,
               rows=None):
    """Exact attention over packed variable-length sequences, fp64, from the
    definition (aegloslab "3.7 어텐션 II", section 3.7.6, the varlen form).

    q [total_q, Hq, d], k/v [total_k, Hkv, d]: uint16 bf16 bit patterns.
    cu_q, cu_k: int [nseq + 1] cumulative lengths.  Sequence s: queries
    [cu_q[s], cu_q[s+1]), keys [cu_k[s], cu_k[s+1]).  Local query i of a
    sequence with Lq queries and Lk keys lines up with local key
    i + Lk - Lq; causal keeps keys j <= i + Lk - Lq, a window (int w or pair
    (left, right)) keeps i + Lk - Lq - left <= j <= i + Lk - Lq + right.
    The score is scale * q.k, masked keys are dropped, and the soft cap
    c * tanh(s / c) applies to the rest.
    rows: None for every row, else int array [n, 2] of (h, i).
    Returns (O, LSE): [total_q, Hq, d] and [Hq, total_q], or [n, d] and [n]
    for selected rows.  A row with no visible key has O = 0, LSE = -inf.
    """
    tq, Hq, d = q.shape
    Hkv = k.shape[1]
    group = Hq // Hkv
    cu_q = np.asarray(cu_q, dtype=np.int64)
    cu_k = np.asarray(cu_k, dtype=np.int64)
    if window is None:
        wl = wr = None
    elif np.isscalar(window):
        wl = wr = int(window)
    else:
        wl, wr = (int(x) for x in window)
    seq_of = np.searchsorted(cu_q, np.arange(tq), side="right") - 1

    def one_row(h, i):
        s = int(seq_of[i])
        q0, q1, k0, k1 = cu_q[s], cu_q[s + 1], cu_k[s], cu_k[s + 1]
        diag = (i - q0) + (k1 - k0) - (q1 - q0)
        j = np.arange(k1 - k0)
        vis = np.ones(j.shape, dtype=bool)
        if causal:
            vis &= j <= diag
        if wl is not None:
            vis &= (j >= diag - wl) & (j <= diag + wr)
        if not vis.any():
            return np.zeros(d), -np.inf
        hk = h // group
        kk = _bf16_to_f64(k[k0:k1, hk, :])[vis]
        vv = _bf16_to_f64(v[k0:k1, hk, :])[vis]
        sc = (kk @ _bf16_to_f64(q[i, h, :])) * scale
        if softcap is not None:
            sc = softcap * np.tanh(sc / softcap)
        m = sc.max()
        e = np.exp(sc - m)
        den = e.sum()
        return (e / den) @ vv, m + np.log(den)

    if rows is not None:
        rows = np.asarray(rows, dtype=np.int64).reshape(-1, 2)
        o = np.empty((rows.shape[0], d))
        lse = np.empty(rows.shape[0])
        for n, (h, i) in enumerate(rows):
            o[n], lse[n] = one_row(int(h), int(i))
        return o, lse
    o = np.empty((tq, Hq, d))
    lse = np.empty((Hq, tq))
    for h in range(Hq):
        for i in range(tq):
            o[i, h], lse[h, i] = one_row(h, i)
    return o, lse


# ---------------------------------------------------------------------------
# FP8 (E4M3) block quantization with incoherent processing (youngju.dev
# "FlashAttention 논문 분석", FlashAttention-3 section "FP8 지원과 정확도
# 유지": a scale per block, and a random orthogonal matrix applied to Q and K
# before quantization).
# ---------------------------------------------------------------------------
E4M3_MAX = 448.0


def e4m3_decode(codes):
    """E4M3 (OCP FP8, bias 7, no infinities, S.1111.111 = NaN) -> float64."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    val = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return sign * val


def e4m3_encode(x):
    """Round-to-nearest-even E4M3 codes of finite values with |x| <= 448."""
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)) or np.any(np.abs(x) > E4M3_MAX):
        raise ValueError("e4m3_encode: values must be finite with |x| <= 448")
    a = np.abs(x)
    sign = np.where(np.signbit(x), 0x80, 0)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0))).astype(np.int64)
    # subnormals (a < 2^-6): multiples of 2^-9
    sub = a < 2.0 ** -6
    msub = np.rint(a / 2.0 ** -9).astype(np.int64)  # 0..8; 8 is the smallest normal
    # normals: (1 + m/8) 2^e, with the mantissa rounded to 3 bits
    e = np.clip(e, -6, 8)
    frac = a / np.exp2(e.astype(np.float64))  # in [1, 2) up to the log2 rounding
    lo = frac < 1.0
    e = np.where(lo, e - 1, e)
    frac = np.where(lo, frac * 2.0, frac)
    hi = frac >= 2.0
    e = np.where(hi, e + 1, e)
    frac = np.where(hi, frac / 2.0, frac)
    m = np.rint((frac - 1.0) * 8.0).astype(np.int64)  # 0..8
    carry = m == 8
    e = np.where(carry, e + 1, e)
    m = np.where(carry, 0, m)
    normal = ((e + 7) << 3) | m
    code = np.where(sub, msub, normal)  # msub == 8 encodes as exponent 1, mantissa 0
    return (code | sign).astype(np.uint8)


def hadamard_rotate(y, signs):
    """Rows of y (float32, last axis d, a power of two) times
    diag(signs) H / sqrt(d), H the Walsh-Hadamard matrix, in float32 with the
    radix-2 butterfly: for stride h = 1, 2, ..., d/2 the element with the
    stride bit clear becomes a + b and its partner a - b."""
    y = np.asarray(y, dtype=np.float32) * np.asarray(signs, dtype=np.float32)
    d = y.shape[-1]
    h = 1
    while h < d:
        z = y.reshape(y.shape[:-1] + (d // (2 * h), 2, h))
        a, b = z[..., 0, :].copy(), z[..., 1, :].copy()
        z[..., 0, :] = a + b
        z[..., 1, :] = a - b
        y = z.reshape(y.shape)
        h *= 2
    return (y * np.float32(1.0 / np.sqrt(d))).astype(np.float32)


def quantize_fp8(x_bits, *, signs=None, per_head=False, block=64):
    """E4M3 codes [B,H,N,d] and power-of-two scales float32 [B,H,ceil(N/block)]
    of a bf16 tensor: every `block` rows of a (b, h) (or the whole head) get
    the scale 2^e, e the smallest integer with max|block| <= 448 * 2^e
    (2^0 for an all-zero block), and the codes are RNE(x / 2^e).  With signs
    the rows are first rotated by diag(signs) H / sqrt(d) in float32."""
    x = (np.asarray(x_bits, dtype=np.uint32) << 16).view(np.float32)
    B, H, N, d = x.shape
    y = hadamard_rotate(x, signs) if signs is not None else x.astype(np.float32)
    nblk = (N + block - 1) // block
    amax = np.zeros((B, H, nblk), dtype=np.float64)
    for i in range(nblk):
        amax[:, :, i] = np.abs(y[:, :, i * block:(i + 1) * block]).max(axis=(2, 3))
    if per_head:
        amax[:] = amax.max(axis=2, keepdims=True)
    e = np.zeros(amax.shape, dtype=np.int64)
    pos = amax > 0
    e[pos] = np.ceil(np.log2(amax[pos] / E4M3_MAX)).astype(np.int64)
    # settle the boundary exactly: smallest e with amax <= 448 * 2^e
    e = np.where(pos & (amax <= E4M3_MAX * np.exp2(e - 1.0)), e - 1, e)
    e = np.where(pos & (amax > E4M3_MAX * np.exp2(e.astype(np.float64))), e + 1, e)
    scales = np.exp2(e.astype(np.float64)).astype(np.float32)
    rows_scale = np.repeat(scales, block, axis=2)[:, :, :N, None].astype(np.float64)
    codes = e4m3_encode(y.astype(np.float64) / rows_scale)
    return codes, scales


def dequantize_fp8(codes, scales, block=64):
    """bf16 bit patterns of codes * scale (exact: E4M3 values times powers of
    two are bf16 values)."""
    N = codes.shape[2]
    v = e4m3_decode(codes) * np.repeat(scales.astype(np.float64), block, axis=2)[:, :, :N, None]
    f = v.astype(np.float32)
    if not np.array_equal(f.astype(np.float64), v):
        raise ValueError("dequantized value not representable")
    bits = f.view(np.uint32)
    if np.any(bits & 0xFFFF):
        raise ValueError("dequantized value not a bf16 value")
    return (bits >> 16).astype(np.uint16)
