"""Host-side checks of the C ABI (no GPU needed).

The library must load, export every function that include/exattn.h
declares, size its buffers consistently, and reject malformed calls with
the documented status before touching the GPU (validation runs before any
HIP call, so these calls are safe without a device).
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "exattn.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    from exact_attention_15_amd import binding
    return binding.library()


def test_header_declares_the_boundary():
    names = _declared_functions()
    for n in ("attn_fwd", "attn_decode", "attn_mask_build", "attn_mask_bytes",
              "attn_fwd_workspace_size", "attn_decode_workspace_size",
              "attn_bwd", "attn_bwd_workspace_size",
              "attn_fwd_varlen", "attn_fwd_varlen_workspace_size",
              "attn_fwd_fp8", "attn_quantize_fp8", "attn_quantize_fp8_workspace_size",
              "attn_decode_noalloc", "attn_status_string", "attn_last_error"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for s in range(5):
        assert lib.attn_status_string(s)
    assert lib.attn_status_string(99) == b"unknown status"


def test_mask_bytes_matches_python_layout(lib):
    from exact_attention_15_amd import binding
    spec = binding.MaskSpec(causal=True)
    for B, N in [(1, 1), (1, 256), (2, 1000), (8, 4096), (4, 16384)]:
        assert lib.attn_mask_bytes(spec.ref(), B, N) == binding.mask_layout(B, N)["bytes"]
    assert lib.attn_mask_bytes(spec.ref(), 0, 10) == 0


def test_decode_workspace_size(lib):
    # m and l: B*Hq*nchunk floats each; O: B*Hq*nchunk*d floats (256-byte aligned sections)
    B, Hq, T, d, chunk = 16, 32, 32768, 128, 1024
    n = B * Hq * (T // chunk)
    assert lib.attn_decode_workspace_size(B, Hq, T, d, chunk) == 4 * n * 2 + 4 * n * d


def _t(ptr=16, sb=0, sh=0, sn=0):
    from exact_attention_15_amd.binding import AttnTensor
    return AttnTensor(ptr, sb, sh, sn)


def _fwd(lib, d=128, Hq=4, Hkv=2, scale=0.1, B=1, N=8, ptr=16, ws=None, ws_bytes=0):
    t = _t(ptr, 0, 0, 128)
    lse = ctypes.c_void_p(16)
    return lib.attn_fwd(t, t, t, t, lse, B, Hq, Hkv, N, d, None, ctypes.c_float(scale),
                        None, ws, ws_bytes, None)


def test_fwd_validation_before_launch(lib):
    from exact_attention_15_amd import binding as b
    assert _fwd(lib, d=96) == b.ATTN_ERR_UNSUPPORTED
    assert b"head dim 96" in lib.attn_last_error()
    assert _fwd(lib, Hq=3, Hkv=2) == b.ATTN_ERR_INVALID
    assert _fwd(lib, scale=0.0) == b.ATTN_ERR_INVALID
    assert _fwd(lib, scale=float("nan")) == b.ATTN_ERR_INVALID
    assert _fwd(lib, ptr=18) == b.ATTN_ERR_INVALID                  # misaligned
    assert _fwd(lib, ws=None) == b.ATTN_ERR_WORKSPACE                # no block mask, no workspace
    assert _fwd(lib, ws=ctypes.c_void_p(16), ws_bytes=8) == b.ATTN_ERR_WORKSPACE
    assert _fwd(lib, B=0) == b.ATTN_OK                               # empty: nothing to do
    assert _fwd(lib, N=0) == b.ATTN_OK
    assert _fwd(lib, N=1 << 30) == b.ATTN_ERR_UNSUPPORTED            # longest sequence is 2^30 - 1


def test_fwd_rejects_bad_specs(lib):
    from exact_attention_15_amd import binding as b
    t = _t(16, 0, 0, 128)
    for spec in (b.AttnMaskSpec(b.ATTN_MASK_DOCS, 0, 0, 0.0, None, 2),
                 b.AttnMaskSpec(b.ATTN_MASK_DOCS, 0, 0, 0.0, 64, 1),
                 b.AttnMaskSpec(b.ATTN_MOD_SOFTCAP, 0, 0, 0.0, None, 0),
                 b.AttnMaskSpec(1 << 10, 0, 0, 0.0, None, 0)):
        st = lib.attn_fwd(t, t, t, t, ctypes.c_void_p(16), 1, 2, 2, 8, 128, ctypes.byref(spec),
                          ctypes.c_float(0.1), None, None, 0, None)
        assert st == b.ATTN_ERR_INVALID


def test_decode_noalloc_validation_before_launch(lib):
    # the allocation-free decode validates like attn_decode and rejects
    # partials larger than its static scratch before any HIP call
    from exact_attention_15_amd import binding as b
    t = _t(16, 0, 0, 128)
    limit = 16 << 20

    def call(B=2, Hq=8, Hkv=2, T=4096, d=128, chunk=1024, lens=16):
        return lib.attn_decode_noalloc(t, t, t, lens, t, ctypes.c_void_p(16), B, Hq, Hkv, T, d, chunk,
                                       ctypes.c_float(0.1), None)
    assert call(d=80) == b.ATTN_ERR_UNSUPPORTED
    assert call(Hq=6, Hkv=4) == b.ATTN_ERR_INVALID
    assert call(chunk=1000) == b.ATTN_ERR_UNSUPPORTED
    assert call(lens=None) == b.ATTN_ERR_INVALID
    assert call(B=0) == b.ATTN_OK
    # the decode workload's partials fit; twice its cache length does not
    assert lib.attn_decode_workspace_size(16, 32, 32768, 128, 1024) <= limit
    assert lib.attn_decode_workspace_size(16, 32, 65536, 128, 1024) > limit
    assert call(B=16, Hq=32, Hkv=8, T=65536) == b.ATTN_ERR_WORKSPACE
    assert b"static" in lib.attn_last_error()


def test_decode_validation_before_launch(lib):
    from exact_attention_15_amd import binding as b
    t = _t(16, 0, 0, 128)

    def call(Hq=8, Hkv=2, d=128, chunk=1024, ws=None, ws_bytes=0, lens=16, T=4096):
        return lib.attn_decode(t, t, t, lens, t, ctypes.c_void_p(16), 2, Hq, Hkv, T, d, chunk,
                               ctypes.c_float(0.1), ws, ws_bytes, None)
    assert call(d=80) == b.ATTN_ERR_UNSUPPORTED
    assert call(Hq=34, Hkv=2) == b.ATTN_ERR_UNSUPPORTED   # group of 17
    assert call(Hq=6, Hkv=4) == b.ATTN_ERR_INVALID
    assert call(chunk=1000) == b.ATTN_ERR_UNSUPPORTED
    assert call(chunk=4096) == b.ATTN_ERR_UNSUPPORTED
    assert call(lens=None) == b.ATTN_ERR_INVALID
    assert call() == b.ATTN_ERR_WORKSPACE
    # cache token stride at 2^20 elements: rows are addressed with 32-bit offsets
    wide = _t(16, 0, 0, 1 << 20)
    assert lib.attn_decode(t, wide, t, 16, t, ctypes.c_void_p(16), 2, 8, 2, 4096, 128, 1024,
                           ctypes.c_float(0.1), None, 0, None) == b.ATTN_ERR_UNSUPPORTED


def test_bwd_workspace_size(lib):
    # forward block mask + transposed (key-block) mask + two fp32 [B][Hq][N] row arrays
    from exact_attention_15_amd import binding as b

    def a256(x):
        return (x + 255) & ~255
    for B, Hq, N in [(1, 1, 1), (2, 3, 1000), (8, 32, 4096)]:
        nkb, nqt64 = (N + 127) // 128, (N + 63) // 64
        kvmask = a256(4 * B * nkb) + a256(4 * B * nkb * nqt64)
        want = b.mask_layout(B, N)["bytes"] + kvmask + 2 * a256(4 * B * Hq * N)
        assert lib.attn_bwd_workspace_size(None, B, Hq, N) == want
    assert lib.attn_bwd_workspace_size(None, 0, 4, 10) == 0


def test_bwd_validation_before_launch(lib):
    from exact_attention_15_amd import binding as b
    t = _t(16, 0, 0, 128)
    lse = ctypes.c_void_p(16)

    def call(d=128, Hq=4, Hkv=2, B=1, N=8, scale=0.1, ws=None, ws_bytes=0, dq=t, lse=lse, wide=None):
        q = wide or t
        return lib.attn_bwd(q, t, t, t, lse, t, dq, t, t, B, Hq, Hkv, N, d, None,
                            ctypes.c_float(scale), ws, ws_bytes, None)
    assert call(d=96) == b.ATTN_ERR_UNSUPPORTED
    assert call(Hq=3, Hkv=2) == b.ATTN_ERR_INVALID
    assert call(scale=-1.0) == b.ATTN_ERR_INVALID
    assert call(dq=_t(0, 0, 0, 128)) == b.ATTN_ERR_INVALID           # null output
    assert call(dq=_t(24, 0, 0, 128)) == b.ATTN_ERR_INVALID          # misaligned output
    assert call(lse=None) == b.ATTN_ERR_INVALID
    assert call(wide=_t(16, 0, 0, 1 << 24)) == b.ATTN_ERR_UNSUPPORTED
    assert call() == b.ATTN_ERR_WORKSPACE
    assert call(ws=ctypes.c_void_p(16), ws_bytes=64) == b.ATTN_ERR_WORKSPACE
    assert call(B=0) == b.ATTN_OK
    assert call(N=0) == b.ATTN_OK


def test_varlen_validation_before_launch(lib):
    from exact_attention_15_amd import binding as b
    t = _t(16, 0, 0, 256)
    lse = ctypes.c_void_p(16)

    def call(d=128, Hq=4, Hkv=2, nseq=2, tq=10, tk=12, cu_q=16, cu_k=16, flags=0, ws=None,
             ws_bytes=0, kt=t):
        spec = b.AttnMaskSpec(flags, 0, 0, 0.0, None, 0)
        return lib.attn_fwd_varlen(t, kt, kt, t, lse, cu_q, cu_k, nseq, tq, tk, Hq, Hkv, d,
                                   ctypes.byref(spec), ctypes.c_float(0.1), ws, ws_bytes, None)
    assert call(d=96) == b.ATTN_ERR_UNSUPPORTED
    assert call(Hq=3, Hkv=2) == b.ATTN_ERR_INVALID
    assert call(nseq=-1) == b.ATTN_ERR_INVALID
    assert call(nseq=0) == b.ATTN_ERR_INVALID            # rows but no sequence
    assert call(cu_q=None) == b.ATTN_ERR_INVALID
    assert call(tq=1 << 30) == b.ATTN_ERR_UNSUPPORTED
    assert call(tk=1 << 30) == b.ATTN_ERR_UNSUPPORTED
    assert call(flags=b.ATTN_MASK_DOCS) == b.ATTN_ERR_INVALID
    assert call() == b.ATTN_ERR_WORKSPACE
    assert call(tq=0) == b.ATTN_OK                         # nothing to do
    # with no keys, k and v are never read and may be null
    assert call(tk=0, kt=_t(0, 0, 0, 0)) == b.ATTN_ERR_WORKSPACE


def test_varlen_workspace_size(lib):
    # the block mask of one batch row: total_q rows over total_k keys
    def a256(x):
        return (x + 255) & ~255
    for tq, tk in [(10, 12), (5000, 300), (300, 5000)]:
        nqt, nkt = (tq + 127) // 128, (tk + 63) // 64
        want = 2 * a256(4 * tq) + 2 * a256(4 * nqt) + a256(4 * nqt * nkt)
        assert lib.attn_fwd_varlen_workspace_size(tq, tk) == want
    assert lib.attn_fwd_varlen_workspace_size(0, 10) == 0


def test_alibi_validation(lib):
    from exact_attention_15_amd import binding as b
    t = _t(16, 0, 0, 128)
    no_slopes = b.AttnMaskSpec(b.ATTN_MOD_ALIBI, 0, 0, 0.0, None, 0, None)
    st = lib.attn_fwd(t, t, t, t, ctypes.c_void_p(16), 1, 2, 2, 8, 128, ctypes.byref(no_slopes),
                      ctypes.c_float(0.1), None, None, 0, None)
    assert st == b.ATTN_ERR_INVALID and b"alibi_slopes" in lib.attn_last_error()
    spec = b.AttnMaskSpec(b.ATTN_MOD_ALIBI, 0, 0, 0.0, None, 0, 64)
    st = lib.attn_bwd(t, t, t, t, ctypes.c_void_p(16), t, t, t, t, 1, 2, 2, 8, 128,
                      ctypes.byref(spec), ctypes.c_float(0.1), None, 0, None)
    assert st == b.ATTN_ERR_UNSUPPORTED
    st = lib.attn_fwd_varlen(t, t, t, t, ctypes.c_void_p(16), 16, 16, 1, 8, 8, 2, 2, 128,
                             ctypes.byref(spec), ctypes.c_float(0.1), None, 0, None)
    assert st == b.ATTN_ERR_UNSUPPORTED


def test_fp8_validation_before_launch(lib):
    from exact_attention_15_amd import binding as b
    t = _t(16, 0, 0, 128)
    f = ctypes.c_void_p(16)

    def fwd8(d=128, Hq=4, Hkv=2, qt=t, flags=0):
        spec = b.AttnMaskSpec(flags, 0, 0, 0.0, None, 0, 64)
        return lib.attn_fwd_fp8(qt, t, t, f, f, f, t, f, 1, Hq, Hkv, 8, d, ctypes.byref(spec),
                                ctypes.c_float(0.1), None, None, 0, None)
    assert fwd8(d=64) == b.ATTN_ERR_UNSUPPORTED
    assert fwd8(Hq=3) == b.ATTN_ERR_INVALID
    assert fwd8(qt=_t(16, 0, 0, 136)) == b.ATTN_ERR_INVALID        # byte strides multiple of 16
    assert fwd8(flags=b.ATTN_MOD_ALIBI) == b.ATTN_ERR_UNSUPPORTED
    assert fwd8() == b.ATTN_ERR_WORKSPACE

    def quant(d=128, out=t, scales=16, ws=None, ws_bytes=0):
        return lib.attn_quantize_fp8(t, out, scales, 1, 2, 100, d, None, 0, ws, ws_bytes, None)
    assert quant(d=64) == b.ATTN_ERR_UNSUPPORTED
    assert quant(scales=None) == b.ATTN_ERR_INVALID
    assert quant(out=_t(16, 0, 0, 8)) == b.ATTN_ERR_INVALID
    assert quant() == b.ATTN_ERR_WORKSPACE
    assert lib.attn_quantize_fp8_workspace_size(2, 3, 100) == 256
