"""ctypes binding of libexattn (argument marshalling only).

Every step of the computation runs in the HIP kernels behind the C ABI in
``include/exattn.h``.  PyTorch only supplies device memory (tensors, the
workspace) and the stream the calls are enqueued on.  If the library is
missing it is built in-tree; if it cannot be built or loaded, import fails --
there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libexattn.so")

ATTN_OK, ATTN_ERR_INVALID, ATTN_ERR_UNSUPPORTED, ATTN_ERR_WORKSPACE, ATTN_ERR_HIP = range(5)
ATTN_MASK_CAUSAL = 1
ATTN_MASK_WINDOW = 2
ATTN_MASK_DOCS = 4
ATTN_MOD_SOFTCAP = 8
ATTN_MASK_NO_SKIP = 16
ATTN_MOD_ALIBI = 32

# Tile sizes of the forward kernel (block-mask granularity).
BLOCK_M = 128
BLOCK_N = 64


class AttnTensor(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("stride_b", ctypes.c_int64),
                ("stride_h", ctypes.c_int64), ("stride_n", ctypes.c_int64)]


class AttnMaskSpec(ctypes.Structure):
    _fields_ = [("flags", ctypes.c_uint32), ("window_left", ctypes.c_int32),
                ("window_right", ctypes.c_int32), ("softcap", ctypes.c_float),
                ("doc_offsets", ctypes.c_void_p), ("doc_stride", ctypes.c_int32),
                ("alibi_slopes", ctypes.c_void_p)]


class AttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(LIB_PATH)
    P, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    T = AttnTensor
    SP = ctypes.POINTER(AttnMaskSpec)
    lib.attn_mask_bytes.restype = sz
    lib.attn_mask_bytes.argtypes = [SP, i32, i32]
    lib.attn_mask_build.restype = i32
    lib.attn_mask_build.argtypes = [SP, i32, i32, P, sz, P]
    lib.attn_fwd_workspace_size.restype = sz
    lib.attn_fwd_workspace_size.argtypes = [SP, i32, i32]
    lib.attn_fwd.restype = i32
    lib.attn_fwd.argtypes = [T, T, T, T, P, i32, i32, i32, i32, i32, SP, f32, P, P, sz, P]
    lib.attn_fwd_varlen_workspace_size.restype = sz
    lib.attn_fwd_varlen_workspace_size.argtypes = [i32, i32]
    lib.attn_fwd_varlen.restype = i32
    lib.attn_fwd_varlen.argtypes = [T, T, T, T, P, P, P, i32, i32, i32, i32, i32, i32, SP, f32, P, sz, P]
    lib.attn_quantize_fp8_workspace_size.restype = sz
    lib.attn_quantize_fp8_workspace_size.argtypes = [i32, i32, i32]
    lib.attn_quantize_fp8.restype = i32
    lib.attn_quantize_fp8.argtypes = [T, T, P, i32, i32, i32, i32, P, i32, P, sz, P]
    lib.attn_fwd_fp8.restype = i32
    lib.attn_fwd_fp8.argtypes = [T, T, T, P, P, P, T, P, i32, i32, i32, i32, i32, SP, f32, P, P, sz, P]
    lib.attn_decode_workspace_size.restype = sz
    lib.attn_decode_workspace_size.argtypes = [i32, i32, i32, i32, i32]
    lib.attn_decode.restype = i32
    lib.attn_decode.argtypes = [T, T, T, P, T, P, i32, i32, i32, i32, i32, i32, f32, P, sz, P]
    lib.attn_decode_noalloc.restype = i32
    lib.attn_decode_noalloc.argtypes = [T, T, T, P, T, P, i32, i32, i32, i32, i32, i32, f32, P]
    lib.attn_bwd_workspace_size.restype = sz
    lib.attn_bwd_workspace_size.argtypes = [SP, i32, i32, i32]
    lib.attn_bwd.restype = i32
    lib.attn_bwd.argtypes = [T, T, T, T, P, T, T, T, T, i32, i32, i32, i32, i32, SP, f32, P, sz, P]
    lib.attn_status_string.restype = ctypes.c_char_p
    lib.attn_status_string.argtypes = [i32]
    lib.attn_last_error.restype = ctypes.c_char_p
    lib.attn_last_error.argtypes = []
    _lib = lib
    return lib


def library():
    """The loaded ctypes library (built on first use if absent)."""
    return _load()


def _check(status: int):
    if status != ATTN_OK:
        lib = _load()
        msg = lib.attn_last_error().decode() or lib.attn_status_string(status).decode()
        raise AttnError(status, msg)


def _tensor4(t: torch.Tensor) -> AttnTensor:
    if t.dim() != 4:
        raise ValueError("expected a 4-D tensor [B, H, N, d]")
    return AttnTensor(t.data_ptr(), t.stride(0), t.stride(1), t.stride(2))


def _check_bf16(name, t):
    if not t.is_cuda or t.dtype != torch.bfloat16:
        raise TypeError(f"{name}: expected a bf16 tensor on a GPU")
    if t.numel() and t.stride(-1) != 1:
        raise ValueError(f"{name}: the head dimension must be contiguous")


def _check_out(name, t, shape, dtype, device, contiguous=False):
    """A caller-supplied output buffer must match what the call writes: the
    C ABI takes only pointers and strides, so a smaller or mistyped buffer
    would be written out of bounds."""
    if not isinstance(t, torch.Tensor) or t.dtype != dtype or t.device != device:
        raise TypeError(f"{name}: expected a {dtype} tensor on {device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if dtype == torch.bfloat16 and t.numel() and t.stride(-1) != 1:
        raise ValueError(f"{name}: the head dimension must be contiguous")


def _check_block_mask(lib, block_mask, spec, B, N, device):
    """A prebuilt block mask must be a uint8 device buffer at least as large
    as the layout for (B, N) (attn_mask_bytes)."""
    if (not isinstance(block_mask, torch.Tensor) or block_mask.dtype != torch.uint8
            or block_mask.device != device or not block_mask.is_contiguous()):
        raise TypeError(f"block_mask: expected a contiguous uint8 tensor on {device} (from mask_build)")
    need = lib.attn_mask_bytes(spec.ref(), B, N)
    if block_mask.numel() < need:
        raise ValueError(f"block_mask: {block_mask.numel()} bytes, the mask for B={B}, N={N} "
                         f"needs {need}")


def _check_spec(spec, B, Hq, device):
    """The spec's device arrays are read per batch row (document offsets) and
    per query head (ALiBi slopes)."""
    if spec.doc_offsets is not None:
        if spec.doc_offsets.device != device:
            raise TypeError(f"doc_offsets: expected a tensor on {device}")
        if spec.doc_offsets.shape[0] < B:
            raise ValueError(f"doc_offsets: {spec.doc_offsets.shape[0]} rows for B={B} batch rows")
    if spec.alibi_slopes is not None:
        if spec.alibi_slopes.device != device:
            raise TypeError(f"alibi_slopes: expected a tensor on {device}")
        if Hq is not None and spec.alibi_slopes.numel() != Hq:
            raise ValueError("alibi_slopes must hold one slope per query head")


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


class MaskSpec:
    """Python holder of an ``attn_mask_spec`` (keeps doc_offsets alive)."""

    def __init__(self, *, causal=False, window=None, doc_offsets=None,
                 softcap=None, no_skip=False, alibi_slopes=None):
        flags = 0
        wl = wr = 0
        if causal:
            flags |= ATTN_MASK_CAUSAL
        if window is not None:
            flags |= ATTN_MASK_WINDOW
            wl, wr = (window, window) if isinstance(window, int) else window
        self.doc_offsets = None
        doc_ptr, doc_stride = None, 0
        if doc_offsets is not None:
            flags |= ATTN_MASK_DOCS
            if doc_offsets.dtype != torch.int32 or not doc_offsets.is_cuda or doc_offsets.dim() != 2:
                raise TypeError("doc_offsets: expected an int32 [B, max_docs+1] GPU tensor")
            self.doc_offsets = doc_offsets.contiguous()
            doc_ptr, doc_stride = self.doc_offsets.data_ptr(), self.doc_offsets.shape[1]
        cap = 0.0
        if softcap is not None:
            flags |= ATTN_MOD_SOFTCAP
            cap = float(softcap)
        if no_skip:
            flags |= ATTN_MASK_NO_SKIP
        self.alibi_slopes = None
        slopes_ptr = None
        if alibi_slopes is not None:
            if alibi_slopes.dtype != torch.float32 or not alibi_slopes.is_cuda or alibi_slopes.dim() != 1:
                raise TypeError("alibi_slopes: expected a float32 [Hq] GPU tensor")
            flags |= ATTN_MOD_ALIBI
            self.alibi_slopes = alibi_slopes.contiguous()
            slopes_ptr = self.alibi_slopes.data_ptr()
        self.c = AttnMaskSpec(flags, int(wl), int(wr), cap, doc_ptr, doc_stride, slopes_ptr)

    def ref(self):
        return ctypes.byref(self.c)


def mask_build(spec: MaskSpec, B: int, N: int, device=None) -> torch.Tensor:
    """Build a reusable block mask (a uint8 device buffer)."""
    lib = _load()
    device = device or torch.device("cuda", torch.cuda.current_device())
    _check_spec(spec, B, None, device)
    nbytes = lib.attn_mask_bytes(spec.ref(), B, N)
    buf = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)
    _check(lib.attn_mask_build(spec.ref(), B, N, buf.data_ptr(), nbytes, _stream(device)))
    return buf


def fwd(q, k, v, *, causal=False, window=None, doc_offsets=None, softcap=None,
        scale=None, block_mask=None, no_skip=False, spec=None, out=None, lse=None,
        alibi_slopes=None):
    """Exact attention forward.  q [B,Hq,N,d], k/v [B,Hkv,N,d] bf16 (any
    batch/head/token strides).  Returns (O [B,Hq,N,d] bf16, LSE [B,Hq,N] fp32)."""
    lib = _load()
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_bf16(name, t)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    if k.shape != (B, Hkv, N, d) or v.shape != (B, Hkv, N, d):
        raise ValueError(f"k/v must be [B, Hkv, N, d]; got {tuple(k.shape)} and {tuple(v.shape)}")
    if spec is None:
        spec = MaskSpec(causal=causal, window=window, doc_offsets=doc_offsets,
                        softcap=softcap, no_skip=no_skip, alibi_slopes=alibi_slopes)
    _check_spec(spec, B, Hq, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, Hq, N, d), dtype=torch.bfloat16, device=q.device)
    _check_out("out", out, (B, Hq, N, d), torch.bfloat16, q.device)
    if lse is None:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    _check_out("lse", lse, (B, Hq, N), torch.float32, q.device, contiguous=True)
    ws = None
    ws_bytes = 0
    if block_mask is None:
        ws_bytes = lib.attn_fwd_workspace_size(spec.ref(), B, N)
        ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
    else:
        _check_block_mask(lib, block_mask, spec, B, N, q.device)
    st = lib.attn_fwd(_tensor4(q), _tensor4(k), _tensor4(v), _tensor4(out), lse.data_ptr(),
                      B, Hq, Hkv, N, d, spec.ref(), float(scale),
                      None if block_mask is None else block_mask.data_ptr(),
                      None if ws is None else ws.data_ptr(), ws_bytes, _stream(q.device))
    _check(st)
    return out, lse


def _tensor3(t: torch.Tensor) -> AttnTensor:
    if t.dim() != 3:
        raise ValueError("expected a 3-D tensor [total, H, d]")
    return AttnTensor(t.data_ptr(), 0, t.stride(1), t.stride(0))


def fwd_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, *, causal=False, window=None,
               softcap=None, scale=None, no_skip=False, out=None, lse=None, workspace=None):
    """Exact attention over packed variable-length sequences.  q [total_q, Hq, d],
    k/v [total_k, Hkv, d] bf16; cu_seqlens_q/k int32 [nseq + 1] on the GPU
    (cumulative lengths).  Returns (O [total_q, Hq, d] bf16, LSE [Hq, total_q] fp32)."""
    lib = _load()
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_bf16(name, t)
    tq, Hq, d = q.shape
    tk, Hkv = k.shape[0], k.shape[1]
    if k.shape != (tk, Hkv, d) or v.shape != (tk, Hkv, d):
        raise ValueError(f"k/v must be [total_k, Hkv, d]; got {tuple(k.shape)} and {tuple(v.shape)}")
    for name, c in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k)):
        if c.dtype != torch.int32 or not c.is_cuda or c.dim() != 1 or not c.is_contiguous():
            raise TypeError(f"{name}: expected a contiguous int32 [nseq + 1] GPU tensor")
    if cu_seqlens_q.numel() != cu_seqlens_k.numel() or cu_seqlens_q.numel() < 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both hold nseq + 1 >= 1 entries")
    nseq = cu_seqlens_q.numel() - 1
    spec = MaskSpec(causal=causal, window=window, softcap=softcap, no_skip=no_skip)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((tq, Hq, d), dtype=torch.bfloat16, device=q.device)
    _check_out("out", out, (tq, Hq, d), torch.bfloat16, q.device)
    if lse is None:
        lse = torch.empty((Hq, tq), dtype=torch.float32, device=q.device)
    _check_out("lse", lse, (Hq, tq), torch.float32, q.device, contiguous=True)
    ws_bytes = lib.attn_fwd_varlen_workspace_size(tq, tk)
    if workspace is not None and (workspace.dtype != torch.uint8 or workspace.device != q.device):
        raise TypeError(f"workspace: expected a uint8 tensor on {q.device}")
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
    st = lib.attn_fwd_varlen(_tensor3(q), _tensor3(k), _tensor3(v), _tensor3(out), lse.data_ptr(),
                             cu_seqlens_q.data_ptr(), cu_seqlens_k.data_ptr(), nseq, tq, tk, Hq, Hkv,
                             d, spec.ref(), float(scale), workspace.data_ptr(), ws_bytes,
                             _stream(q.device))
    _check(st)
    return out, lse


def fwd_varlen_workspace_bytes(total_q, total_k) -> int:
    return _load().attn_fwd_varlen_workspace_size(total_q, total_k)


def bwd(q, k, v, o, lse, dout, *, causal=False, window=None, doc_offsets=None,
        softcap=None, scale=None, no_skip=False, spec=None, dq=None, dk=None, dv=None,
        workspace=None):
    """Gradients of exact attention.  q, k, v and the mask arguments as given
    to ``fwd``; o, lse its outputs; dout [B,Hq,N,d] bf16 the gradient of the
    loss with respect to o.  Returns (dQ [B,Hq,N,d], dK, dV [B,Hkv,N,d]) bf16."""
    lib = _load()
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        _check_bf16(name, t)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    if k.shape != (B, Hkv, N, d) or v.shape != (B, Hkv, N, d):
        raise ValueError(f"k/v must be [B, Hkv, N, d]; got {tuple(k.shape)} and {tuple(v.shape)}")
    if o.shape != q.shape or dout.shape != q.shape:
        raise ValueError("o and dout must have the shape of q")
    if lse.dtype != torch.float32 or not lse.is_contiguous() or lse.shape != (B, Hq, N):
        raise TypeError("lse: expected a contiguous fp32 [B, Hq, N] tensor")
    if spec is None:
        spec = MaskSpec(causal=causal, window=window, doc_offsets=doc_offsets,
                        softcap=softcap, no_skip=no_skip)
    _check_spec(spec, B, Hq, q.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if dq is None:
        dq = torch.empty((B, Hq, N, d), dtype=torch.bfloat16, device=q.device)
    if dk is None:
        dk = torch.empty((B, Hkv, N, d), dtype=torch.bfloat16, device=q.device)
    if dv is None:
        dv = torch.empty((B, Hkv, N, d), dtype=torch.bfloat16, device=q.device)
    if lse.device != q.device:
        raise TypeError(f"lse: expected a tensor on {q.device}")
    for name, t, shape in (("dq", dq, (B, Hq, N, d)), ("dk", dk, (B, Hkv, N, d)), ("dv", dv, (B, Hkv, N, d))):
        _check_out(name, t, shape, torch.bfloat16, q.device)
    ws_bytes = lib.attn_bwd_workspace_size(spec.ref(), B, Hq, N)
    if workspace is not None and (workspace.dtype != torch.uint8 or workspace.device != q.device):
        raise TypeError(f"workspace: expected a uint8 tensor on {q.device}")
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
    st = lib.attn_bwd(_tensor4(q), _tensor4(k), _tensor4(v), _tensor4(o), lse.data_ptr(),
                      _tensor4(dout), _tensor4(dq), _tensor4(dk), _tensor4(dv),
                      B, Hq, Hkv, N, d, spec.ref(), float(scale), workspace.data_ptr(),
                      ws_bytes, _stream(q.device))
    _check(st)
    return dq, dk, dv


def bwd_workspace_bytes(B, Hq, N, spec=None) -> int:
    return _load().attn_bwd_workspace_size(None if spec is None else spec.ref(), B, Hq, N)


def _tensor4u8(t: torch.Tensor) -> AttnTensor:
    if t.dim() != 4 or t.dtype != torch.uint8 or not t.is_cuda:
        raise TypeError("expected a uint8 [B, H, N, d] GPU tensor of E4M3 codes")
    if t.stride(-1) != 1:
        raise ValueError("the head dimension must be contiguous")
    return AttnTensor(t.data_ptr(), t.stride(0), t.stride(1), t.stride(2))


def quantize_fp8(x, *, signs=None, per_head=False, out=None, scales=None):
    """E4M3 block quantization of a bf16 [B, H, N, 128] tensor.  signs: an
    int8 [128] GPU tensor of +-1 for the random Hadamard rotation (the same
    for Q and K), or None.  Returns (codes uint8 [B,H,N,128], scales fp32
    [B, H, ceil(N/64)])."""
    lib = _load()
    _check_bf16("x", x)
    B, H, N, d = x.shape
    if out is None:
        out = torch.empty((B, H, N, d), dtype=torch.uint8, device=x.device)
    elif tuple(out.shape) != (B, H, N, d):
        raise ValueError(f"out must be {(B, H, N, d)}; got {tuple(out.shape)}")
    if scales is None:
        scales = torch.empty((B, H, (N + 63) // 64), dtype=torch.float32, device=x.device)
    elif (tuple(scales.shape) != (B, H, (N + 63) // 64) or scales.dtype != torch.float32
          or not scales.is_contiguous()):
        raise ValueError("scales must be a contiguous fp32 [B, H, ceil(N/64)] tensor")
    if signs is not None and (signs.dtype != torch.int8 or not signs.is_cuda or signs.numel() != d):
        raise TypeError("signs: expected an int8 [d] GPU tensor of +-1")
    ws_bytes = lib.attn_quantize_fp8_workspace_size(B, H, N)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=x.device)
    st = lib.attn_quantize_fp8(_tensor4(x), _tensor4u8(out), scales.data_ptr(), B, H, N, d,
                               None if signs is None else signs.data_ptr(), int(bool(per_head)),
                               ws.data_ptr(), ws_bytes, _stream(x.device))
    _check(st)
    return out, scales


def fwd_fp8(q8, k8, v8, q_scales, k_scales, v_scales, *, causal=False, window=None,
            doc_offsets=None, softcap=None, scale=None, block_mask=None, no_skip=False,
            spec=None, out=None, lse=None):
    """Forward attention on E4M3 codes from quantize_fp8 (v quantized per
    head).  Returns (O [B,Hq,N,128] bf16, LSE [B,Hq,N] fp32)."""
    lib = _load()
    for name, t in (("q8", q8), ("k8", k8), ("v8", v8)):
        _tensor4u8(t)
    B, Hq, N, d = q8.shape
    Hkv = k8.shape[1]
    if k8.shape != (B, Hkv, N, d) or v8.shape != (B, Hkv, N, d):
        raise ValueError(f"k8/v8 must be [B, Hkv, N, d]; got {tuple(k8.shape)} and {tuple(v8.shape)}")
    nblk = (N + 63) // 64
    for name, t, H in (("q_scales", q_scales, Hq), ("k_scales", k_scales, Hkv), ("v_scales", v_scales, Hkv)):
        if tuple(t.shape) != (B, H, nblk):
            raise ValueError(f"{name} must be [B, H, ceil(N/64)] = {(B, H, nblk)}; got {tuple(t.shape)}")
    if spec is None:
        spec = MaskSpec(causal=causal, window=window, doc_offsets=doc_offsets, softcap=softcap,
                        no_skip=no_skip)
    _check_spec(spec, B, Hq, q8.device)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, Hq, N, d), dtype=torch.bfloat16, device=q8.device)
    _check_out("out", out, (B, Hq, N, d), torch.bfloat16, q8.device)
    if lse is None:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q8.device)
    _check_out("lse", lse, (B, Hq, N), torch.float32, q8.device, contiguous=True)
    for name, t in (("q_scales", q_scales), ("k_scales", k_scales), ("v_scales", v_scales)):
        if t.dtype != torch.float32 or t.device != q8.device or not t.is_contiguous():
            raise TypeError(f"{name}: expected a contiguous fp32 tensor on {q8.device}")
    ws = None
    ws_bytes = 0
    if block_mask is None:
        ws_bytes = lib.attn_fwd_workspace_size(spec.ref(), B, N)
        ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q8.device)
    else:
        _check_block_mask(lib, block_mask, spec, B, N, q8.device)
    st = lib.attn_fwd_fp8(_tensor4u8(q8), _tensor4u8(k8), _tensor4u8(v8), q_scales.data_ptr(),
                          k_scales.data_ptr(), v_scales.data_ptr(), _tensor4(out), lse.data_ptr(),
                          B, Hq, Hkv, N, d, spec.ref(), float(scale),
                          None if block_mask is None else block_mask.data_ptr(),
                          None if ws is None else ws.data_ptr(), ws_bytes, _stream(q8.device))
    _check(st)
    return out, lse


def decode(q, k_cache, v_cache, lens, *, scale=None, chunk=1024, out=None, lse=None,
           workspace=None):
    """Split-KV decode.  q [B,Hq,d] (or [B,Hq,1,d]), caches [B,Hkv,T,d] bf16,
    lens int32 [B] on the GPU.  Returns (O [B,Hq,d] bf16, LSE [B,Hq] fp32)."""
    lib = _load()
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache)):
        _check_bf16(name, t)
    if q.dim() not in (3, 4) or (q.dim() == 4 and q.shape[2] != 1):
        raise ValueError(f"q: expected [B, Hq, d] or [B, Hq, 1, d], got {tuple(q.shape)}")
    q4 = q if q.dim() == 4 else q.unsqueeze(2)
    B, Hq, _, d = q4.shape
    if k_cache.dim() != 4:
        raise ValueError(f"k_cache: expected [B, Hkv, T, d], got {tuple(k_cache.shape)}")
    Hkv, T = k_cache.shape[1], k_cache.shape[2]
    if tuple(k_cache.shape) != (B, Hkv, T, d) or tuple(v_cache.shape) != (B, Hkv, T, d):
        raise ValueError(f"k_cache and v_cache must both be [B, Hkv, T, d] = {(B, Hkv, T, d)}; "
                         f"got {tuple(k_cache.shape)} and {tuple(v_cache.shape)}")
    if k_cache.device != q.device or v_cache.device != q.device:
        raise TypeError("q, k_cache and v_cache must be on the same device")
    if (lens.dtype != torch.int32 or lens.device != q.device or lens.dim() != 1
            or lens.numel() != B or not lens.is_contiguous()):
        raise TypeError(f"lens: expected a contiguous int32 [B] tensor on {q.device}")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.bfloat16, device=q.device)
    o4 = out if out.dim() == 4 else out.unsqueeze(2)
    _check_out("out", o4, (B, Hq, 1, d), torch.bfloat16, q.device)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    _check_out("lse", lse, (B, Hq), torch.float32, q.device, contiguous=True)
    ws_bytes = lib.attn_decode_workspace_size(B, Hq, T, d, chunk)
    if workspace is not None and (workspace.dtype != torch.uint8 or workspace.device != q.device):
        raise TypeError(f"workspace: expected a uint8 tensor on {q.device}")
    if workspace is None or workspace.numel() < ws_bytes:
        workspace = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=q.device)
    st = lib.attn_decode(_tensor4(q4), _tensor4(k_cache), _tensor4(v_cache),
                         lens.data_ptr(), _tensor4(o4), lse.data_ptr(), B, Hq, Hkv, T, d,
                         int(chunk), float(scale), workspace.data_ptr(), ws_bytes,
                         _stream(q.device))
    _check(st)
    return out, lse


def decode_noalloc(q, k_cache, v_cache, lens, *, out, lse, scale=None, chunk=1024):
    """``decode`` through attn_decode_noalloc: the chunk partials live in the
    library's static per-GPU scratch, and nothing is allocated -- not here
    either, so the caller passes ``out`` [B,Hq,d] bf16 and ``lse`` [B,Hq]
    fp32.  Calls that may overlap on one GPU race on that scratch.
    Returns (out, lse)."""
    lib = _load()
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache)):
        _check_bf16(name, t)
    if q.dim() not in (3, 4) or (q.dim() == 4 and q.shape[2] != 1):
        raise ValueError(f"q: expected [B, Hq, d] or [B, Hq, 1, d], got {tuple(q.shape)}")
    q4 = q if q.dim() == 4 else q.unsqueeze(2)
    B, Hq, _, d = q4.shape
    if k_cache.dim() != 4:
        raise ValueError(f"k_cache: expected [B, Hkv, T, d], got {tuple(k_cache.shape)}")
    Hkv, T = k_cache.shape[1], k_cache.shape[2]
    if tuple(k_cache.shape) != (B, Hkv, T, d) or tuple(v_cache.shape) != (B, Hkv, T, d):
        raise ValueError(f"k_cache and v_cache must both be [B, Hkv, T, d] = {(B, Hkv, T, d)}; "
                         f"got {tuple(k_cache.shape)} and {tuple(v_cache.shape)}")
    if k_cache.device != q.device or v_cache.device != q.device:
        raise TypeError("q, k_cache and v_cache must be on the same device")
    if (lens.dtype != torch.int32 or lens.device != q.device or lens.dim() != 1
            or lens.numel() != B or not lens.is_contiguous()):
        raise TypeError(f"lens: expected a contiguous int32 [B] tensor on {q.device}")
    o4 = out if out.dim() == 4 else out.unsqueeze(2)
    _check_out("out", o4, (B, Hq, 1, d), torch.bfloat16, q.device)
    _check_out("lse", lse, (B, Hq), torch.float32, q.device, contiguous=True)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    st = lib.attn_decode_noalloc(_tensor4(q4), _tensor4(k_cache), _tensor4(v_cache), lens.data_ptr(),
                                 _tensor4(o4), lse.data_ptr(), B, Hq, Hkv, T, d, int(chunk),
                                 float(scale), _stream(q.device))
    _check(st)
    return out, lse


def decode_workspace_bytes(B, Hq, T, d, chunk=1024) -> int:
    return _load().attn_decode_workspace_size(B, Hq, T, d, chunk)


def mask_layout(B: int, N: int) -> dict:
    """Offsets (bytes) of the block-mask sections, mirroring the C layout."""
    def a256(x):
        return (x + 255) & ~255
    nqt = (N + BLOCK_M - 1) // BLOCK_M
    nkt = (N + BLOCK_N - 1) // BLOCK_N
    rows, items = B * N, B * nqt
    off = 0
    lay = {"nqt": nqt, "nkt": nkt}
    lay["lo"] = off; off = a256(off + 4 * rows)
    lay["hi"] = off; off = a256(off + 4 * rows)
    lay["count"] = off; off = a256(off + 4 * items)
    lay["list"] = off; off = a256(off + 4 * items * nkt)
    lay["order"] = off; off = a256(off + 4 * items)
    lay["bytes"] = off
    return lay


def mask_unpack(buf: torch.Tensor, B: int, N: int) -> dict:
    """Host copy of a block mask's sections (for inspection and tests)."""
    lay = mask_layout(B, N)
    raw = buf.cpu()

    def sect(name, n):
        return raw[lay[name]: lay[name] + 4 * n].view(torch.int32).clone()
    nqt, nkt = lay["nqt"], lay["nkt"]
    return {
        "lo": sect("lo", B * N).view(B, N),
        "hi": sect("hi", B * N).view(B, N),
        "count": sect("count", B * nqt).view(B, nqt),
        "list": sect("list", B * nqt * nkt).view(B, nqt, nkt),
        "order": sect("order", B * nqt),
        "nqt": nqt, "nkt": nkt,
    }
