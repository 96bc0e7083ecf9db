"""Exact attention for AMD MI355X (gfx950): tiled online-softmax forward and
its backward, register-level masks and score mods, and split-KV decode, as
hand-written HIP kernels behind a small C ABI (``include/exattn.h``).

The Python surface is a thin ctypes binding: PyTorch provides device memory
and streams, the kernels do all of the work.
"""
from .binding import (  # noqa: F401
    ATTN_MASK_CAUSAL, ATTN_MASK_DOCS, ATTN_MASK_NO_SKIP, ATTN_MASK_WINDOW,
    ATTN_MOD_ALIBI, ATTN_MOD_SOFTCAP, BLOCK_M, BLOCK_N, AttnError, MaskSpec, bwd, bwd_workspace_bytes,
    decode, decode_noalloc, decode_workspace_bytes, fwd, fwd_fp8, fwd_varlen, fwd_varlen_workspace_bytes, library,
    mask_build, mask_layout, mask_unpack, quantize_fp8,
)
