/*
 * exattn.h -- C ABI of the MI355X (gfx950) exact-attention library.
 *
 * The library computes exact softmax(Q K^T * scale) V tile by tile with an
 * online softmax (running row max m and running sum l, rescaling the output
 * block by block), so the N x N score and probability matrices never reach
 * HBM.  Sources for the operation:
 *   - the attention definition and its tiling/online-softmax form:
 *     youngju.dev "FlashAttention 논문 분석: IO-Aware Exact Attention...",
 *     sections "수학적 정의", "Online Softmax와 블록 단위 누적" and
 *     "알고리즘 의사코드";
 *   - register-level score modifications and masks (causal, sliding window,
 *     document boundaries) and block-level skipping of fully masked tiles:
 *     it-trends-board "PyTorch FlexAttention 도입 분석", section 2;
 *   - GQA, soft cap, packed documents and split-KV decode with a combine:
 *     aegloslab "3.7 어텐션 II — 융합 커널·실전 라이브러리", sections 3.7.4
 *     to 3.7.6.
 *
 * Conventions shared by every entry point
 *   - Device pointers are HIP device memory owned by the caller.  The library
 *     never allocates, frees or synchronises; it enqueues work on `stream`
 *     (a hipStream_t passed as void*, NULL = the default stream) and returns.
 *     Buffers must stay valid until that work completes.
 *   - Tensors are bf16 (stored as raw 16-bit values) with a unit stride on
 *     the head dimension d and explicit element strides for batch, head and
 *     token, so [B,H,N,d] and [B,N,H,d] layouts both work without copies.
 *     Pointers must be 16-byte aligned and strides multiples of 8 elements.
 *   - A non-OK status means nothing was enqueued, except ATTN_ERR_HIP (a
 *     launch failed after validation).  attn_last_error() gives a message
 *     for the calling thread's last non-OK status.  There is no fallback
 *     path: unsupported input is an error.
 *   - Calls on one stream are ordered; calls that share a workspace or block
 *     mask buffer on different streams race.
 */
#ifndef EXATTN_H
#define EXATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    ATTN_OK = 0,
    ATTN_ERR_INVALID = 1,     /* malformed argument (null pointer, bad size, misaligned) */
    ATTN_ERR_UNSUPPORTED = 2, /* well-formed but not implemented (head dim, group size) */
    ATTN_ERR_WORKSPACE = 3,   /* workspace / block-mask buffer too small */
    ATTN_ERR_HIP = 4          /* a kernel launch failed */
} attn_status;

/* Mask and score-modification flags (attn_mask_spec.flags), combined by AND. */
enum {
    ATTN_MASK_CAUSAL = 1u,  /* key j visible to query i only if j <= i */
    ATTN_MASK_WINDOW = 2u,  /* visible only if i - window_left <= j <= i + window_right */
    ATTN_MASK_DOCS = 4u,    /* visible only inside the query's document */
    ATTN_MOD_SOFTCAP = 8u,  /* visible scores s -> softcap * tanh(s / softcap) */
    ATTN_MASK_NO_SKIP = 16u, /* diagnostic: visit every key tile (none skipped,
                                all element-masked); results are bitwise equal */
    ATTN_MOD_ALIBI = 32u     /* distance bias: s -> s - slope[h] * |i - j| (attn_fwd only) */
};

/*
 * Mask specification.  Every supported mask gives each query row one
 * contiguous interval of visible keys, which is what the block mask stores.
 * The scaled score gets the ALiBi bias (if any), is masked to -inf, and the
 * soft cap then applies to the remaining scores only, so masked keys get
 * weight exactly 0.  ALiBi adds a distance-based bias before the softmax
 * (aegloslab "3.7 어텐션 II", section 3.7.5): query head h subtracts
 * alibi_slopes[h] * |i - j|; the slopes are the caller's (the usual choice
 * is a geometric sequence over the heads).  It does not change which tiles
 * the block mask skips.
 */
typedef struct {
    uint32_t flags;
    int32_t window_left;        /* ATTN_MASK_WINDOW: keys before i that stay visible */
    int32_t window_right;       /* ATTN_MASK_WINDOW: keys after i that stay visible */
    float softcap;              /* ATTN_MOD_SOFTCAP: cap c > 0 */
    const int32_t *doc_offsets; /* ATTN_MASK_DOCS: device int32 [B][doc_stride], per
                                   row 0 = o_0 < o_1 < ... < o_n = N, padded with N
                                   (cumulative document boundaries) */
    int32_t doc_stride;         /* entries per batch row (max documents + 1), >= 2 */
    const float *alibi_slopes;  /* ATTN_MOD_ALIBI: device fp32 [Hq], finite */
} attn_mask_spec;

/* A strided bf16 tensor view: element (b, h, n, t) lives at
 * ptr + b*stride_b + h*stride_h + n*stride_n + t (in 2-byte elements). */
typedef struct {
    void *ptr;
    int64_t stride_b, stride_h, stride_n;
} attn_tensor;

/*
 * Block mask: per-row visible key intervals, and for every 128-query tile
 * the list of 64-key tiles that hold at least one visible key, each marked
 * FULL (no element mask needed) or PARTIAL, plus a heavy-first order of the
 * query tiles of each batch row.  Fully masked tiles are never visited (it-trends-board
 * "PyTorch FlexAttention 도입 분석", section 2, the block-mask early-out;
 * youngju.dev "FlashAttention 논문 분석", FlashAttention-2 improvement 1:
 * blocks that need no mask skip the masking).
 *
 * attn_mask_bytes: size in bytes of the block mask for (spec, B, N).
 * attn_mask_build: builds it into `out` (device memory, >= attn_mask_bytes)
 *   on `stream`.  Depends only on the spec, B and N (never on heads or data),
 *   so one build serves any number of attn_fwd calls with the same mask.
 *   Errors: ATTN_ERR_INVALID (null spec/out with B*N > 0, B < 0, N < 0, bad
 *   doc_stride, softcap <= 0 with ATTN_MOD_SOFTCAP), ATTN_ERR_UNSUPPORTED
 *   (N >= 2^30), ATTN_ERR_WORKSPACE (bytes too small), ATTN_ERR_HIP.
 */
size_t attn_mask_bytes(const attn_mask_spec *spec, int B, int N);
attn_status attn_mask_build(const attn_mask_spec *spec, int B, int N, void *out,
                            size_t bytes, void *stream);

/*
 * Forward attention (prefill, Nq = Nk = N): O = softmax(Q K^T * scale) V
 * per (batch row, query head), computed tile by tile with a running row
 * max and sum so that no score or probability matrix is stored
 * (youngju.dev "FlashAttention 논문 분석", sections "수학적 정의",
 * "Online Softmax와 블록 단위 누적" and "알고리즘 의사코드"; the
 * FlashAttention-2 section for normalising once at the end and for the
 * grid over query tiles).  Masks and score mods per attn_mask_spec
 * (it-trends-board "PyTorch FlexAttention 도입 분석", section 2; aegloslab
 * "3.7 어텐션 II", section 3.7.5).
 *   q [B,Hq,N,d], k and v [B,Hkv,N,d]: bf16 inputs; query head h reads KV
 *     head h / (Hq/Hkv) (grouped-query attention, no K/V copies).
 *   o [B,Hq,N,d]: bf16 output, normalised (O = P V with rows of P summing
 *     to 1), rounded to nearest even.
 *   lse: fp32 [B][Hq][N] contiguous, natural-log log-sum-exp of the final
 *     (scaled, masked, capped) scores of each row; -inf (and O = 0) for a
 *     row with no visible key.
 *   scale: multiplies q.k before masking; finite and > 0 (1/sqrt(d) is the
 *     usual choice).
 *   block_mask: a buffer built by attn_mask_build with the same spec, B and
 *     N, or NULL.  If NULL the call builds one in `workspace` first, which
 *     then needs attn_fwd_workspace_size bytes; otherwise workspace may be
 *     NULL with ws_bytes 0.
 * Supported: d in {64, 128}; Hq % Hkv == 0; 0 <= N < 2^30; B >= 0 (B*N == 0
 * is a no-op).  Errors: ATTN_ERR_INVALID, ATTN_ERR_UNSUPPORTED (other d),
 * ATTN_ERR_WORKSPACE, ATTN_ERR_HIP.
 */
size_t attn_fwd_workspace_size(const attn_mask_spec *spec, int B, int N);
attn_status attn_fwd(attn_tensor q, attn_tensor k, attn_tensor v, attn_tensor o,
                     float *lse, int B, int Hq, int Hkv, int N, int d,
                     const attn_mask_spec *spec, float scale,
                     const void *block_mask, void *workspace, size_t ws_bytes,
                     void *stream);

/*
 * Forward attention over packed variable-length sequences (no padding):
 * the flash-attn varlen form of aegloslab "3.7 어텐션 II", section 3.7.6.
 * Sequence s owns query rows [cu_seqlens_q[s], cu_seqlens_q[s+1]) and keys
 * [cu_seqlens_k[s], cu_seqlens_k[s+1]); a query sees only its own
 * sequence's keys.
 *   q [total_q, Hq, d], k and v [total_k, Hkv, d], o [total_q, Hq, d]: bf16,
 *     given as attn_tensor with stride_h and stride_n (stride_b is ignored).
 *   lse: fp32 [Hq][total_q] contiguous (natural log; -inf and O = 0 for a
 *     row with no visible key).
 *   cu_seqlens_q, cu_seqlens_k: device int32 [nseq + 1], nondecreasing from
 *     0 to total_q (total_k): the cumulative lengths.  Values outside
 *     [0, total] are clamped (never read out of bounds); other malformed
 *     offsets give unspecified results.
 *   spec: ATTN_MASK_CAUSAL, ATTN_MASK_WINDOW, ATTN_MOD_SOFTCAP and
 *     ATTN_MASK_NO_SKIP apply inside each sequence (ATTN_MASK_DOCS is
 *     rejected, ATTN_MOD_ALIBI unsupported).  With Lq queries and Lk keys in a sequence, local query i
 *     lines up with local key i + Lk - Lq (the last query with the last
 *     key): causal keeps keys j <= i + Lk - Lq, the window is taken about
 *     that key.  For Lq = Lk this is the usual square mask.
 *   workspace: >= attn_fwd_varlen_workspace_size(total_q, total_k) bytes,
 *     16-byte aligned (the block mask is built there).
 * Supported: d in {64, 128}; Hq % Hkv == 0; total_q, total_k < 2^30.
 * total_q == 0 is a no-op.
 * Errors: ATTN_ERR_INVALID, ATTN_ERR_UNSUPPORTED, ATTN_ERR_WORKSPACE,
 * ATTN_ERR_HIP.
 */
size_t attn_fwd_varlen_workspace_size(int total_q, int total_k);
attn_status attn_fwd_varlen(attn_tensor q, attn_tensor k, attn_tensor v, attn_tensor o,
                            float *lse, const int32_t *cu_seqlens_q,
                            const int32_t *cu_seqlens_k, int nseq, int total_q, int total_k,
                            int Hq, int Hkv, int d, const attn_mask_spec *spec, float scale,
                            void *workspace, size_t ws_bytes, void *stream);

/*
 * Split-KV decode: one new query per (batch row, query head) against the
 * first lens[b] keys of a KV cache (aegloslab "3.7 어텐션 II", section
 * 3.7.4).  The valid keys are cut into chunks of `chunk` keys; every
 * (b, KV head, chunk) is processed in parallel, producing partial row max,
 * sum and unnormalised output for the whole GQA group, and a second kernel
 * merges the partials by rescaling each with exp(m_c - max_c m_c).
 *   q [B,Hq,1,d] (stride_n unused), k_cache and v_cache [B,Hkv,T,d] bf16.
 *   lens: device int32 [B], 0 <= lens[b] <= T (values outside are clamped
 *     into [0, T]); keys at positions >= lens[b] are never read.
 *   o [B,Hq,1,d] bf16 (stride_n unused); lse fp32 [B][Hq] contiguous
 *     (natural log; -inf and O = 0 when lens[b] == 0).
 *   chunk: keys per split, a multiple of 64 in [64, 2048].
 *   k_cache / v_cache token strides (stride_n) must be below 2^20 elements.
 *   workspace: >= attn_decode_workspace_size(B, Hq, T, d, chunk) bytes.
 * Supported: d in {64, 128}; Hq % Hkv == 0 with Hq/Hkv <= 16.
 * Errors: ATTN_ERR_INVALID, ATTN_ERR_UNSUPPORTED, ATTN_ERR_WORKSPACE,
 * ATTN_ERR_HIP.
 */
size_t attn_decode_workspace_size(int B, int Hq, int T, int d, int chunk);
attn_status attn_decode(attn_tensor q, attn_tensor k_cache, attn_tensor v_cache,
                        const int32_t *lens, attn_tensor o, float *lse, int B,
                        int Hq, int Hkv, int T, int d, int chunk, float scale,
                        void *workspace, size_t ws_bytes, void *stream);

/*
 * attn_decode without a workspace, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops and harnesses
 * that forbid hipMalloc.  The chunk partials live in a static device array
 * of ATTN_DECODE_NOALLOC_SCRATCH_BYTES inside the library, one copy per GPU,
 * held from the library's load until the process ends.  The call makes no
 * allocation of any kind.
 *   Arguments, layouts, results and the other errors: as attn_decode (the
 *   caller still owns q, the caches, lens, o and lse).
 *   The partials need attn_decode_workspace_size(B, Hq, T, d, chunk) bytes;
 *   a call needing more than ATTN_DECODE_NOALLOC_SCRATCH_BYTES returns
 *   ATTN_ERR_WORKSPACE and enqueues nothing (use attn_decode then).
 *   Every call on one GPU shares that GPU's scratch: calls that may overlap
 *   on the same GPU (different streams or host threads) race; calls on one
 *   stream are ordered and safe.  Nothing in the scratch needs clearing
 *   between calls.  The first call on a device looks up that device's
 *   scratch address (hipGetSymbolAddress); ATTN_ERR_HIP if that fails.
 */
#define ATTN_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
attn_status attn_decode_noalloc(attn_tensor q, attn_tensor k_cache, attn_tensor v_cache,
                                const int32_t *lens, attn_tensor o, float *lse, int B,
                                int Hq, int Hkv, int T, int d, int chunk, float scale,
                                void *stream);

/*
 * Backward of attn_fwd: the gradients dQ, dK, dV of a loss given its
 * gradient dO with respect to O.  The probabilities are recomputed tile by
 * tile from lse instead of being stored (youngju.dev "FlashAttention 논문
 * 분석", section "Recomputation 전략"); with dP = dO V^T and
 * D_i = sum_t dO_it O_it, dS = P * (dP - D) (times 1 - tanh^2 of the capped
 * score under ATTN_MOD_SOFTCAP), dQ = scale dS K, dK = scale dS^T Q,
 * dV = P^T dO.
 *   q, k, v, spec, scale, B, Hq, Hkv, N, d: exactly as given to attn_fwd.
 *   o [B,Hq,N,d] and lse fp32 [B][Hq][N] contiguous: attn_fwd's outputs.
 *   dout [B,Hq,N,d]: gradient of the loss with respect to o.
 *   dq [B,Hq,N,d], dk and dv [B,Hkv,N,d]: bf16 outputs, fully overwritten
 *     (no accumulation into existing values); dk and dv of a KV head sum
 *     over the Hq/Hkv query heads that share it.  They must not overlap any
 *     input.  Keys that no query sees get zero gradient, as do rows with no
 *     visible key.
 *   workspace: >= attn_bwd_workspace_size(spec, B, Hq, N) bytes, 16-byte
 *     aligned (the call builds its block masks and per-row data there).
 *   q, k, v, o and dout token strides must be below 2^24 elements.
 * Supported: d in {64, 128}; Hq % Hkv == 0; N < 2^30; not ATTN_MOD_ALIBI
 * (ATTN_ERR_UNSUPPORTED).  Errors: ATTN_ERR_INVALID, ATTN_ERR_UNSUPPORTED,
 * ATTN_ERR_WORKSPACE, ATTN_ERR_HIP.
 */
size_t attn_bwd_workspace_size(const attn_mask_spec *spec, int B, int Hq, int N);
attn_status attn_bwd(attn_tensor q, attn_tensor k, attn_tensor v, attn_tensor o,
                     const float *lse, attn_tensor dout, attn_tensor dq, attn_tensor dk,
                     attn_tensor dv, int B, int Hq, int Hkv, int N, int d,
                     const attn_mask_spec *spec, float scale, void *workspace,
                     size_t ws_bytes, void *stream);

/*
 * FP8 (E4M3) forward, FlashAttention-3's FP8 variant (youngju.dev
 * "FlashAttention 논문 분석", FlashAttention-3 sections "FP8 텐서 코어" and
 * "FP8 지원과 정확도 유지"): block quantization and incoherent processing.
 *
 * attn_quantize_fp8: E4M3 codes of a bf16 [B,H,N,d] tensor (d = 128).
 *   Every 64-row block of a (b, h) gets a scale 2^e, the smallest power of
 *   two with max|block| <= 448 * 2^e (per_head != 0: one scale per (b, h),
 *   written to each of its blocks); codes are round-to-nearest-even of
 *   value / 2^e.  With signs (device int8 [d] of +1/-1, the caller's random
 *   draws) each row is first multiplied by the random orthogonal matrix
 *   diag(signs) H / sqrt(d), H the Walsh-Hadamard matrix (fast butterfly,
 *   strides 1, 2, ..., d/2, in fp32): apply the same signs to Q and K (the
 *   product Q K^T is unchanged) and none to V.
 *   x: bf16 attn_tensor; out: byte strides (stride_b/h/n in bytes, multiples
 *   of 16), 16-byte aligned; scales: device fp32 [B][H][ceil(N/64)];
 *   workspace: >= attn_quantize_fp8_workspace_size(B, H, N) bytes.
 *
 * attn_fwd_fp8: attn_fwd on E4M3 inputs (d = 128): S = (q8 . k8) * sq * sk
 *   * scale with sq, sk the blocks' scales.  For the P V product each
 *   probability, taken against a reference max that trails the row max by
 *   at most a factor 4, is rounded to E4M3 as p * 2^6 (<= 256);
 *   O = sum(p~ v8) * sv / l with l the sum of the unrounded p, and the LSE
 *   uses the unrounded p as well.
 *   q [B,Hq,N,128], k, v [B,Hkv,N,128]: codes from attn_quantize_fp8 (byte
 *   strides, multiples of 16; token strides below 2^24 bytes);
 *   q_scales [B][Hq][ceil(N/64)], k_scales and v_scales [B][Hkv][ceil(N/64)]
 *   device fp32, as written by attn_quantize_fp8; v must be quantized with
 *   per_head set (its first block's scale is used for the whole head).
 *   o, lse, spec (not ATTN_MOD_ALIBI), scale, block_mask, workspace: as for
 *   attn_fwd.
 * Errors: ATTN_ERR_INVALID, ATTN_ERR_UNSUPPORTED (d != 128, N >= 2^30, ALiBi),
 * ATTN_ERR_WORKSPACE, ATTN_ERR_HIP.
 */
size_t attn_quantize_fp8_workspace_size(int B, int H, int N);
attn_status attn_quantize_fp8(attn_tensor x, attn_tensor out, float *scales, int B, int H, int N,
                              int d, const int8_t *signs, int per_head, void *workspace,
                              size_t ws_bytes, void *stream);
attn_status attn_fwd_fp8(attn_tensor q, attn_tensor k, attn_tensor v, const float *q_scales,
                         const float *k_scales, const float *v_scales, attn_tensor o, float *lse,
                         int B, int Hq, int Hkv, int N, int d, const attn_mask_spec *spec,
                         float scale, const void *block_mask, void *workspace, size_t ws_bytes,
                         void *stream);

/*
 * Errors.  Unsupported input is refused with a status and a message that
 * names what is unsupported (head dim, group size, layout, alignment), and
 * nothing runs in its place: the pages' troubleshooting material shows the
 * same convention (an exception that names the unsupported architecture or
 * tensor shape: youngju.dev "FlashAttention 논문 분석", section "트러블슈팅:
 * 실패 사례와 복구", cases 1 and 2) and names the silent fall back to a
 * slower N x N path as the most common hidden loss (aegloslab "3.7 어텐션
 * II", sections 3.7.3 and 3.7.9).
 *
 * attn_status_string: a static, never-null description of a status code
 *   ("unknown status" for values outside the enum).
 * attn_last_error: the message of the calling thread's most recent non-OK
 *   status ("" if there was none); thread-local storage owned by the
 *   library, valid until that thread's next call.
 */
const char *attn_status_string(attn_status status);
const char *attn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* EXATTN_H */
