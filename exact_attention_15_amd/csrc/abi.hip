// C ABI of libexattn: validation, buffer sizing and kernel launches.
// Every check runs before any launch; the library never allocates or
// synchronises.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "common.h"

using namespace exattn;

// ---- static scratch of attn_decode_noalloc ----
// The chunk partials (m, l, O) of attn_decode_noalloc live in this array
// instead of a caller workspace.  Each GPU holds its own copy, at its own
// address, from the library's load until the process ends.  In host code
// the name `scratch` denotes a host-side stand-in, not device memory: the
// device address is taken once per device with hipGetSymbolAddress (that
// device current) and only that address is ever passed to a kernel.  Every
// call on a GPU shares its copy; the combine reads only what the split of
// the same call wrote, so nothing has to start at zero, and calls that
// overlap on one GPU (different streams, or host threads) race.
static __device__ __align__(256) uint8_t scratch[ATTN_DECODE_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local char g_last_error[512] = "";

attn_status fail(attn_status s, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
attn_status fail(attn_status s, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return s;
}

attn_status hip_fail(hipError_t e, const char *what) {
    return fail(ATTN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

attn_status check_tensor(const attn_tensor &t, const char *name, bool need_n_stride) {
    if (!t.ptr) return fail(ATTN_ERR_INVALID, "%s: null pointer", name);
    if (!aligned16(t.ptr)) return fail(ATTN_ERR_INVALID, "%s: pointer not 16-byte aligned", name);
    if (t.stride_b < 0 || t.stride_h < 0 || t.stride_n < 0)
        return fail(ATTN_ERR_INVALID, "%s: negative stride", name);
    if (t.stride_b % 8 || t.stride_h % 8 || (need_n_stride && t.stride_n % 8))
        return fail(ATTN_ERR_INVALID, "%s: strides must be multiples of 8 elements", name);
    return ATTN_OK;
}

// Longest sequence the forward kernels index (keys and rows stay below 2^30
// so that the element mask's unsigned interval test cannot wrap); far beyond
// what fits in one GPU's memory.
const int MAX_TOKENS = 1 << 30;

const uint32_t KNOWN_FLAGS = ATTN_MASK_CAUSAL | ATTN_MASK_WINDOW | ATTN_MASK_DOCS | ATTN_MOD_SOFTCAP |
                             ATTN_MASK_NO_SKIP | ATTN_MOD_ALIBI;

attn_status check_spec(const attn_mask_spec *spec) {
    if (!spec) return ATTN_OK;
    if (spec->flags & ~KNOWN_FLAGS) return fail(ATTN_ERR_INVALID, "mask spec: unknown flag bits 0x%x", spec->flags);
    if (spec->flags & ATTN_MASK_DOCS) {
        if (!spec->doc_offsets) return fail(ATTN_ERR_INVALID, "mask spec: ATTN_MASK_DOCS needs doc_offsets");
        if (spec->doc_stride < 2) return fail(ATTN_ERR_INVALID, "mask spec: doc_stride must be >= 2");
    }
    if (spec->flags & ATTN_MOD_SOFTCAP) {
        if (!(spec->softcap > 0.f) || !std::isfinite(spec->softcap))
            return fail(ATTN_ERR_INVALID, "mask spec: softcap must be finite and > 0");
    }
    if ((spec->flags & ATTN_MOD_ALIBI) && !spec->alibi_slopes)
        return fail(ATTN_ERR_INVALID, "mask spec: ATTN_MOD_ALIBI needs alibi_slopes");
    return ATTN_OK;
}

// Scale and soft-cap constants of the score path, in base-2 units.
void set_score_params(FwdParams &p, const attn_mask_spec &sp, float scale) {
    const float log2e = 1.4426950408889634f;
    p.scale_log2 = scale * log2e;
    const bool softcap = sp.flags & ATTN_MOD_SOFTCAP;
    p.cap_inv_scale_2log2e = softcap ? 2.f * log2e * (scale / sp.softcap) : 0.f;
    p.cap_log2 = softcap ? sp.softcap * log2e : 0.f;
    p.cap_log2_2 = 2.f * p.cap_log2;
    p.cap_inv2 = softcap ? 2.f / sp.softcap : 0.f;
    // tanh(x) = x - x^3/3 + 2x^5/15 - ..., x = scale * raw / c: coefficients
    // of raw * poly(raw^2), times c * log2(e) * (scale / c)
    {
        const double sc = softcap ? double(scale) / double(sp.softcap) : 0.0, k = sc * sc;
        const double l2 = 1.4426950408889634 * double(scale);
        p.cap_poly_lim = softcap ? float(0.15 / sc) : 0.f;
        p.cap_poly[0] = float(l2);
        p.cap_poly[1] = float(l2 * (-1.0 / 3.0) * k);
        p.cap_poly[2] = float(l2 * (2.0 / 15.0) * k * k);
    }
    p.alibi_slopes = (sp.flags & ATTN_MOD_ALIBI) ? sp.alibi_slopes : nullptr;
}

attn_mask_spec spec_or_default(const attn_mask_spec *spec) {
    attn_mask_spec s;
    std::memset(&s, 0, sizeof s);
    if (spec) s = *spec;
    return s;
}

// ---- decode: validation and launch shared by attn_decode and
// attn_decode_noalloc ----
attn_status decode_setup(const char *fn, attn_tensor q, attn_tensor k_cache, attn_tensor v_cache,
                         const int32_t *lens, attn_tensor o, float *lse, int B, int Hq, int Hkv, int T, int d,
                         int chunk, float scale, DecodeParams &p, size_t &need, size_t &off_l, size_t &off_o,
                         bool &noop) {
    noop = false;
    if (B < 0 || T < 0) return fail(ATTN_ERR_INVALID, "%s: B=%d T=%d", fn, B, T);
    if (Hq <= 0 || Hkv <= 0) return fail(ATTN_ERR_INVALID, "%s: Hq=%d Hkv=%d", fn, Hq, Hkv);
    if (Hq % Hkv) return fail(ATTN_ERR_INVALID, "%s: Hq=%d is not a multiple of Hkv=%d", fn, Hq, Hkv);
    if (Hq / Hkv > 16) return fail(ATTN_ERR_UNSUPPORTED, "%s: group size %d > 16", fn, Hq / Hkv);
    if (d != 64 && d != 128) return fail(ATTN_ERR_UNSUPPORTED, "%s: head dim %d (supported: 64, 128)", fn, d);
    if (chunk < 64 || chunk > 2048 || chunk % 64)
        return fail(ATTN_ERR_UNSUPPORTED, "%s: chunk %d (multiple of 64 in [64, 2048])", fn, chunk);
    if (!std::isfinite(scale) || !(scale > 0.f)) return fail(ATTN_ERR_INVALID, "%s: scale must be finite and > 0", fn);
    if (B == 0) {
        noop = true;
        return ATTN_OK;
    }
    attn_status st;
    if ((st = check_tensor(q, "q", false)) != ATTN_OK) return st;
    if ((st = check_tensor(k_cache, "k_cache", true)) != ATTN_OK) return st;
    if ((st = check_tensor(v_cache, "v_cache", true)) != ATTN_OK) return st;
    if ((st = check_tensor(o, "o", false)) != ATTN_OK) return st;
    if (k_cache.stride_n >= (int64_t(1) << 20) || v_cache.stride_n >= (int64_t(1) << 20))
        return fail(ATTN_ERR_UNSUPPORTED, "%s: k/v cache token stride must be below 2^20 elements", fn);
    if (!lens) return fail(ATTN_ERR_INVALID, "%s: null lens", fn);
    if (!lse) return fail(ATTN_ERR_INVALID, "%s: null lse", fn);
    const int nchunk = T > 0 ? (T + chunk - 1) / chunk : 1;
    need = decode_ws_bytes(B, Hq, nchunk, d, &off_l, &off_o);
    p.q = static_cast<const uint16_t *>(q.ptr);
    p.k = static_cast<const uint16_t *>(k_cache.ptr);
    p.v = static_cast<const uint16_t *>(v_cache.ptr);
    p.o = static_cast<uint16_t *>(o.ptr);
    p.lse = lse;
    p.lens = lens;
    p.q_sb = q.stride_b; p.q_sh = q.stride_h;
    p.k_sb = k_cache.stride_b; p.k_sh = k_cache.stride_h; p.k_sn = k_cache.stride_n;
    p.v_sb = v_cache.stride_b; p.v_sh = v_cache.stride_h; p.v_sn = v_cache.stride_n;
    p.o_sb = o.stride_b; p.o_sh = o.stride_h;
    p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.T = T; p.chunk = chunk; p.nchunk = nchunk;
    p.scale_log2 = scale * 1.4426950408889634f;
    return ATTN_OK;
}

attn_status decode_launch(const char *fn, DecodeParams &p, char *ws, size_t off_l, size_t off_o, int d,
                          void *stream) {
    p.part_m = reinterpret_cast<float *>(ws);
    p.part_l = reinterpret_cast<float *>(ws + off_l);
    p.part_o = reinterpret_cast<float *>(ws + off_o);
    hipError_t e = launch_decode(p, d, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, fn);
    return ATTN_OK;
}

constexpr int MAX_SCRATCH_DEVICES = 64;
std::mutex g_scratch_mu;
char *g_scratch_dev[MAX_SCRATCH_DEVICES] = {};

// Device address of this library's scratch on the GPU that `stream` runs on
// (the current device for the null stream).
attn_status noalloc_scratch(void *stream, char **out) {
    int dev = -1;
    hipError_t e = stream ? hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "attn_decode_noalloc: device of the stream");
    if (dev < 0 || dev >= MAX_SCRATCH_DEVICES)
        return fail(ATTN_ERR_UNSUPPORTED, "attn_decode_noalloc: device %d (at most %d devices)", dev,
                    MAX_SCRATCH_DEVICES);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        int cur = -1;
        if ((e = hipGetDevice(&cur)) != hipSuccess) return hip_fail(e, "attn_decode_noalloc: hipGetDevice");
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess)
            return hip_fail(e, "attn_decode_noalloc: hipSetDevice");
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (cur != dev) {
            hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess && e2 != hipSuccess) e = e2;
        }
        if (e != hipSuccess) return hip_fail(e, "attn_decode_noalloc: hipGetSymbolAddress of the scratch");
        if (!ptr || !aligned16(ptr)) return fail(ATTN_ERR_HIP, "attn_decode_noalloc: bad scratch address");
        g_scratch_dev[dev] = static_cast<char *>(ptr);
    }
    *out = g_scratch_dev[dev];
    return ATTN_OK;
}

} // namespace

extern "C" {


const char *attn_status_string(attn_status s) {
    switch (s) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_INVALID: return "invalid argument";
    case ATTN_ERR_UNSUPPORTED: return "unsupported configuration";
    case ATTN_ERR_WORKSPACE: return "workspace too small";
    case ATTN_ERR_HIP: return "HIP launch failure";
    }
    return "unknown status";
}

const char *attn_last_error(void) { return g_last_error; }

size_t attn_mask_bytes(const attn_mask_spec *spec, int B, int N) {
    (void)spec;
    if (B <= 0 || N <= 0) return 0;
    return mask_layout(B, N).bytes;
}

attn_status attn_mask_build(const attn_mask_spec *spec, int B, int N, void *out, size_t bytes,
                            void *stream) {
    if (B < 0 || N < 0) return fail(ATTN_ERR_INVALID, "attn_mask_build: B=%d N=%d", B, N);
    if (N >= MAX_TOKENS) return fail(ATTN_ERR_UNSUPPORTED, "attn_mask_build: N=%d (supported: below 2^30)", N);
    attn_status st = check_spec(spec);
    if (st != ATTN_OK) return st;
    if (int64_t(B) * N == 0) return ATTN_OK;
    if (!out) return fail(ATTN_ERR_INVALID, "attn_mask_build: null output buffer");
    if (!aligned16(out)) return fail(ATTN_ERR_INVALID, "attn_mask_build: buffer not 16-byte aligned");
    const MaskLayout L = mask_layout(B, N);
    if (bytes < L.bytes)
        return fail(ATTN_ERR_WORKSPACE, "attn_mask_build: need %zu bytes, got %zu", L.bytes, bytes);
    hipError_t e = launch_mask_build(spec_or_default(spec), L, out, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "attn_mask_build");
    return ATTN_OK;
}

size_t attn_fwd_workspace_size(const attn_mask_spec *spec, int B, int N) {
    return attn_mask_bytes(spec, B, N);
}

attn_status attn_fwd(attn_tensor q, attn_tensor k, attn_tensor v, attn_tensor o, float *lse, int B,
                     int Hq, int Hkv, int N, int d, const attn_mask_spec *spec, float scale,
                     const void *block_mask, void *workspace, size_t ws_bytes, void *stream) {
    if (B < 0 || N < 0) return fail(ATTN_ERR_INVALID, "attn_fwd: B=%d N=%d", B, N);
    if (N >= MAX_TOKENS) return fail(ATTN_ERR_UNSUPPORTED, "attn_fwd: N=%d (supported: below 2^30)", N);
    if (Hq <= 0 || Hkv <= 0) return fail(ATTN_ERR_INVALID, "attn_fwd: Hq=%d Hkv=%d", Hq, Hkv);
    if (Hq % Hkv) return fail(ATTN_ERR_INVALID, "attn_fwd: Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
    if (d != 64 && d != 128) return fail(ATTN_ERR_UNSUPPORTED, "attn_fwd: head dim %d (supported: 64, 128)", d);
    if (!std::isfinite(scale) || !(scale > 0.f)) return fail(ATTN_ERR_INVALID, "attn_fwd: scale must be finite and > 0");
    attn_status st = check_spec(spec);
    if (st != ATTN_OK) return st;
    if (int64_t(B) * N == 0) return ATTN_OK;
    if ((st = check_tensor(q, "q", true)) != ATTN_OK) return st;
    if ((st = check_tensor(k, "k", true)) != ATTN_OK) return st;
    if ((st = check_tensor(v, "v", true)) != ATTN_OK) return st;
    if ((st = check_tensor(o, "o", true)) != ATTN_OK) return st;
    if (!lse) return fail(ATTN_ERR_INVALID, "attn_fwd: null lse");
    if (k.stride_n >= (int64_t(1) << 24) || v.stride_n >= (int64_t(1) << 24))
        return fail(ATTN_ERR_UNSUPPORTED, "attn_fwd: k/v token stride must be below 2^24 elements");
    const MaskLayout L = mask_layout(B, N);
    if (int64_t(B) * L.nqt * Hq > 0x7FFFFFFFLL) return fail(ATTN_ERR_UNSUPPORTED, "attn_fwd: grid too large");
    const attn_mask_spec sp = spec_or_default(spec);
    const void *mask = block_mask;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (!mask) {
        if (!workspace || ws_bytes < L.bytes)
            return fail(ATTN_ERR_WORKSPACE, "attn_fwd: workspace needs %zu bytes, got %zu", L.bytes,
                        workspace ? ws_bytes : size_t(0));
        if (!aligned16(workspace)) return fail(ATTN_ERR_INVALID, "attn_fwd: workspace not 16-byte aligned");
        hipError_t e = launch_mask_build(sp, L, workspace, s);
        if (e != hipSuccess) return hip_fail(e, "attn_fwd (mask build)");
        mask = workspace;
    }
    FwdParams p;
    p.q = static_cast<const uint16_t *>(q.ptr);
    p.k = static_cast<const uint16_t *>(k.ptr);
    p.v = static_cast<const uint16_t *>(v.ptr);
    p.o = static_cast<uint16_t *>(o.ptr);
    p.lse = lse;
    p.q_sb = q.stride_b; p.q_sh = q.stride_h; p.q_sn = q.stride_n;
    p.k_sb = k.stride_b; p.k_sh = k.stride_h; p.k_sn = k.stride_n;
    p.v_sb = v.stride_b; p.v_sh = v.stride_h; p.v_sn = v.stride_n;
    p.o_sb = o.stride_b; p.o_sh = o.stride_h; p.o_sn = o.stride_n;
    p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.N = N; p.Nk = N; p.nqt = L.nqt; p.nkt = L.nkt;
    set_score_params(p, sp, scale);
    p.mask = mask_view(mask, L);
    hipError_t e = launch_fwd(p, d, sp.flags & ATTN_MOD_SOFTCAP, sp.flags & ATTN_MOD_ALIBI, s);
    if (e != hipSuccess) return hip_fail(e, "attn_fwd");
    return ATTN_OK;
}

size_t attn_fwd_varlen_workspace_size(int total_q, int total_k) {
    if (total_q <= 0 || total_k < 0) return 0;
    return mask_layout(1, total_q, total_k).bytes;
}

attn_status attn_fwd_varlen(attn_tensor q, attn_tensor k, attn_tensor v, attn_tensor o, float *lse,
                            const int32_t *cu_seqlens_q, const int32_t *cu_seqlens_k, int nseq, int total_q,
                            int total_k, int Hq, int Hkv, int d, const attn_mask_spec *spec, float scale,
                            void *workspace, size_t ws_bytes, void *stream) {
    if (nseq < 0 || total_q < 0 || total_k < 0)
        return fail(ATTN_ERR_INVALID, "attn_fwd_varlen: nseq=%d total_q=%d total_k=%d", nseq, total_q, total_k);
    if (total_q >= MAX_TOKENS || total_k >= MAX_TOKENS)
        return fail(ATTN_ERR_UNSUPPORTED, "attn_fwd_varlen: total_q=%d total_k=%d (supported: below 2^30)", total_q,
                    total_k);
    if (Hq <= 0 || Hkv <= 0) return fail(ATTN_ERR_INVALID, "attn_fwd_varlen: Hq=%d Hkv=%d", Hq, Hkv);
    if (Hq % Hkv) return fail(ATTN_ERR_INVALID, "attn_fwd_varlen: Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
    if (d != 64 && d != 128)
        return fail(ATTN_ERR_UNSUPPORTED, "attn_fwd_varlen: head dim %d (supported: 64, 128)", d);
    if (!std::isfinite(scale) || !(scale > 0.f))
        return fail(ATTN_ERR_INVALID, "attn_fwd_varlen: scale must be finite and > 0");
    attn_status st = check_spec(spec);
    if (st != ATTN_OK) return st;
    if (spec && (spec->flags & ATTN_MASK_DOCS))
        return fail(ATTN_ERR_INVALID, "attn_fwd_varlen: ATTN_MASK_DOCS does not apply (sequences come from cu_seqlens)");
    if (spec && (spec->flags & ATTN_MOD_ALIBI))
        return fail(ATTN_ERR_UNSUPPORTED, "attn_fwd_varlen: ATTN_MOD_ALIBI is supported by attn_fwd only");
    if (total_q == 0) return ATTN_OK;
    if (nseq == 0) return fail(ATTN_ERR_INVALID, "attn_fwd_varlen: total_q=%d rows but no sequence", total_q);
    if (!cu_seqlens_q || !cu_seqlens_k) return fail(ATTN_ERR_INVALID, "attn_fwd_varlen: null cu_seqlens");
    if ((st = check_tensor(q, "q", true)) != ATTN_OK) return st;
    if ((st = check_tensor(o, "o", true)) != ATTN_OK) return st;
    if (total_k > 0) {
        if ((st = check_tensor(k, "k", true)) != ATTN_OK) return st;
        if ((st = check_tensor(v, "v", true)) != ATTN_OK) return st;
    }
    if (!lse) return fail(ATTN_ERR_INVALID, "attn_fwd_varlen: null lse");
    if (k.stride_n >= (int64_t(1) << 24) || v.stride_n >= (int64_t(1) << 24))
        return fail(ATTN_ERR_UNSUPPORTED, "attn_fwd_varlen: k/v token stride must be below 2^24 elements");
    const MaskLayout L = mask_layout(1, total_q, total_k);
    if (int64_t(L.nqt) * Hq > 0x7FFFFFFFLL) return fail(ATTN_ERR_UNSUPPORTED, "attn_fwd_varlen: grid too large");
    if (!workspace || ws_bytes < L.bytes)
        return fail(ATTN_ERR_WORKSPACE, "attn_fwd_varlen: workspace needs %zu bytes, got %zu", L.bytes,
                    workspace ? ws_bytes : size_t(0));
    if (!aligned16(workspace)) return fail(ATTN_ERR_INVALID, "attn_fwd_varlen: workspace not 16-byte aligned");
    const attn_mask_spec sp = spec_or_default(spec);
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = launch_mask_build(sp, L, workspace, s, VarlenView{cu_seqlens_q, cu_seqlens_k, nseq});
    if (e != hipSuccess) return hip_fail(e, "attn_fwd_varlen (mask build)");
    // With no keys at all every row is empty and no key tile is listed; the
    // kernel then never reads k or v.
    FwdParams p;
    p.q = static_cast<const uint16_t *>(q.ptr);
    p.k = static_cast<const uint16_t *>(total_k > 0 ? k.ptr : q.ptr);
    p.v = static_cast<const uint16_t *>(total_k > 0 ? v.ptr : q.ptr);
    p.o = static_cast<uint16_t *>(o.ptr);
    p.lse = lse;
    p.q_sb = 0; p.q_sh = q.stride_h; p.q_sn = q.stride_n;
    p.k_sb = 0; p.k_sh = k.stride_h; p.k_sn = k.stride_n;
    p.v_sb = 0; p.v_sh = v.stride_h; p.v_sn = v.stride_n;
    p.o_sb = 0; p.o_sh = o.stride_h; p.o_sn = o.stride_n;
    p.B = 1; p.Hq = Hq; p.Hkv = Hkv; p.N = total_q; p.Nk = total_k; p.nqt = L.nqt; p.nkt = L.nkt;
    set_score_params(p, sp, scale);
    p.mask = mask_view(workspace, L);
    e = launch_fwd(p, d, sp.flags & ATTN_MOD_SOFTCAP, false, s);
    if (e != hipSuccess) return hip_fail(e, "attn_fwd_varlen");
    return ATTN_OK;
}

size_t attn_bwd_workspace_size(const attn_mask_spec *spec, int B, int Hq, int N) {
    (void)spec;
    if (B <= 0 || Hq <= 0 || N <= 0) return 0;
    const size_t rows = size_t(B) * size_t(Hq) * size_t(N);
    return mask_layout(B, N).bytes + bwd_mask_layout(B, N).bytes + 2 * align256(4 * rows);
}

attn_status attn_bwd(attn_tensor q, attn_tensor k, attn_tensor v, attn_tensor o, const float *lse,
                     attn_tensor dout, attn_tensor dq, attn_tensor dk, attn_tensor dv, int B, int Hq, int Hkv,
                     int N, int d, const attn_mask_spec *spec, float scale, void *workspace, size_t ws_bytes,
                     void *stream) {
    if (B < 0 || N < 0) return fail(ATTN_ERR_INVALID, "attn_bwd: B=%d N=%d", B, N);
    if (N >= MAX_TOKENS) return fail(ATTN_ERR_UNSUPPORTED, "attn_bwd: N=%d (supported: below 2^30)", N);
    if (Hq <= 0 || Hkv <= 0) return fail(ATTN_ERR_INVALID, "attn_bwd: Hq=%d Hkv=%d", Hq, Hkv);
    if (Hq % Hkv) return fail(ATTN_ERR_INVALID, "attn_bwd: Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
    if (d != 64 && d != 128) return fail(ATTN_ERR_UNSUPPORTED, "attn_bwd: head dim %d (supported: 64, 128)", d);
    if (!std::isfinite(scale) || !(scale > 0.f)) return fail(ATTN_ERR_INVALID, "attn_bwd: scale must be finite and > 0");
    attn_status st = check_spec(spec);
    if (st != ATTN_OK) return st;
    if (spec && (spec->flags & ATTN_MOD_ALIBI))
        return fail(ATTN_ERR_UNSUPPORTED, "attn_bwd: ATTN_MOD_ALIBI is supported by attn_fwd only");
    if (int64_t(B) * N == 0) return ATTN_OK;
    const attn_tensor *ts[] = {&q, &k, &v, &o, &dout, &dq, &dk, &dv};
    const char *names[] = {"q", "k", "v", "o", "dout", "dq", "dk", "dv"};
    for (int i = 0; i < 8; ++i)
        if ((st = check_tensor(*ts[i], names[i], true)) != ATTN_OK) return st;
    if (!lse) return fail(ATTN_ERR_INVALID, "attn_bwd: null lse");
    for (int i = 0; i < 5; ++i)
        if (ts[i]->stride_n >= (int64_t(1) << 24))
            return fail(ATTN_ERR_UNSUPPORTED, "attn_bwd: %s token stride must be below 2^24 elements", names[i]);
    const MaskLayout L = mask_layout(B, N);
    const BwdMaskLayout BL = bwd_mask_layout(B, N);
    if (int64_t(B) * L.nqt * Hq > 0x7FFFFFFFLL || int64_t(B) * BL.nkb * Hkv > 0x7FFFFFFFLL)
        return fail(ATTN_ERR_UNSUPPORTED, "attn_bwd: grid too large");
    const size_t rows = size_t(B) * size_t(Hq) * size_t(N);
    const size_t need = attn_bwd_workspace_size(spec, B, Hq, N);
    if (!workspace || ws_bytes < need)
        return fail(ATTN_ERR_WORKSPACE, "attn_bwd: workspace needs %zu bytes, got %zu", need,
                    workspace ? ws_bytes : size_t(0));
    if (!aligned16(workspace)) return fail(ATTN_ERR_INVALID, "attn_bwd: workspace not 16-byte aligned");
    const attn_mask_spec sp = spec_or_default(spec);
    hipStream_t s = static_cast<hipStream_t>(stream);
    char *ws = static_cast<char *>(workspace);
    char *kv_mask = ws + L.bytes;
    float *lse2 = reinterpret_cast<float *>(kv_mask + BL.bytes);
    float *dvec = reinterpret_cast<float *>(kv_mask + BL.bytes + align256(4 * rows));
    hipError_t e = launch_mask_build(sp, L, ws, s);
    if (e != hipSuccess) return hip_fail(e, "attn_bwd (mask build)");
    BwdParams p;
    p.q = static_cast<const uint16_t *>(q.ptr);
    p.k = static_cast<const uint16_t *>(k.ptr);
    p.v = static_cast<const uint16_t *>(v.ptr);
    p.o = static_cast<const uint16_t *>(o.ptr);
    p.dout = static_cast<const uint16_t *>(dout.ptr);
    p.lse = lse;
    p.lse2 = lse2;
    p.dvec = dvec;
    p.dq = static_cast<uint16_t *>(dq.ptr);
    p.dk = static_cast<uint16_t *>(dk.ptr);
    p.dv = static_cast<uint16_t *>(dv.ptr);
    p.q_sb = q.stride_b; p.q_sh = q.stride_h; p.q_sn = q.stride_n;
    p.k_sb = k.stride_b; p.k_sh = k.stride_h; p.k_sn = k.stride_n;
    p.v_sb = v.stride_b; p.v_sh = v.stride_h; p.v_sn = v.stride_n;
    p.o_sb = o.stride_b; p.o_sh = o.stride_h; p.o_sn = o.stride_n;
    p.do_sb = dout.stride_b; p.do_sh = dout.stride_h; p.do_sn = dout.stride_n;
    p.dq_sb = dq.stride_b; p.dq_sh = dq.stride_h; p.dq_sn = dq.stride_n;
    p.dk_sb = dk.stride_b; p.dk_sh = dk.stride_h; p.dk_sn = dk.stride_n;
    p.dv_sb = dv.stride_b; p.dv_sh = dv.stride_h; p.dv_sn = dv.stride_n;
    p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.N = N; p.nqt = L.nqt; p.nkt = L.nkt; p.nkb = BL.nkb; p.nqt64 = BL.nqt64;
    const float log2e = 1.4426950408889634f;
    p.scale = scale;
    p.scale_log2 = scale * log2e;
    const bool softcap = sp.flags & ATTN_MOD_SOFTCAP;
    p.cap_inv_scale_2log2e = softcap ? 2.f * log2e * (scale / sp.softcap) : 0.f;
    p.cap_log2 = softcap ? sp.softcap * log2e : 0.f;
    p.cap_log2_2 = 2.f * p.cap_log2;
    p.inv_cap_log2 = softcap ? 1.f / p.cap_log2 : 0.f;
    p.mask = mask_view(ws, L);
    p.kv_count = reinterpret_cast<const int32_t *>(kv_mask + BL.off_count);
    p.kv_list = reinterpret_cast<const int32_t *>(kv_mask + BL.off_list);
    e = launch_bwd(p, d, softcap, sp.flags, L, BL, kv_mask, s);
    if (e != hipSuccess) return hip_fail(e, "attn_bwd");
    return ATTN_OK;
}

size_t attn_quantize_fp8_workspace_size(int B, int H, int N) {
    if (B <= 0 || H <= 0 || N <= 0) return 0;
    return align256(4 * size_t(B) * size_t(H) * size_t((N + 63) / 64));
}

attn_status attn_quantize_fp8(attn_tensor x, attn_tensor out, float *scales, int B, int H, int N, int d,
                              const int8_t *signs, int per_head, void *workspace, size_t ws_bytes, void *stream) {
    if (B < 0 || H <= 0 || N < 0) return fail(ATTN_ERR_INVALID, "attn_quantize_fp8: B=%d H=%d N=%d", B, H, N);
    if (d != 128) return fail(ATTN_ERR_UNSUPPORTED, "attn_quantize_fp8: head dim %d (supported: 128)", d);
    if (int64_t(B) * N == 0) return ATTN_OK;
    attn_status st;
    if ((st = check_tensor(x, "x", true)) != ATTN_OK) return st;
    if (!out.ptr || !aligned16(out.ptr)) return fail(ATTN_ERR_INVALID, "attn_quantize_fp8: out null or not 16-byte aligned");
    if (out.stride_b < 0 || out.stride_h < 0 || out.stride_n < 0 || out.stride_b % 16 || out.stride_h % 16 ||
        out.stride_n % 16)
        return fail(ATTN_ERR_INVALID, "attn_quantize_fp8: out strides must be non-negative multiples of 16 bytes");
    if (!scales) return fail(ATTN_ERR_INVALID, "attn_quantize_fp8: null scales");
    const size_t need = attn_quantize_fp8_workspace_size(B, H, N);
    if (!workspace || ws_bytes < need)
        return fail(ATTN_ERR_WORKSPACE, "attn_quantize_fp8: workspace needs %zu bytes, got %zu", need,
                    workspace ? ws_bytes : size_t(0));
    if (int64_t(B) > 65535 || int64_t(H) > 65535)
        return fail(ATTN_ERR_UNSUPPORTED, "attn_quantize_fp8: B and H must be below 65536");
    QuantParams p;
    p.x = static_cast<const uint16_t *>(x.ptr);
    p.x_sb = x.stride_b; p.x_sh = x.stride_h; p.x_sn = x.stride_n;
    p.out = static_cast<uint8_t *>(out.ptr);
    p.o_sb = out.stride_b; p.o_sh = out.stride_h; p.o_sn = out.stride_n;
    p.scales = scales;
    p.amax = static_cast<float *>(workspace);
    p.signs = signs;
    p.B = B; p.H = H; p.N = N; p.nblk = (N + 63) / 64; p.per_head = per_head ? 1 : 0;
    p.inv_sqrt_d = float(1.0 / std::sqrt(double(d)));
    hipError_t e = launch_quant(p, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "attn_quantize_fp8");
    return ATTN_OK;
}

attn_status attn_fwd_fp8(attn_tensor q, attn_tensor k, attn_tensor v, const float *q_scales,
                         const float *k_scales, const float *v_scales, attn_tensor o, float *lse, int B, int Hq,
                         int Hkv, int N, int d, const attn_mask_spec *spec, float scale, const void *block_mask,
                         void *workspace, size_t ws_bytes, void *stream) {
    if (B < 0 || N < 0) return fail(ATTN_ERR_INVALID, "attn_fwd_fp8: B=%d N=%d", B, N);
    if (N >= MAX_TOKENS) return fail(ATTN_ERR_UNSUPPORTED, "attn_fwd_fp8: N=%d (supported: below 2^30)", N);
    if (Hq <= 0 || Hkv <= 0) return fail(ATTN_ERR_INVALID, "attn_fwd_fp8: Hq=%d Hkv=%d", Hq, Hkv);
    if (Hq % Hkv) return fail(ATTN_ERR_INVALID, "attn_fwd_fp8: Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
    if (d != 128) return fail(ATTN_ERR_UNSUPPORTED, "attn_fwd_fp8: head dim %d (supported: 128)", d);
    if (!std::isfinite(scale) || !(scale > 0.f)) return fail(ATTN_ERR_INVALID, "attn_fwd_fp8: scale must be finite and > 0");
    attn_status st = check_spec(spec);
    if (st != ATTN_OK) return st;
    if (spec && (spec->flags & ATTN_MOD_ALIBI))
        return fail(ATTN_ERR_UNSUPPORTED, "attn_fwd_fp8: ATTN_MOD_ALIBI is supported by attn_fwd only");
    if (int64_t(B) * N == 0) return ATTN_OK;
    const attn_tensor *ts[] = {&q, &k, &v};
    const char *names[] = {"q", "k", "v"};
    for (int i = 0; i < 3; ++i) {
        const attn_tensor &t = *ts[i];
        if (!t.ptr || !aligned16(t.ptr)) return fail(ATTN_ERR_INVALID, "attn_fwd_fp8: %s null or not 16-byte aligned", names[i]);
        if (t.stride_b < 0 || t.stride_h < 0 || t.stride_n < 0 || t.stride_b % 16 || t.stride_h % 16 ||
            t.stride_n % 16)
            return fail(ATTN_ERR_INVALID, "attn_fwd_fp8: %s strides must be non-negative multiples of 16 bytes", names[i]);
        if (t.stride_n >= (int64_t(1) << 24))
            return fail(ATTN_ERR_UNSUPPORTED, "attn_fwd_fp8: %s token stride must be below 2^24 bytes", names[i]);
    }
    if ((st = check_tensor(o, "o", true)) != ATTN_OK) return st;
    if (!lse || !q_scales || !k_scales || !v_scales) return fail(ATTN_ERR_INVALID, "attn_fwd_fp8: null lse or scales");
    const MaskLayout L = mask_layout(B, N);
    if (int64_t(B) * L.nqt * Hq > 0x7FFFFFFFLL) return fail(ATTN_ERR_UNSUPPORTED, "attn_fwd_fp8: grid too large");
    const attn_mask_spec sp = spec_or_default(spec);
    const void *mask = block_mask;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (!mask) {
        if (!workspace || ws_bytes < L.bytes)
            return fail(ATTN_ERR_WORKSPACE, "attn_fwd_fp8: workspace needs %zu bytes, got %zu", L.bytes,
                        workspace ? ws_bytes : size_t(0));
        if (!aligned16(workspace)) return fail(ATTN_ERR_INVALID, "attn_fwd_fp8: workspace not 16-byte aligned");
        hipError_t e = launch_mask_build(sp, L, workspace, s);
        if (e != hipSuccess) return hip_fail(e, "attn_fwd_fp8 (mask build)");
        mask = workspace;
    }
    Fwd8Params p;
    p.q = static_cast<const uint8_t *>(q.ptr);
    p.k = static_cast<const uint8_t *>(k.ptr);
    p.v = static_cast<const uint8_t *>(v.ptr);
    p.o = static_cast<uint16_t *>(o.ptr);
    p.lse = lse;
    p.q_scales = q_scales; p.k_scales = k_scales; p.v_scales = v_scales;
    p.q_sb = q.stride_b; p.q_sh = q.stride_h; p.q_sn = q.stride_n;
    p.k_sb = k.stride_b; p.k_sh = k.stride_h; p.k_sn = k.stride_n;
    p.v_sb = v.stride_b; p.v_sh = v.stride_h; p.v_sn = v.stride_n;
    p.o_sb = o.stride_b; p.o_sh = o.stride_h; p.o_sn = o.stride_n;
    p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.N = N; p.nqt = L.nqt; p.nkt = L.nkt; p.nblk64 = (N + 63) / 64;
    const float log2e = 1.4426950408889634f;
    p.scale_log2 = scale * log2e;
    const bool softcap = sp.flags & ATTN_MOD_SOFTCAP;
    p.cap_inv_scale_2log2e = softcap ? 2.f * log2e * (scale / sp.softcap) : 0.f;
    p.cap_log2 = softcap ? sp.softcap * log2e : 0.f;
    p.cap_log2_2 = 2.f * p.cap_log2;
    p.mask = mask_view(mask, L);
    hipError_t e = launch_fwd8(p, softcap, s);
    if (e != hipSuccess) return hip_fail(e, "attn_fwd_fp8");
    return ATTN_OK;
}

size_t attn_decode_workspace_size(int B, int Hq, int T, int d, int chunk) {
    if (B <= 0 || Hq <= 0 || T < 0 || d <= 0 || chunk <= 0) return 0;
    const int nchunk = T > 0 ? (T + chunk - 1) / chunk : 1;
    return decode_ws_bytes(B, Hq, nchunk, d, nullptr, nullptr);
}

attn_status attn_decode(attn_tensor q, attn_tensor k_cache, attn_tensor v_cache, const int32_t *lens,
                        attn_tensor o, float *lse, int B, int Hq, int Hkv, int T, int d, int chunk,
                        float scale, void *workspace, size_t ws_bytes, void *stream) {
    DecodeParams p;
    size_t need = 0, off_l = 0, off_o = 0;
    bool noop = false;
    attn_status st = decode_setup("attn_decode", q, k_cache, v_cache, lens, o, lse, B, Hq, Hkv, T, d, chunk,
                                  scale, p, need, off_l, off_o, noop);
    if (st != ATTN_OK || noop) return st;
    if (!workspace || ws_bytes < need)
        return fail(ATTN_ERR_WORKSPACE, "attn_decode: workspace needs %zu bytes, got %zu", need,
                    workspace ? ws_bytes : size_t(0));
    if (!aligned16(workspace)) return fail(ATTN_ERR_INVALID, "attn_decode: workspace not 16-byte aligned");
    return decode_launch("attn_decode", p, static_cast<char *>(workspace), off_l, off_o, d, stream);
}

attn_status attn_decode_noalloc(attn_tensor q, attn_tensor k_cache, attn_tensor v_cache, const int32_t *lens,
                                attn_tensor o, float *lse, int B, int Hq, int Hkv, int T, int d, int chunk,
                                float scale, void *stream) {
    DecodeParams p;
    size_t need = 0, off_l = 0, off_o = 0;
    bool noop = false;
    attn_status st = decode_setup("attn_decode_noalloc", q, k_cache, v_cache, lens, o, lse, B, Hq, Hkv, T, d,
                                  chunk, scale, p, need, off_l, off_o, noop);
    if (st != ATTN_OK || noop) return st;
    if (need > ATTN_DECODE_NOALLOC_SCRATCH_BYTES)
        return fail(ATTN_ERR_WORKSPACE,
                    "attn_decode_noalloc: the chunk partials need %zu bytes, more than the %zu-byte static "
                    "scratch (B * Hq * ceil(T / chunk) * (d + 2) * 4 bytes plus alignment); use attn_decode "
                    "with a workspace",
                    need, size_t(ATTN_DECODE_NOALLOC_SCRATCH_BYTES));
    char *ws = nullptr;
    if ((st = noalloc_scratch(stream, &ws)) != ATTN_OK) return st;
    return decode_launch("attn_decode_noalloc", p, ws, off_l, off_o, d, stream);
}

} // extern "C"
