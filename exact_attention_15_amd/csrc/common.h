// Internal declarations shared by the HIP translation units of libexattn.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "exattn.h" // include/ is on the include path

namespace exattn {

// Forward tiling: a workgroup owns BLOCK_M query rows (4 waves x 32 rows)
// and sweeps key tiles of BLOCK_N keys.
constexpr int BLOCK_M = 128;
constexpr int BLOCK_N = 64;

// Block-mask entry: (key tile index << 1) | partial-bit.
constexpr int32_t TILE_PARTIAL = 1;

// Device layout of a block mask (all int32, each section 256-byte aligned)
// for B batch rows of N query rows over Nk keys (Nk = N except for packed
// variable-length input).
struct MaskLayout {
    int B, N, Nk, nqt, nkt;
    size_t off_lo, off_hi, off_count, off_list, off_order, bytes;
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

inline MaskLayout mask_layout(int B, int N, int Nk = -1) {
    MaskLayout L;
    L.B = B;
    L.N = N;
    L.Nk = Nk < 0 ? N : Nk;
    L.nqt = (N + BLOCK_M - 1) / BLOCK_M;
    L.nkt = (L.Nk + BLOCK_N - 1) / BLOCK_N;
    size_t rows = size_t(B) * size_t(N);
    size_t items = size_t(B) * size_t(L.nqt);
    size_t off = 0;
    L.off_lo = off;    off = align256(off + 4 * rows);
    L.off_hi = off;    off = align256(off + 4 * rows);
    L.off_count = off; off = align256(off + 4 * items);
    L.off_list = off;  off = align256(off + 4 * items * size_t(L.nkt));
    L.off_order = off; off = align256(off + 4 * items); // [B][nqt]
    L.bytes = off;
    return L;
}

struct MaskView {
    const int32_t *lo, *hi, *count, *list, *order;
};

inline MaskView mask_view(const void *base, const MaskLayout &L) {
    const char *p = static_cast<const char *>(base);
    MaskView v;
    v.lo = reinterpret_cast<const int32_t *>(p + L.off_lo);
    v.hi = reinterpret_cast<const int32_t *>(p + L.off_hi);
    v.count = reinterpret_cast<const int32_t *>(p + L.off_count);
    v.list = reinterpret_cast<const int32_t *>(p + L.off_list);
    v.order = reinterpret_cast<const int32_t *>(p + L.off_order);
    return v;
}

// Packed variable-length sequences (one batch row): sequence s holds query
// rows [cu_q[s], cu_q[s+1]) and keys [cu_k[s], cu_k[s+1]).  Null cu_q means
// a regular [B, N] layout.
struct VarlenView {
    const int32_t *cu_q, *cu_k;
    int nseq;
};

// Launchers (each returns hipSuccess or the launch error).
hipError_t launch_mask_build(const attn_mask_spec &spec, const MaskLayout &L,
                             void *out, hipStream_t stream, VarlenView vl = VarlenView{nullptr, nullptr, 0});

struct FwdParams {
    const uint16_t *q, *k, *v;
    uint16_t *o;
    float *lse;
    int64_t q_sb, q_sh, q_sn;
    int64_t k_sb, k_sh, k_sn;
    int64_t v_sb, v_sh, v_sn;
    int64_t o_sb, o_sh, o_sn;
    int B, Hq, Hkv, N, nqt, nkt;
    int Nk;              // keys per batch row (N except for packed variable-length input)
    float scale_log2;    // scale * log2(e): scores in base-2 units
    float cap_inv_scale_2log2e; // 2 * log2(e) * scale / c (softcap mode only)
    float cap_log2;             // c * log2(e)     (softcap mode only)
    float cap_log2_2;           // 2 * c * log2(e) (softcap mode only)
    float cap_inv2;             // 2 / c           (softcap with ALiBi)
    // Polynomial form of the cap (softcap mode only): for |raw| <= cap_poly_lim
    // (|x| <= 0.15 with x = scale * raw / c), c tanh(x) * log2(e) =
    // raw * (cap_poly[0] + r2 (cap_poly[1] + r2 cap_poly[2])), r2 = raw^2:
    // tanh's Taylor series to x^5, whose remainder is below 17/315 x^7, a
    // relative 6.1e-7 at |x| = 0.15.
    float cap_poly_lim;
    float cap_poly[3];
    const float *alibi_slopes;  // [Hq], natural units (ALiBi mode only)
    MaskView mask;
};

hipError_t launch_fwd(const FwdParams &p, int d, bool softcap, bool alibi, hipStream_t stream);

// Backward tiling.  The dQ kernel uses the forward decomposition and block
// mask.  The dK/dV kernel gives a workgroup BWD_KB keys (4 waves x 32) and
// streams 64-row query tiles; its per-(b, key block) list of query tiles is
// the block mask transposed at that granularity: count [B][nkb], list
// [B][nkb][nqt64] of (query tile << 1) | partial-bit.
constexpr int BWD_KB = 128;
struct BwdMaskLayout {
    int nkb, nqt64;
    size_t off_count, off_list, bytes;
};
inline BwdMaskLayout bwd_mask_layout(int B, int N) {
    BwdMaskLayout L;
    L.nkb = (N + BWD_KB - 1) / BWD_KB;
    L.nqt64 = (N + BLOCK_N - 1) / BLOCK_N;
    size_t items = size_t(B) * size_t(L.nkb);
    size_t off = 0;
    L.off_count = off; off = align256(off + 4 * items);
    L.off_list = off;  off = align256(off + 4 * items * size_t(L.nqt64));
    L.bytes = off;
    return L;
}

struct BwdParams {
    const uint16_t *q, *k, *v, *o, *dout;
    const float *lse;                  // [B][Hq][N] natural log, from the forward
    float *lse2, *dvec;                // workspace [B][Hq][N]: base-2 LSE (+inf: no key), rowsum(dO * O)
    uint16_t *dq, *dk, *dv;
    int64_t q_sb, q_sh, q_sn, k_sb, k_sh, k_sn, v_sb, v_sh, v_sn;
    int64_t o_sb, o_sh, o_sn, do_sb, do_sh, do_sn;
    int64_t dq_sb, dq_sh, dq_sn, dk_sb, dk_sh, dk_sn, dv_sb, dv_sh, dv_sn;
    int B, Hq, Hkv, N, nqt, nkt, nkb, nqt64;
    float scale, scale_log2;
    float cap_inv_scale_2log2e, cap_log2, cap_log2_2, inv_cap_log2; // softcap mode only
    MaskView mask;                     // forward block mask (row intervals, dQ tile lists)
    const int32_t *kv_count, *kv_list; // transposed lists (dK/dV)
};

hipError_t launch_bwd(const BwdParams &p, int d, bool softcap, uint32_t flags, const MaskLayout &L,
                      const BwdMaskLayout &BL, void *kv_mask, hipStream_t stream);

// FP8 (E4M3) block quantization of a bf16 [B, H, N, d] tensor (d = 128):
// codes [B, H, N, d] bytes, scales fp32 [B][H][nblk] (powers of two, one per
// 64-row block; all equal within a head when per_head is set).
struct QuantParams {
    const uint16_t *x;
    int64_t x_sb, x_sh, x_sn;
    uint8_t *out;
    int64_t o_sb, o_sh, o_sn;
    float *scales;
    float *amax;         // workspace [B][H][nblk]
    const int8_t *signs; // [d] of +-1 for the rotation, or null
    int B, H, N, nblk, per_head;
    float inv_sqrt_d;
};
hipError_t launch_quant(const QuantParams &p, hipStream_t stream);

// FP8 forward (d = 128): q, k, v are E4M3 codes with per-64-row-block
// scales for q and k and one scale per (b, KV head) for v.
struct Fwd8Params {
    const uint8_t *q, *k, *v;
    uint16_t *o;
    float *lse;
    const float *q_scales, *k_scales, *v_scales; // [B][Hq][nblk64], [B][Hkv][nblk64] (v: per head, all equal)
    int64_t q_sb, q_sh, q_sn;
    int64_t k_sb, k_sh, k_sn;
    int64_t v_sb, v_sh, v_sn;
    int64_t o_sb, o_sh, o_sn;
    int B, Hq, Hkv, N, nqt, nkt, nblk64;
    float scale_log2;
    float cap_inv_scale_2log2e, cap_log2, cap_log2_2; // softcap mode only
    MaskView mask;
};
hipError_t launch_fwd8(const Fwd8Params &p, bool softcap, hipStream_t stream);

struct DecodeParams {
    const uint16_t *q, *k, *v;
    uint16_t *o;
    float *lse;
    const int32_t *lens;
    int64_t q_sb, q_sh;
    int64_t k_sb, k_sh, k_sn;
    int64_t v_sb, v_sh, v_sn;
    int64_t o_sb, o_sh;
    int B, Hq, Hkv, T, chunk, nchunk;
    float scale_log2;
    float *part_m, *part_l, *part_o; // workspace partials
};

hipError_t launch_decode(const DecodeParams &p, int d, hipStream_t stream);

// Workspace layout of attn_decode: m, l [B][Hq][nchunk], O [B][Hq][nchunk][d].
inline size_t decode_ws_bytes(int B, int Hq, int nchunk, int d, size_t *off_l,
                              size_t *off_o) {
    size_t n = size_t(B) * size_t(Hq) * size_t(nchunk);
    size_t off = align256(4 * n);
    if (off_l) *off_l = off;
    off = align256(off + 4 * n);
    if (off_o) *off_o = off;
    off = align256(off + 4 * n * size_t(d));
    return off;
}

} // namespace exattn
