// FP8 (E4M3) forward pass for gfx950, d = 128: the FlashAttention-3 FP8
// variant (youngju.dev "FlashAttention 논문 분석", FlashAttention-3 sections
// "FP8 텐서 코어" and "FP8 지원과 정확도 유지") re-derived for CDNA4's
// v_mfma_f32_32x32x64_f8f6f4.
//
// Same decomposition, block mask, online softmax and transposed
// formulation as the bf16 kernel (one workgroup of 4 waves per 128 query
// rows, 64-key tiles through a two-stage LDS buffer):
//   S^T = K Q^T   A = 32 keys x 64 dims of K (two ds_read_b128 per lane),
//                 B = the wave's 32 query rows (registers), in E4M3;
//                 two k-steps cover d = 128;
//   O^T += V^T P^T  A = 32 dims x 64 keys of V^T, assembled with four
//                 ds_read_b64_tr_b8 per lane; B = the probabilities, rounded
//                 to E4M3 in the lane's own accumulator order; one MFMA per
//                 32-dim block covers the whole tile.
// Any assignment of the k index to (lane half, byte) works for an MFMA as
// long as A and B use the same one: for S it is dims 32h .. 32h+31 of the
// k-step in byte order, for P V it is the accumulator's key order.
//
// Scales: S = s_raw * sq(row block) * sk(key tile) * scale, folded into the
// exponent's FMA (per lane and tile).  The reference max m moves lazily: it
// trails a row's running max by at most 2^RESCALE8 = 4 (it is raised only
// when a tile's max exceeds it by more), so p = 2^(s - m) <= 4 and the P V
// operand p * 2^6 = 2^(s - m + 6) stays <= 256, within E4M3's range;
// O = acc * sv / l, with acc and l both in units of 2^6 p and l summed from
// the unrounded values.
#include "tile.h"

namespace exattn {

namespace {

constexpr int ROW8 = 128;                 // bytes per K/V row (d = 128 in E4M3)
constexpr int TILE8 = BLOCK_N * ROW8;     // 8 KiB
constexpr int STAGE8 = 2 * TILE8;         // K tile + V tile
constexpr int LOADS8 = TILE8 / 1024 / 4;  // 1 KiB DMAs per wave per tile (2)
constexpr int RPL8 = 1024 / ROW8;         // rows per 1 KiB load (8)
constexpr size_t LDS8 = size_t(2) * STAGE8;
constexpr float LOG2E8 = 1.4426950408889634f;
constexpr float LN2_8 = 0.6931471805599453f;
// The reference max trails a row's running max by at most this many powers
// of two, so p <= 2^RESCALE8 and p * 2^(8 - RESCALE8) stays within 256.
constexpr int RESCALE8 = 2;

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef int i32x2v_t __attribute__((__vector_size__(2 * sizeof(int))));

// 128-byte rows: 8 chunks of 16 bytes, the bf16 d = 64 geometry.
__device__ __forceinline__ int swz8(int r) { return swz<64>(r); }

__device__ __forceinline__ i32x8_t mfma8_operand(u32x4_t lo, u32x4_t hi) {
    return i32x8_t{int(lo[0]), int(lo[1]), int(lo[2]), int(lo[3]), int(hi[0]), int(hi[1]), int(hi[2]), int(hi[3])};
}

} // namespace

extern __shared__ __attribute__((aligned(1024))) uint8_t smem_raw[];

template <bool SOFTCAP>
__device__ __forceinline__ void attn_fwd8_body(const Fwd8Params &p) {
    lds_u8 *smem = (lds_u8 *)(smem_raw);
    const int tid = __builtin_amdgcn_workitem_id_x();
    const int bid = __builtin_amdgcn_workgroup_id_x();
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int col = lane & 31, half = lane >> 5;

    // Work assignment: as the bf16 forward (groups sharing K/V on one XCD,
    // heavy-first query tiles).
    const int G = p.Hq / p.Hkv;
    const int per_group = G * p.nqt;
    const int ngroups = p.B * p.Hkv;
    int group, within;
    if ((ngroups & 7) == 0) {
        const int x = bid & 7, j = bid >> 3;
        group = x + 8 * (j / per_group);
        within = j % per_group;
    } else {
        group = bid / per_group;
        within = bid % per_group;
    }
    const int b = group / p.Hkv, hk = group % p.Hkv;
    const int qt = __builtin_amdgcn_readfirstlane(p.mask.order[int64_t(b) * p.nqt + within / G]);
    const int h = hk * G + within % G;
    const int item = b * p.nqt + qt;
    const int row = qt * BLOCK_M + wave * 32 + col;
    const bool row_ok = row < p.N;

    // Q fragment (B operand of S^T): lane (col, half) holds, for k-step s,
    // bytes [64s + 32*half, +32) of its query row.
    i32x8_t qf[2];
    {
        const uint8_t *qrow = p.q + b * p.q_sb + h * p.q_sh + int64_t(row) * p.q_sn;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            u32x4_t lo = {0u, 0u, 0u, 0u}, hi = {0u, 0u, 0u, 0u};
            if (row_ok) {
                lo = *reinterpret_cast<const u32x4_t *>(qrow + 64 * s + 32 * half);
                hi = *reinterpret_cast<const u32x4_t *>(qrow + 64 * s + 32 * half + 16);
            }
            qf[s] = mfma8_operand(lo, hi);
        }
    }
    int lo = 1, hi = 0;
    float qscale = 0.f;
    if (row_ok) {
        lo = p.mask.lo[int64_t(b) * p.N + row];
        hi = p.mask.hi[int64_t(b) * p.N + row];
        qscale = p.q_scales[(int64_t(b) * p.Hq + h) * p.nblk64 + row / BLOCK_N];
    }
    // Element mask of PARTIAL tiles: the width of the row's interval, and an
    // offset that puts every key outside it for a row with none (lo > hi;
    // keys and N stay below 2^30)
    const uint32_t vis_w = hi >= lo ? uint32_t(hi - lo) : 0u;
    const uint32_t vis_pad = hi >= lo ? 0u : 0x40000000u;
    // per-lane base-2 factor of the raw dot products, before the key scale
    const float c_row = p.scale_log2 * qscale;
    const float *kscales = p.k_scales + (int64_t(b) * p.Hkv + hk) * p.nblk64;
    const float vscale = p.v_scales[(int64_t(b) * p.Hkv + hk) * p.nblk64]; // one scale per head: block 0's

    const int ntiles = __builtin_amdgcn_readfirstlane(p.mask.count[item]);
    const int32_t *tiles = p.mask.list + int64_t(item) * p.nkt;
    const uint8_t *kbase = p.k + b * p.k_sb + hk * p.k_sh;
    const uint8_t *vbase = p.v + b * p.v_sb + hk * p.v_sh;

    // HBM -> LDS: wave w, load u fills bytes [(LOADS8*w + u) KiB, +1 KiB) of
    // a tile: row RPL8*(LOADS8*w + u) + lane/8, physical chunk lane%8, which
    // holds logical chunk (lane%8) ^ swz8(row).
    auto ld_row = [&](int u) { return RPL8 * (LOADS8 * wave + u) + lane / 8; };
    auto ld_col = [&](int u) { return 16u * uint32_t((lane % 8) ^ swz8(ld_row(u))); };
    uint32_t ld_koff[LOADS8], ld_voff[LOADS8];
#pragma unroll
    for (int u = 0; u < LOADS8; ++u) {
        ld_koff[u] = uint32_t(ld_row(u)) * uint32_t(p.k_sn) + ld_col(u);
        ld_voff[u] = uint32_t(ld_row(u)) * uint32_t(p.v_sn) + ld_col(u);
    }
    auto issue_tile = [&](int kt, const int stage) {
        const int key0 = kt * BLOCK_N;
        const uint8_t *kt_base = kbase + int64_t(key0) * p.k_sn;
        const uint8_t *vt_base = vbase + int64_t(key0) * p.v_sn;
        lds_u8 *kdst = smem + stage * STAGE8 + LOADS8 * wave * 1024;
        lds_u8 *vdst = kdst + TILE8;
        if (key0 + BLOCK_N <= p.N) {
#pragma unroll
            for (int u = 0; u < LOADS8; ++u) {
                dma16_saddr(kt_base, ld_koff[u], lds_addr(kdst + u * 1024));
                dma16_saddr(vt_base, ld_voff[u], lds_addr(vdst + u * 1024));
            }
        } else {
            const int last = p.N - 1 - key0; // rows past N re-read row N-1 (always masked)
#pragma unroll
            for (int u = 0; u < LOADS8; ++u) {
                const int r = min(ld_row(u), last);
                dma16(kt_base + int64_t(r) * p.k_sn + ld_col(u), lds_addr(kdst + u * 1024));
                dma16(vt_base + int64_t(r) * p.v_sn + ld_col(u), lds_addr(vdst + u * 1024));
            }
        }
    };

    // K reads (A of S^T): row 32*kb + col, logical chunks 4s + 2*half and
    // 4s + 2*half + 1; swz8 depends on row % 16 only, so kb adds 32 rows.
    int k_rd[2][2];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int c = 0; c < 2; ++c) k_rd[s][c] = col * ROW8 + 16 * ((4 * s + 2 * half + c) ^ swz8(col));
    // V^T reads (A of O^T): read t (bytes 8t .. 8t+7 of the operand) of
    // d-block db.  ds_read_b64_tr_b8 gives lane i of each 16-lane group byte
    // i%8 of the 8 bytes addressed by lane 2e + i/8, as element e.  Source
    // lane j = lane%16 addresses key row r_e (e = j/2) at dims
    // 32*db + 16*((lane/16)%2) + 8*(j%2), so lane l receives dim
    // 32*db + l%32 of keys r_0 .. r_7, where for read t
    // r_e = 32(t/2) + 16(t%2) + 8(e/4) + 4*half + e%4: the keys whose
    // probabilities sit in bytes 8t .. 8t+7 of the B operand.
    // Rows of reads t = 0..3 differ by 16t and share r % 16, hence the
    // swizzle: read t is read 0 plus 16t rows (an immediate offset).
    int v_rd[4];
    {
        const int j = lane & 15, e = j >> 1, par = j & 1, g2 = (lane >> 4) & 1;
        const int r = 8 * (e >> 2) + 4 * half + (e & 3);
#pragma unroll
        for (int db = 0; db < 4; ++db) {
            const int cb = 32 * db + 16 * g2 + 8 * par; // byte offset inside the row
            v_rd[db] = r * ROW8 + 16 * ((cb >> 4) ^ swz8(r)) + (cb & 15);
        }
    }

    f32x16_t acc_o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc_o[i] = f32x16_t{};
    float m_run = -INFINITY; // reference max (base-2 units), within RESCALE8 of the running max
    float l_run = 0.f;       // this half's share of the running sum

    int ent_cur = 0, ent_next_v = 0;
    float ksc_cur = 0.f; // key scale of the current tile, loaded a tile ahead
    auto step = [&](int it, const int stage) {
        const int ent = ent_cur;
        const int kt = ent >> 1;
        const bool partial = ent & TILE_PARTIAL;
        const int ent_next = __builtin_amdgcn_readfirstlane(ent_next_v);
        const int ent_next2_v = tiles[min(it + 2, ntiles - 1)];
        const float ksc_next = kscales[ent_next >> 1];
        if (it + 1 < ntiles) issue_tile(ent_next >> 1, 1 - stage);
        const lds_u8 *ks = smem + stage * STAGE8;
        const lds_u8 *vs = ks + TILE8;

        // ---- S^T = K Q^T: 2 key blocks x 2 k-steps, all K reads first ----
        u32x4_t kr[2][2][2]; // [k-step][key block][chunk]
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int c = 0; c < 2; ++c)
                    kr[s][kb][c] = *reinterpret_cast<const __attribute__((address_space(3))) u32x4_t *>(
                        ks + k_rd[s][c] + 32 * kb * ROW8);
        f32x16_t s0 = f32x16_t{}, s1 = f32x16_t{};
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            s0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(mfma8_operand(kr[s][0][0], kr[s][0][1]), qf[s], s0,
                                                                  0, 0, 0, 0, 0, 0);
            s1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(mfma8_operand(kr[s][1][0], kr[s][1][1]), qf[s], s1,
                                                                  0, 0, 0, 0, 0, 0);
        }

        // ---- scale, score mod, mask ----
        const float c = c_row * ksc_cur; // base-2 factor of this tile's raw dot products
        float t[32];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            t[r] = s0[r];
            t[16 + r] = s1[r];
        }
        if constexpr (SOFTCAP) {
            // c * tanh(scale * s / c) in base-2 units from the dequantized
            // dot product (the raw one times sq * sk)
            const float k2 = p.cap_inv_scale_2log2e * qscale * ksc_cur;
#pragma unroll
            for (int j = 0; j < 32; ++j) {
                const float e = __builtin_amdgcn_exp2f(t[j] * k2);
                t[j] = p.cap_log2 - p.cap_log2_2 * __builtin_amdgcn_rcpf(e + 1.f);
            }
        }
        if (partial) {
            // key = kb0 + 4*half + off_j is visible iff key - lo <= hi - lo
            // as unsigned numbers: one add, one compare and one select
            const uint32_t nl = uint32_t(kt * BLOCK_N + 4 * half - lo) + vis_pad;
#pragma unroll
            for (int j = 0; j < 32; ++j)
                if (uint32_t(32 * (j >> 4) + acc_row(j & 15, 0)) + nl > vis_w) t[j] = -INFINITY;
        }

        // ---- online softmax; the reference max moves only when a row's max
        // exceeds it by more than a factor 2^RESCALE8 ----
        float mx[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) mx[k] = fmaxf(t[k], t[k + 4]);
#pragma unroll
        for (int i = 8; i < 32; i += 4)
#pragma unroll
            for (int k = 0; k < 4; ++k) mx[k] = fmaxf(mx[k], t[i + k]);
        float mt = fmaxf(fmaxf(mx[0], mx[1]), fmaxf(mx[2], mx[3]));
        mt = fmaxf(mt, wave_swap_halves(mt, half));
        if constexpr (!SOFTCAP) mt *= c; // c > 0, so the max commutes with it
        // the accumulator's rescale waits for the previous tile's P V
        // products: it is applied after the exponentials
        const bool grow = __any(row_ok && mt > m_run + RESCALE8);
        float alpha = 1.f;
        if (grow) {
            const float m_new = fmaxf(m_run, mt);
            alpha = __builtin_amdgcn_exp2f(m_run - (m_new == -INFINITY ? 0.f : m_new));
            m_run = m_new;
        }
        // p * 2^(8 - RESCALE8) = 2^(s - m + 8 - RESCALE8) <= 256: the E4M3
        // operand directly (the sum l is kept in the same units)
        const float m8 = ((m_run == -INFINITY) ? 0.f : m_run) - float(8 - RESCALE8);
        float ps[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 32; ++j) {
            if constexpr (SOFTCAP)
                t[j] = __builtin_amdgcn_exp2f(t[j] - m8);
            else
                t[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(t[j], c, -m8));
            ps[j & 3] += t[j];
        }
        // one explicit FMA (alpha = 1 without a rescale): the sum rounds the
        // same way in both unrolled copies of the step
        l_run = __builtin_fmaf(l_run, alpha, (ps[0] + ps[1]) + (ps[2] + ps[3]));

        // ---- P to E4M3, byte b = 16kb + r, then O^T += V^T P^T ----
        i32x8_t pk;
#pragma unroll
        for (int w = 0; w < 8; ++w) {
            int v = __builtin_amdgcn_cvt_pk_fp8_f32(t[4 * w], t[4 * w + 1], 0, false);
            v = __builtin_amdgcn_cvt_pk_fp8_f32(t[4 * w + 2], t[4 * w + 3], v, true);
            pk[w] = v;
        }
        // an opaque copy of the flag that depends on the packed probabilities
        // keeps the compiler from merging this branch into the one above
        int grow_late = __builtin_amdgcn_readfirstlane(int(grow));
        asm volatile("" : "+s"(grow_late)
                     : "v"(pk[0]), "v"(pk[1]), "v"(pk[2]), "v"(pk[3]), "v"(pk[4]), "v"(pk[5]), "v"(pk[6]),
                       "v"(pk[7]));
        if (grow_late) {
#pragma unroll
            for (int i = 0; i < 4; ++i) acc_o[i] *= alpha;
        }
        // V^T operands for the four 32-dim blocks, read right before their
        // MFMAs (read during the exponentials they held 32 more registers
        // and the kernel ran 6-9% slower)
        i32x8_t va[4];
#pragma unroll
        for (int db = 0; db < 4; ++db) {
            u32x2_t r8[4];
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                const auto v2 = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                    reinterpret_cast<__attribute__((address_space(3))) i32x2v_t *>(const_cast<lds_u8 *>(vs) +
                                                                                   v_rd[db] + 16 * ROW8 * tt));
                r8[tt] = __builtin_bit_cast(u32x2_t, v2);
            }
            va[db] = i32x8_t{int(r8[0][0]), int(r8[0][1]), int(r8[1][0]), int(r8[1][1]),
                             int(r8[2][0]), int(r8[2][1]), int(r8[3][0]), int(r8[3][1])};
        }
#pragma unroll
        for (int db = 0; db < 4; ++db)
            acc_o[db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va[db], pk, acc_o[db], 0, 0, 0, 0, 0, 0);

        wait_vmem_all();
        __syncthreads();
        ent_cur = ent_next;
        ent_next_v = ent_next2_v;
        ksc_cur = ksc_next;
    };

    if (ntiles > 0) {
        ent_cur = __builtin_amdgcn_readfirstlane(tiles[0]);
        ksc_cur = kscales[ent_cur >> 1];
        issue_tile(ent_cur >> 1, 0);
        ent_next_v = tiles[min(1, ntiles - 1)];
    }
    wait_vmem_all();
    __syncthreads();
    for (int it = 0; it < ntiles; it += 2) {
        step(it, 0);
        if (it + 1 < ntiles) step(it + 1, 1);
    }

    // ---- epilogue: O = acc * sv / l, LSE = ln 2 * (m + log2 l - 8 + RESCALE8)
    // (acc and l both hold p * 2^(8 - RESCALE8)) ----
    const float l_tot = l_run + wave_swap_halves(l_run, half);
    if (row_ok) {
        const float inv = l_tot > 0.f ? vscale / l_tot : 0.f;
        uint16_t *orow = p.o + b * p.o_sb + h * p.o_sh + int64_t(row) * p.o_sn;
#pragma unroll
        for (int db = 0; db < 4; ++db) {
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
                const int d0 = 32 * db + 8 * rq + 4 * half;
                u32x2_t w;
                w[0] = pack_bf16x2(acc_o[db][4 * rq + 0] * inv, acc_o[db][4 * rq + 1] * inv);
                w[1] = pack_bf16x2(acc_o[db][4 * rq + 2] * inv, acc_o[db][4 * rq + 3] * inv);
                *reinterpret_cast<u32x2_t *>(orow + d0) = w;
            }
        }
        if (half == 0) {
            const float lse = l_tot > 0.f ? (m_run + __builtin_amdgcn_logf(l_tot) - float(8 - RESCALE8)) * LN2_8 : -INFINITY;
            p.lse[(int64_t(b) * p.Hq + h) * p.N + row] = lse;
        }
    }
}

__global__ __launch_bounds__(256, 2) void k_attn_fwd8_d128(Fwd8Params p) { attn_fwd8_body<false>(p); }
__global__ __launch_bounds__(256, 2) void k_attn_fwd8_d128_softcap(Fwd8Params p) { attn_fwd8_body<true>(p); }

hipError_t launch_fwd8(const Fwd8Params &p, bool softcap, hipStream_t stream) {
    void (*kernel)(Fwd8Params) = softcap ? k_attn_fwd8_d128_softcap : k_attn_fwd8_d128;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, int(LDS8));
    if (e != hipSuccess) return e;
    const int64_t nblocks = int64_t(p.B) * p.nqt * p.Hq;
    hipLaunchKernelGGL(kernel, dim3(unsigned(nblocks)), dim3(256), LDS8, stream, p);
    return hipGetLastError();
}

static_assert(LOADS8 == 2 && RPL8 == 8, "fp8 tile loads");

} // namespace exattn
