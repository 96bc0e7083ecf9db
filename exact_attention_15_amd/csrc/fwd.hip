// Tiled exact-attention forward pass for gfx950 (CDNA4, wave64, bf16 MFMA).
//
// One workgroup (4 waves) owns 128 query rows of one (batch, head); each wave
// owns 32 of them.  The workgroup sweeps the key tiles that its block-mask
// entry lists (64 keys per tile), staging K and V tiles through LDS with a
// double buffer, and keeps per-row running max m and running sum l so that
// every tile's scores are turned into probabilities immediately and folded
// into the output accumulator with a rescale by exp(m_old - m_new)
// (youngju.dev "FlashAttention 논문 분석", sections "Online Softmax와 블록
// 단위 누적" and "알고리즘 의사코드"; the FlashAttention-2 changes of the same
// page: normalise once at the end, parallelise over query tiles, and keep
// each wave's rows private so waves never reduce through shared memory).
//
// Data movement.  K and V tiles go from HBM straight into LDS with
// global_load_lds_dwordx4 (no register staging, no VALU work): every wave
// instruction writes 1 KiB of LDS contiguously, lane l at byte 16*l.  Rows
// are not padded; instead the 16-byte chunks of row r are XOR-swizzled
// (chunk c stored at c ^ swz(r)), which the loading lanes realise by picking
// which global chunk they fetch.  The next tile is requested before the
// current one is consumed, so its latency hides behind a tile of MFMA work.
//
// MFMA formulation.  Scores are computed transposed, S^T = K Q^T, with
// v_mfma_f32_32x32x16_bf16: K rows are the A operand (ds_read_b128 from LDS),
// the wave's 32 query rows are the B operand (held in registers for the whole
// kernel).  In the 32x32 accumulator, lane l holds column l%32 -- one query
// -- and 16 keys, so a row's max and sum need only an in-lane reduction and
// one exchange between the two 32-lane halves (v_permlane32_swap).  The
// output is accumulated transposed too, O^T = V^T P^T: the probabilities
// already sit in the B-operand layout (lane = query, register = key), and
// the V^T operand is read from the row-major V tile with the LDS transpose
// read ds_read_b64_tr_b16.
//
// Scores are kept in base-2 units (scale * log2 e folded into one FMA), so
// every exponential is one v_exp_f32.
//
// ALiBi (a distance bias added before the softmax, aegloslab "3.7 어텐션 II",
// section 3.7.5) is a compile-time variant: the score becomes
// scale * q.k - slope_h * |i - j| in base-2 units before the cap and mask.
#include "tile.h"

namespace exattn {

constexpr float LN2 = 0.6931471805599453f;
// Lazy rescaling threshold (base-2 units): probabilities stay <= 2^8.
constexpr float RESCALE_LOG2 = 8.f;
// LDS operand reads in flight ahead of the MFMAs that consume them.
constexpr int QK_AHEAD = 2;
constexpr int PV_AHEAD = 3;
// Instruction classes of __builtin_amdgcn_sched_group_barrier.
constexpr int SCHED_MFMA = 0x0008;
constexpr int SCHED_DS_READ = 0x0100;

extern __shared__ __attribute__((aligned(1024))) uint8_t smem_raw[];

// The kernel body is a device template; the __global__ entry points below
// are plain (non-template) functions, one per head dim and score mod.
template <int D, bool SOFTCAP, bool ALIBI>
__device__ __forceinline__ void attn_fwd_body(const FwdParams &p) {
    // Without the cap or the bias, raw dot products are kept until the
    // exponent's FMA applies the scale; otherwise scores are formed in
    // base-2 units first.
    constexpr bool SCALED = SOFTCAP || ALIBI;
    using C = FwdCfg<D>;
    lds_u8 *smem = (lds_u8 *)(smem_raw); // generic -> LDS address space

    // Builtins rather than threadIdx/blockIdx: the latter may be lowered to
    // device-library calls.  The wave index is made a scalar so that all
    // per-wave addresses (LDS destinations of the tile loads) are SGPRs.
    const int tid = __builtin_amdgcn_workitem_id_x();
    const int bid = __builtin_amdgcn_workgroup_id_x();
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int col = lane & 31, half = lane >> 5;

    // Work assignment.  A "group" is everything that reads the same K/V:
    // one (batch row, KV head) with all its query tiles and all Hq/Hkv query
    // heads, ordered heavy-first by query tile, heads adjacent.  Workgroups
    // are dispatched round-robin over the 8 XCDs (id % 8), each with its own
    // L2, so group g is given to XCD g % 8: an XCD then streams whole groups
    // and their K/V tiles are fetched into its L2 once and reused there.
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
    // Values read from memory are not known to be wave-uniform; readfirstlane
    // makes them scalars so all per-tile address arithmetic stays on the SALU.
    const int qt = __builtin_amdgcn_readfirstlane(p.mask.order[int64_t(b) * p.nqt + within / G]);
    const int h = hk * G + within % G;
    const int item = b * p.nqt + qt;
    const int row = qt * BLOCK_M + wave * 32 + col; // this lane's query row
    const bool row_ok = row < p.N;

    // Q fragment: B operand of S^T = K Q^T.  Lane (col, half) holds, for
    // k-step s, elements [16s + 8*half, 16s + 8*half + 8) of its query row.
    bf16x8_t qf[C::KSTEPS];
    {
        const uint16_t *qrow = p.q + b * p.q_sb + h * p.q_sh + int64_t(row) * p.q_sn;
#pragma unroll
        for (int s = 0; s < C::KSTEPS; ++s) {
            u32x4_t x = {0u, 0u, 0u, 0u};
            if (row_ok) x = *reinterpret_cast<const u32x4_t *>(qrow + 16 * s + 8 * half);
            qf[s] = __builtin_bit_cast(bf16x8_t, x);
        }
    }
    int lo = 1, hi = 0;
    if (row_ok) {
        lo = p.mask.lo[int64_t(b) * p.N + row];
        hi = p.mask.hi[int64_t(b) * p.N + row];
    }
    // Element mask of PARTIAL tiles: the width of the row's interval, and an
    // offset that puts every key outside it for a row with none (lo > hi;
    // keys and N stay below 2^30)
    const uint32_t vis_w = hi >= lo ? uint32_t(hi - lo) : 0u;
    const uint32_t vis_pad = hi >= lo ? 0u : 0x40000000u;

    // ALiBi slope of this query head, base-2 units
    float slope = 0.f;
    if constexpr (ALIBI) slope = p.alibi_slopes[h] * 1.4426950408889634f;

    const int ntiles = __builtin_amdgcn_readfirstlane(p.mask.count[item]);
    const int32_t *tiles = p.mask.list + int64_t(item) * p.nkt;
    // With the distance bias the key tiles are visited from the last listed
    // (nearest the diagonal under a causal mask, where the bias is smallest)
    // down, so that a row's max is met early and later tiles rarely raise
    // it: in ascending order a steep slope raised it at every tile and each
    // raise rescaled the accumulator.
    auto tile_at = [&](int i) { return ALIBI ? tiles[ntiles - 1 - i] : tiles[i]; };
    const uint16_t *kbase = p.k + b * p.k_sb + hk * p.k_sh;
    const uint16_t *vbase = p.v + b * p.v_sb + hk * p.v_sh;

    // ---- HBM -> LDS tile loads ----
    // Wave w, load u fills LDS bytes [(LOADS*w + u) KiB, +1 KiB) of a tile:
    // row ROWS_PER_LOAD*(LOADS*w + u) + lane/CHUNKS, physical chunk
    // lane%CHUNKS, which holds logical chunk (lane%CHUNKS) ^ swz(row).  The
    // per-lane byte offsets inside a tile fit 32 bits (stride_n < 2^24).
    auto ld_row = [&](int u) { return C::ROWS_PER_LOAD * (C::LOADS * wave + u) + lane / C::CHUNKS; };
    auto ld_col = [&](int u) { return 8u * uint32_t((lane % C::CHUNKS) ^ swz<D>(ld_row(u))); };
    // Byte offsets, so that each load is a scalar base plus a 32-bit
    // per-lane offset (the saddr + voffset form: no 64-bit VALU adds).
    uint32_t ld_koff[C::LOADS], ld_voff[C::LOADS];
#pragma unroll
    for (int u = 0; u < C::LOADS; ++u) {
        ld_koff[u] = 2u * (uint32_t(ld_row(u)) * uint32_t(p.k_sn) + ld_col(u));
        ld_voff[u] = 2u * (uint32_t(ld_row(u)) * uint32_t(p.v_sn) + ld_col(u));
    }
    auto issue_tile = [&](int kt, const int stage) {
        const int key0 = kt * BLOCK_N;
        const uint16_t *kt_base = kbase + int64_t(key0) * p.k_sn;
        const uint16_t *vt_base = vbase + int64_t(key0) * p.v_sn;
        lds_u8 *kdst = smem + stage * C::STAGE_BYTES + C::LOADS * wave * 1024;
        lds_u8 *vdst = kdst + C::TILE_BYTES;
        if (key0 + BLOCK_N <= p.Nk) {
#pragma unroll
            for (int u = 0; u < C::LOADS; ++u) {
                dma16_saddr(kt_base, ld_koff[u], lds_addr(kdst + u * 1024));
                dma16_saddr(vt_base, ld_voff[u], lds_addr(vdst + u * 1024));
            }
        } else {
            const int last = p.Nk - 1 - key0; // rows past Nk re-read row Nk-1 (always masked)
#pragma unroll
            for (int u = 0; u < C::LOADS; ++u) {
                const int r = min(ld_row(u), last);
                dma16(kt_base + int64_t(r) * p.k_sn + ld_col(u), lds_addr(kdst + u * 1024));
                dma16(vt_base + int64_t(r) * p.v_sn + ld_col(u), lds_addr(vdst + u * 1024));
            }
        }
    };

    // ---- per-lane LDS read offsets (bytes, inside one tile) ----
    // K (A operand of S^T): lane reads row 32*kb + col, logical chunk 2s + half;
    // swz depends on row % 16 only, so kb just adds 32 rows.
    int k_rd[C::KSTEPS];
#pragma unroll
    for (int s = 0; s < C::KSTEPS; ++s)
        k_rd[s] = col * C::ROW_BYTES + 16 * ((2 * s + half) ^ swz<D>(col));
    // V (A operand of O^T, via transpose reads): for the probabilities of
    // keys k0..k0+3 (k0 = 32kb + 16hh + 4*half + 8j) and d-block db, lane
    // reads 8 bytes of row k0 + (lane%16)/4 at elements 32*db + 16*dh +
    // 4*(lane%4); the transpose read then returns, in element e, V[k0+e] at
    // column 32*db + lane%32.  swz of those rows depends on (lane, j) only,
    // so (kb, hh) just add 32kb + 16hh rows.
    const int s16 = lane & 15, dh = (lane >> 4) & 1;
    int v_rd[2][C::DBLK];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int db = 0; db < C::DBLK; ++db) {
            const int r = 4 * half + 8 * j + (s16 >> 2);
            const int cb = 64 * db + 32 * dh + 8 * (s16 & 3); // byte offset inside the row
            v_rd[j][db] = r * C::ROW_BYTES + 16 * ((cb >> 4) ^ swz<D>(r)) + (cb & 15);
        }

    f32x16_t acc_o[C::DBLK];
#pragma unroll
    for (int i = 0; i < C::DBLK; ++i) acc_o[i] = f32x16_t{};
    float m_run = -INFINITY; // reference max (base-2 units), shared by both halves
    float l_run = 0.f;       // this half's share of the running sum

    // One tile: compute on buffer `stage` while the next tile (if any)
    // streams into the other buffer.  The loop below is unrolled by two and
    // the lambda is inlined with stage = 0 and 1, so every LDS address folds
    // into a per-lane register plus an immediate offset.
    // Tile-list entries are read one iteration before they are needed: the
    // entry of tile it+1 was loaded during iteration it-1 and has arrived by
    // the end-of-iteration wait, so no list read is ever waited on alone.
    int ent_cur = 0, ent_next_v = 0;
    auto step = [&](int it, const int stage) {
        const int ent = ent_cur;
        const int kt = ent >> 1;
        const bool partial = ent & TILE_PARTIAL;
        const int ent_next = __builtin_amdgcn_readfirstlane(ent_next_v);
        const int ent_next2_v = tile_at(min(it + 2, ntiles - 1));
        // The other buffer was last read in iteration it-1, which every wave
        // has finished (barrier at the end of it), so it can be refilled now.
        if (it + 1 < ntiles) issue_tile(ent_next >> 1, 1 - stage);

        const lds_u8 *ks = smem + stage * C::STAGE_BYTES;
        const lds_u8 *vs = ks + C::TILE_BYTES;

        // ---- S^T = K Q^T for the tile's two 32-key blocks ----
        // The K operands are read QK_AHEAD k-steps ahead of the MFMAs that
        // use them, so LDS latency overlaps matrix work; the scheduling
        // groups pin that interleave (DS reads, then MFMAs, k-step by k-step).
        f32x16_t s0 = f32x16_t{}, s1 = f32x16_t{};
        // The wave's priority is raised while it issues its MFMA blocks, so
        // that a SIMD whose other wave is in its softmax issues the MFMAs
        // first (+1% measured; raising it for the softmax instead gained
        // nothing).
        __builtin_amdgcn_s_setprio(1);
        {
            bf16x8_t ka[C::KSTEPS][2];
            auto kread = [&](int s) {
                ka[s][0] = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8_t *>(ks + k_rd[s]);
                ka[s][1] = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8_t *>(
                    ks + k_rd[s] + 32 * C::ROW_BYTES);
            };
#pragma unroll
            for (int s = 0; s < QK_AHEAD; ++s) kread(s);
#pragma unroll
            for (int s = 0; s < C::KSTEPS; ++s) {
                if (s + QK_AHEAD < C::KSTEPS) kread(s + QK_AHEAD);
                s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[s][0], qf[s], s0, 0, 0, 0);
                s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[s][1], qf[s], s1, 0, 0, 0);
            }
            __builtin_amdgcn_sched_group_barrier(SCHED_DS_READ, 2 * QK_AHEAD, 0);
#pragma unroll
            for (int s = 0; s < C::KSTEPS; ++s) {
                if (s + QK_AHEAD < C::KSTEPS) __builtin_amdgcn_sched_group_barrier(SCHED_DS_READ, 2, 0);
                __builtin_amdgcn_sched_group_barrier(SCHED_MFMA, 2, 0);
            }
        }
        __builtin_amdgcn_s_setprio(0);

        // ---- score_mod and mask in registers ----
        // Without a cap the raw dot products are kept and the scale is folded
        // into the exponent's FMA (max commutes with a positive scale); with
        // the cap, c * tanh(scale * s / c) is formed first, in base-2 units,
        // using tanh(x) = 1 - 2 / (exp(2x) + 1).
        float t[32];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            t[r] = s0[r];
            t[16 + r] = s1[r];
        }
        if constexpr (ALIBI) {
            // key - row for register j is rel + c_j, c_j = 32 * (j / 16) +
            // acc_row(j % 16, 0); the bias -slope * |key - row| is
            // -|y| (slope >= 0) or +|y| with y = slope * (key - row), one FMA
            // each, the absolute value being an operand modifier
            const float srel = slope * float(kt * BLOCK_N + 4 * half - row);
            if (slope >= 0.f) {
#pragma unroll
                for (int j = 0; j < 32; ++j) {
                    const float y = __builtin_fmaf(float(32 * (j >> 4) + acc_row(j & 15, 0)), slope, srel);
                    t[j] = __builtin_fmaf(t[j], p.scale_log2, -fabsf(y));
                }
            } else {
#pragma unroll
                for (int j = 0; j < 32; ++j) {
                    const float y = __builtin_fmaf(float(32 * (j >> 4) + acc_row(j & 15, 0)), slope, srel);
                    t[j] = __builtin_fmaf(t[j], p.scale_log2, fabsf(y));
                }
            }
        }
        // Without the bias, a tile whose raw scores all lie in
        // |scale * s / c| <= 0.15 (a wave-uniform test) takes the polynomial
        // form of the cap instead of an exponential and a reciprocal.
        // Without the bias the cap is also fused into the exponent (CAPFUSE):
        // the row max is taken on the raw scores and capped once (the cap is
        // increasing), and each score's capped value minus the reference max
        // is a single FMA.
        constexpr bool CAPFUSE = SOFTCAP && !ALIBI;
        bool poly = false;
        if constexpr (CAPFUSE) {
            float am[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) am[k] = fmaxf(fabsf(t[k]), fabsf(t[k + 4]));
#pragma unroll
            for (int i = 8; i < 32; i += 4)
#pragma unroll
                for (int k = 0; k < 4; ++k) am[k] = fmaxf(am[k], fabsf(t[i + k]));
            const float a = fmaxf(fmaxf(am[0], am[1]), fmaxf(am[2], am[3]));
            poly = __all(a <= p.cap_poly_lim);
        }
        if constexpr (SOFTCAP && ALIBI) {
            // with the bias the score is already scaled (base-2 units)
#pragma unroll
            for (int j = 0; j < 32; ++j) {
                const float e = __builtin_amdgcn_exp2f(t[j] * p.cap_inv2);
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

        // ---- online softmax ----
        // The exponentials are formed first against the current reference
        // max.  If every lane's 32 probabilities sum below 2^RESCALE_LOG2,
        // none of them reaches it, so no row's max has risen past the
        // reference by RESCALE_LOG2 and nothing is rescaled: the row-max
        // tree is skipped.  Otherwise (and while some row has no reference
        // yet) the max is taken and the rescale decided as before, and the
        // exponentials are formed again if the reference moved.  The result
        // is the same either way.
        auto exps = [&](float m_use, float (&pv)[32], float (&ps)[4]) {
#pragma unroll
            for (int k = 0; k < 4; ++k) ps[k] = 0.f;
            if constexpr (CAPFUSE) {
                if (poly) {
                    // s (a0 + s^2 (a1 + s^2 a2)) - m as one FMA; a masked
                    // score (-inf) gives -inf * +inf - m = -inf
#pragma unroll
                    for (int j = 0; j < 32; ++j) {
                        const float r2 = t[j] * t[j];
                        const float q = __builtin_fmaf(__builtin_fmaf(p.cap_poly[2], r2, p.cap_poly[1]), r2, p.cap_poly[0]);
                        pv[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(t[j], q, -m_use));
                        ps[j & 3] += pv[j];
                    }
                } else {
                    // c log2e - 2 c log2e / (exp(2 scale s / c) + 1) - m, with
                    // the masked scores (finite here) put back to -inf
                    const float cm = p.cap_log2 - m_use;
#pragma unroll
                    for (int j = 0; j < 32; ++j) {
                        const float e = __builtin_amdgcn_exp2f(t[j] * p.cap_inv_scale_2log2e);
                        float x = __builtin_fmaf(-p.cap_log2_2, __builtin_amdgcn_rcpf(e + 1.f), cm);
                        if (partial && t[j] == -INFINITY) x = -INFINITY;
                        pv[j] = __builtin_amdgcn_exp2f(x);
                        ps[j & 3] += pv[j];
                    }
                }
            } else {
#pragma unroll
                for (int j = 0; j < 32; ++j) {
                    if constexpr (SCALED)
                        pv[j] = __builtin_amdgcn_exp2f(t[j] - m_use);
                    else
                        pv[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(t[j], p.scale_log2, -m_use));
                    ps[j & 3] += pv[j];
                }
            }
        };
        float pv[32], ps[4];
        float alpha = 1.f;
        const bool fresh = __any(row_ok && m_run == -INFINITY);
        bool need_max = fresh;
        if (!fresh) {
            exps(m_run, pv, ps);
            const float lsum = (ps[0] + ps[1]) + (ps[2] + ps[3]);
            need_max = __any(row_ok && !(lsum < float(1 << int(RESCALE_LOG2))));
        }
        if (need_max) {
            // Row max and sum as 4-way trees: short dependency chains.
            float mx[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) mx[k] = fmaxf(t[k], t[k + 4]);
#pragma unroll
            for (int i = 8; i < 32; i += 4)
#pragma unroll
                for (int k = 0; k < 4; ++k) mx[k] = fmaxf(mx[k], t[i + k]);
            float mt = fmaxf(fmaxf(mx[0], mx[1]), fmaxf(mx[2], mx[3]));
            mt = fmaxf(mt, wave_swap_halves(mt, half));
            if constexpr (!SCALED) mt *= p.scale_log2;
            if constexpr (CAPFUSE) {
                // the cap of the raw row max (-inf stays -inf in the polynomial
                // form: its highest coefficient is positive)
                if (poly) {
                    const float r2 = mt * mt;
                    mt *= __builtin_fmaf(__builtin_fmaf(p.cap_poly[2], r2, p.cap_poly[1]), r2, p.cap_poly[0]);
                } else if (mt != -INFINITY) {
                    const float e = __builtin_amdgcn_exp2f(mt * p.cap_inv_scale_2log2e);
                    mt = p.cap_log2 - p.cap_log2_2 * __builtin_amdgcn_rcpf(e + 1.f);
                }
            }
            // Rescale O and l only when some valid row's max grew by more than
            // RESCALE_LOG2 (a wave-uniform decision); otherwise keep the older,
            // smaller reference max: p stays <= 2^RESCALE_LOG2 and the result is
            // exact, since O, l and the LSE all use the same reference.  Rows
            // past N never vote, so the decision does not depend on whether
            // fully visible tiles are element-masked.
            const float m_new = fmaxf(m_run, mt);
            bool moved = false;
            if (__any(row_ok && m_new > m_run + RESCALE_LOG2)) {
                alpha = __builtin_amdgcn_exp2f(m_run - (m_new == -INFINITY ? 0.f : m_new));
#pragma unroll
                for (int i = 0; i < C::DBLK; ++i) acc_o[i] *= alpha;
                m_run = m_new;
                moved = true;
            }
            if (fresh || moved) exps((m_run == -INFINITY) ? 0.f : m_run, pv, ps);
        }
#pragma unroll
        for (int j = 0; j < 32; ++j) t[j] = pv[j];
        // one explicit FMA (alpha = 1 without a rescale), so that the sum
        // rounds the same way in both unrolled copies of the step whatever
        // the compiler contracts
        l_run = __builtin_fmaf(l_run, alpha, (ps[0] + ps[1]) + (ps[2] + ps[3]));

        // ---- O^T += V^T P^T ----
        u32x4_t pk[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            pk[i][0] = pack_bf16x2(t[8 * i + 0], t[8 * i + 1]);
            pk[i][1] = pack_bf16x2(t[8 * i + 2], t[8 * i + 3]);
            pk[i][2] = pack_bf16x2(t[8 * i + 4], t[8 * i + 5]);
            pk[i][3] = pack_bf16x2(t[8 * i + 6], t[8 * i + 7]);
        }
        // MFMA m = (2*kb + hh)*DBLK + db uses the probabilities of keys
        // k0 + {0..3} and k0 + 8 + {0..3}, k0 = 32kb + 16hh + 4*half, and the
        // V^T operand of those keys for d-block db; operands are read PV_AHEAD
        // MFMAs ahead.
        __builtin_amdgcn_s_setprio(1);
        {
            constexpr int NM = 4 * C::DBLK;
            u32x4_t va[NM];
            auto vread = [&](int m) {
                const int kbhh = m / C::DBLK, db = m % C::DBLK;
                const lds_u8 *vrow = vs + 16 * kbhh * C::ROW_BYTES;
                const u32x2_t l2 = lds_read_tr16(vrow, v_rd[0][db]);
                const u32x2_t h2 = lds_read_tr16(vrow, v_rd[1][db]);
                va[m] = u32x4_t{l2[0], l2[1], h2[0], h2[1]};
            };
#pragma unroll
            for (int m = 0; m < PV_AHEAD; ++m) vread(m);
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                if (m + PV_AHEAD < NM) vread(m + PV_AHEAD);
                const int db = m % C::DBLK;
                acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    __builtin_bit_cast(bf16x8_t, va[m]), __builtin_bit_cast(bf16x8_t, pk[m / C::DBLK]),
                    acc_o[db], 0, 0, 0);
            }
            __builtin_amdgcn_sched_group_barrier(SCHED_DS_READ, 2 * PV_AHEAD, 0);
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                if (m + PV_AHEAD < NM) __builtin_amdgcn_sched_group_barrier(SCHED_DS_READ, 2, 0);
                __builtin_amdgcn_sched_group_barrier(SCHED_MFMA, 1, 0);
            }
        }
        __builtin_amdgcn_s_setprio(0);

        // The next tile's LDS writes must land before anyone reads them, and
        // this tile's buffer must be free before it is refilled.
        wait_vmem_all();
        __syncthreads();
        ent_cur = ent_next;
        ent_next_v = ent_next2_v;
    };

    if (ntiles > 0) {
        ent_cur = __builtin_amdgcn_readfirstlane(tile_at(0));
        issue_tile(ent_cur >> 1, 0);
        ent_next_v = tile_at(min(1, ntiles - 1));
    }
    wait_vmem_all();
    __syncthreads();
    for (int it = 0; it < ntiles; it += 2) {
        step(it, 0);
        if (it + 1 < ntiles) step(it + 1, 1);
    }

    // ---- epilogue: O / l, LSE = ln 2 * (m + log2 l) ----
    const float l_tot = l_run + wave_swap_halves(l_run, half);
    if (row_ok) {
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        uint16_t *orow = p.o + b * p.o_sb + h * p.o_sh + int64_t(row) * p.o_sn;
#pragma unroll
        for (int db = 0; db < C::DBLK; ++db) {
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
            const float lse = l_tot > 0.f ? (m_run + __builtin_amdgcn_logf(l_tot)) * LN2 : -INFINITY;
            p.lse[(int64_t(b) * p.Hq + h) * p.N + row] = lse;
        }
    }
}

#define EXATTN_FWD_KERNEL(NAME, D, SOFTCAP, ALIBI)                                             \
    __global__ __launch_bounds__(256, 2) void NAME(FwdParams p) { attn_fwd_body<D, SOFTCAP, ALIBI>(p); }
EXATTN_FWD_KERNEL(k_attn_fwd_d128, 128, false, false)
EXATTN_FWD_KERNEL(k_attn_fwd_d128_softcap, 128, true, false)
EXATTN_FWD_KERNEL(k_attn_fwd_d64, 64, false, false)
EXATTN_FWD_KERNEL(k_attn_fwd_d64_softcap, 64, true, false)
EXATTN_FWD_KERNEL(k_attn_fwd_d128_alibi, 128, false, true)
EXATTN_FWD_KERNEL(k_attn_fwd_d128_softcap_alibi, 128, true, true)
EXATTN_FWD_KERNEL(k_attn_fwd_d64_alibi, 64, false, true)
EXATTN_FWD_KERNEL(k_attn_fwd_d64_softcap_alibi, 64, true, true)
#undef EXATTN_FWD_KERNEL

static hipError_t launch_kernel(void (*kernel)(FwdParams), size_t lds_bytes, const FwdParams &p,
                                hipStream_t stream) {
    // More than 64 KiB of dynamic LDS must be allowed explicitly (per device).
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, int(lds_bytes));
    if (e != hipSuccess) return e;
    const int64_t nblocks = int64_t(p.B) * p.nqt * p.Hq;
    hipLaunchKernelGGL(kernel, dim3(unsigned(nblocks)), dim3(256), lds_bytes, stream, p);
    return hipGetLastError();
}

hipError_t launch_fwd(const FwdParams &p, int d, bool softcap, bool alibi, hipStream_t stream) {
    void (*kernel)(FwdParams);
    if (d == 128)
        kernel = alibi ? (softcap ? k_attn_fwd_d128_softcap_alibi : k_attn_fwd_d128_alibi)
                       : (softcap ? k_attn_fwd_d128_softcap : k_attn_fwd_d128);
    else
        kernel = alibi ? (softcap ? k_attn_fwd_d64_softcap_alibi : k_attn_fwd_d64_alibi)
                       : (softcap ? k_attn_fwd_d64_softcap : k_attn_fwd_d64);
    return launch_kernel(kernel, d == 128 ? FwdCfg<128>::LDS_BYTES : FwdCfg<64>::LDS_BYTES, p, stream);
}

static_assert(FwdCfg<128>::LOADS == 4 && FwdCfg<64>::LOADS == 2, "tile loads per wave");
static_assert(FwdCfg<128>::LDS_BYTES == 65536, "two 32 KiB stages at d = 128");

} // namespace exattn
