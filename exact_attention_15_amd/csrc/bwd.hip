// Backward pass of tiled exact attention for gfx950: dQ, dK and dV from Q,
// K, V, the output O, its gradient dO and the forward's per-row log-sum-exp.
//
// The probabilities are recomputed tile by tile from the saved LSE instead of
// being stored (youngju.dev "FlashAttention 논문 분석", section
// "Recomputation 전략"): P = exp(S - LSE).  With dP = dO V^T and
// D_i = rowsum(dO_i * O_i), the softmax backward is dS = P * (dP - D); the
// soft cap multiplies it by 1 - tanh^2 = 1 - (s' / c)^2; then
// dQ = scale * dS K, dK = scale * dS^T Q and dV = P^T dO.
//
// Two gradient kernels, after the transposed block mask (k_bwd_mask_kv):
//   k_bwd_dq     the forward's decomposition (128 query rows per workgroup,
//                64-key tiles from the forward block mask): first, per row,
//                D = dO . O and the base-2 LSE (+inf for a row with no
//                visible key, so its recomputed P is 0), kept and written
//                for the next kernel; then S^T = K Q^T and dP^T = V dO^T on
//                the MFMA pipe, dS^T in registers, and dQ^T += K^T dS^T with
//                K^T from LDS transpose reads;
//   k_bwd_dkdv   128 keys per workgroup (K and V fragments held in registers,
//                one key per lane column), streaming the 64-row Q and dO
//                tiles of every query head of the GQA group: S = Q K^T,
//                dV^T += dO^T P, dP = dO V^T, dK^T += Q^T dS.
// The mirrored formulations keep every accumulator in the layout the next
// MFMA takes as its B operand, as in the forward pass.
#include "tile.h"

namespace exattn {

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));

constexpr float LOG2E = 1.4426950408889634f;
constexpr int B_AHEAD = 2; // LDS operand reads in flight ahead of their MFMAs
// The dK/dV kernel runs one wave per SIMD, so nothing else hides its LDS
// operand latency: at d = 128 its reads go six k-steps ahead, held there by
// scheduling groups (left to itself the scheduler put a wait before almost
// every MFMA).  Measured on the causal MHA backward (d = 128): 4.38 -> 4.18
// ms; at d = 64 (four k-steps) the unpinned order measured 1.3% faster.
template <int D> constexpr int dkdv_ahead() { return D == 128 ? 6 : B_AHEAD; }

extern __shared__ __attribute__((aligned(1024))) uint8_t smem_raw[];

// ---------------------------------------------------------------------------
// Transposed block mask: for every (b, 128-key block), the 64-row query tiles
// holding a visible (row, key) pair, ascending, each FULL or PARTIAL.  A tile
// is FULL when all its 64 rows exist and see every key of the block that
// exists.  Wave w classifies query tiles w*64 + j (j = 0..63) of each round
// of 256, one after another with lane = row and two ballots (the rows'
// intervals loaded eight tiles at a time); the visited tiles are compacted
// in order with a ballot/popcount prefix.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_bwd_mask_kv(int N, int nkb, int nqt64, uint32_t flags,
                                                     const int32_t *lo_in, const int32_t *hi_in,
                                                     int32_t *count_out, int32_t *list_out) {
    __shared__ int32_t s_wcnt[4];
    const int kb = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
    const int lane = t & 63, w = t >> 6;
    const int c0 = kb * BWD_KB, c1 = min(c0 + BWD_KB, N) - 1; // existing keys of the block
    const bool no_skip = flags & ATTN_MASK_NO_SKIP;
    const int64_t item = int64_t(b) * nkb + kb;
    int32_t *list = list_out + item * nqt64;
    int base = 0;
    for (int k0 = 0; k0 < nqt64; k0 += 256) {
        bool my_any = false, my_full = false;
        const int kw = k0 + w * 64;
        // eight query tiles per batch: their row intervals are all requested
        // before the first is used, one memory round trip per batch
        for (int j0 = 0; j0 < 64; j0 += 8) {
            if (kw + j0 >= nqt64) break; // wave-uniform
            int lo[8], hi[8];
            bool ok[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int row = (kw + j0 + u) * BLOCK_N + lane;
                ok[u] = kw + j0 + u < nqt64 && row < N;
                lo[u] = 1;
                hi[u] = 0;
                if (ok[u]) {
                    lo[u] = lo_in[int64_t(b) * N + row];
                    hi[u] = hi_in[int64_t(b) * N + row];
                }
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                if (kw + j0 + u >= nqt64) break; // wave-uniform
                const bool seen = ok[u] && max(lo[u], c0) <= min(hi[u], c1);
                const bool gap = !ok[u] || !(lo[u] <= c0 && hi[u] >= c1);
                bool any = __any(seen), full = !__any(gap);
                if (no_skip) {
                    any = true;
                    full = false;
                }
                if (lane == j0 + u) {
                    my_any = any;
                    my_full = full;
                }
            }
        }
        const uint64_t vis = __ballot(my_any);
        if (lane == 0) s_wcnt[w] = __popcll(vis);
        __syncthreads();
        int woff = base;
        for (int x = 0; x < w; ++x) woff += s_wcnt[x];
        const int total = s_wcnt[0] + s_wcnt[1] + s_wcnt[2] + s_wcnt[3];
        if (my_any) {
            const int pos = woff + __popcll(vis & ((uint64_t(1) << lane) - 1));
            list[pos] = ((kw + lane) << 1) | (my_full ? 0 : TILE_PARTIAL);
        }
        base += total;
        __syncthreads();
    }
    if (t == 0) count_out[item] = base;
}

// ---------------------------------------------------------------------------
// Shared pieces of the two gradient kernels.
// ---------------------------------------------------------------------------
// AHEAD: operand reads in flight ahead of the MFMAs; PIN: hold that order
// with scheduling groups.
template <int D, int AHEAD = B_AHEAD, bool PIN = false> struct BwdTile {
    using C = FwdCfg<D>;
    // Per-lane LDS offsets.  Row reads (A operand of a "rows x fragment"
    // product): lane reads row 32*kb + col, logical chunk 2s + half.
    // Transpose reads (A operand of a "d x rows" product): see the forward.
    int rd[C::KSTEPS];
    int tr[2][C::DBLK];
    __device__ void init(int col, int half, int lane) {
#pragma unroll
        for (int s = 0; s < C::KSTEPS; ++s) rd[s] = col * C::ROW_BYTES + 16 * ((2 * s + half) ^ swz<D>(col));
        const int s16 = lane & 15, dh = (lane >> 4) & 1;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int db = 0; db < C::DBLK; ++db) {
                const int r = 4 * half + 8 * j + (s16 >> 2);
                const int cb = 64 * db + 32 * dh + 8 * (s16 & 3);
                tr[j][db] = r * C::ROW_BYTES + 16 * ((cb >> 4) ^ swz<D>(r)) + (cb & 15);
            }
    }
    // X^T-block products: acc_kb = tile rows [32kb, 32kb+32) times frag^T
    // (lane column = the fragment's row), for kb = 0, 1.
    __device__ void rows_times_frag(const lds_u8 *tile, const bf16x8_t *frag, f32x16_t &s0, f32x16_t &s1) const {
        bf16x8_t a[C::KSTEPS][2];
        auto rd_s = [&](int s) {
            a[s][0] = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8_t *>(tile + rd[s]);
            a[s][1] = *reinterpret_cast<const __attribute__((address_space(3))) bf16x8_t *>(tile + rd[s] +
                                                                                           32 * C::ROW_BYTES);
        };
        s0 = f32x16_t{};
        s1 = f32x16_t{};
#pragma unroll
        for (int s = 0; s < AHEAD && s < C::KSTEPS; ++s) rd_s(s);
#pragma unroll
        for (int s = 0; s < C::KSTEPS; ++s) {
            if (s + AHEAD < C::KSTEPS) rd_s(s + AHEAD);
            s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s][0], frag[s], s0, 0, 0, 0);
            s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s][1], frag[s], s1, 0, 0, 0);
        }
        if constexpr (PIN) {
            // keep the operand reads AHEAD k-steps ahead of their MFMAs
            __builtin_amdgcn_sched_group_barrier(0x0100, 2 * (AHEAD < C::KSTEPS ? AHEAD : C::KSTEPS), 0);
#pragma unroll
            for (int s = 0; s < C::KSTEPS; ++s) {
                if (s + AHEAD < C::KSTEPS) __builtin_amdgcn_sched_group_barrier(0x0100, 2, 0);
                __builtin_amdgcn_sched_group_barrier(0x0008, 2, 0);
            }
        }
    }
    // acc[db] += tile^T (d-block db x 64 rows) times pk (64 rows x 32 lane
    // columns, packed in the accumulator's row order).
    __device__ void tile_t_times(const lds_u8 *tile, const u32x4_t *pk, f32x16_t *acc) const {
        constexpr int NM = 4 * C::DBLK;
        u32x4_t va[NM];
        auto vread = [&](int m) {
            const int kbhh = m / C::DBLK, db = m % C::DBLK;
            const lds_u8 *vrow = tile + 16 * kbhh * C::ROW_BYTES;
            const u32x2_t l2 = lds_read_tr16(vrow, tr[0][db]);
            const u32x2_t h2 = lds_read_tr16(vrow, tr[1][db]);
            va[m] = u32x4_t{l2[0], l2[1], h2[0], h2[1]};
        };
#pragma unroll
        for (int m = 0; m < AHEAD; ++m) vread(m);
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            if (m + AHEAD < NM) vread(m + AHEAD);
            const int db = m % C::DBLK;
            acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, va[m]),
                                                               __builtin_bit_cast(bf16x8_t, pk[m / C::DBLK]), acc[db],
                                                               0, 0, 0);
        }
        if constexpr (PIN) {
            __builtin_amdgcn_sched_group_barrier(0x0100, 2 * AHEAD, 0);
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                if (m + AHEAD < NM) __builtin_amdgcn_sched_group_barrier(0x0100, 2, 0);
                __builtin_amdgcn_sched_group_barrier(0x0008, 1, 0);
            }
        }
    }
};

// Fragment of row `row` (zero if !ok): lane (col, half) holds, for k-step s,
// elements [16s + 8*half, +8) -- the B-operand layout of the products above.
template <int D>
__device__ __forceinline__ void load_frag(const uint16_t *rowp, bool ok, int half, bf16x8_t *f) {
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
        u32x4_t x = {0u, 0u, 0u, 0u};
        if (ok) x = *reinterpret_cast<const u32x4_t *>(rowp + 16 * s + 8 * half);
        f[s] = __builtin_bit_cast(bf16x8_t, x);
    }
}

__device__ __forceinline__ void pack4(const float *t, u32x4_t *pk) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        pk[i][0] = pack_bf16x2(t[8 * i + 0], t[8 * i + 1]);
        pk[i][1] = pack_bf16x2(t[8 * i + 2], t[8 * i + 3]);
        pk[i][2] = pack_bf16x2(t[8 * i + 4], t[8 * i + 5]);
        pk[i][3] = pack_bf16x2(t[8 * i + 6], t[8 * i + 7]);
    }
}

// Store a transposed accumulator (rows = d, column = this lane's row `row`)
// times `mul` as bf16 into out[row][d].
template <int D>
__device__ __forceinline__ void store_rowmajor(uint16_t *outrow, const f32x16_t *acc, float mul, int half) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
            const int d0 = 32 * db + 8 * rq + 4 * half;
            u32x2_t w;
            w[0] = pack_bf16x2(acc[db][4 * rq + 0] * mul, acc[db][4 * rq + 1] * mul);
            w[1] = pack_bf16x2(acc[db][4 * rq + 2] * mul, acc[db][4 * rq + 3] * mul);
            *reinterpret_cast<u32x2_t *>(outrow + d0) = w;
        }
}

// Issue the DMA of a 64-row tile of a [rows, D] matrix (row stride sn) into
// LDS `dst` (this wave's LOADS KiB; rows past N re-read row N-1).
template <int D>
__device__ __forceinline__ void dma_tile(const uint16_t *base, int64_t sn, int row0, int N, const uint32_t *off,
                                         lds_u8 *dst, int wave, int lane) {
    using C = FwdCfg<D>;
    const uint16_t *tb = base + int64_t(row0) * sn;
    lds_u8 *d = dst + C::LOADS * wave * 1024;
    if (row0 + BLOCK_N <= N) {
#pragma unroll
        for (int u = 0; u < C::LOADS; ++u) dma16_saddr(tb, off[u], lds_addr(d + u * 1024));
    } else {
        const int last = N - 1 - row0;
#pragma unroll
        for (int u = 0; u < C::LOADS; ++u) {
            const int r = min(C::ROWS_PER_LOAD * (C::LOADS * wave + u) + lane / C::CHUNKS, last);
            const uint32_t c = 8u * uint32_t((lane % C::CHUNKS) ^
                                             swz<D>(C::ROWS_PER_LOAD * (C::LOADS * wave + u) + lane / C::CHUNKS));
            dma16(tb + int64_t(r) * sn + c, lds_addr(d + u * 1024));
        }
    }
}
template <int D> __device__ __forceinline__ void dma_offsets(int64_t sn, int wave, int lane, uint32_t *off) {
    using C = FwdCfg<D>;
#pragma unroll
    for (int u = 0; u < C::LOADS; ++u) {
        const int r = C::ROWS_PER_LOAD * (C::LOADS * wave + u) + lane / C::CHUNKS;
        off[u] = 2u * (uint32_t(r) * uint32_t(sn) + 8u * uint32_t((lane % C::CHUNKS) ^ swz<D>(r)));
    }
}

// ---------------------------------------------------------------------------
// dQ.  One workgroup per (128-row query tile, query head, b), work mapped as
// in the forward (groups sharing K/V on one XCD, heavy-first query tiles).
// ---------------------------------------------------------------------------
// SAME_SN: K and V have the same token stride, so their tile DMAs share
// one set of per-lane offsets (four fewer VGPRs held through the loop).
template <int D, bool SOFTCAP, bool SAME_SN>
__device__ __forceinline__ void bwd_dq_body(const BwdParams &p) {
    using C = FwdCfg<D>;
    lds_u8 *smem = (lds_u8 *)(smem_raw);
    const int tid = __builtin_amdgcn_workitem_id_x();
    const int bid = __builtin_amdgcn_workgroup_id_x();
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int col = lane & 31, half = lane >> 5;

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

    bf16x8_t qf[C::KSTEPS], gf[C::KSTEPS];
    load_frag<D>(p.q + b * p.q_sb + h * p.q_sh + int64_t(row) * p.q_sn, row_ok, half, qf);
    load_frag<D>(p.dout + b * p.do_sb + h * p.do_sh + int64_t(row) * p.do_sn, row_ok, half, gf);
    int lo = 1, hi = 0;
    float lse2 = INFINITY, dd = 0.f;
    {
        // The row's D = rowsum(dO * O) and base-2 LSE are formed here, from
        // the dO fragment already in registers and the row of O read in the
        // same layout, and written for the dK/dV kernel that runs next.
        bf16x8_t of[C::KSTEPS];
        load_frag<D>(p.o + b * p.o_sb + h * p.o_sh + int64_t(row) * p.o_sn, row_ok, half, of);
        float acc = 0.f;
#pragma unroll
        for (int s2 = 0; s2 < C::KSTEPS; ++s2)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc = __builtin_fmaf(float(gf[s2][e]), float(of[s2][e]), acc);
        dd = acc + wave_swap_halves(acc, half);
        if (row_ok) {
            lo = p.mask.lo[int64_t(b) * p.N + row];
            hi = p.mask.hi[int64_t(b) * p.N + row];
            const int64_t r = (int64_t(b) * p.Hq + h) * p.N + row;
            const float l = p.lse[r];
            lse2 = l == -INFINITY ? INFINITY : l * LOG2E;
            if (half == 0) {
                p.dvec[r] = dd;
                p.lse2[r] = lse2;
            }
        }
    }
    // Element mask of PARTIAL tiles, as in the forward: key is visible iff
    // key - lo <= hi - lo as unsigned numbers; a row with no visible key
    // gets an offset that puts every key outside (keys stay below 2^30).
    const uint32_t vis_w = hi >= lo ? uint32_t(hi - lo) : 0u;
    const uint32_t vis_pad = hi >= lo ? 0u : 0x40000000u;

    const int ntiles = __builtin_amdgcn_readfirstlane(p.mask.count[item]);
    const int32_t *tiles = p.mask.list + int64_t(item) * p.nkt;
    const uint16_t *kbase = p.k + b * p.k_sb + hk * p.k_sh;
    const uint16_t *vbase = p.v + b * p.v_sb + hk * p.v_sh;
    uint32_t koff[C::LOADS], voff[SAME_SN ? 1 : C::LOADS];
    dma_offsets<D>(p.k_sn, wave, lane, koff);
    if constexpr (!SAME_SN) dma_offsets<D>(p.v_sn, wave, lane, voff);
    const uint32_t *voffs = SAME_SN ? koff : voff;
    auto issue_tile = [&](int kt, int stage) {
        lds_u8 *kdst = smem + stage * C::STAGE_BYTES;
        dma_tile<D>(kbase, p.k_sn, kt * BLOCK_N, p.N, koff, kdst, wave, lane);
        dma_tile<D>(vbase, p.v_sn, kt * BLOCK_N, p.N, voffs, kdst + C::TILE_BYTES, wave, lane);
    };
    BwdTile<D> tl;
    tl.init(col, half, lane);

    f32x16_t acc[C::DBLK];
#pragma unroll
    for (int i = 0; i < C::DBLK; ++i) acc[i] = f32x16_t{};

    int ent_cur = 0, ent_next_v = 0;
    auto step = [&](int it, const int stage) {
        const int ent = ent_cur;
        const int kt = ent >> 1;
        const bool partial = ent & TILE_PARTIAL;
        const int ent_next = __builtin_amdgcn_readfirstlane(ent_next_v);
        const int ent_next2_v = tiles[min(it + 2, ntiles - 1)];
        if (it + 1 < ntiles) issue_tile(ent_next >> 1, 1 - stage);
        const lds_u8 *ks = smem + stage * C::STAGE_BYTES;
        const lds_u8 *vs = ks + C::TILE_BYTES;

        // S^T = K Q^T (lane = query, registers = keys), then P^T (with the
        // soft cap's derivative folded in), then dP^T = V dO^T
        float ds[32];
        {
            f32x16_t s0, s1;
            tl.rows_times_frag(ks, qf, s0, s1);
#pragma unroll
            for (int j = 0; j < 32; ++j) {
                const float s = j < 16 ? s0[j] : s1[j - 16];
                float pj, fac = 1.f;
                if constexpr (SOFTCAP) {
                    const float e = __builtin_amdgcn_exp2f(s * p.cap_inv_scale_2log2e);
                    const float tc = p.cap_log2 - p.cap_log2_2 * __builtin_amdgcn_rcpf(e + 1.f);
                    const float r = tc * p.inv_cap_log2;
                    fac = 1.f - r * r;
                    pj = __builtin_amdgcn_exp2f(tc - lse2);
                } else {
                    pj = __builtin_amdgcn_exp2f(__builtin_fmaf(s, p.scale_log2, -lse2));
                }
                ds[j] = pj * fac;
            }
            // The mask is a loop of its own under one branch: tested inside
            // the loop above, the compiler turned it into selects that ran
            // on every tile.
            if (partial) {
                const uint32_t nl = uint32_t(kt * BLOCK_N + 4 * half - lo) + vis_pad;
#pragma unroll
                for (int j = 0; j < 32; ++j)
                    if (uint32_t(32 * (j >> 4) + acc_row(j & 15, 0)) + nl > vis_w) ds[j] = 0.f;
            }
        }
        {
            f32x16_t g0, g1;
            tl.rows_times_frag(vs, gf, g0, g1);
#pragma unroll
            for (int j = 0; j < 32; ++j) ds[j] *= (j < 16 ? g0[j] : g1[j - 16]) - dd;
        }
        u32x4_t pk[4];
        pack4(ds, pk);
        // dQ^T += K^T dS^T
        tl.tile_t_times(ks, pk, acc);

        wait_vmem_all();
        __syncthreads();
        ent_cur = ent_next;
        ent_next_v = ent_next2_v;
    };

    if (ntiles > 0) {
        ent_cur = __builtin_amdgcn_readfirstlane(tiles[0]);
        issue_tile(ent_cur >> 1, 0);
        ent_next_v = tiles[min(1, ntiles - 1)];
    }
    wait_vmem_all();
    __syncthreads();
    for (int it = 0; it < ntiles; it += 2) {
        step(it, 0);
        if (it + 1 < ntiles) step(it + 1, 1);
    }
    if (row_ok) store_rowmajor<D>(p.dq + b * p.dq_sb + h * p.dq_sh + int64_t(row) * p.dq_sn, acc, p.scale, half);
}

// ---------------------------------------------------------------------------
// dK, dV.  One workgroup per (128-key block, KV head, b); wave w owns keys
// 32w .. 32w+31 of the block (lane column = key).  The stream is every
// listed 64-row query tile of every query head of the group; each stage
// holds the Q tile, the dO tile and the tile rows' base-2 LSE, D and
// visible-key interval (4 x 256 bytes).
// ---------------------------------------------------------------------------
template <int D, bool SOFTCAP>
__device__ __forceinline__ void bwd_dkdv_body(const BwdParams &p) {
    using C = FwdCfg<D>;
    constexpr int ROWDATA = 4 * BLOCK_N * 4;                // lse2, D, lo, hi of 64 rows
    constexpr int STAGE = 2 * C::TILE_BYTES + ROWDATA;
    lds_u8 *smem = (lds_u8 *)(smem_raw);
    const int tid = __builtin_amdgcn_workitem_id_x();
    const int bid = __builtin_amdgcn_workgroup_id_x();
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int col = lane & 31, half = lane >> 5;

    // Work assignment: the key blocks of one (b, KV head) share every Q and
    // dO tile, so they run on one XCD (workgroups are dispatched round-robin
    // over the 8 XCDs by id % 8, each XCD with its own L2) in ascending
    // block order, which is heaviest first under a causal mask.
    const int ngroups = p.B * p.Hkv;
    int group, kb;
    if ((ngroups & 7) == 0) {
        const int x = bid & 7, j = bid >> 3;
        group = x + 8 * (j / p.nkb);
        kb = j % p.nkb;
    } else {
        group = bid / p.nkb;
        kb = bid % p.nkb;
    }
    const int b = group / p.Hkv, hk = group % p.Hkv;
    const int G = p.Hq / p.Hkv;
    const int key = kb * BWD_KB + wave * 32 + col;
    const bool key_ok = key < p.N;

    bf16x8_t kf[C::KSTEPS], vf[C::KSTEPS];
    load_frag<D>(p.k + b * p.k_sb + hk * p.k_sh + int64_t(key) * p.k_sn, key_ok, half, kf);
    load_frag<D>(p.v + b * p.v_sb + hk * p.v_sh + int64_t(key) * p.v_sn, key_ok, half, vf);

    const int64_t item = int64_t(b) * p.nkb + kb;
    const int cnt = __builtin_amdgcn_readfirstlane(p.kv_count[item]);
    const int ntiles = cnt * G;
    const int32_t *qlist = p.kv_list + item * p.nqt64;
    uint32_t qoff[C::LOADS], goff[C::LOADS];
    dma_offsets<D>(p.q_sn, wave, lane, qoff);
    dma_offsets<D>(p.do_sn, wave, lane, goff);
    // tile it -> query head hk * G + it / cnt and list entry it % cnt
    auto head = [&](int it) { return hk * G + it / cnt; };
    auto issue_tile = [&](int it, int ent, int stage) {
        const int h = head(it), qt = ent >> 1, row0 = qt * BLOCK_N;
        lds_u8 *dst = smem + stage * STAGE;
        dma_tile<D>(p.q + b * p.q_sb + h * p.q_sh, p.q_sn, row0, p.N, qoff, dst, wave, lane);
        dma_tile<D>(p.dout + b * p.do_sb + h * p.do_sh, p.do_sn, row0, p.N, goff, dst + C::TILE_BYTES, wave, lane);
        // row data: wave w loads array w (4 bytes per row, rows past N clamped)
        const int r = min(row0 + lane, p.N - 1);
        const int64_t rr = (int64_t(b) * p.Hq + h) * p.N + r;
        const void *src = wave == 0 ? (const void *)(p.lse2 + rr)
                        : wave == 1 ? (const void *)(p.dvec + rr)
                        : wave == 2 ? (const void *)(p.mask.lo + int64_t(b) * p.N + r)
                                    : (const void *)(p.mask.hi + int64_t(b) * p.N + r);
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, off"
                     :
                     : "s"(lds_addr(dst + 2 * C::TILE_BYTES + wave * 256)), "v"(src)
                     : "memory", "m0");
    };
    BwdTile<D, dkdv_ahead<D>(), D == 128> tl;
    tl.init(col, half, lane);

    f32x16_t adk[C::DBLK], adv[C::DBLK];
#pragma unroll
    for (int i = 0; i < C::DBLK; ++i) {
        adk[i] = f32x16_t{};
        adv[i] = f32x16_t{};
    }

    // List entries are read one step before they are needed: the entry of
    // tile it+1 was loaded during step it-1 and has arrived by that step's
    // end-of-step wait, so no entry read is ever waited on alone (with one
    // wave per SIMD nothing else would hide that latency).
    int ent_cur = 0, ent_next_v = 0;
    auto step = [&](int it, const int stage) {
        const int ent = ent_cur;
        const int row0 = (ent >> 1) * BLOCK_N;
        const bool partial = ent & TILE_PARTIAL;
        const int ent_next = __builtin_amdgcn_readfirstlane(ent_next_v);
        const int ent_next2_v = qlist[min(it + 2, ntiles - 1) % cnt];
        if (it + 1 < ntiles) issue_tile(it + 1, ent_next, 1 - stage);
        const lds_u8 *qs = smem + stage * STAGE;
        const lds_u8 *gs = qs + C::TILE_BYTES;
        const lds_u8 *rowd = gs + C::TILE_BYTES;
        // per-register row data: rows 32kb + 8i + 4*half + {0..3}
        auto rowvec = [&](int arr, int kbk, int i) {
            return *reinterpret_cast<const __attribute__((address_space(3))) f32x4_t *>(
                rowd + arr * 256 + 4 * (32 * kbk + 8 * i + 4 * half));
        };
        auto rowvec_i = [&](int arr, int kbk, int i) {
            return *reinterpret_cast<const __attribute__((address_space(3))) i32x4_t *>(
                rowd + arr * 256 + 4 * (32 * kbk + 8 * i + 4 * half));
        };

        // S = Q K^T (lane = key, registers = query rows), then dP = dO V^T,
        // whose MFMAs run while the probabilities are formed
        f32x16_t s0, s1;
        tl.rows_times_frag(qs, kf, s0, s1);
        f32x16_t g0, g1;
        tl.rows_times_frag(gs, vf, g0, g1);
        float pr[32], fac[32];
#pragma unroll
        for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const f32x4_t l2 = rowvec(0, kbk, i);
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const int j = 16 * kbk + 4 * i + c;
                    const float s = kbk == 0 ? s0[4 * i + c] : s1[4 * i + c];
                    if constexpr (SOFTCAP) {
                        const float e = __builtin_amdgcn_exp2f(s * p.cap_inv_scale_2log2e);
                        const float tc = p.cap_log2 - p.cap_log2_2 * __builtin_amdgcn_rcpf(e + 1.f);
                        const float r = tc * p.inv_cap_log2;
                        fac[j] = 1.f - r * r;
                        pr[j] = __builtin_amdgcn_exp2f(tc - l2[c]);
                    } else {
                        fac[j] = 1.f;
                        pr[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(s, p.scale_log2, -l2[c]));
                    }
                }
            }
        if (partial) {
#pragma unroll
            for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const i32x4_t lov = rowvec_i(2, kbk, i), hiv = rowvec_i(3, kbk, i);
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const int j = 16 * kbk + 4 * i + c;
                        const int rq = row0 + 32 * kbk + 8 * i + 4 * half + c;
                        const int lo = lov[c], hi = hiv[c];
                        if (rq >= p.N || key < lo || key > hi) pr[j] = 0.f;
                    }
                }
        }
        // dV^T += dO^T P
        u32x4_t pk[4];
        pack4(pr, pk);
        tl.tile_t_times(gs, pk, adv);
        // dS = P (dP - D) * cap factor
        float ds[32];
#pragma unroll
        for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const f32x4_t dv = rowvec(1, kbk, i);
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const int j = 16 * kbk + 4 * i + c;
                    const float dp = kbk == 0 ? g0[4 * i + c] : g1[4 * i + c];
                    ds[j] = pr[j] * (dp - dv[c]) * fac[j];
                }
            }
        // dK^T += Q^T dS
        pack4(ds, pk);
        tl.tile_t_times(qs, pk, adk);

        wait_vmem_all();
        __syncthreads();
        ent_cur = ent_next;
        ent_next_v = ent_next2_v;
    };

    if (ntiles > 0) {
        ent_cur = __builtin_amdgcn_readfirstlane(qlist[0]);
        issue_tile(0, ent_cur, 0);
        ent_next_v = qlist[min(1, ntiles - 1) % cnt];
    }
    wait_vmem_all();
    __syncthreads();
    for (int it = 0; it < ntiles; it += 2) {
        step(it, 0);
        if (it + 1 < ntiles) step(it + 1, 1);
    }
    if (key_ok) {
        store_rowmajor<D>(p.dk + b * p.dk_sb + hk * p.dk_sh + int64_t(key) * p.dk_sn, adk, p.scale, half);
        store_rowmajor<D>(p.dv + b * p.dv_sb + hk * p.dv_sh + int64_t(key) * p.dv_sn, adv, 1.f, half);
    }
}

// Register budgets: the dQ kernel keeps Q and dO fragments and a d x 32
// accumulator per wave; two waves per SIMD fit except with the soft cap at
// d = 128.  At d = 128 without the cap, separate K and V DMA offsets leave
// a few registers to spill, and each reload waits (vmcnt) on the tile DMAs
// already in flight; with equal K and V token strides the offsets are
// shared and nothing spills.  The dK/dV kernel keeps K and V fragments and
// two accumulators: one wave per SIMD, accumulators in AGPRs.
#define EXATTN_BWD_KERNELS(SUFFIX, D, SOFTCAP, DQ_WAVES)                                                     \
    __global__ __launch_bounds__(256, DQ_WAVES) void k_bwd_dq_##SUFFIX(BwdParams p) {                        \
        bwd_dq_body<D, SOFTCAP, false>(p);                                                                   \
    }                                                                                                          \
    __global__ __launch_bounds__(256, DQ_WAVES) void k_bwd_dq_same_##SUFFIX(BwdParams p) {                   \
        bwd_dq_body<D, SOFTCAP, true>(p);                                                                    \
    }                                                                                                          \
    __global__ __launch_bounds__(256, 1) void k_bwd_dkdv_##SUFFIX(BwdParams p) { bwd_dkdv_body<D, SOFTCAP>(p); }
EXATTN_BWD_KERNELS(d128, 128, false, 2)
EXATTN_BWD_KERNELS(d128_softcap, 128, true, 1)
EXATTN_BWD_KERNELS(d64, 64, false, 2)
EXATTN_BWD_KERNELS(d64_softcap, 64, true, 2)
#undef EXATTN_BWD_KERNELS

static hipError_t launch_with_lds(void (*kernel)(BwdParams), int64_t nblocks, size_t lds, const BwdParams &p,
                                  hipStream_t stream) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kernel, dim3(unsigned(nblocks)), dim3(256), lds, stream, p);
    return hipGetLastError();
}

template <int D>
static hipError_t launch_bwd_d(const BwdParams &p, bool softcap, hipStream_t stream) {
    using C = FwdCfg<D>;
    hipError_t e;
    void (*dq)(BwdParams);
    void (*dkdv)(BwdParams);
    const bool same = p.k_sn == p.v_sn; // K and V DMAs can share their offsets
    if constexpr (D == 128) {
        dq = softcap ? (same ? k_bwd_dq_same_d128_softcap : k_bwd_dq_d128_softcap)
                     : (same ? k_bwd_dq_same_d128 : k_bwd_dq_d128);
        dkdv = softcap ? k_bwd_dkdv_d128_softcap : k_bwd_dkdv_d128;
    } else {
        dq = softcap ? (same ? k_bwd_dq_same_d64_softcap : k_bwd_dq_d64_softcap)
                     : (same ? k_bwd_dq_same_d64 : k_bwd_dq_d64);
        dkdv = softcap ? k_bwd_dkdv_d64_softcap : k_bwd_dkdv_d64;
    }
    e = launch_with_lds(dq, int64_t(p.B) * p.nqt * p.Hq, C::LDS_BYTES, p, stream);
    if (e != hipSuccess) return e;
    const size_t lds_kv = 2 * (2 * size_t(C::TILE_BYTES) + 4 * BLOCK_N * 4);
    return launch_with_lds(dkdv, int64_t(p.B) * p.Hkv * p.nkb, lds_kv, p, stream);
}

hipError_t launch_bwd(const BwdParams &p, int d, bool softcap, uint32_t flags, const MaskLayout &L,
                      const BwdMaskLayout &BL, void *kv_mask, hipStream_t stream) {
    char *base = static_cast<char *>(kv_mask);
    hipLaunchKernelGGL(k_bwd_mask_kv, dim3(BL.nkb, L.B), dim3(256), 0, stream, L.N, BL.nkb, BL.nqt64, flags,
                       p.mask.lo, p.mask.hi, reinterpret_cast<int32_t *>(base + BL.off_count),
                       reinterpret_cast<int32_t *>(base + BL.off_list));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return d == 128 ? launch_bwd_d<128>(p, softcap, stream) : launch_bwd_d<64>(p, softcap, stream);
}

} // namespace exattn
