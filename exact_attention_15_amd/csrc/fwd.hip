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
// MFMA formulation.  Scores are computed transposed, S^T = K Q^T, with
// v_mfma_f32_32x32x16_bf16: K rows are the A operand (read from LDS), the
// wave's 32 query rows are the B operand (held in registers for the whole
// kernel).  In the 32x32 accumulator, lane l holds column l%32 -- one query
// -- and 16 keys, so a row's max and sum need only an in-lane reduction and
// one exchange between the two 32-lane halves.  The output is accumulated
// transposed too, O^T = V^T P^T: the probabilities already sit in the B
// operand layout (lane = query, register = key), and V^T is the A operand,
// read from a transposed copy of the V tile in LDS.
//
// Scores are kept in base-2 units (scale * log2 e folded in), so every
// exponential is one v_exp_f32.
#include "common.h"

namespace exattn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

template <int D> struct FwdCfg {
    static constexpr int KSTEPS = D / 16;            // k-steps of the S^T MFMAs
    static constexpr int DBLK = D / 32;              // 32-row blocks of O^T
    static constexpr int K_ROW = D + 8;              // K tile row stride in LDS (elements)
    static constexpr int VT_ROW = BLOCK_N + 4;       // V^T tile row stride in LDS (elements)
    static constexpr int K_ELEMS = BLOCK_N * K_ROW;
    static constexpr int VT_ELEMS = D * VT_ROW;
    static constexpr int STAGE = K_ELEMS + VT_ELEMS; // one buffer, elements
    static constexpr int CHUNKS = D / 8;             // 16-byte chunks per row
    static constexpr int K_LOADS = BLOCK_N * CHUNKS / 256;       // per thread
    static constexpr int V_ITEMS = (BLOCK_N / 2) * CHUNKS / 256; // row pairs per thread
    static constexpr size_t LDS_BYTES = size_t(2) * STAGE * 2;
};

// 32x32 accumulator layout of v_mfma_f32_32x32x16_bf16: register r of lane l
// holds row 8*(r/4) + 4*(l/32) + r%4 and column l%32.
__device__ __forceinline__ int acc_row(int r, int half) { return 8 * (r >> 2) + 4 * half + (r & 3); }

__device__ __forceinline__ float wave_swap_halves(float x) {
    // Value of lane l^32 (the other 32-lane half of the wave).
    return __shfl_xor(x, 32);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    // Round-to-nearest-even to bf16 (v_cvt_pk_bf16_f32).
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    bf16x2_t v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}

template <int D, bool SOFTCAP>
__global__ __launch_bounds__(256, 2) void k_attn_fwd(FwdParams p) {
    using C = FwdCfg<D>;
    extern __shared__ __attribute__((aligned(16))) uint16_t smem[];

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int col = lane & 31, half = lane >> 5;

    const int item = p.mask.order[blockIdx.x / p.Hq];
    const int h = blockIdx.x % p.Hq;
    const int b = item / p.nqt, qt = item % p.nqt;
    const int hk = h / (p.Hq / p.Hkv);
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

    const int ntiles = p.mask.count[item];
    const int32_t *tiles = p.mask.list + int64_t(item) * p.nkt;
    const uint16_t *kbase = p.k + b * p.k_sb + hk * p.k_sh;
    const uint16_t *vbase = p.v + b * p.v_sb + hk * p.v_sh;

    f32x16_t acc_o[C::DBLK];
#pragma unroll
    for (int i = 0; i < C::DBLK; ++i) acc_o[i] = f32x16_t{};
    float m_run = -INFINITY; // running max (base-2 units), shared by both halves
    float l_run = 0.f;       // this half's share of the running sum

    // Register staging of the next tile.
    u32x4_t kreg[C::K_LOADS];
    u32x4_t vreg[C::V_ITEMS][2];

    auto gload = [&](int kt) {
        const int key0 = kt * BLOCK_N;
#pragma unroll
        for (int u = 0; u < C::K_LOADS; ++u) {
            const int ci = tid + 256 * u;
            const int key = ci / C::CHUNKS, c = ci % C::CHUNKS;
            const int gk = key0 + key;
            u32x4_t x = {0u, 0u, 0u, 0u};
            if (gk < p.N) x = *reinterpret_cast<const u32x4_t *>(kbase + int64_t(gk) * p.k_sn + 8 * c);
            kreg[u] = x;
        }
#pragma unroll
        for (int u = 0; u < C::V_ITEMS; ++u) {
            const int it = tid + 256 * u;
            const int pr = it % (BLOCK_N / 2), c = it / (BLOCK_N / 2);
            const int gk = key0 + 2 * pr;
            u32x4_t x0 = {0u, 0u, 0u, 0u}, x1 = {0u, 0u, 0u, 0u};
            if (gk < p.N) x0 = *reinterpret_cast<const u32x4_t *>(vbase + int64_t(gk) * p.v_sn + 8 * c);
            if (gk + 1 < p.N) x1 = *reinterpret_cast<const u32x4_t *>(vbase + int64_t(gk + 1) * p.v_sn + 8 * c);
            vreg[u][0] = x0;
            vreg[u][1] = x1;
        }
    };
    auto swrite = [&](int stage) {
        uint16_t *ks = smem + stage * C::STAGE;
        uint16_t *vts = ks + C::K_ELEMS;
#pragma unroll
        for (int u = 0; u < C::K_LOADS; ++u) {
            const int ci = tid + 256 * u;
            const int key = ci / C::CHUNKS, c = ci % C::CHUNKS;
            *reinterpret_cast<u32x4_t *>(ks + key * C::K_ROW + 8 * c) = kreg[u];
        }
        // V^T[d][key]: pair keys (2pr, 2pr+1) of the same d into one dword.
#pragma unroll
        for (int u = 0; u < C::V_ITEMS; ++u) {
            const int it = tid + 256 * u;
            const int pr = it % (BLOCK_N / 2), c = it / (BLOCK_N / 2);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint32_t a = vreg[u][0][j >> 1], bb = vreg[u][1][j >> 1];
                const uint32_t w = (j & 1) ? ((a >> 16) | (bb & 0xFFFF0000u))
                                           : ((a & 0xFFFFu) | (bb << 16));
                *reinterpret_cast<uint32_t *>(vts + (8 * c + j) * C::VT_ROW + 2 * pr) = w;
            }
        }
    };

    if (ntiles > 0) {
        gload(tiles[0] >> 1);
        swrite(0);
    }
    __syncthreads();

    for (int it = 0; it < ntiles; ++it) {
        const int ent = tiles[it];
        const int kt = ent >> 1;
        const bool partial = ent & TILE_PARTIAL;
        if (it + 1 < ntiles) gload(tiles[it + 1] >> 1);

        const uint16_t *ks = smem + (it & 1) * C::STAGE;
        const uint16_t *vts = ks + C::K_ELEMS;

        // ---- S^T = K Q^T for the tile's two 32-key blocks ----
        f32x16_t s0 = f32x16_t{}, s1 = f32x16_t{};
#pragma unroll
        for (int s = 0; s < C::KSTEPS; ++s) {
            const bf16x8_t a0 = *reinterpret_cast<const bf16x8_t *>(ks + col * C::K_ROW + 16 * s + 8 * half);
            const bf16x8_t a1 = *reinterpret_cast<const bf16x8_t *>(ks + (32 + col) * C::K_ROW + 16 * s + 8 * half);
            s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[s], s0, 0, 0, 0);
            s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[s], s1, 0, 0, 0);
        }

        // ---- score_mod and mask in registers ----
        float t[32];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            t[r] = s0[r];
            t[16 + r] = s1[r];
        }
#pragma unroll
        for (int j = 0; j < 32; ++j) {
            if constexpr (SOFTCAP) {
                // c * tanh(scale * s / c) with tanh(x) = 1 - 2 / (exp(2x) + 1),
                // then to base-2 units.
                const float e = __builtin_amdgcn_exp2f(t[j] * (p.cap_inv_scale * 2.f * LOG2E));
                const float th = 1.f - 2.f * __builtin_amdgcn_rcpf(e + 1.f);
                t[j] = th * p.cap_log2;
            } else {
                t[j] *= p.scale_log2;
            }
        }
        if (partial) {
            const int kb0 = kt * BLOCK_N;
#pragma unroll
            for (int j = 0; j < 32; ++j) {
                const int key = kb0 + 32 * (j >> 4) + acc_row(j & 15, half);
                if (key < lo || key > hi) t[j] = -INFINITY;
            }
        }

        // ---- online softmax ----
        float mt = t[0];
#pragma unroll
        for (int j = 1; j < 32; ++j) mt = fmaxf(mt, t[j]);
        mt = fmaxf(mt, wave_swap_halves(mt));
        const float m_new = fmaxf(m_run, mt);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
        m_run = m_new;
        float psum = 0.f;
#pragma unroll
        for (int j = 0; j < 32; ++j) {
            t[j] = __builtin_amdgcn_exp2f(t[j] - m_use);
            psum += t[j];
        }
        l_run = l_run * alpha + psum;
#pragma unroll
        for (int i = 0; i < C::DBLK; ++i) acc_o[i] *= alpha;

        // ---- O^T += V^T P^T ----
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const int base = 16 * kb + 8 * hh;
                u32x4_t pk;
                pk[0] = pack_bf16x2(t[base + 0], t[base + 1]);
                pk[1] = pack_bf16x2(t[base + 2], t[base + 3]);
                pk[2] = pack_bf16x2(t[base + 4], t[base + 5]);
                pk[3] = pack_bf16x2(t[base + 6], t[base + 7]);
                const bf16x8_t pb = __builtin_bit_cast(bf16x8_t, pk);
                // Keys of these 8 probabilities: key0 + {0..3} and key0 + 8 + {0..3}.
                const int key0 = 32 * kb + 16 * hh + 4 * half;
#pragma unroll
                for (int db = 0; db < C::DBLK; ++db) {
                    const uint16_t *vp = vts + (32 * db + col) * C::VT_ROW + key0;
                    const u32x2_t lo4 = *reinterpret_cast<const u32x2_t *>(vp);
                    const u32x2_t hi4 = *reinterpret_cast<const u32x2_t *>(vp + 8);
                    const u32x4_t av = {lo4[0], lo4[1], hi4[0], hi4[1]};
                    acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(bf16x8_t, av), pb, acc_o[db], 0, 0, 0);
                }
            }
        }

        if (it + 1 < ntiles) swrite((it + 1) & 1);
        __syncthreads();
    }

    // ---- epilogue: O / l, LSE = ln 2 * (m + log2 l) ----
    const float l_tot = l_run + wave_swap_halves(l_run);
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

template <int D, bool SOFTCAP> static hipError_t launch_fwd_t(const FwdParams &p, hipStream_t stream) {
    using C = FwdCfg<D>;
    // More than 64 KiB of dynamic LDS must be allowed explicitly (per device).
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_attn_fwd<D, SOFTCAP>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       int(C::LDS_BYTES));
    if (e != hipSuccess) return e;
    const int64_t nblocks = int64_t(p.B) * p.nqt * p.Hq;
    hipLaunchKernelGGL((k_attn_fwd<D, SOFTCAP>), dim3(unsigned(nblocks)), dim3(256), C::LDS_BYTES,
                       stream, p);
    return hipGetLastError();
}

hipError_t launch_fwd(const FwdParams &p, int d, bool softcap, hipStream_t stream) {
    if (d == 128) return softcap ? launch_fwd_t<128, true>(p, stream) : launch_fwd_t<128, false>(p, stream);
    return softcap ? launch_fwd_t<64, true>(p, stream) : launch_fwd_t<64, false>(p, stream);
}

} // namespace exattn
