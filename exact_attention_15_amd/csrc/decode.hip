// Split-KV decode for gfx950: one new query per (batch row, query head)
// against the first lens[b] keys of a KV cache.
//
// A single query row gives too little parallelism if each (b, head) is one
// workgroup, so the valid keys are cut into chunks and every
// (b, KV head, chunk) becomes a workgroup that computes a partial softmax --
// local max m_c, local sum l_c and the unnormalised output -- for all query
// heads of the GQA group at once, so the group's K/V bytes are read once.  A
// second kernel merges the partials of each (b, query head) by rescaling
// them with exp(m_c - max m) (aegloslab "3.7 어텐션 II", sections 3.7.4 and
// 3.7.5).
//
// The split kernel is bound by HBM: K and V of the chunk are streamed once
// with 16-byte loads.  Each wave owns a slice of the chunk (128 keys) and
// streams it on its own (no workgroup barrier until the final merge): first
// K, with several 16-key groups in flight, scoring the group's queries with
// bf16 MFMA (v_mfma_f32_16x16x32_bf16: queries as the A operand, 16 keys as
// the B operand); then the slice's softmax; then V, whose first loads are
// already in flight, accumulating P.V in fp32 on the vector ALU.  The wave
// partials are merged through LDS at the end.
#include "common.h"

namespace exattn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr float LN2_D = 0.6931471805599453f;
constexpr int MAX_CHUNK = 2048;
constexpr int K_AHEAD = 4; // 16-key K groups in flight per wave
constexpr int V_PAIRS = 4; // V row pairs (two 16-byte loads each) in flight per lane


__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
    return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
    return x;
}

// Work items are the valid (b, KV head, chunk) triples, enumerated batch row
// by batch row, chunk fastest.  Workgroup i takes item i, so the valid items
// occupy the first workgroup ids.  Consecutive ids go to different XCDs
// (round-robin dispatch), so each XCD gets an equal share of the KV bytes
// whatever the mix of lengths; a grid indexed directly by (chunk, head, b)
// would give the low XCDs up to one extra chunk per (b, head).  Returns false
// for the ids past the last item.  Wave-uniform; lens is scanned 64 rows at a
// time with a wave prefix sum, which also gives the row's length.
__device__ __forceinline__ bool decode_item(const DecodeParams &p, int &b, int &g, int &c, int &len_b) {
    int i = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
    const int lane = threadIdx.x & 63;
    for (int b0 = 0; b0 < p.B; b0 += 64) {
        const int bb = b0 + lane;
        int nc = 0, len = 0;
        if (bb < p.B) {
            len = p.lens[bb];
            len = len < 0 ? 0 : (len > p.T ? p.T : len);
            nc = (len + p.chunk - 1) / p.chunk;
        }
        const int items = nc * p.Hkv;
        int incl = items;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int t = __shfl_up(incl, o);
            if (lane >= o) incl += t;
        }
        const int total = __shfl(incl, 63);
        if (i < total) {
            const int l = __ffsll((unsigned long long)__ballot(incl > i)) - 1;
            const int j = i - __shfl(incl - items, l);
            const int ncl = __shfl(nc, l);
            b = __builtin_amdgcn_readfirstlane(b0 + l);
            g = __builtin_amdgcn_readfirstlane(j / ncl);
            c = __builtin_amdgcn_readfirstlane(j % ncl);
            len_b = __builtin_amdgcn_readfirstlane(__shfl(len, l)); // clamped into [0, T]
            return true;
        }
        i -= total;
    }
    return false;
}

// G: query heads per KV head, rounded up to a supported size (<= 16).
// Scores live in LDS per wave, key-major: sc[key * GP + q], GP = max(G, 4).
// Up to G = 4 a workgroup has up to 8 waves (two per SIMD).  From G = 8
// the G x 8 fp32 accumulators per lane raise the register count (G = 8: 155
// VGPRs, three waves per SIMD; G = 16: the whole register file), and a
// workgroup has at most 4 waves, one per SIMD, so that as many workgroups as
// the registers allow share a CU (an 8-wave workgroup at G = 8 left one CU
// with a single workgroup).
template <int G> constexpr int decode_max_waves() { return G > 4 ? 4 : 8; }
template <int D, int G>
__global__ __launch_bounds__(64 * decode_max_waves<G>()) void k_decode_split(DecodeParams p, int group) {
    constexpr int GP = G < 4 ? 4 : G;
    constexpr int KS = D / 32;   // k-steps of the 16x16x32 score MFMA
    constexpr int CH = D / 8;    // 16-byte chunks per row
    constexpr int KPI = 64 / CH; // keys covered by one wave-wide V load
    constexpr int KP = 2 * KPI;  // keys per V iteration (each lane takes a pair)
    extern __shared__ __attribute__((aligned(16))) float sm[];

    int b, g, c, len;
    if (!decode_item(p, b, g, c, len)) return;
    const int k0 = c * p.chunk;
    const int nk = min(p.chunk, len - k0);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nwaves = blockDim.x >> 6;
    const int cw = p.chunk / nwaves;                    // keys per wave slice (multiple of 16)
    const int wk0 = wave * cw;                          // slice start inside the chunk
    const int nkw = max(0, min(cw, nk - wk0));          // keys in this wave's slice
    float *sc = sm + size_t(wave) * cw * GP;            // this wave's scores
    const uint16_t *kbase = p.k + b * p.k_sb + g * p.k_sh + int64_t(k0 + wk0) * p.k_sn;
    const uint16_t *vbase = p.v + b * p.v_sb + g * p.v_sh + int64_t(k0 + wk0) * p.v_sn;

    // Both streams keep their loads unconditional (rows past the slice are
    // clamped to its last key and their results discarded) and their trip
    // counts padded to the prefetch depth, so the loop bodies have a single
    // path and the compiler can count loads in flight instead of draining.
    float m_w[G], l_w[G];
    float acc[G][8];
#pragma unroll
    for (int q = 0; q < G; ++q) {
        m_w[q] = -INFINITY;
        l_w[q] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[q][e] = 0.f;
    }
    const int dc = lane % CH, ksub = lane / CH;
    if (nkw > 0) {
        // ---- pass 1: scores S = Q K^T, 16 keys per MFMA group ----
        // A operand: lane l holds query row l%16 (zero beyond the group), and
        // for k-step s the 8 elements [32s + 8(l/16), +8).  B operand: lane l
        // holds key l%16 of the 16-key group with the same element ranges, so
        // each load instruction reads 64 contiguous bytes of each of 16 rows.
        const int r16 = lane & 15, g4 = lane >> 4;
        bf16x8_t qa[KS];
        {
            const bool ok = r16 < group;
            const uint16_t *qrow = p.q + b * p.q_sb + int64_t(g * group + (ok ? r16 : 0)) * p.q_sh;
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                const u32x4_t x = *reinterpret_cast<const u32x4_t *>(qrow + 32 * s + 8 * g4);
                qa[s] = ok ? __builtin_bit_cast(bf16x8_t, x) : bf16x8_t{};
            }
        }
        auto kload = [&](int grp, u32x4_t *dst) {
            const int key = min(grp * 16 + r16, nkw - 1);
            const uint16_t *src = kbase + int64_t(key) * p.k_sn + 8 * g4;
#pragma unroll
            for (int s = 0; s < KS; ++s) dst[s] = *reinterpret_cast<const u32x4_t *>(src + 32 * s);
        };
        const int ngroups = (nkw + 15) >> 4;
        const int ngroups_pad = (ngroups + K_AHEAD - 1) / K_AHEAD * K_AHEAD;
        u32x4_t kb[K_AHEAD][KS];
        // Issue the prologue in group order (the loop waits for the oldest
        // group only, which requires it to be the first one issued).
#pragma unroll
        for (int i = 0; i < K_AHEAD; ++i) {
            kload(i, kb[i]);
            __builtin_amdgcn_sched_barrier(0);
        }
        for (int grp0 = 0; grp0 < ngroups_pad; grp0 += K_AHEAD) {
#pragma unroll
            for (int i = 0; i < K_AHEAD; ++i) {
                const int grp = grp0 + i;
                f32x4_t sacc = f32x4_t{};
#pragma unroll
                for (int s = 0; s < KS; ++s)
                    sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[s], __builtin_bit_cast(bf16x8_t, kb[i][s]),
                                                                    sacc, 0, 0, 0);
                // refill this buffer with the group K_AHEAD further on
                kload(grp + K_AHEAD, kb[i]);
                // Lane l holds rows (queries) 4*(l/16)+r of column (key) l%16.
                const int key = grp * 16 + r16;
                if (key < nkw && 4 * g4 < GP)
                    *reinterpret_cast<f32x4_t *>(sc + key * GP + 4 * g4) = sacc * p.scale_log2;
            }
        }

        // Start the V stream before the softmax so its latency overlaps it.
        // Lane l covers d-chunk l%CH of the key pair 2*(l/CH) + KP*it and
        // the key after it (KP keys per wave per iteration, two row loads).
        // Rows are addressed with 32-bit byte offsets from the slice base:
        // key < 2048 and the token stride is below 2^20 elements.
        const uint8_t *vb8 = reinterpret_cast<const uint8_t *>(vbase);
        const uint32_t vrow = 2u * uint32_t(p.v_sn), vcol = 16u * uint32_t(dc);
        auto vload2 = [&](int it, u32x4_t &xa, u32x4_t &xb) {
            const int ka = 2 * ksub + KP * it;
            xa = *reinterpret_cast<const u32x4_t *>(vb8 + (__umul24(uint32_t(min(ka, nkw - 1)), vrow) + vcol));
            xb = *reinterpret_cast<const u32x4_t *>(vb8 + (__umul24(uint32_t(min(ka + 1, nkw - 1)), vrow) + vcol));
        };
        u32x4_t va[V_PAIRS], vb[V_PAIRS];
#pragma unroll
        for (int i = 0; i < V_PAIRS; ++i) {
            vload2(i, va[i], vb[i]);
            __builtin_amdgcn_sched_barrier(0);
        }

        // ---- slice softmax: per query, max and exp over the wave's keys ----
        // (wave-private LDS, so only the wave's own ordering matters)
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
#pragma unroll
        for (int q = 0; q < G; ++q) {
            float m = -INFINITY;
            for (int j = lane; j < nkw; j += 64) m = fmaxf(m, sc[j * GP + q]);
            m_w[q] = wave_max(m);
        }
#pragma unroll
        for (int q = 0; q < G; ++q) {
            float l = 0.f;
            for (int j = lane; j < nkw; j += 64) {
                const float e = __builtin_amdgcn_exp2f(sc[j * GP + q] - m_w[q]);
                sc[j * GP + q] = e;
                l += e;
            }
            l_w[q] = wave_sum(l);
        }
        // Zero the probabilities of the padding keys the V loop runs over,
        // [nkw, round up to KP * V_PAIRS), which stay inside the slice (its
        // length is a multiple of that), so the loop needs no key checks.
        const int nkw_pad = (nkw + KP * V_PAIRS - 1) / (KP * V_PAIRS) * (KP * V_PAIRS);
        for (int j = nkw + lane; j < nkw_pad; j += 64)
#pragma unroll
            for (int q = 0; q < GP; ++q) sc[j * GP + q] = 0.f;
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");

        // ---- pass 2: partial O = P V on the vector ALU, two keys at a time ----
        // The two rows are interleaved into bf16 pairs (V[ka][e], V[kb][e])
        // with v_perm and dotted with the matching probability pair (P
        // rounded to bf16, as the P V product of the forward pass uses it)
        // by v_dot2_f32_bf16, which accumulates in fp32.
        const int nit = nkw_pad / KP;
        for (int it0 = 0; it0 < nit; it0 += V_PAIRS) {
#pragma unroll
            for (int i = 0; i < V_PAIRS; ++i) {
                const int it = it0 + i;
                const int ka = 2 * ksub + KP * it;
                // Interleave first, so that the row registers are free when
                // the refill loads (V_PAIRS pairs ahead) are issued into them.
                bf16x2_t vp[8];
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    vp[2 * w] = __builtin_bit_cast(bf16x2_t, __builtin_amdgcn_perm(vb[i][w], va[i][w], 0x05040100u));
                    vp[2 * w + 1] = __builtin_bit_cast(bf16x2_t, __builtin_amdgcn_perm(vb[i][w], va[i][w], 0x07060302u));
                }
                __builtin_amdgcn_sched_barrier(0);
                vload2(it + V_PAIRS, va[i], vb[i]);
#pragma unroll
                for (int q4 = 0; q4 < GP; q4 += 4) {
                    const f32x4_t pa = *reinterpret_cast<const f32x4_t *>(sc + ka * GP + q4);
                    const f32x4_t pb = *reinterpret_cast<const f32x4_t *>(sc + (ka + 1) * GP + q4);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        if (q4 + r < G) {
                            const bf16x2_t pp = {(__bf16)pa[r], (__bf16)pb[r]};
#pragma unroll
                            for (int e = 0; e < 8; ++e)
                                acc[q4 + r][e] = __builtin_amdgcn_fdot2_f32_bf16(vp[e], pp, acc[q4 + r][e], false);
                        }
                    }
                }
            }
        }
    }
    // Reduce over the lanes that share a d-chunk (equal dc).
#pragma unroll
    for (int o = CH; o < 64; o <<= 1)
#pragma unroll
        for (int q = 0; q < G; ++q)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[q][e] += __shfl_xor(acc[q][e], o);

    // ---- merge the wave partials (LDS reused after the barrier) ----
    __syncthreads();
    float *red = sm;                       // [nwaves][G][D]
    float *wm = sm + nwaves * G * D;       // [nwaves][G]
    float *wl = wm + nwaves * G;           // [nwaves][G]
    if (ksub == 0) {
#pragma unroll
        for (int q = 0; q < G; ++q)
#pragma unroll
            for (int e = 0; e < 8; ++e) red[(wave * G + q) * D + 8 * dc + e] = acc[q][e];
    }
    if (lane < G) {
#pragma unroll
        for (int q = 0; q < G; ++q)
            if (lane == q) {
                wm[wave * G + q] = m_w[q];
                wl[wave * G + q] = l_w[q];
            }
    }
    __syncthreads();
    const int64_t part_base = (int64_t(b) * p.Hq + int64_t(g) * group) * p.nchunk + c;
    for (int i = tid; i < group * D; i += blockDim.x) {
        const int q = i / D, d = i % D;
        float M = -INFINITY;
        for (int w = 0; w < nwaves; ++w) M = fmaxf(M, wm[w * G + q]);
        float o = 0.f;
        for (int w = 0; w < nwaves; ++w) {
            const float mw = wm[w * G + q];
            if (mw != -INFINITY) o += __builtin_amdgcn_exp2f(mw - M) * red[(w * G + q) * D + d];
        }
        p.part_o[(part_base + int64_t(q) * p.nchunk) * D + d] = o;
        if (d == 0) {
            float L = 0.f;
            for (int w = 0; w < nwaves; ++w) {
                const float mw = wm[w * G + q];
                if (mw != -INFINITY) L += __builtin_amdgcn_exp2f(mw - M) * wl[w * G + q];
            }
            p.part_m[part_base + int64_t(q) * p.nchunk] = M;
            p.part_l[part_base + int64_t(q) * p.nchunk] = L;
        }
    }
}

// One workgroup of D threads per (query head, b): merge the chunk partials.
// The chunks are taken in batches of COMBINE_BATCH.  Every thread issues the
// loads of its output element for the whole batch at once (rows past the
// last chunk are clamped and weighted 0) while the first wave loads the
// batch's maxima and sums, one chunk per lane, reduces them and leaves the
// chunk weights exp(m_c - M) in LDS; the running max / sum / output are
// rescaled once per batch, so a (b, head) with up to COMBINE_BATCH chunks
// costs one round trip to memory and each thread makes COMBINE_BATCH loads.
constexpr int COMBINE_BATCH = 32;
template <int D>
__global__ __launch_bounds__(D) void k_decode_combine(DecodeParams p) {
    __shared__ float w_sh[COMBINE_BATCH];
    __shared__ float stat_sh[2]; // the batch's new running max and weighted sum
    const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x, lane = d & 63;
    int len = p.lens[b];
    len = len < 0 ? 0 : (len > p.T ? p.T : len);
    const int nch = (len + p.chunk - 1) / p.chunk;
    const int64_t base = (int64_t(b) * p.Hq + h) * p.nchunk;
    uint16_t *orow = p.o + b * p.o_sb + h * p.o_sh;
    float M = -INFINITY, L = 0.f, acc = 0.f;
    for (int c0 = 0; c0 < nch; c0 += COMBINE_BATCH) {
        float ov[COMBINE_BATCH];
#pragma unroll
        for (int j = 0; j < COMBINE_BATCH; ++j) ov[j] = p.part_o[(base + min(c0 + j, nch - 1)) * D + d];
        if (d < 64) {
            const bool ok = lane < COMBINE_BATCH && c0 + lane < nch;
            const int cc = ok ? c0 + lane : 0;
            const float mv = ok ? p.part_m[base + cc] : -INFINITY;
            const float lv = ok ? p.part_l[base + cc] : 0.f;
            // a chunk holds at least one key, so its max is finite unless
            // scores overflowed
            const float Mb = fmaxf(M, wave_max(mv));
            const float w = ok ? __builtin_amdgcn_exp2f(mv - Mb) : 0.f;
            if (lane < COMBINE_BATCH) w_sh[lane] = w;
            const float Lb = wave_sum(w * lv);
            if (lane == 0) {
                stat_sh[0] = Mb;
                stat_sh[1] = Lb;
            }
        }
        __syncthreads();
        const float Mb = stat_sh[0];
        const float r = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - Mb);
        L = __builtin_fmaf(L, r, stat_sh[1]);
        acc *= r;
#pragma unroll
        for (int j = 0; j < COMBINE_BATCH; ++j) acc = __builtin_fmaf(w_sh[j], ov[j], acc);
        M = Mb;
        __syncthreads(); // the next batch rewrites the weights
    }
    const float o = L > 0.f ? acc / L : 0.f;
    __bf16 ob = (__bf16)o;
    orow[d] = __builtin_bit_cast(uint16_t, ob);
    if (d == 0)
        p.lse[int64_t(b) * p.Hq + h] = L > 0.f ? (M + __builtin_amdgcn_logf(L)) * LN2_D : -INFINITY;
}

// Waves per split workgroup: about one per DECODE_WAVE_KEYS keys of the
// chunk, a power of two in [1, max_waves] that leaves a multiple of 64 keys
// per wave (chunk is a multiple of 64; the V loop pads a slice to 32 or 64
// keys).
constexpr int DECODE_WAVE_KEYS = 128;
static int decode_waves(int chunk, int max_waves) {
    int n = 1;
    while (n < max_waves && 2 * n * DECODE_WAVE_KEYS <= chunk) n *= 2;
    while ((chunk / 64) % n) n /= 2;
    return n;
}

template <int D, int G> static hipError_t launch_split(const DecodeParams &p, int group, hipStream_t stream) {
    constexpr int GP = G < 4 ? 4 : G;
    const int nwaves = decode_waves(p.chunk, decode_max_waves<G>());
    const size_t lds_scores = size_t(p.chunk) * GP * sizeof(float);
    const size_t lds_merge = (size_t(nwaves) * G * D + 2 * size_t(nwaves) * G) * sizeof(float);
    const size_t lds = lds_scores > lds_merge ? lds_scores : lds_merge;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_decode_split<D, G>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_decode_split<D, G>), dim3(p.nchunk, p.Hkv, p.B), dim3(64 * nwaves), lds, stream, p,
                       group);
    return hipGetLastError();
}

template <int D> static hipError_t launch_decode_d(const DecodeParams &p, hipStream_t stream) {
    const int group = p.Hq / p.Hkv;
    hipError_t e;
    if (group <= 1) e = launch_split<D, 1>(p, group, stream);
    else if (group <= 2) e = launch_split<D, 2>(p, group, stream);
    else if (group <= 4) e = launch_split<D, 4>(p, group, stream);
    else if (group <= 8) e = launch_split<D, 8>(p, group, stream);
    else e = launch_split<D, 16>(p, group, stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_decode_combine<D>), dim3(p.Hq, p.B), dim3(D), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_decode(const DecodeParams &p, int d, hipStream_t stream) {
    return d == 128 ? launch_decode_d<128>(p, stream) : launch_decode_d<64>(p, stream);
}

static_assert(MAX_CHUNK * 16 * 4 <= 160 * 1024, "decode scores must fit in LDS");
static_assert((8 * 16 * 128 + 2 * 8 * 16) * 4 <= 160 * 1024, "decode merge buffers must fit in LDS");

} // namespace exattn
