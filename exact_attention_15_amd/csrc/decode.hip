// Split-KV decode for gfx950: one new query per (batch row, query head)
// against the first lens[b] keys of a KV cache.
//
// A single query row gives too little parallelism if each (b, head) is one
// workgroup, so the valid keys are cut into chunks and every
// (b, KV head, chunk) becomes a workgroup that computes a partial online
// softmax -- local max m_c, local sum l_c and the unnormalised output -- for
// all query heads of the GQA group at once, so the group's K/V bytes are
// read once.  A second kernel merges the partials of each (b, query head) by
// rescaling them with exp(m_c - max m) (aegloslab "3.7 어텐션 II", sections
// 3.7.4 and 3.7.5).
//
// The split kernel is bound by HBM: K and V of the chunk are streamed once
// with 16-byte loads.  Scores use bf16 MFMA (v_mfma_f32_16x16x32_bf16, the
// group's queries as the A operand, 16 keys per instruction as the B
// operand), probabilities stay fp32, and P.V runs on the vector ALU with the
// V row chunk each lane loaded.
#include "common.h"

namespace exattn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr float LN2_D = 0.6931471805599453f;
constexpr int MAX_CHUNK = 2048;

__device__ __forceinline__ float bf16lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

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

// G: query heads per KV head, rounded up to a supported size (<= 16).
// Scores live in LDS as sc[key * GP + q], GP = max(G, 4).
template <int D, int G>
__global__ __launch_bounds__(256) void k_decode_split(DecodeParams p, int group) {
    constexpr int GP = G < 4 ? 4 : G;
    constexpr int KS = D / 32;     // k-steps of the 16x16x32 score MFMA
    constexpr int CH = D / 8;      // 16-byte chunks per row
    constexpr int KPI = 64 / CH;   // keys covered by one wave-wide load
    extern __shared__ __attribute__((aligned(16))) float sm[];
    float *sc = sm; // [chunk][GP]; reused for the wave sums after P.V
    __shared__ float s_m[GP], s_l[GP];

    const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    int len = p.lens[b];
    len = len < 0 ? 0 : (len > p.T ? p.T : len);
    const int k0 = c * p.chunk;
    if (k0 >= len) return;
    const int nk = min(p.chunk, len - k0);

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const uint16_t *kbase = p.k + b * p.k_sb + g * p.k_sh + int64_t(k0) * p.k_sn;
    const uint16_t *vbase = p.v + b * p.v_sb + g * p.v_sh + int64_t(k0) * p.v_sn;

    // ---- scores: S = Q K^T, 16 keys per MFMA ----
    // A operand: lane l holds query row l%16 (zero beyond the group), and for
    // k-step s the 8 elements [(D/4)*(l/16) + 8s, +8).  B operand: lane l
    // holds key l%16 of the 16-key group with the same element ranges, so
    // each lane reads D/2 contiguous bytes of one K row.
    const int r16 = lane & 15, g4 = lane >> 4;
    bf16x8_t qa[KS];
    {
        const bool ok = r16 < group;
        const uint16_t *qrow = p.q + b * p.q_sb + int64_t(g * group + (ok ? r16 : 0)) * p.q_sh;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            u32x4_t x = {0u, 0u, 0u, 0u};
            if (ok) x = *reinterpret_cast<const u32x4_t *>(qrow + (D / 4) * g4 + 8 * s);
            qa[s] = __builtin_bit_cast(bf16x8_t, x);
        }
    }
    const int ngroups = (nk + 15) >> 4;
    constexpr int UNR = 4;
    for (int kg0 = wave * UNR; kg0 < ngroups; kg0 += 4 * UNR) {
        u32x4_t kb[UNR][KS];
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
            const int key = (kg0 + u) * 16 + r16;
            const bool ok = (kg0 + u) < ngroups && key < nk;
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                u32x4_t x = {0u, 0u, 0u, 0u};
                if (ok) x = *reinterpret_cast<const u32x4_t *>(kbase + int64_t(key) * p.k_sn + (D / 4) * g4 + 8 * s);
                kb[u][s] = x;
            }
        }
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
            if (kg0 + u >= ngroups) break;
            f32x4_t acc = f32x4_t{};
#pragma unroll
            for (int s = 0; s < KS; ++s)
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa[s], __builtin_bit_cast(bf16x8_t, kb[u][s]), acc, 0, 0, 0);
            // Lane l holds rows (queries) 4*(l/16)+r of column (key) l%16.
            const int key = (kg0 + u) * 16 + r16;
            if (key < nk) {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int q = 4 * g4 + r;
                    if (q < GP) sc[key * GP + q] = acc[r] * p.scale_log2;
                }
            }
        }
    }
    __syncthreads();

    // ---- chunk-local softmax: one wave per query ----
    for (int q = wave; q < group; q += 4) {
        float m = -INFINITY;
        for (int j = lane; j < nk; j += 64) m = fmaxf(m, sc[j * GP + q]);
        m = wave_max(m);
        float l = 0.f;
        for (int j = lane; j < nk; j += 64) {
            const float e = __builtin_amdgcn_exp2f(sc[j * GP + q] - m);
            sc[j * GP + q] = e;
            l += e;
        }
        l = wave_sum(l);
        if (lane == 0) {
            s_m[q] = m;
            s_l[q] = l;
        }
    }
    __syncthreads();

    // ---- partial O = P V on the vector ALU ----
    // Lane l covers d-chunk l%CH of key (l/CH) within each wave-wide load.
    const int dc = lane % CH, ksub = lane / CH;
    float acc[G][8];
#pragma unroll
    for (int q = 0; q < G; ++q)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[q][e] = 0.f;
    constexpr int VUNR = 4;
    for (int j0 = wave * KPI; j0 < nk; j0 += 4 * KPI * VUNR) {
        u32x4_t vv[VUNR];
#pragma unroll
        for (int u = 0; u < VUNR; ++u) {
            const int key = j0 + 4 * KPI * u + ksub;
            u32x4_t x = {0u, 0u, 0u, 0u};
            if (key < nk) x = *reinterpret_cast<const u32x4_t *>(vbase + int64_t(key) * p.v_sn + 8 * dc);
            vv[u] = x;
        }
#pragma unroll
        for (int u = 0; u < VUNR; ++u) {
            const int key = j0 + 4 * KPI * u + ksub;
            if (key < nk) {
                float vf[8];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    vf[2 * e] = bf16lo(vv[u][e]);
                    vf[2 * e + 1] = bf16hi(vv[u][e]);
                }
#pragma unroll
                for (int q = 0; q < G; ++q) {
                    const float pq = sc[key * GP + q];
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[q][e] += pq * vf[e];
                }
            }
        }
    }
    // Reduce over the KPI keys of a wave-wide load (lanes with equal dc).
#pragma unroll
    for (int o = CH; o < 64; o <<= 1)
#pragma unroll
        for (int q = 0; q < G; ++q)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[q][e] += __shfl_xor(acc[q][e], o);
    __syncthreads(); // scores are no longer needed: reuse LDS for the wave sums
    float *red = sm;  // [4 waves][G][D]
    if (ksub == 0) {
#pragma unroll
        for (int q = 0; q < G; ++q)
#pragma unroll
            for (int e = 0; e < 8; ++e) red[(wave * G + q) * D + 8 * dc + e] = acc[q][e];
    }
    __syncthreads();
    const int64_t part_base = (int64_t(b) * p.Hq + int64_t(g) * group) * p.nchunk + c;
    for (int i = tid; i < group * D; i += 256) {
        const int q = i / D, d = i % D;
        const float s = red[(0 * G + q) * D + d] + red[(1 * G + q) * D + d] + red[(2 * G + q) * D + d] +
                        red[(3 * G + q) * D + d];
        p.part_o[(part_base + int64_t(q) * p.nchunk) * D + d] = s;
    }
    if (tid < group) {
        p.part_m[part_base + int64_t(tid) * p.nchunk] = s_m[tid];
        p.part_l[part_base + int64_t(tid) * p.nchunk] = s_l[tid];
    }
}

// One workgroup of D threads per (query head, b): merge the chunk partials.
template <int D>
__global__ __launch_bounds__(D) void k_decode_combine(DecodeParams p) {
    const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
    int len = p.lens[b];
    len = len < 0 ? 0 : (len > p.T ? p.T : len);
    const int nch = (len + p.chunk - 1) / p.chunk;
    const int64_t base = (int64_t(b) * p.Hq + h) * p.nchunk;
    uint16_t *orow = p.o + b * p.o_sb + h * p.o_sh;
    float M = -INFINITY;
    for (int c = 0; c < nch; ++c) M = fmaxf(M, p.part_m[base + c]);
    float L = 0.f, acc = 0.f;
    for (int c = 0; c < nch; ++c) {
        const float w = __builtin_amdgcn_exp2f(p.part_m[base + c] - M);
        L += w * p.part_l[base + c];
        acc += w * p.part_o[(base + c) * D + d];
    }
    const float o = L > 0.f ? acc / L : 0.f;
    __bf16 ob = (__bf16)o;
    orow[d] = __builtin_bit_cast(uint16_t, ob);
    if (d == 0)
        p.lse[int64_t(b) * p.Hq + h] = L > 0.f ? (M + __builtin_amdgcn_logf(L)) * LN2_D : -INFINITY;
}

template <int D, int G> static hipError_t launch_split(const DecodeParams &p, int group, hipStream_t stream) {
    constexpr int GP = G < 4 ? 4 : G;
    size_t lds_scores = size_t(p.chunk) * GP * sizeof(float);
    size_t lds_red = size_t(4) * G * D * sizeof(float);
    size_t lds = lds_scores > lds_red ? lds_scores : lds_red;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_decode_split<D, G>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_decode_split<D, G>), dim3(p.nchunk, p.Hkv, p.B), dim3(256), lds, stream, p, group);
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

static_assert(MAX_CHUNK * 16 * 4 + 2 * 16 * 4 <= 160 * 1024, "decode scores and row stats must fit in LDS");

} // namespace exattn
