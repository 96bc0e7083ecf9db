// FP8 (E4M3) block quantization of a bf16 [B, H, N, d] tensor, with optional
// incoherent processing, for the FP8 forward (youngju.dev "FlashAttention
// 논문 분석", FlashAttention-3 section "FP8 지원과 정확도 유지"):
//   - block quantization: every block of 64 rows of one (b, h) gets its own
//     scale, so a block's largest magnitude maps near the top of the E4M3
//     range (or one scale per (b, h) when per_head is set);
//   - incoherent processing: rows are multiplied by a random orthogonal
//     matrix before quantization.  The matrix used is R = diag(signs) * H /
//     sqrt(d) with H the Walsh-Hadamard matrix, applied with the fast
//     butterfly.  Q and K rotated by the same R keep Q K^T unchanged.
// Scales are powers of two: a value is divided exactly, so the only
// rounding is the E4M3 conversion (round to nearest even).
//
// One workgroup of 256 threads per 64-row block: thread t handles 32
// consecutive elements of row t/4 (d = 128), so the butterfly stages 1..16
// are in registers and 32, 64 are exchanges with lanes t^1, t^2.  With a
// scale per block, one kernel reduces the block's largest magnitude in LDS
// and writes the codes.  With one scale per head, a first kernel writes every
// block's largest magnitude to the workspace and a second recomputes the
// rotation, takes the head's largest and writes the codes.
#include "tile.h"

namespace exattn {

constexpr int QROWS = 64;    // rows per quantization block
constexpr float E4M3_MAX = 448.f;

// The rotated (or plain) 32 values of this thread, in fp32.
__device__ __forceinline__ void quant_load_row(const QuantParams &p, int b, int h, int row, int part, float *y) {
    const bool ok = row < p.N;
    // 64 bytes per thread as four 16-byte loads (rows are 16-byte aligned)
    const u32x4_t *src = reinterpret_cast<const u32x4_t *>(p.x + b * p.x_sb + h * p.x_sh +
                                                           int64_t(ok ? row : 0) * p.x_sn + 32 * part);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const u32x4_t v = ok ? src[w] : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            y[8 * w + 2 * e] = __builtin_bit_cast(float, v[e] << 16);
            y[8 * w + 2 * e + 1] = __builtin_bit_cast(float, v[e] & 0xFFFF0000u);
        }
    }
    if (p.signs) {
#pragma unroll
        for (int i = 0; i < 32; ++i)
            if (p.signs[32 * part + i] < 0) y[i] = -y[i];
        // Walsh-Hadamard butterflies, stride 1, 2, ..., 64: the element with
        // the stride bit clear becomes a + b, the other a - b
#pragma unroll
        for (int hs = 1; hs < 32; hs <<= 1)
#pragma unroll
            for (int i = 0; i < 32; ++i)
                if (!(i & hs)) {
                    const float a = y[i], c = y[i + hs];
                    y[i] = a + c;
                    y[i + hs] = a - c;
                }
#pragma unroll
        for (int lanebit = 1; lanebit <= 2; lanebit <<= 1) {
            const bool upper = part & lanebit;
#pragma unroll
            for (int i = 0; i < 32; ++i) {
                const float other = __shfl_xor(y[i], lanebit);
                y[i] = upper ? other - y[i] : y[i] + other;
            }
        }
#pragma unroll
        for (int i = 0; i < 32; ++i) y[i] *= p.inv_sqrt_d;
    }
}

// Smallest e with amax <= 448 * 2^e (e = 0 for an all-zero block): the
// scale is 2^e and the block's values divided by it stay within E4M3.
__device__ __forceinline__ int quant_exponent(float amax) {
    if (!(amax > 0.f)) return 0;
    int e;
    frexpf(amax / E4M3_MAX, &e); // amax/448 = m * 2^e, m in [0.5, 1): 2^(e-1) < amax/448 <= 2^e ...
    // ... except when amax/448 is a power of two (m = 0.5), where 2^(e-1) suffices;
    // the division rounds, so settle the boundary with exact comparisons
    while (e > -126 && amax <= E4M3_MAX * ldexpf(1.f, e - 1)) --e;
    while (amax > E4M3_MAX * ldexpf(1.f, e)) ++e;
    return e;
}

// Codes of this thread's 32 values divided by 2^e, 32 bytes to row `row`.
__device__ __forceinline__ void quant_store(const QuantParams &p, int b, int h, int row, int part, const float *y,
                                            int e) {
    const float inv = ldexpf(1.f, -e);
    uint32_t w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        int v = __builtin_amdgcn_cvt_pk_fp8_f32(y[4 * i] * inv, y[4 * i + 1] * inv, 0, false);
        v = __builtin_amdgcn_cvt_pk_fp8_f32(y[4 * i + 2] * inv, y[4 * i + 3] * inv, v, true);
        w[i] = uint32_t(v);
    }
    uint8_t *dst = p.out + b * p.o_sb + h * p.o_sh + int64_t(row) * p.o_sn + 32 * part;
    *reinterpret_cast<u32x4_t *>(dst) = u32x4_t{w[0], w[1], w[2], w[3]};
    *reinterpret_cast<u32x4_t *>(dst + 16) = u32x4_t{w[4], w[5], w[6], w[7]};
}

// Largest |y| over the workgroup's 64-row block (all 256 threads call it).
__device__ __forceinline__ float quant_block_max(const float *y, float *s_max) {
    const int t = threadIdx.x;
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) m = fmaxf(m, fabsf(y[i]));
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    if ((t & 63) == 0) s_max[t >> 6] = m;
    __syncthreads();
    return fmaxf(fmaxf(s_max[0], s_max[1]), fmaxf(s_max[2], s_max[3]));
}

// Per-block scales in one pass: the block is the workgroup's, so its max is
// reduced in LDS and the codes are written from the same registers.
__global__ __launch_bounds__(256) void k_quant_block(QuantParams p) {
    __shared__ float s_max[4];
    const int blk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int t = threadIdx.x, row = blk * QROWS + t / 4, part = t % 4;
    float y[32];
    quant_load_row(p, b, h, row, part, y);
    const int e = quant_exponent(quant_block_max(y, s_max));
    if (t == 0) p.scales[(int64_t(b) * p.H + h) * p.nblk + blk] = ldexpf(1.f, e);
    if (row < p.N) quant_store(p, b, h, row, part, y, e);
}

// First pass of the per-head mode: every block's max |y| to the workspace.
__global__ __launch_bounds__(256) void k_quant_amax(QuantParams p) {
    __shared__ float s_max[4];
    const int blk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int t = threadIdx.x, row = blk * QROWS + t / 4, part = t % 4;
    float y[32];
    quant_load_row(p, b, h, row, part, y);
    const float m = quant_block_max(y, s_max);
    if (t == 0) p.amax[(int64_t(b) * p.H + h) * p.nblk + blk] = m;
}

// One scale per head: the second pass takes the max over the head's blocks.
__global__ __launch_bounds__(256) void k_quant_apply(QuantParams p) {
    const int blk = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int t = threadIdx.x, row = blk * QROWS + t / 4, part = t % 4;
    const float *am = p.amax + (int64_t(b) * p.H + h) * p.nblk;
    float amax = 0.f;
    for (int i = 0; i < p.nblk; ++i) amax = fmaxf(amax, am[i]);
    const int e = quant_exponent(amax);
    if (t == 0) p.scales[(int64_t(b) * p.H + h) * p.nblk + blk] = ldexpf(1.f, e);
    if (row >= p.N) return;
    float y[32];
    quant_load_row(p, b, h, row, part, y);
    quant_store(p, b, h, row, part, y, e);
}

hipError_t launch_quant(const QuantParams &p, hipStream_t stream) {
    const dim3 grid(p.nblk, p.H, p.B);
    if (!p.per_head) {
        hipLaunchKernelGGL(k_quant_block, grid, dim3(256), 0, stream, p);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(k_quant_amax, grid, dim3(256), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_quant_apply, grid, dim3(256), 0, stream, p);
    return hipGetLastError();
}

} // namespace exattn
