// Issue rates on gfx950 with register operands only: VALU FMA, v_exp_f32,
// v_mfma_f32_32x32x16_bf16, MFMA and VALU in one wave, and MFMA in one wave
// beside VALU in the other wave of the same SIMD, and chains of dependent
// MFMAs (the accumulator of each the input of the next).  One 4- or 8-wave
// workgroup per CU (96 KiB of LDS each), so each SIMD holds 1 or 2 of them;
// in an 8-wave workgroup waves w and w+4 share a SIMD (the map is printed
// first).  Times are s_memtime ticks per loop iteration per wave, and the
// tick rate against wall time.  Every result feeds a store that a condition
// the values never meet guards.
#include <hip/hip_runtime.h>
#include <cstdio>
#include <cstdlib>
#include <vector>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
constexpr int ITERS = 4096;
#define CHECK(x)                                                                                                    \
    do {                                                                                                            \
        hipError_t e_ = (x);                                                                                        \
        if (e_ != hipSuccess) {                                                                                     \
            printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__);                                  \
            exit(1);                                                                                                \
        }                                                                                                           \
    } while (0)

__device__ __forceinline__ void fma16(float (&a)[16], float x) {
#pragma unroll
    for (int i = 0; i < 16; ++i) a[i] = __builtin_fmaf(a[i], x, 1.0f);
}
__device__ __forceinline__ void exp16(float (&a)[16]) {
#pragma unroll
    for (int i = 0; i < 16; ++i) a[i] = __builtin_amdgcn_exp2f(a[i]);
}
__device__ __forceinline__ void mfma8(f32x16 (&c)[4], bf16x8 a, bf16x8 b) {
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int i = 0; i < 4; ++i) c[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[i], 0, 0, 0);
}

// 8 MFMAs on NACC accumulators taken in turn: each MFMA depends on the one
// NACC places before it (NACC = 1: one chain of dependent MFMAs).
template <int NACC> __device__ __forceinline__ void mfma8_chains(f32x16 (&c)[4], bf16x8 a, bf16x8 b) {
#pragma unroll
    for (int r = 0; r < 8 / NACC; ++r)
#pragma unroll
        for (int i = 0; i < NACC; ++i) c[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[i], 0, 0, 0);
}

// MODE 0: 32 FMA; 1: 16 exp; 2: 8 MFMA; 3: waves 0-3 8 MFMA, 4-7 32 FMA;
// 4: waves 0-3 8 MFMA, 4-7 16 exp; 5: 8 MFMA and 32 FMA in every wave;
// 6: 8 MFMA in one dependent chain; 7: 8 MFMA in two chains taken in turn
template <int MODE>
__global__ __launch_bounds__(512) void k_units(float x, long long *ticks, float *sink) {
    __shared__ float pad[24 * 1024]; // 96 KiB: one workgroup per CU
    const int w = threadIdx.x >> 6;
    if (x == 12345.f) pad[threadIdx.x] = x;
    float a[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) a[i] = x * (i + 1) * 1e-3f;
    f32x16 c[4] = {};
    bf16x8 av, bv;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        av[i] = (__bf16)(x * i);
        bv[i] = (__bf16)(x + i);
    }
    __syncthreads();
    const long long t0 = __builtin_amdgcn_s_memtime();
#pragma unroll 4
    for (int it = 0; it < ITERS; ++it) {
        if constexpr (MODE == 0) { fma16(a, x); fma16(a, x); }
        else if constexpr (MODE == 1) { exp16(a); }
        else if constexpr (MODE == 2) { mfma8(c, av, bv); }
        else if constexpr (MODE == 3) { if (w < 4) mfma8(c, av, bv); else { fma16(a, x); fma16(a, x); } }
        else if constexpr (MODE == 4) { if (w < 4) mfma8(c, av, bv); else exp16(a); }
        else if constexpr (MODE == 5) { mfma8(c, av, bv); fma16(a, x); fma16(a, x); }
        else if constexpr (MODE == 6) { mfma8_chains<1>(c, av, bv); }
        else { mfma8_chains<2>(c, av, bv); }
    }
    const long long t1 = __builtin_amdgcn_s_memtime();
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) s += a[i];
#pragma unroll
    for (int i = 0; i < 4; ++i) s += c[i][0] + c[i][5];
    if (s == 12345.678f) sink[threadIdx.x] = s;
    if (pad[threadIdx.x & 1023] == 12345.f) sink[0] = 1.f;
    if ((threadIdx.x & 63) == 0) ticks[blockIdx.x * 8 + w] = t1 - t0;
}

__global__ __launch_bounds__(512) void k_simdmap(int *out) {
    // HW_REG_HW_ID (hwreg 4): simd id in bits [5:4]
    const int hw = __builtin_amdgcn_s_getreg((31 << 11) | (0 << 6) | 4);
    if ((threadIdx.x & 63) == 0) out[blockIdx.x * 8 + (threadIdx.x >> 6)] = (hw >> 4) & 3;
    __syncthreads();
}

int main() {
    int ncu = 0;
    CHECK(hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, 0));
    const int nb = ncu;
    {
        int *d;
        CHECK(hipMalloc(&d, nb * 8 * sizeof(int)));
        hipLaunchKernelGGL(k_simdmap, dim3(nb), dim3(512), 0, 0, d);
        CHECK(hipDeviceSynchronize());
        std::vector<int> h(nb * 8);
        CHECK(hipMemcpy(h.data(), d, h.size() * sizeof(int), hipMemcpyDeviceToHost));
        int same = 0;
        for (int b = 0; b < nb; ++b) {
            bool ok = true;
            for (int w = 0; w < 4; ++w) ok &= h[b * 8 + w] == h[b * 8 + w + 4];
            same += ok;
        }
        printf("8-wave workgroups in which waves w and w+4 share a SIMD for every w: %d of %d\n", same, nb);
    }
    long long *ticks;
    float *sink;
    CHECK(hipMalloc(&ticks, nb * 8 * sizeof(long long)));
    CHECK(hipMalloc(&sink, 512 * sizeof(float)));
    const char *names[] = {"32 FMA", "16 v_exp_f32", "8 MFMA 32x32x16 bf16", "8 MFMA (waves 0-3) | 32 FMA (waves 4-7)",
                           "8 MFMA (waves 0-3) | 16 exp (waves 4-7)", "8 MFMA + 32 FMA in every wave",
                           "8 MFMA, one dependent chain", "8 MFMA, two chains in turn"};
    void (*kern[8])(float, long long *, float *) = {k_units<0>, k_units<1>, k_units<2>, k_units<3>,
                                                     k_units<4>, k_units<5>, k_units<6>, k_units<7>};
    hipEvent_t e0, e1;
    CHECK(hipEventCreate(&e0));
    CHECK(hipEventCreate(&e1));
    printf("%-8s %-44s %14s %14s %10s\n", "waves/WG", "per loop iteration", "ticks w0-3", "ticks w4-7", "tick GHz");
    for (int waves : {4, 8}) {
        for (int mode = 0; mode < 8; ++mode) {
            if (waves == 4 && (mode == 3 || mode == 4)) continue;
            hipLaunchKernelGGL(kern[mode], dim3(nb), dim3(64 * waves), 0, 0, 1.0001f, ticks, sink);
            CHECK(hipDeviceSynchronize());
            CHECK(hipEventRecord(e0));
            hipLaunchKernelGGL(kern[mode], dim3(nb), dim3(64 * waves), 0, 0, 1.0001f, ticks, sink);
            CHECK(hipEventRecord(e1));
            CHECK(hipEventSynchronize(e1));
            float ms;
            CHECK(hipEventElapsedTime(&ms, e0, e1));
            std::vector<long long> h(nb * 8);
            CHECK(hipMemcpy(h.data(), ticks, h.size() * sizeof(long long), hipMemcpyDeviceToHost));
            double s0 = 0, s1 = 0;
            int n0 = 0, n1 = 0;
            long long mx = 0;
            for (int b = 0; b < nb; ++b)
                for (int w = 0; w < waves; ++w) {
                    const long long v = h[b * 8 + w];
                    mx = v > mx ? v : mx;
                    if (w < 4) { s0 += v; ++n0; } else { s1 += v; ++n1; }
                }
            printf("%-8d %-44s %14.1f %14.1f %10.2f\n", waves, names[mode], s0 / n0 / ITERS,
                   n1 ? s1 / n1 / ITERS : 0.0, double(mx) / (ms * 1e6));
        }
    }
    return 0;
}
