// LDS read rates on gfx950, one workgroup per CU (64 KiB of LDS), 8 or 16
// waves, 8 reads in flight per wave:
//   b128   ds_read_b128, 1 KiB per wave instruction, lanes at consecutive
//          16-byte chunks (no bank conflict);
//   tr16   ds_read_b64_tr_b16, 512 bytes per wave instruction, with the
//          forward kernel's V-operand addressing in its XOR-swizzled
//          64-row x 256-byte tiles (no bank conflict);
//   mfma   v_mfma_f32_32x32x16_bf16 whose A operand comes from one
//          ds_read_b128 each (the forward's score products), 4 reads ahead.
// Every address stays inside the 64 KiB buffer.
#include <hip/hip_runtime.h>
#include <cstdio>
#include <cstdlib>
#include <vector>

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) uint8_t lds8;
constexpr int ITERS = 2048;
constexpr uint32_t LDS_MASK = 0xFFFF; // 64 KiB
#define CHECK(x)                                                                                                    \
    do {                                                                                                            \
        hipError_t e_ = (x);                                                                                        \
        if (e_ != hipSuccess) {                                                                                     \
            printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__);                                  \
            exit(1);                                                                                                \
        }                                                                                                           \
    } while (0)

__device__ __forceinline__ int swz128(int r) { return 4 * (r & 3) + ((r >> 2) & 3); }

template <int MODE>
__global__ __launch_bounds__(1024) void k_lds(float x, int salt, long long *ticks, float *sink) {
    __shared__ __attribute__((aligned(1024))) uint8_t buf[98304]; // 96 KiB: one workgroup per CU; reads use the first 64 KiB
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    for (int i = tid; i < 65536 / 4; i += blockDim.x) reinterpret_cast<float *>(buf)[i] = x * (i & 255);
    __syncthreads();
    lds8 *lb = (lds8 *)buf;
    u32x4 acc = {0, 0, 0, 0};
    f32x16 c[4] = {};
    bf16x8 bq;
#pragma unroll
    for (int i = 0; i < 8; ++i) bq[i] = (__bf16)(x + i);
    // tr16 offsets: the forward's V^T reads of one 32-key block
    const int s16 = lane & 15, dh = (lane >> 4) & 1, half = lane >> 5;
    int trofs[8];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int db = 0; db < 4; ++db) {
            const int r = 4 * half + 8 * j + (s16 >> 2);
            const int cb = 64 * db + 32 * dh + 8 * (s16 & 3);
            trofs[4 * j + db] = r * 256 + 16 * ((cb >> 4) ^ swz128(r)) + (cb & 15);
        }
    __syncthreads();
    const long long t0 = __builtin_amdgcn_s_memtime();
    for (int it = 0; it < ITERS; ++it) {
        const uint32_t base = uint32_t((it * 8 + w) * 1024 + salt);
        if constexpr (MODE == 0) {
            u32x4 v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u)
                v[u] = *reinterpret_cast<const __attribute__((address_space(3))) u32x4 *>(
                    lb + ((base + u * 1024 + lane * 16) & LDS_MASK));
#pragma unroll
            for (int u = 0; u < 8; ++u) acc += v[u]; // a sum: nothing cancels across iterations
            asm volatile("" : "+v"(acc));             // and the sum is formed every iteration
        } else if constexpr (MODE == 1) {
            i16x4 v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u)
                v[u] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(reinterpret_cast<__attribute__((address_space(3))) i16x4 *>(
                    lb + ((base * 4 + (u >> 2) * 4096 + trofs[u]) & LDS_MASK)));
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                acc.x += uint32_t(uint16_t(v[u][0])) | (uint32_t(uint16_t(v[u][1])) << 16);
                acc.y += uint32_t(uint16_t(v[u][2])) | (uint32_t(uint16_t(v[u][3])) << 16);
            }
            asm volatile("" : "+v"(acc));
        } else {
            u32x4 v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u)
                v[u] = *reinterpret_cast<const __attribute__((address_space(3))) u32x4 *>(
                    lb + ((base + u * 1024 + lane * 16) & LDS_MASK));
#pragma unroll
            for (int u = 0; u < 8; ++u)
                c[u & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, v[u]), bq, c[u & 3], 0, 0, 0);
            __builtin_amdgcn_sched_group_barrier(0x0100, 4, 0);
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                if (u + 4 < 8) __builtin_amdgcn_sched_group_barrier(0x0100, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x0008, 1, 0);
            }
        }
    }
    const long long t1 = __builtin_amdgcn_s_memtime();
    float s = float(acc.x + acc.y + acc.z + acc.w);
#pragma unroll
    for (int i = 0; i < 4; ++i) s += c[i][0] + c[i][7];
    if (s == 12345.678f) sink[tid] = s;
    if (lane == 0) ticks[blockIdx.x * 16 + w] = t1 - t0;
}

int main() {
    int ncu = 0;
    CHECK(hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, 0));
    const int nb = ncu;
    long long *ticks;
    float *sink;
    CHECK(hipMalloc(&ticks, nb * 16 * sizeof(long long)));
    CHECK(hipMalloc(&sink, 1024 * sizeof(float)));
    hipEvent_t e0, e1;
    CHECK(hipEventCreate(&e0));
    CHECK(hipEventCreate(&e1));
    const char *names[] = {"ds_read_b128 (1 KiB/instr)", "ds_read_b64_tr_b16 (512 B/instr)", "MFMA fed by one ds_read_b128 each"};
    void (*kern[3])(float, int, long long *, float *) = {k_lds<0>, k_lds<1>, k_lds<2>};
    const double bytes_per_instr[3] = {1024, 512, 1024};
    printf("%-6s %-36s %12s %16s %14s %14s\n", "waves", "probe", "ticks/instr", "bytes/tick/CU", "GB/s per CU", "MFMA TFLOP/s");
    for (int waves : {8, 16}) {
        for (int mode = 0; mode < 3; ++mode) {
            hipLaunchKernelGGL(kern[mode], dim3(nb), dim3(64 * waves), 0, 0, 1.0001f, 0, ticks, sink);
            CHECK(hipDeviceSynchronize());
            CHECK(hipEventRecord(e0));
            hipLaunchKernelGGL(kern[mode], dim3(nb), dim3(64 * waves), 0, 0, 1.0001f, 0, ticks, sink);
            CHECK(hipEventRecord(e1));
            CHECK(hipEventSynchronize(e1));
            float ms;
            CHECK(hipEventElapsedTime(&ms, e0, e1));
            std::vector<long long> h(nb * 16);
            CHECK(hipMemcpy(h.data(), ticks, h.size() * sizeof(long long), hipMemcpyDeviceToHost));
            double sum = 0;
            for (int b = 0; b < nb; ++b)
                for (int w = 0; w < waves; ++w) sum += h[b * 16 + w];
            const double ticks_per_iter = sum / (nb * waves) / ITERS;
            const double instr = 8.0 * waves * ITERS;                     // per CU
            const double bytes = instr * bytes_per_instr[mode];           // per CU
            const double gbs = bytes / (ms * 1e-3) / 1e9;
            const double tflops = mode == 2 ? instr * nb * 32768.0 / (ms * 1e-3) / 1e12 : 0.0;
            printf("%-6d %-36s %12.2f %16.1f %14.1f %14.1f\n", waves, names[mode], ticks_per_iter / 8.0,
                   bytes / (ticks_per_iter * ITERS), gbs, tflops);
        }
    }
    return 0;
}
