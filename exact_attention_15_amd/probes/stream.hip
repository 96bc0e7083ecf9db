// HBM read bandwidth on gfx950: the ceilings the decode kernel's
// HBM-bound roofline is read against.  Every access stays inside its 1 GiB
// buffer.
//   gridstride  every thread reads 16 bytes per load, 8 loads in flight,
//               the grid strides over the whole buffer;
//   items       the decode split kernel's access pattern: items of 256 KiB
//               of one buffer (K) and 256 KiB of another (V), each of 8
//               waves of a workgroup streaming a contiguous eighth of an
//               item's K then of its V, with 4 or 8 loads in flight per
//               lane; one workgroup per item, or a persistent grid of 512
//               workgroups taking items round-robin.
#include <hip/hip_runtime.h>
#include <cstdio>
#include <cstdlib>

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
#define CHECK(x)                                                                                                    \
    do {                                                                                                            \
        hipError_t e_ = (x);                                                                                        \
        if (e_ != hipSuccess) {                                                                                     \
            printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__);                                  \
            exit(1);                                                                                                \
        }                                                                                                           \
    } while (0)

template <int UNR>
__global__ __launch_bounds__(256) void k_gridstride(const u32x4 *__restrict__ a, size_t n16, uint32_t *out) {
    size_t i = (size_t)blockIdx.x * 256 * UNR + threadIdx.x;
    const size_t step = (size_t)gridDim.x * 256 * UNR;
    u32x4 acc = {0, 0, 0, 0};
    for (; i + 256 * (UNR - 1) < n16; i += step) {
        u32x4 v[UNR];
#pragma unroll
        for (int u = 0; u < UNR; ++u) v[u] = a[i + 256 * u];
#pragma unroll
        for (int u = 0; u < UNR; ++u) acc ^= v[u];
    }
    if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x12345678u) out[0] = 1;
}

template <int UNR>
__global__ __launch_bounds__(512) void k_items(const u32x4 *__restrict__ a, const u32x4 *__restrict__ b, int nitems,
                                               int item16, uint32_t *out) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, nw = blockDim.x >> 6;
    const int slice = item16 / nw;
    u32x4 acc = {0, 0, 0, 0};
    for (int it = blockIdx.x; it < nitems; it += gridDim.x) {
        for (int buf = 0; buf < 2; ++buf) {
            const u32x4 *base = (buf ? b : a) + (size_t)it * item16 + (size_t)wave * slice;
            for (int j = lane; j + 64 * (UNR - 1) < slice; j += 64 * UNR) {
                u32x4 v[UNR];
#pragma unroll
                for (int u = 0; u < UNR; ++u) v[u] = base[j + 64 * u];
#pragma unroll
                for (int u = 0; u < UNR; ++u) acc ^= v[u];
            }
        }
    }
    if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x12345678u) out[0] = 1;
}

int main() {
    const size_t bytes = size_t(1) << 30;
    const size_t n16 = bytes / 16;
    u32x4 *a, *b;
    uint32_t *out;
    CHECK(hipMalloc(&a, bytes));
    CHECK(hipMalloc(&b, bytes));
    CHECK(hipMalloc(&out, 64));
    CHECK(hipMemset(a, 1, bytes));
    CHECK(hipMemset(b, 2, bytes));
    hipEvent_t e0, e1;
    CHECK(hipEventCreate(&e0));
    CHECK(hipEventCreate(&e1));
    auto timeit = [&](const char *name, double nbytes, auto launch) {
        for (int w = 0; w < 20; ++w) launch();
        CHECK(hipDeviceSynchronize());
        const int reps = 30;
        CHECK(hipEventRecord(e0));
        for (int r = 0; r < reps; ++r) launch();
        CHECK(hipEventRecord(e1));
        CHECK(hipEventSynchronize(e1));
        float ms;
        CHECK(hipEventElapsedTime(&ms, e0, e1));
        const double us = ms * 1e3 / reps;
        printf("%-58s %8.1f us %7.0f GB/s\n", name, us, nbytes / (us * 1e-6) / 1e9);
        fflush(stdout);
    };
    for (int grid : {1024, 4096, 8192}) {
        char nm[96];
        snprintf(nm, sizeof nm, "gridstride 1 GiB, 8 loads in flight, grid %d", grid);
        timeit(nm, double(bytes), [&] { hipLaunchKernelGGL((k_gridstride<8>), dim3(grid), dim3(256), 0, 0, a, n16, out); });
    }
    const int item16 = (256 * 1024) / 16; // per buffer
    const int nitems = 1880;              // 0.985 GB in all
    if ((size_t)nitems * item16 > n16) return 1;
    const double item_bytes = 2.0 * nitems * item16 * 16;
    for (int grid : {512, 1880}) {
        char nm[96];
        snprintf(nm, sizeof nm, "items K+V (decode pattern), 4 loads/lane, grid %d", grid);
        timeit(nm, item_bytes, [&] { hipLaunchKernelGGL((k_items<4>), dim3(grid), dim3(512), 0, 0, a, b, nitems, item16, out); });
        snprintf(nm, sizeof nm, "items K+V (decode pattern), 8 loads/lane, grid %d", grid);
        timeit(nm, item_bytes, [&] { hipLaunchKernelGGL((k_items<8>), dim3(grid), dim3(512), 0, 0, a, b, nitems, item16, out); });
    }
    return 0;
}
