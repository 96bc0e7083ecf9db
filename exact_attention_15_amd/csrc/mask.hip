// Block-mask builder: per-row visible key intervals, per-query-tile lists of
// visited key tiles (FULL or PARTIAL), and a heavy-first order of the query
// tiles of each batch row.
//
// Every mask the library supports (causal, sliding window, document
// boundaries, and their combinations) leaves each query row i one interval
// [lo_i, hi_i] of visible keys.  The block mask precomputes, per 128-row
// query tile, which 64-key tiles hold any visible key, so the forward kernel
// never visits fully masked tiles (it-trends-board "PyTorch FlexAttention
// 도입 분석", section 2, the block-mask early-out), and which of them need no
// element mask at all (youngju.dev "FlashAttention 논문 분석",
// FlashAttention-2 improvement 1).
#include "common.h"

namespace exattn {

// One thread per (b, i): the visible interval of query row i.
__global__ void k_mask_rows(attn_mask_spec spec, int B, int N, int32_t *lo_out,
                            int32_t *hi_out) {
    const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
    if (idx >= int64_t(B) * N) return;
    const int b = int(idx / N);
    const int i = int(idx % N);
    int64_t lo = 0, hi = int64_t(N) - 1;
    if (spec.flags & ATTN_MASK_CAUSAL) hi = min(hi, int64_t(i));
    if (spec.flags & ATTN_MASK_WINDOW) {
        lo = max(lo, int64_t(i) - spec.window_left);
        hi = min(hi, int64_t(i) + spec.window_right);
    }
    if (spec.flags & ATTN_MASK_DOCS) {
        // Last boundary at or below i (binary search over the padded row).
        const int32_t *off = spec.doc_offsets + int64_t(b) * spec.doc_stride;
        int a = 0, z = spec.doc_stride - 1; // invariant: answer in [a, z]
        if (off[0] > i) {
            a = z = -1;
        } else {
            while (a < z) {
                int mid = (a + z + 1) >> 1;
                if (off[mid] <= i) a = mid; else z = mid - 1;
            }
        }
        int64_t start = a >= 0 ? off[a] : 0;
        int64_t end = (a >= 0 && a + 1 < spec.doc_stride) ? off[a + 1] : N;
        if (end > N) end = N;
        lo = max(lo, start);
        hi = min(hi, end - 1);
    }
    if (lo > hi) { lo = 1; hi = 0; } // empty row
    lo_out[idx] = int32_t(lo);
    hi_out[idx] = int32_t(hi);
}

// One workgroup per (query tile, b).  Thread t classifies a contiguous run of
// key tiles; a block-wide prefix sum then writes the visited tiles in order.
__global__ __launch_bounds__(256) void k_mask_tiles(uint32_t flags, int N, int nqt, int nkt,
                                                    const int32_t *lo_in, const int32_t *hi_in,
                                                    int32_t *count_out, int32_t *list_out) {
    __shared__ int32_t s_lo[BLOCK_M], s_hi[BLOCK_M];
    __shared__ int32_t s_valid[BLOCK_M];
    __shared__ int32_t s_cnt[256];
    const int qt = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
    const int r0 = qt * BLOCK_M;
    if (t < BLOCK_M) {
        const int row = r0 + t;
        const bool ok = row < N;
        s_valid[t] = ok;
        s_lo[t] = ok ? lo_in[int64_t(b) * N + row] : 1;
        s_hi[t] = ok ? hi_in[int64_t(b) * N + row] : 0;
    }
    __syncthreads();
    const bool no_skip = flags & ATTN_MASK_NO_SKIP;
    const int per = (nkt + 255) / 256;
    const int kt0 = min(nkt, t * per), kt1 = min(nkt, kt0 + per);
    // Count this thread's visited tiles; the classification is repeated in
    // the write pass below (it is cheap) instead of being stored.
    int n_mine = 0;
    for (int kt = kt0; kt < kt1; ++kt) {
        const int c0 = kt * BLOCK_N, c1 = c0 + BLOCK_N - 1;
        bool any = false, full = true;
        for (int r = 0; r < BLOCK_M; ++r) {
            if (!s_valid[r]) continue;
            const int lo = s_lo[r], hi = s_hi[r];
            if (max(lo, c0) <= min(hi, c1)) any = true;
            if (!(lo <= c0 && hi >= c1)) full = false;
        }
        if (no_skip) { any = true; full = false; }
        n_mine += any;
    }
    s_cnt[t] = n_mine;
    __syncthreads();
    // Exclusive prefix over 256 counts (Hillis-Steele in shared memory).
    for (int s = 1; s < 256; s <<= 1) {
        int add = t >= s ? s_cnt[t - s] : 0;
        __syncthreads();
        s_cnt[t] += add;
        __syncthreads();
    }
    const int base = s_cnt[t] - n_mine;
    const int64_t item = int64_t(b) * nqt + qt;
    int32_t *list = list_out + item * nkt;
    int w = base;
    for (int kt = kt0; kt < kt1; ++kt) {
        const int c0 = kt * BLOCK_N, c1 = c0 + BLOCK_N - 1;
        bool any = false, full = true;
        for (int r = 0; r < BLOCK_M; ++r) {
            if (!s_valid[r]) continue;
            const int lo = s_lo[r], hi = s_hi[r];
            if (max(lo, c0) <= min(hi, c1)) any = true;
            if (!(lo <= c0 && hi >= c1)) full = false;
        }
        if (no_skip) { any = true; full = false; }
        if (any) list[w++] = (kt << 1) | (full ? 0 : TILE_PARTIAL);
    }
    if (t == 255) count_out[item] = s_cnt[255];
}

// One workgroup per batch row: order[b][rank] = query tile, ranked by
// descending visited-tile count (ties keep tile order), so the forward
// kernel can hand out the heaviest query tiles of each batch row first.
__global__ __launch_bounds__(1024) void k_mask_order(int nqt, const int32_t *count, int32_t *order) {
    const int b = blockIdx.x;
    const int32_t *cb = count + int64_t(b) * nqt;
    int32_t *ob = order + int64_t(b) * nqt;
    for (int i = threadIdx.x; i < nqt; i += blockDim.x) {
        const int ci = cb[i];
        int rank = 0;
        for (int j = 0; j < nqt; ++j) {
            const int cj = cb[j];
            rank += (cj > ci) || (cj == ci && j < i);
        }
        ob[rank] = i;
    }
}

hipError_t launch_mask_build(const attn_mask_spec &spec, const MaskLayout &L, void *out,
                             hipStream_t stream) {
    char *base = static_cast<char *>(out);
    int32_t *lo = reinterpret_cast<int32_t *>(base + L.off_lo);
    int32_t *hi = reinterpret_cast<int32_t *>(base + L.off_hi);
    int32_t *cnt = reinterpret_cast<int32_t *>(base + L.off_count);
    int32_t *list = reinterpret_cast<int32_t *>(base + L.off_list);
    int32_t *order = reinterpret_cast<int32_t *>(base + L.off_order);
    const int64_t rows = int64_t(L.B) * L.N;
    const int64_t nblk = (rows + 255) / 256;
    hipLaunchKernelGGL(k_mask_rows, dim3(unsigned(nblk)), dim3(256), 0, stream, spec, L.B, L.N,
                       lo, hi);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_mask_tiles, dim3(L.nqt, L.B), dim3(256), 0, stream, spec.flags, L.N,
                       L.nqt, L.nkt, lo, hi, cnt, list);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_mask_order, dim3(L.B), dim3(1024), 0, stream, L.nqt, cnt, order);
    return hipGetLastError();
}

} // namespace exattn
