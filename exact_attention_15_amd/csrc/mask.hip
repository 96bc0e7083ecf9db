// Block-mask builder: per-row visible key intervals, per-query-tile lists of
// visited key tiles (FULL or PARTIAL), and a heavy-first order of the query
// tiles of each batch row.
//
// Every mask the library supports (causal, sliding window, document
// boundaries, packed variable-length sequences, and their combinations)
// leaves each query row i one interval
// [lo_i, hi_i] of visible keys.  The block mask precomputes, per 128-row
// query tile, which 64-key tiles hold any visible key, so the forward kernel
// never visits fully masked tiles (it-trends-board "PyTorch FlexAttention
// 도입 분석", section 2, the block-mask early-out), and which of them need no
// element mask at all (youngju.dev "FlashAttention 논문 분석",
// FlashAttention-2 improvement 1).
#include "common.h"

namespace exattn {

// Packed variable-length input: query row i belongs to the sequence s with
// cu_q[s] <= i < cu_q[s+1] and sees that sequence's keys [cu_k[s],
// cu_k[s+1]).  With Lq queries and Lk keys in the sequence, query iq lines
// up with key iq + Lk - Lq (the last query with the last key), and the
// causal limit and the window are taken about that key.  Offsets are
// clamped into [0, N] and [0, Nk], so malformed ones cannot move an
// interval outside the keys that exist.
__device__ __forceinline__ void varlen_interval(const attn_mask_spec &spec, const VarlenView &vl, int N, int Nk,
                                                int i, int64_t &lo, int64_t &hi) {
    // last sequence s in [0, nseq) with cu_q[s] <= i
    int a = 0, z = vl.nseq - 1;
    if (z < 0 || vl.cu_q[0] > i) {
        lo = 1;
        hi = 0;
        return;
    }
    while (a < z) {
        const int mid = (a + z + 1) >> 1;
        if (vl.cu_q[mid] <= i) a = mid; else z = mid - 1;
    }
    const int64_t q0 = min(max(int64_t(vl.cu_q[a]), int64_t(0)), int64_t(N));
    const int64_t q1 = min(max(int64_t(vl.cu_q[a + 1]), q0), int64_t(N));
    const int64_t k0 = min(max(int64_t(vl.cu_k[a]), int64_t(0)), int64_t(Nk));
    const int64_t k1 = min(max(int64_t(vl.cu_k[a + 1]), k0), int64_t(Nk));
    if (i >= q1) { // past the last sequence's queries
        lo = 1;
        hi = 0;
        return;
    }
    const int64_t diag = (i - q0) + (k1 - k0) - (q1 - q0); // local key on this query's diagonal
    int64_t l = 0, h = k1 - k0 - 1;
    if (spec.flags & ATTN_MASK_CAUSAL) h = min(h, diag);
    if (spec.flags & ATTN_MASK_WINDOW) {
        l = max(l, diag - spec.window_left);
        h = min(h, diag + spec.window_right);
    }
    lo = k0 + l;
    hi = k0 + h;
}

// The visible interval [lo, hi] of query row i of batch row b (lo > hi when
// no key is visible: then lo = 1, hi = 0).
__device__ __forceinline__ void row_interval(const attn_mask_spec &spec, const VarlenView &vl, int b, int N, int Nk,
                                             int i, int &lo_out, int &hi_out) {
    int64_t lo = 0, hi = int64_t(N) - 1;
    if (vl.cu_q) {
        varlen_interval(spec, vl, N, Nk, i, lo, hi);
        if (lo > hi) { lo = 1; hi = 0; }
        lo_out = int(lo);
        hi_out = int(hi);
        return;
    }
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
    if (lo > hi) { lo = 1; hi = 0; }
    lo_out = int(lo);
    hi_out = int(hi);
}

// One workgroup (4 waves) per (query tile, b).  Threads 0..127 compute and
// store the intervals of the tile's rows.  The key tiles are then classified
// 256 at a time, thread t taking tile k0 + t:
// - FULL (every row sees every key of the tile) holds exactly when the
//   largest lo is at or before the tile's first key and the smallest hi at
//   or after its last, both over the existing rows (a row with no visible
//   key has lo > hi and so rules FULL out everywhere);
// - visited (some row sees some key of it): row r touches the tiles
//   lo_r/64 .. hi_r/64, so each row adds +1 and -1 at the two ends of that
//   range in an LDS difference array, and a prefix sum gives every tile the
//   number of rows that touch it.
// The visited tiles are written in key order with a ballot/popcount
// compaction.
// order_direct: the heavy-first order, written here (and k_mask_order not
// run) when it has a closed form: under a plain causal mask over equal
// query and key counts, query tile qt visits floor(last row / 64) + 1 key
// tiles, a count that grows strictly with qt, so the order is the reverse
// tile order.
__global__ __launch_bounds__(256) void k_mask_tiles(attn_mask_spec spec, VarlenView vl, int N, int Nk, int nqt,
                                                    int nkt, int32_t *lo_out, int32_t *hi_out, int32_t *count_out,
                                                    int32_t *list_out, int32_t *order_direct) {
    __shared__ int32_t s_lo[BLOCK_M], s_hi[BLOCK_M];
    __shared__ int32_t s_diff[257];
    __shared__ int32_t s_wsum[4];
    __shared__ int32_t s_ext[2][4];
    const int qt = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
    const int lane = t & 63, w = t >> 6;
    const int r0 = qt * BLOCK_M;
    if (t < BLOCK_M) {
        int lo = 1, hi = 0;
        const int row = r0 + t;
        if (row < N) {
            row_interval(spec, vl, b, N, Nk, row, lo, hi);
            lo_out[int64_t(b) * N + row] = lo;
            hi_out[int64_t(b) * N + row] = hi;
        }
        s_lo[t] = lo;
        s_hi[t] = hi;
    }
    __syncthreads();
    // Largest lo and smallest hi over the existing rows (waves 0 and 1 hold
    // rows 0..127; rows past N do not count).
    if (w < 2) {
        const bool ok = r0 + t < N;
        int mlo = ok ? s_lo[t] : INT32_MIN, mhi = ok ? s_hi[t] : INT32_MAX;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) {
            mlo = max(mlo, __shfl_xor(mlo, o));
            mhi = min(mhi, __shfl_xor(mhi, o));
        }
        if (lane == 0) {
            s_ext[0][w] = mlo;
            s_ext[1][w] = mhi;
        }
    }
    __syncthreads();
    const int max_lo = max(s_ext[0][0], s_ext[0][1]), min_hi = min(s_ext[1][0], s_ext[1][1]);
    const bool no_skip = spec.flags & ATTN_MASK_NO_SKIP;
    const int64_t item = int64_t(b) * nqt + qt;
    int32_t *list = list_out + item * nkt;
    int base = 0;
    for (int k0 = 0; k0 < nkt; k0 += 256) {
        s_diff[t] = 0;
        if (t == 0) s_diff[256] = 0;
        __syncthreads();
        if (t < BLOCK_M && r0 + t < N) {
            const int lo = s_lo[t], hi = s_hi[t];
            if (lo <= hi) {
                const int a = max(lo / BLOCK_N, k0), z = min(hi / BLOCK_N, k0 + 255);
                if (a <= z) {
                    atomicAdd(&s_diff[a - k0], 1);
                    atomicAdd(&s_diff[z - k0 + 1], -1);
                }
            }
        }
        __syncthreads();
        // inclusive prefix sum of s_diff[0..255]: wave scan, then wave totals
        int v = s_diff[t];
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int u = __shfl_up(v, o);
            if (lane >= o) v += u;
        }
        if (lane == 63) s_wsum[w] = v;
        __syncthreads();
        for (int x = 0; x < w; ++x) v += s_wsum[x];
        const int kt = k0 + t;
        const int c0 = kt * BLOCK_N, c1 = c0 + BLOCK_N - 1;
        bool any = kt < nkt && v > 0;
        bool full = max_lo <= c0 && min_hi >= c1;
        if (no_skip) {
            any = kt < nkt;
            full = false;
        }
        __syncthreads(); // s_wsum is reused for the compaction counts
        const uint64_t vis = __ballot(any);
        if (lane == 0) s_wsum[w] = __popcll(vis);
        __syncthreads();
        int woff = base;
        for (int x = 0; x < w; ++x) woff += s_wsum[x];
        const int total = s_wsum[0] + s_wsum[1] + s_wsum[2] + s_wsum[3];
        if (any) {
            const int pos = woff + __popcll(vis & ((uint64_t(1) << lane) - 1));
            list[pos] = (kt << 1) | (full ? 0 : TILE_PARTIAL);
        }
        base += total;
        __syncthreads(); // s_diff and s_wsum are rewritten by the next round
    }
    if (t == 0) {
        count_out[item] = base;
        if (order_direct) order_direct[int64_t(b) * nqt + (nqt - 1 - qt)] = qt;
    }
}

// One workgroup per batch row: order[b][rank] = query tile, ranked by
// descending visited-tile count (ties keep tile order), so the forward
// kernel can hand out the heaviest query tiles of each batch row first.
// With documents or varlen sequences the tiles are first grouped by the
// start of their first row's visible interval (its document), documents in
// order: the workgroups that run at once then read one or two documents'
// K/V, which stay in the XCD's L2, where heavy-first across all documents
// ran the heaviest tiles of every document together (the packed GQA
// document workload fetched 1.8x its compulsory bytes that way).
// The row's keys are staged in LDS when they fit (ORDER_LDS_TILES), so the
// rank loop reads LDS broadcasts instead of global memory.
constexpr int ORDER_LDS_TILES = 8192;
__global__ __launch_bounds__(1024) void k_mask_order(int nqt, int N, bool by_doc, const int32_t *count,
                                                     const int32_t *lo, int32_t *order) {
    extern __shared__ int32_t s_key[]; // [0, nqt): counts; [nqt, 2 nqt): document keys
    const int b = blockIdx.x;
    const int32_t *cb = count + int64_t(b) * nqt;
    const int32_t *lb = lo + int64_t(b) * N;
    int32_t *ob = order + int64_t(b) * nqt;
    const bool in_lds = nqt <= ORDER_LDS_TILES;
    auto doc_key = [&](int i) { return by_doc ? lb[int64_t(i) * BLOCK_M] : 0; };
    if (in_lds) {
        for (int i = threadIdx.x; i < nqt; i += blockDim.x) {
            s_key[i] = cb[i];
            s_key[nqt + i] = doc_key(i);
        }
        __syncthreads();
    }
    auto rank_all = [&](auto cnt_at, auto key_at) {
        for (int i = threadIdx.x; i < nqt; i += blockDim.x) {
            const int ci = cnt_at(i), ki = key_at(i);
            int rank = 0;
            for (int j = 0; j < nqt; ++j) {
                const int cj = cnt_at(j), kj = key_at(j);
                rank += (kj < ki) || (kj == ki && ((cj > ci) || (cj == ci && j < i)));
            }
            ob[rank] = i;
        }
    };
    if (in_lds) {
        const __attribute__((address_space(3))) int32_t *sk = (const __attribute__((address_space(3))) int32_t *)(s_key);
        rank_all([&](int i) { return sk[i]; }, [&](int i) { return sk[nqt + i]; });
    } else {
        rank_all([&](int i) { return cb[i]; }, doc_key);
    }
}

hipError_t launch_mask_build(const attn_mask_spec &spec, const MaskLayout &L, void *out,
                             hipStream_t stream, VarlenView vl) {
    char *base = static_cast<char *>(out);
    int32_t *lo = reinterpret_cast<int32_t *>(base + L.off_lo);
    int32_t *hi = reinterpret_cast<int32_t *>(base + L.off_hi);
    int32_t *cnt = reinterpret_cast<int32_t *>(base + L.off_count);
    int32_t *list = reinterpret_cast<int32_t *>(base + L.off_list);
    int32_t *order = reinterpret_cast<int32_t *>(base + L.off_order);
    const uint32_t mask_bits = spec.flags & (ATTN_MASK_CAUSAL | ATTN_MASK_WINDOW | ATTN_MASK_DOCS | ATTN_MASK_NO_SKIP);
    const bool causal_only = mask_bits == ATTN_MASK_CAUSAL && vl.cu_q == nullptr && L.N == L.Nk;
    hipLaunchKernelGGL(k_mask_tiles, dim3(L.nqt, L.B), dim3(256), 0, stream, spec, vl, L.N, L.Nk, L.nqt, L.nkt,
                       lo, hi, cnt, list, causal_only ? order : nullptr);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || causal_only) return e;
    const size_t order_lds = L.nqt <= ORDER_LDS_TILES ? 2 * size_t(L.nqt) * sizeof(int32_t) : 0;
    const bool by_doc = (spec.flags & ATTN_MASK_DOCS) || vl.cu_q != nullptr;
    hipLaunchKernelGGL(k_mask_order, dim3(L.B), dim3(1024), order_lds, stream, L.nqt, L.N, by_doc, cnt, lo,
                       order);
    return hipGetLastError();
}

} // namespace exattn
