// Device helpers shared by the forward and backward kernels: MFMA operand
// types, the LDS tile layout (XOR-swizzled 16-byte chunks), the 32x32
// accumulator layout, LDS transpose reads and the HBM -> LDS DMA.
#pragma once
#include "common.h"

namespace exattn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;

// Tile geometry for head dim D: 64-row tiles of K, V (forward) or of Q, dO
// (backward) staged in LDS.
template <int D> struct FwdCfg {
    static constexpr int KSTEPS = D / 16;              // k-steps of the S^T MFMAs
    static constexpr int DBLK = D / 32;                // 32-row blocks of O^T
    static constexpr int ROW_BYTES = D * 2;            // one K or V row
    static constexpr int CHUNKS = D / 8;               // 16-byte chunks per row
    static constexpr int TILE_BYTES = BLOCK_N * ROW_BYTES;
    static constexpr int STAGE_BYTES = 2 * TILE_BYTES; // K tile + V tile
    static constexpr int LOADS = TILE_BYTES / 1024 / 4; // 1 KiB loads per wave per tile
    static constexpr int ROWS_PER_LOAD = 1024 / ROW_BYTES;
    static constexpr size_t LDS_BYTES = size_t(2) * STAGE_BYTES;
};

// Chunk swizzle.  D = 128 (16 chunks per row; 4 rows span the 64 banks):
// swz(r) = 4*(r%4) + (r/4)%4 gives 16 consecutive rows distinct values
// (conflict-free K reads of one chunk column) and gives 4 consecutive rows
// disjoint groups of 4 chunks (conflict-free transpose reads of V).  D = 64
// (8 chunks per row; two rows span the banks): the same two properties with
// swz(r) = 4*((r/2)%2) + (r/4)%4.
template <int D> __device__ __forceinline__ int swz(int r) {
    if constexpr (D == 128) return 4 * (r & 3) + ((r >> 2) & 3);
    else return 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
}

// 32x32 accumulator layout of v_mfma_f32_32x32x16_bf16: register r of lane l
// holds row 8*(r/4) + 4*(l/32) + r%4 and column l%32.
__device__ __forceinline__ int acc_row(int r, int half) { return 8 * (r >> 2) + 4 * half + (r & 3); }

__device__ __forceinline__ float wave_swap_halves(float x, int half) {
    // Value of lane l^32 (the other 32-lane half of the wave): after
    // v_permlane32_swap(x, x) the first result holds the low half twice and
    // the second the high half twice.
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __builtin_bit_cast(float, half ? r[0] : r[1]);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    // Round-to-nearest-even to bf16 (v_cvt_pk_bf16_f32).
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    bf16x2_t v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ u32x2_t lds_read_tr16(const lds_u8 *base, int off) {
    // ds_read_b64_tr_b16: within each 16-lane group, element e of lane i is
    // element i%4 of the 8 bytes addressed by lane 4e + i/4.
    const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        reinterpret_cast<__attribute__((address_space(3))) i16x4_t *>(const_cast<lds_u8 *>(base) + off));
    return __builtin_bit_cast(u32x2_t, v);
}

// HBM -> LDS DMA: lane l writes `bytes` bytes at LDS address m0 + bytes*l.
// Issued through inline assembly so that the compiler does not take later
// LDS reads as dependent on it: it cannot tell the two tile buffers apart
// and would wait for every DMA in flight before the V transpose reads,
// halving the time a tile load has to arrive.  The kernel orders these
// writes itself (s_waitcnt vmcnt, then a workgroup barrier, before a buffer
// is read).  One wait state separates the M0 write from the DMA.
__device__ __forceinline__ void dma16_saddr(const void *base, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
                 :
                 : "s"(lds), "v"(voff), "s"(base)
                 : "memory", "m0");
}
__device__ __forceinline__ void dma16(const void *addr, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                 :
                 : "s"(lds), "v"(addr)
                 : "memory", "m0");
}
// Wait until every vector-memory operation of this wave has completed.  The
// inline-assembly wait covers the DMA above, which the compiler does not
// see; the builtin tells the compiler's own bookkeeping that nothing is in
// flight any more, so it adds no waits of its own later.
__device__ __forceinline__ void wait_vmem_all() {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0x0F70); // vmcnt(0), expcnt and lgkmcnt unconstrained
}
__device__ __forceinline__ uint32_t lds_addr(const __attribute__((address_space(3))) uint8_t *p) {
    return uint32_t(reinterpret_cast<uintptr_t>(p));
}

} // namespace exattn
