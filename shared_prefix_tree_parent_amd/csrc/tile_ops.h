// LDS tiles and bf16 MFMA operand helpers for gfx950 (CDNA4), shared by device sources.
//
// Tiles are row-major [rows][D] bf16 in LDS; the 16-byte chunks of each row are permuted by
// XOR with sw(row), exactly as the HBM rows are copied in.  sw is chosen so that both kinds of
// fragment read hit distinct LDS banks (a row read: 32 rows, one chunk each; a transposed
// read: 4 rows x 64 bytes per half-wave), and so that it repeats every 16 rows: row offsets
// that are multiples of 16 become instruction immediates.
//
// 32x32x16 bf16 MFMA: lane l supplies A[m = l%32][k = 8(l/32) .. +7] and B[k = 8(l/32) .. +7]
// [n = l%32]; accumulator element i of lane l is C[8(i/4) + 4(l/32) + i%4][l%32].  acc_frag
// turns accumulator registers 8 ks .. 8 ks + 7 into a B operand whose k slots hold the rows
// 16 ks + 4(l/32) + {0..3} and 16 ks + 8 + 4(l/32) + {0..3}; an A operand paired with it must
// supply the same k order (Tile::perm_frag / Tile::tr_frag).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>
#include <utility>

namespace treeattn {
namespace tile {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef int int32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ floatx16 zero16() {
    floatx16 z;
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = 0.f;
    return z;
}

__device__ __forceinline__ floatx16 mfma(bf16x8_t a, bf16x8_t b, floatx16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Calls f(std::integral_constant<int, I>) for I = 0 .. N-1: compile-time indices, so register
// arrays indexed by them stay in registers.
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F &&f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// bf16 operand from accumulator registers 8 ks .. 8 ks + 7.
__device__ __forceinline__ bf16x8_t acc_frag(const floatx16 &x, int ks) {
    bf16x8_t f;
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = static_cast<__bf16>(x[8 * ks + e]);
    return f;
}

template <int D>
struct Tile {
    static constexpr int CPR = D / 8;                 // 16-byte chunks per row
    static constexpr int ROWB = D * 2;                // bytes per row
    static constexpr int NDS = D / 16;                // k-steps over D per 32x32x16 MFMA
    static constexpr int NDB = D / 32;                // 32-wide column blocks
    static __device__ __forceinline__ int sw(int row) {
        if constexpr (CPR == 16) return (row & 15) ^ ((row & 3) << 2);
        else return ((row >> 1) & 7) ^ (((row >> 1) & 1) << 2);
    }
    // Byte offset of the chunk that holds (row, 8-element column group c).
    static __device__ __forceinline__ int chunk_at(int row, int c) { return row * ROWB + ((c ^ sw(row)) << 4); }
    // Row operand of rows rb + l%32 (A rows or B columns), k = columns 16 ds + 8 (l/32) .. +7.
    static __device__ __forceinline__ bf16x8_t row_frag(const char *tile, int rb, int lane, int ds) {
        return *reinterpret_cast<const bf16x8_t *>(tile + chunk_at(rb + (lane & 31), 2 * ds + (lane >> 5)));
    }
    // A operand of rows rb + l%32 whose k slots are columns 16 c16 + 4(l/32) + {0..3} and
    // 16 c16 + 8 + 4(l/32) + {0..3} (the order acc_frag gives a B operand).
    static __device__ __forceinline__ bf16x8_t perm_frag(const char *tile, int rb, int lane, int c16) {
        const int row = rb + (lane & 31), h = lane >> 5;
        const bf16x4_t y0 = *reinterpret_cast<const bf16x4_t *>(tile + chunk_at(row, 2 * c16) + 8 * h);
        const bf16x4_t y1 = *reinterpret_cast<const bf16x4_t *>(tile + chunk_at(row, 2 * c16 + 1) + 8 * h);
        return __builtin_shufflevector(y0, y1, 0, 1, 2, 3, 4, 5, 6, 7);
    }
    // Transposed A operand of a 32-row block at rb: lane l holds column 32 db + l%32 of rows
    // rb + 16 ks + 4(l/32) + 0..3 and rb + 16 ks + 8 + 4(l/32) + 0..3 (two LDS transpose reads).
    static __device__ __forceinline__ bf16x8_t tr_frag(const char *tile, int rb, int lane, int ks, int db) {
        typedef shortx4 __attribute__((address_space(3))) *lds_p;
        const int grp = lane >> 4, j = lane & 15, h = grp >> 1;
        const int col = 32 * db + 16 * (grp & 1) + 4 * (j & 3);
        bf16x4_t y[2];
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int row = rb + 16 * ks + 8 * r + 4 * h + (j >> 2);
            const char *p = tile + chunk_at(row, col >> 3) + (col & 7) * 2;
            y[r] = __builtin_bit_cast(bf16x4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_p)(p)));
        }
        return __builtin_shufflevector(y[0], y[1], 0, 1, 2, 3, 4, 5, 6, 7);
    }
    // Element (row, col) of the tile.
    static __device__ __forceinline__ float at(const char *tile, int row, int col) {
        return float(*reinterpret_cast<const __bf16 *>(tile + chunk_at(row, col >> 3) + (col & 7) * 2));
    }
    // Split forms of row_frag / tr_frag for kernels that keep the lane part of every address
    // in a register and add the rest as an instruction immediate.
    // Row operand: lane part for block row 0; add 32 * block * ROWB.
    static __device__ __forceinline__ int row_lane(int lane, int ds) {
        return chunk_at(lane & 31, 2 * ds + (lane >> 5));
    }
    // Transposed operand, read r (0, 1) of the two: in each 16-lane group, lane j points at row
    // 8 r + 4 h + j/4, columns 4(j%4) .. +3 of a 16-column group and receives one column of 4
    // rows.  Lane part for block row 0, ks = 0; add (32 * block + 16 ks) * ROWB.
    static __device__ __forceinline__ int tr_lane(int lane, int db, int r) {
        const int grp = lane >> 4, j = lane & 15, h = grp >> 1;
        const int col = 32 * db + 16 * (grp & 1) + 4 * (j & 3);
        return chunk_at(8 * r + 4 * h + (j >> 2), col >> 3) + (col & 7) * 2;
    }
    static __device__ __forceinline__ bf16x8_t row_at(const char *p) {
        return *reinterpret_cast<const bf16x8_t *>(p);
    }
    static __device__ __forceinline__ bf16x8_t tr_at(const char *p0, const char *p1) {
        typedef shortx4 __attribute__((address_space(3))) *lds_p;
        const bf16x4_t y0 = __builtin_bit_cast(bf16x4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_p)(p0)));
        const bf16x4_t y1 = __builtin_bit_cast(bf16x4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_p)(p1)));
        return __builtin_shufflevector(y0, y1, 0, 1, 2, 3, 4, 5, 6, 7);
    }
};

// Per-lane parts of the fragment addresses of a Tile<D> (computed once per kernel).
template <int D>
struct LaneOffsets {
    int row[Tile<D>::NDS];
    int tr[Tile<D>::NDB][2];
    __device__ __forceinline__ explicit LaneOffsets(int lane) {
#pragma unroll
        for (int ds = 0; ds < Tile<D>::NDS; ++ds) row[ds] = Tile<D>::row_lane(lane, ds);
#pragma unroll
        for (int db = 0; db < Tile<D>::NDB; ++db) {
            tr[db][0] = Tile<D>::tr_lane(lane, db, 0);
            tr[db][1] = Tile<D>::tr_lane(lane, db, 1);
        }
    }
};

// Direct-to-LDS buffer loads, issued as inline asm so that the compiler does not wait for them
// before unrelated LDS reads (it cannot tell which LDS bytes they write).  Offsets past
// num_records read as zeros.
constexpr int kBufFlags = 0x00020000;
__device__ __forceinline__ int32x4_t buf_rsrc(const void *base, uint32_t num_records) {
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    int32x4_t r;
    r[0] = __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(b)));
    r[1] = __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(b >> 32) & 0xffffu));
    r[2] = __builtin_amdgcn_readfirstlane(static_cast<int>(num_records));
    r[3] = kBufFlags;
    return r;
}
// The LDS address is wave-uniform; readfirstlane keeps it in an SGPR for the "s" operand.
// The asm writes M0 and names it as clobbered.  The compiler warns that it does not save a
// reserved register around such a statement; nothing needs saving, because no code in these
// kernels keeps a value in M0 across them (on gfx950 M0 is read only by LDS-DMA, GWS, message
// and interpolation instructions, and the only LDS-DMA loads are these).
__device__ __forceinline__ void buf_to_lds16(int32x4_t r, uint32_t lds, int voff) {
    const uint32_t m = __builtin_amdgcn_readfirstlane(lds);
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %2, %0, 0 offen lds"
                 :: "s"(r), "s"(m), "v"(voff) : "memory", "m0");
}
__device__ __forceinline__ void buf_to_lds4(int32x4_t r, uint32_t lds, int voff) {
    const uint32_t m = __builtin_amdgcn_readfirstlane(lds);
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dword %2, %0, 0 offen lds"
                 :: "s"(r), "s"(m), "v"(voff) : "memory", "m0");
}
__device__ __forceinline__ uint32_t lds_base(const char *p) {
    return __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(
        reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char *)p)));
}
// Wait until this wave's vector loads (including the ones into LDS) have landed, or all but
// the newest N of them (vmcnt; lgkmcnt and expcnt are not waited for).
__device__ __forceinline__ void wait_loads() { __builtin_amdgcn_s_waitcnt(0x0f70); }
template <int N>
__device__ __forceinline__ void wait_loads_but() {
    static_assert(N >= 0 && N < 64, "vmcnt field (6 bits: immediate bits 3:0 and 15:14)");
    __builtin_amdgcn_s_waitcnt(0x0f70 | (N & 15) | ((N >> 4) << 14));
}
__device__ __forceinline__ void block_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Resource for a tile of rows with HBM row stride `stride` bytes whose rows past n_valid read
// as zero.
__device__ __forceinline__ int32x4_t tile_rsrc(const char *src, int n_valid, int stride) {
    return buf_rsrc(src, uint32_t(n_valid > 0 ? n_valid : 0) * uint32_t(stride));
}
// One 1 KB instruction of a tile copy: block blk (1024 / (2 D) rows) into the swizzled LDS tile
// at dst.
template <int D>
__device__ __forceinline__ void copy_block(int32x4_t rs, int stride, uint32_t dst, int blk, int lane) {
    using TL = Tile<D>;
    constexpr int ROWS_PER_KB = 1024 / (D * 2);
    const int row = blk * ROWS_PER_KB + lane / TL::CPR;
    const int c = (lane % TL::CPR) ^ TL::sw(row);
    buf_to_lds16(rs, dst + blk * 1024, row * stride + c * 16);
}
// Copy `rows` rows of D bf16 (HBM row stride `stride` bytes, rows past n_valid read as zero)
// into a swizzled LDS tile; the nw waves of the workgroup split the 1 KB instructions.
template <int D>
__device__ __forceinline__ void copy_tile(const char *src, int n_valid, int stride, uint32_t dst, int rows,
                                          int wave, int nw, int lane) {
    constexpr int ROWS_PER_KB = 1024 / (D * 2);
    const int32x4_t rs = tile_rsrc(src, n_valid, stride);
    for (int blk = wave; blk < rows / ROWS_PER_KB; blk += nw) copy_block<D>(rs, stride, dst, blk, lane);
}

}  // namespace tile
}  // namespace treeattn
