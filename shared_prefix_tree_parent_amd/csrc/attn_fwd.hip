// Tree-masked attention forward for gfx950 (CDNA4): QK^T and PV on MFMA, K/V tiles staged in
// LDS, online softmax, grouped-query head mapping, FULL / PARTIAL / SKIP tile dispatch.
//
// What is computed ("Prefix tree packing", furtherai.github.io, attention-mask passage; "ART-
// Optimized Megatron (AOM)", section "How do we implement shared prefix?"): every real token
// attends to itself, the earlier tokens of its segment and all tokens of its ancestor
// segments, and nothing else:  O = softmax(scale * q k^T over visible keys) v,  LSE = log-sum-
// exp of the visible scores.  Key j is visible to query i iff j <= i < kend[j] (pre-order
// interval form of the page's [enter, exit] ancestor test); FULL tiles skip the test, PARTIAL
// tiles apply it, SKIP tiles are never visited (the mask passage's block skipping).
//
// Work decomposition: one workgroup owns 256 (query head, position) rows = 8 blocks of 32.
//   * item = (row, q-tile of BQ positions, KV head g, chunk of HCH query heads of group g);
//     BQ * HCH = 256, so every item owns the same number of rows and each staged K/V tile is
//     shared by all HCH heads of the group (grouped-query reuse);
//   * 8 waves, one 32-row block each, two waves per SIMD: while one wave runs its softmax on
//     the VALU the other's MFMAs issue (the template also allows 4 waves of two blocks);
//   * K/V tiles (64 keys) are copied HBM -> LDS with direct-to-LDS loads into four buffer
//     slots, two tiles ahead, so the copies run under the compute with no registers; one wave
//     per SIMD issues them.
// MFMA orientation: S^T = K Q^T and O^T = V^T P^T, so each lane owns one query (column) of
// every 32x32 accumulator: row max / row sum are in-lane plus one exchange with lane^32
// (v_permlane32_swap), and the P^T operand of the second product is the first product's
// accumulator, converted in place.  V stays row-major in LDS; its V^T operand comes from
// LDS transpose reads (ds_read_b64_tr_b16).
// Softmax: the reference max only moves when a tile's max exceeds it by more than 2^8 in
// the exponent domain (a wave-uniform branch), so the accumulator rescale is rare; O is
// normalized by the sum of the bf16-rounded weights actually fed to the MFMA, and the LSE is
// the log of that same sum (the normalizer of the weights O was made from; an fp32 sum beside
// it would cost one add per score).  The fp32 instantiation sums the weights in fp32.
// Scheduling: persistent workgroups, about one per CU.  Workgroup b serves KV lane
// b % n_kv_lanes and takes that lane's items one after another, in work-list order (rows in
// order, a row's q-tiles longest list first), from a counter in the workspace; with 8 KV
// heads every XCD (blockIdx round-robin over 8 XCDs) works on one KV head and keeps that
// head's K/V in its own L2.  O leaves through LDS as whole rows.
#include <algorithm>
#include <type_traits>

#include "internal.h"
#include "tile_ops.h"

namespace treeattn {
namespace {

using tile::bf16x8_t;
using tile::floatx16;

struct FwdArgs {
    const void *q, *k, *v;
    void *o;
    float *lse;
    const int32_t *qt_ptr, *kt_idx;
    const uint8_t *kt_kind;
    const int32_t *kend, *work, *n_real, *status;
    int32_t *ctr;         // [2 L]: items handed out per lane, then workgroups finished per lane
    int32_t n_items;      // rows * q-tiles
    int32_t T, Hq, Hkv, G, HCH, nQ, L, BQ;
    float c;       // scale * log2(e): exponent scale for exp2
    float scale;   // softmax scale (for the natural-log LSE)
};

using tile::block_barrier;
using tile::buf_rsrc;
using tile::buf_to_lds16;
using tile::buf_to_lds4;
using tile::int32x4_t;
using tile::static_for;
using tile::wait_loads;
using tile::wait_loads_but;
using tile::zero16;

// Next item of a lane's queue (device-scope counter; values come in work-list order).
__device__ __forceinline__ int fetch_add(int32_t *p) {
    return __hip_atomic_fetch_add(p, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Wait until this wave's LDS reads and writes have completed (vmcnt, expcnt not waited for).
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xc07f); }

// ----------------------------------------------------------------------------- element traits
//
// K and V tiles live in LDS row-major ([64 keys][D]) exactly as in HBM, with the 16-byte chunk
// index of each row XOR-swizzled (ksw / vsw) so the fragment reads below are bank-conflict
// free; tiles are copied HBM -> LDS with direct-to-LDS loads (no registers involved).

template <int D_>
struct Bf16Traits {
    static constexpr int D = D_;
    static constexpr int kEsz = 2;
    static constexpr int NDS = D / 16;        // MFMA k-steps over head_dim for S^T
    static constexpr int NKS = 2;             // MFMA k-steps per 32-key block for O^T
    static constexpr int NDB = D / 32;        // 32-row blocks of O^T
    static constexpr int CPR = D / 8;         // 16-byte chunks per K/V row
    using frag = bf16x8_t;
    using elem = uint16_t;

    static __device__ __forceinline__ floatx16 mfma(frag a, frag b, floatx16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    // K reads: a half-wave reads one chunk of 32 consecutive keys -> spread chunks by key.
    static __device__ __forceinline__ int ksw(int row) { return row & (CPR - 1); }
    // V reads: a wave reads 4 chunks of 8 consecutive keys (4 per half) -> spread by key & 3.
    static __device__ __forceinline__ int vsw(int row) { return (4 * (row & 3)) & (CPR - 1); }
    static __device__ __forceinline__ frag k_frag(const elem *K, int key, int ds, int h) {
        return *reinterpret_cast<const frag *>(K + key * D + (((2 * ds + h) ^ ksw(key)) << 3));
    }
    // V^T operand of O^T = V^T P^T for d-block db, key step ks of 32-key block kb.  Two LDS
    // transpose reads: in each 16-lane group, lane j points at row K0 + j/4, columns
    // dbase + 4 (j%4) .. +3, and receives column dbase + j of rows K0 .. K0+3, so lane l holds
    // V[key][d = 32 db + l%32] for the 8 keys its P^T operand covers (keys 16ks + 4h + 0..3
    // and 16ks + 8 + 4h + 0..3 of the block, h = lane / 32).
    static __device__ __forceinline__ frag v_frag(const elem *V, int lane, int db, int kb, int ks) {
        const int grp = lane >> 4, j = lane & 15, h = grp >> 1;
        const int d = 32 * db + 16 * (grp & 1) + 4 * (j & 3);
        typedef short shortx4 __attribute__((ext_vector_type(4)));
        typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
        typedef shortx4 __attribute__((address_space(3))) *lds_p;
        bf16x4_t y[2];
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int row = 32 * kb + 16 * ks + 8 * r + 4 * h + (j >> 2);
            const elem *p = V + row * D + (((d >> 3) ^ vsw(row)) << 3) + (d & 7);
            // whole-vector bit cast (a bit cast of a single vector element is not used)
            y[r] = __builtin_bit_cast(bf16x4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_p)(p)));
        }
        return __builtin_shufflevector(y[0], y[1], 0, 1, 2, 3, 4, 5, 6, 7);
    }
    static __device__ __forceinline__ frag q_frag(const elem *q, int ds, int h) {
        return *reinterpret_cast<const frag *>(q + (2 * ds + h) * 8);
    }
    // Byte offsets inside a K / V tile split into a lane part (kept in a register) and a
    // compile-time part (the instruction's immediate offset).
    static constexpr int K_KB_BYTES = 32 * D * kEsz;
    static __device__ __forceinline__ int k_lane(int ds, int l32, int h) {
        return l32 * D * kEsz + (((2 * ds + h) ^ ksw(l32)) << 4);
    }
    static __device__ __forceinline__ frag k_frag_at(const char *p) { return *reinterpret_cast<const frag *>(p); }
    static __device__ __forceinline__ int v_lane(int db, int lane) {
        const int grp = lane >> 4, j = lane & 15, h = grp >> 1;
        const int row0 = 4 * h + (j >> 2), d = 32 * db + 16 * (grp & 1) + 4 * (j & 3);
        return (row0 * D + (((d >> 3) ^ vsw(row0)) << 3) + (d & 7)) * kEsz;
    }
    static constexpr int v_imm(int kb, int ks, int r) { return (32 * kb + 16 * ks + 8 * r) * D * kEsz; }
    template <int KB, int KS>
    static __device__ __forceinline__ frag v_frag_at(const char *p) {
        typedef short shortx4 __attribute__((ext_vector_type(4)));
        typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
        typedef shortx4 __attribute__((address_space(3))) *lds_p;
        const bf16x4_t y0 = __builtin_bit_cast(bf16x4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_p)(p + v_imm(KB, KS, 0))));
        const bf16x4_t y1 = __builtin_bit_cast(bf16x4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_p)(p + v_imm(KB, KS, 1))));
        return __builtin_shufflevector(y0, y1, 0, 1, 2, 3, 4, 5, 6, 7);
    }
    // P^T operand for key step ks of a 32-key block: accumulator registers 8ks .. 8ks+7.
    static __device__ __forceinline__ frag p_frag(const floatx16 &p, int ks) {
        frag f;
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = static_cast<__bf16>(p[8 * ks + e]);
        return f;
    }
    // Sum of the (rounded) weights one P^T operand feeds to the MFMA, added to acc.
    static __device__ __forceinline__ float wsum(frag f, float acc) {
        typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
        const bf16x2_t one2 = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(f, f, 0, 1), one2, acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(f, f, 2, 3), one2, acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(f, f, 4, 5), one2, acc, false);
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(f, f, 6, 7), one2, acc, false);
        return acc;
    }
    static constexpr bool kRoundedP = true;
};

template <int D_>
struct F32Traits {
    static constexpr int D = D_;
    static constexpr int kEsz = 4;
    static constexpr int NDS = D / 2;
    static constexpr int NKS = 16;
    static constexpr int NDB = D / 32;
    static constexpr int CPR = D / 4;
    using frag = float;
    using elem = float;

    static __device__ __forceinline__ floatx16 mfma(frag a, frag b, floatx16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ int ksw(int row) { return row & (CPR - 1); }
    static __device__ __forceinline__ int vsw(int) { return 0; }
    static __device__ __forceinline__ frag k_frag(const elem *K, int key, int ds, int h) {
        const int col = 2 * ds + h;
        return K[key * D + (((col >> 2) ^ ksw(key)) << 2) + (col & 3)];
    }
    // key of lane-half h, element of key step ks inside a 32-key block (accumulator layout).
    static __device__ __forceinline__ frag v_frag(const elem *V, int lane, int db, int kb, int ks) {
        const int key = 32 * kb + 8 * (ks >> 2) + 4 * (lane >> 5) + (ks & 3);
        return V[key * D + 32 * db + (lane & 31)];
    }
    static __device__ __forceinline__ frag q_frag(const elem *q, int ds, int h) { return q[2 * ds + h]; }
    static constexpr int K_KB_BYTES = 32 * D * kEsz;
    static __device__ __forceinline__ int k_lane(int ds, int l32, int h) {
        const int col = 2 * ds + h;
        return l32 * D * kEsz + ((((col >> 2) ^ ksw(l32)) << 2) + (col & 3)) * kEsz;
    }
    static __device__ __forceinline__ frag k_frag_at(const char *p) { return *reinterpret_cast<const frag *>(p); }
    static __device__ __forceinline__ int v_lane(int db, int lane) {
        return (4 * (lane >> 5) * D + 32 * db + (lane & 31)) * kEsz;
    }
    template <int KB, int KS>
    static __device__ __forceinline__ frag v_frag_at(const char *p) {
        return *reinterpret_cast<const frag *>(p + (32 * KB + 8 * (KS >> 2) + (KS & 3)) * D * kEsz);
    }
    static __device__ __forceinline__ frag p_frag(const floatx16 &p, int ks) { return p[ks]; }
    static __device__ __forceinline__ float wsum(frag f, float acc) { return acc + f; }
    static constexpr bool kRoundedP = false;
};

// LDS layout: four K tiles, then four V tiles, then the four tiles' kend (64 ints each), four
// control words, then the q-tile's k-tile list.  Tile t lives in buffer slot t % 4.  With K and V in regions of
// their own, every fragment read inside a 64 KB region is one per-lane base register plus an
// instruction immediate (slot and block offsets are compile-time), so reads cost no address
// arithmetic.
template <class Tr>
struct Lds {
    static constexpr int NBUF = 4;
    static constexpr int TILE = 64 * Tr::D * Tr::kEsz;   // one K (or V) tile of 64 keys
    static constexpr int K_OFF = 0;
    static constexpr int V_OFF = NBUF * TILE;
    static constexpr int KE_OFF = 2 * NBUF * TILE;
    static constexpr int CTRL_OFF = KE_OFF + NBUF * 256;
    static constexpr int LIST_OFF = CTRL_OFF + 16;
    static_assert(NBUF * TILE <= 65536, "a region must be reachable by 16-bit LDS offsets");
};

#ifndef TREEATTN_FWD_BLOCKS_PER_WAVE
#define TREEATTN_FWD_BLOCKS_PER_WAVE 1
#endif
constexpr int kNBlk = TREEATTN_FWD_BLOCKS_PER_WAVE;   // 32-row blocks per wave
constexpr int kWaves = 8 / kNBlk;                     // 256 rows per workgroup

// Maxima use IEEE maximum (NaN-propagating; v_maximum3_f32 on gfx950), which needs no
// canonicalizing moves in front of each operand, unlike fmaxf in IEEE mode.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float xchg_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xchg_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// Max of elements [8i, 8i+8) of x as a tree (short dependency chains).
__device__ __forceinline__ float max8(const floatx16 &x, int i) {
    const float a = vmax(vmax(x[8 * i + 0], x[8 * i + 1]), x[8 * i + 2]);
    const float b = vmax(vmax(x[8 * i + 3], x[8 * i + 4]), x[8 * i + 5]);
    return vmax(vmax(a, b), vmax(x[8 * i + 6], x[8 * i + 7]));
}

// ------------------------------------------------------------------------------------ kernel
//
// A workgroup takes items one at a time; an item = 256 (query head, position) rows = 8 blocks
// of 32.  By default 8 waves own one block each, two waves per SIMD; built with
// TREEATTN_FWD_BLOCKS_PER_WAVE=2 it is 4 waves of two blocks (one per SIMD), where every K / V
// fragment read from LDS feeds two MFMAs.
//
// Software pipeline over 32-key steps.  Step u covers block u % 2 (32 keys) of the u / 2-th
// k-tile of the q-tile's list.  In step u a wave issues the MFMAs of S(u+1) = K Q^T and of
// O^T += V^T P^T for step u-1, and, slot by slot between them, the VALU softmax of S(u)
// (computed in step u-1) that yields the P^T operands of step u: the softmax runs under the
// wave's own MFMAs.  Two register sets hold S and P (A: even steps, B: odd steps); one loop
// iteration = one 64-key tile = an even and an odd step, so the sets swap roles without
// copies.  K/V tiles are copied HBM -> LDS two tiles ahead; one barrier per tile.
template <class Tr>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(kWaves / 4, kWaves / 4)))
void tree_attn_fwd_kernel(FwdArgs a) {
    using elem = typename Tr::elem;
    using frag = typename Tr::frag;
    using LD = Lds<Tr>;
    constexpr int D = Tr::D;
    constexpr int NB = LD::NBUF;
    // Grow the reference max only when a block's max exceeds it by more than 2^8 in the
    // exponent domain; otherwise keep the stale reference (weights stay <= 256), which spares
    // the accumulator rescale.
    constexpr float kGrow = 8.0f;

    extern __shared__ __attribute__((aligned(1024))) char smem[];

    if (a.status[0] != 0) return;   // invalid segment table: write nothing

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, h = lane >> 5;
    const int u = blockIdx.x % a.L;
    const int g = u % a.Hkv, chunk = u / a.Hkv;
    int32_t *const take = a.ctr + u;          // items of this lane handed out after the first round
    int32_t *const done = a.ctr + a.L + u;    // workgroups of this lane finished
    int32_t *const ctrl = reinterpret_cast<int32_t *>(smem + LD::CTRL_OFF);
    // Workgroups on this lane; the k-th of them starts with the lane's k-th item, and the rest
    // are handed out by the counter (so the launch does not start with every workgroup
    // contending for it).
    const int n_wg = int(gridDim.x) / a.L + (u < int(gridDim.x) % a.L ? 1 : 0);
    int item = blockIdx.x / a.L;
    while (item < a.n_items) {
    const int tile = a.work[item];
    const int r = tile / a.nQ, qt = tile % a.nQ;
    const int T = a.T;
    const int n_real = a.n_real[r];

    // The wave's two row blocks: block b -> query head of the group (b % HCH) and 32 positions.
    int head[kNBlk], qpos[kNBlk];
#pragma unroll
    for (int j = 0; j < kNBlk; ++j) {
        const int b = kNBlk * wave + j;
        head[j] = g * a.G + chunk * a.HCH + b % a.HCH;
        qpos[j] = qt * a.BQ + (b / a.HCH) * 32 + l32;
    }

    // Q fragments (B operand of S^T = K Q^T): lane holds query l32, head_dim chunk (2ds + h).
    frag qf[kNBlk][Tr::NDS];
#pragma unroll
    for (int j = 0; j < kNBlk; ++j) {
        const elem *qrow = reinterpret_cast<const elem *>(a.q) + ((int64_t(r) * T + qpos[j]) * a.Hq + head[j]) * D;
#pragma unroll
        for (int ds = 0; ds < Tr::NDS; ++ds) qf[j][ds] = Tr::q_frag(qrow, ds, h);
    }

    floatx16 acc[kNBlk][Tr::NDB];
#pragma unroll
    for (int j = 0; j < kNBlk; ++j)
#pragma unroll
        for (int db = 0; db < Tr::NDB; ++db) acc[j][db] = zero16();
    // m_run: reference max (raw score units); w_run: sum of the weights as rounded for the PV
    // product (normalizes O, so the weights applied to V sum to one exactly as used, and gives
    // the LSE); l_run: fp32 sum of the exponentials, kept only where P is not rounded.
    float m_run[kNBlk], l_run[kNBlk], w_run[kNBlk];
#pragma unroll
    for (int j = 0; j < kNBlk; ++j) {
        m_run[j] = -INFINITY;
        l_run[j] = 0.f;
        w_run[j] = 0.f;
    }

    const int32_t t_begin = a.qt_ptr[tile];
    const int N = a.qt_ptr[tile + 1] - t_begin;
    // The q-tile's k-tile list (index * 4 + kind), staged in LDS: list reads in the loop are
    // LDS reads, never a vector-memory wait that would also wait for the K/V copies in flight.
    int32_t *const lst = reinterpret_cast<int32_t *>(smem + LD::LIST_OFF);
    for (int i = tid; i < N; i += kWaves * 64) lst[i] = a.kt_idx[t_begin + i] * 4 + a.kt_kind[t_begin + i];
    wait_lds();
    block_barrier();

    const int row_stride = a.Hkv * D * Tr::kEsz;   // bytes between keys
    const char *kbase0 = reinterpret_cast<const char *>(a.k) + ((int64_t(r) * T) * a.Hkv + g) * D * Tr::kEsz;
    const char *vbase0 = reinterpret_cast<const char *>(a.v) + ((int64_t(r) * T) * a.Hkv + g) * D * Tr::kEsz;
    const int32_t *kend_row = a.kend + int64_t(r) * T;

    // Copy plan of one 64-key tile: one wave instruction moves 64 chunks of 16 bytes into 1 KB
    // of consecutive LDS (lane l at byte 16 l); each lane's source is the chunk that belongs
    // there after swizzling.  The per-lane source offsets never change; the tile base lives in
    // the buffer descriptor, whose size stops at the row's last real key, so pad keys read as
    // zeros (NaN pads cannot reach PV).
    // Copying waves: one per SIMD (waves 0-3 sit on SIMDs 0-3).  A wave that issues a
    // direct-to-LDS copy waits while the CU's memory pipeline is full; with one copying wave per
    // SIMD the other wave of the SIMD keeps issuing meanwhile.
    constexpr int kCW = kWaves >= 8 ? kWaves / 2 : kWaves;
    const bool cw = wave < kCW;
    constexpr int ROWS = 1024 / (D * Tr::kEsz), INSTR = LD::TILE / 1024, PER_WAVE = 2 * INSTR / kCW;
    static_assert((2 * INSTR) % kCW == 0, "waves must split the tile evenly");
    static_assert(PER_WAVE + 1 < 16, "vmcnt field");
    int voff[PER_WAVE];
#pragma unroll
    for (int jj = 0; jj < PER_WAVE; ++jj) {
        const bool isv = jj >= INSTR / kCW;
        const int blk = isv ? wave + kCW * (jj - INSTR / kCW) : wave + kCW * jj;
        const int row = blk * ROWS + lane / Tr::CPR;
        const int c = (lane % Tr::CPR) ^ (isv ? Tr::vsw(row) : Tr::ksw(row));
        voff[jj] = row * row_stride + c * 16;
    }
    // LDS byte address of smem (the dynamic allocation starts at LDS address 0 in practice;
    // taken from the pointer to stay correct either way).
    const uint32_t lds0 = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(
        reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char *)smem)));
    auto issue = [&](int t) __attribute__((always_inline)) {
        const int kt = __builtin_amdgcn_readfirstlane(lst[t]) >> 2;
        const int slot = t & (NB - 1);
        const int n_valid = __builtin_amdgcn_readfirstlane(min(max(n_real - kt * 64, 0), 64));
        const int64_t tb = int64_t(kt) * 64 * row_stride;
        const int32x4_t rk = buf_rsrc(kbase0 + tb, n_valid * row_stride);
        const int32x4_t rv = buf_rsrc(vbase0 + tb, n_valid * row_stride);
        if (cw) {
#pragma unroll
            for (int jj = 0; jj < PER_WAVE; ++jj) {
                const bool isv = jj >= INSTR / kCW;
                const int blk = isv ? wave + kCW * (jj - INSTR / kCW) : wave + kCW * jj;
                const uint32_t dst = lds0 + (isv ? LD::V_OFF : LD::K_OFF) + slot * LD::TILE + blk * 1024;
                buf_to_lds16(isv ? rv : rk, dst, voff[jj]);
            }
        }
        if (wave == kCW - 1)
            buf_to_lds4(buf_rsrc(kend_row + kt * 64, 256), lds0 + LD::KE_OFF + slot * 256, lane * 4);
    };

    // Lane-dependent byte offsets of the K / V fragments inside a tile (loop invariant).
    int klane[Tr::NDS], vlane[Tr::NDB];
#pragma unroll
    for (int ds = 0; ds < Tr::NDS; ++ds) klane[ds] = Tr::k_lane(ds, l32, h);
#pragma unroll
    for (int db = 0; db < Tr::NDB; ++db) vlane[db] = LD::V_OFF + Tr::v_lane(db, lane);   // V region base folded in

    constexpr int NLOAD = 2 * Tr::NDS;          // fragment loads per step: K and V alternate
    static_assert(Tr::NDS == Tr::NDB * Tr::NKS, "S and PV fragments of a step must pair up");
    static_assert(NLOAD >= 8, "the softmax needs at least 8 load slots per step");
    constexpr int EPF = 16 / Tr::NKS;           // accumulator elements per P^T operand
    constexpr int kAhead = 8;                   // LDS fragment reads issued this many slots early
    static_assert(NLOAD % kAhead == 0, "the ring carries over steps only when kAhead divides NLOAD");
    floatx16 sA[kNBlk], sB[kNBlk];
    frag pA[kNBlk][Tr::NKS], pB[kNBlk][Tr::NKS];
    bool pending = false;                       // the last step grew the reference max of a lane
    float alpha_p[kNBlk];                       // ... by these factors (1 where not grown)
    // mc: the reference in exp2 units (0 while it is -inf); thr: the raw score that would
    // grow it (m_run + 8 / c, -inf at first so the first visible score sets it)
    float mc[kNBlk], thr[kNBlk];
    const float grow_raw = kGrow / a.c;
#pragma unroll
    for (int j = 0; j < kNBlk; ++j) {
        alpha_p[j] = 1.f;
        mc[j] = 0.f;
        thr[j] = -INFINITY;
    }

    // Step u-1 of step 0 (the first 32 keys) multiplies zero weights by V block 1 of slot
    // NB-1; clear that block so it holds finite values.
    {
        char *z = smem + LD::V_OFF + (NB - 1) * LD::TILE + 32 * D * Tr::kEsz;
        for (int off = tid * 16; off < 32 * D * Tr::kEsz; off += kWaves * 64 * 16)
            *reinterpret_cast<uint4 *>(z + off) = make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int j = 0; j < kNBlk; ++j)
#pragma unroll
        for (int ks = 0; ks < Tr::NKS; ++ks) {
            if constexpr (Tr::kRoundedP) {
#pragma unroll
                for (int e = 0; e < EPF; ++e) pB[j][ks][e] = static_cast<__bf16>(0.f);
            } else {
                pB[j][ks] = frag{};
            }
        }

    // Interval mask of key block KB of tile t on both row blocks: key j is visible to query i
    // iff j <= i < kend[j].  Register i holds key 32 KB + 4h + 8(i/4) + i%4 of the tile, so the
    // first test is against an immediate; kend comes four keys at a time.
    auto mask = [&](auto kbc, int t, int kt, floatx16 (&sc)[kNBlk]) __attribute__((always_inline)) {
        constexpr int KB = decltype(kbc)::value;
        const int32_t *KEs = reinterpret_cast<const int32_t *>(smem + LD::KE_OFF + (t & (NB - 1)) * 256) + 4 * h;
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
            const int4 ke = *reinterpret_cast<const int4 *>(KEs + 32 * KB + 8 * i4);
            const int kev[4] = {ke.x, ke.y, ke.z, ke.w};
#pragma unroll
            for (int j = 0; j < kNBlk; ++j) {
                const int dq = qpos[j] - kt * 64 - 4 * h;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int c = 32 * KB + 8 * i4 + e;
                    const bool vis = (c <= dq) & (qpos[j] < kev[e]);
                    sc[j][4 * i4 + e] = vis ? sc[j][4 * i4 + e] : -INFINITY;
                }
            }
        }
    };
    auto rescale = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < kNBlk; ++j)
#pragma unroll
            for (int db = 0; db < Tr::NDB; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[j][db][i] *= alpha_p[j];
    };

    // LDS offsets of a step's fragments: step (t, KB) computes S(u+1) from block 1-KB of tile
    // t+KB (past the last tile: stale LDS, never used) and PV(u-1) from block 1-KB of tile
    // t-1+KB.  V offsets are relative to vlane (which holds the V region base).
    auto koff = [&](int t, int KB) __attribute__((always_inline)) {
        return LD::K_OFF + ((t + KB) & (NB - 1)) * LD::TILE + (1 - KB) * Tr::K_KB_BYTES;
    };
    auto voff_of = [&](int t, int KB) __attribute__((always_inline)) {
        return ((t + KB + NB - 1) & (NB - 1)) * LD::TILE;
    };
    // Fragment of load slot i of a step whose V block is VB: even slots K, odd slots V.
    auto load = [&](auto ic, auto vbc, int ko, int vo) __attribute__((always_inline)) -> frag {
        constexpr int i = decltype(ic)::value, n = i / 2, VB = decltype(vbc)::value;
        if constexpr (i % 2 == 0) {
            return Tr::k_frag_at(smem + klane[n] + ko);
        } else {
            constexpr int db = n % Tr::NDB, ks = n / Tr::NDB;
            return Tr::template v_frag_at<VB, ks>(smem + vlane[db] + vo);
        }
    };
    frag ring[kAhead];              // operand reads in flight, carried from step to step

    // One pipeline step (u = 2t + KB): softmax of sc = S(u) into pc; S(u+1) into sn; PV(u-1)
    // with weights pp.  VALU work is spread over the load slots: block maxima in slots 0-1,
    // the reference update in slot 2, the exponentials (with their bf16 operands and weight
    // sums) over slots 3 .. NLOAD-2.  The last kAhead slots read the first operands of the
    // next step, so no step starts by waiting for LDS.
    auto step = [&](auto kbc, int t, int ent, floatx16 (&sc)[kNBlk], floatx16 (&sn)[kNBlk],
                    frag (&pc)[kNBlk][Tr::NKS], const frag (&pp)[kNBlk][Tr::NKS]) __attribute__((always_inline)) {
        constexpr int KB = decltype(kbc)::value;
        using vb_this = std::integral_constant<int, 1 - KB>;
        using vb_next = std::integral_constant<int, KB>;          // the next step has KB' = 1 - KB
        const int ko = koff(t, KB), vo = voff_of(t, KB);
        const int tn = t + KB;                                     // tile of the next step
        const int ko_n = koff(tn, 1 - KB), vo_n = voff_of(tn, 1 - KB);
        if (pending) rescale();   // rare: the reference max grew in the previous step
        if ((ent & 3) == kTilePartial) mask(kbc, t, ent >> 2, sc);
        float mx[kNBlk][2];
        static_for<NLOAD>([&](auto ic) __attribute__((always_inline)) {
            constexpr int i = decltype(ic)::value, n = i / 2;
            const frag op = ring[i % kAhead];
            if constexpr (i + kAhead < NLOAD) ring[i % kAhead] = load(std::integral_constant<int, i + kAhead>{}, vb_this{}, ko, vo);
            else ring[i % kAhead] = load(std::integral_constant<int, i + kAhead - NLOAD>{}, vb_next{}, ko_n, vo_n);
#pragma unroll
            for (int j = 0; j < kNBlk; ++j) {
                if constexpr (i % 2 == 0) {
                    if constexpr (n == 0) sn[j] = Tr::mfma(op, qf[j][0], zero16());
                    else sn[j] = Tr::mfma(op, qf[j][n], sn[j]);
                } else {
                    constexpr int db = n % Tr::NDB, ks = n / Tr::NDB;
                    acc[j][db] = Tr::mfma(op, pp[j][ks], acc[j][db]);
                }
            }
            // Block maxima: partial maxima of 8 elements each over slots 0 and 1.
            if constexpr (i == 0 || i == 1) {
#pragma unroll
                for (int j = 0; j < kNBlk; ++j) mx[j][i] = max8(sc[j], i);
            }
            if constexpr (i == 2) {
                // Grow the reference max only when a block's max exceeds it by more than 2^8 in
                // the exponent domain; otherwise keep the stale reference (weights stay <= 256),
                // which spares the accumulator rescale.  The common case costs one compare per
                // lane against thr = m_run + 8 / c; only when some lane's partial maximum passes
                // it does the wave take the update (row max across the lane halves, alphas).
                float mxl[kNBlk];
                bool need = false;
#pragma unroll
                for (int j = 0; j < kNBlk; ++j) {
                    mxl[j] = vmax(mx[j][0], mx[j][1]);
                    need |= mxl[j] > thr[j];
                }
                pending = false;
                if (__builtin_amdgcn_ballot_w64(need) != 0) {
                    bool any_grow = false;
#pragma unroll
                    for (int j = 0; j < kNBlk; ++j) {
                        const float m = xchg_max(mxl[j]);
                        const bool grow = m * a.c > m_run[j] * a.c + kGrow;
                        const float m_new = grow ? m : m_run[j];
                        alpha_p[j] = grow ? __builtin_amdgcn_exp2f((m_run[j] - m_new) * a.c) : 1.f;
                        l_run[j] *= alpha_p[j];
                        w_run[j] *= alpha_p[j];
                        m_run[j] = m_new;
                        mc[j] = (m_new == -INFINITY ? 0.f : m_new) * a.c;
                        thr[j] = m_new + grow_raw;
                        any_grow |= grow;
                    }
                    pending = __builtin_amdgcn_ballot_w64(any_grow) != 0;
                }
            }
            static_for<16 * kNBlk>([&](auto ec) __attribute__((always_inline)) {
                constexpr int e = decltype(ec)::value, j = e % kNBlk, k = e / kNBlk;
                if constexpr (3 + (e * (NLOAD - 4)) / (16 * kNBlk) == i) {
                    const float x = __builtin_amdgcn_exp2f(fmaf(sc[j][k], a.c, -mc[j]));
                    sc[j][k] = x;
                    if constexpr (!Tr::kRoundedP) l_run[j] += x;
                    if constexpr (k % EPF == EPF - 1) {
                        pc[j][k / EPF] = Tr::p_frag(sc[j], k / EPF);
                        if constexpr (Tr::kRoundedP) w_run[j] = Tr::wsum(pc[j][k / EPF], w_run[j]);
                    }
                }
            });
            __builtin_amdgcn_sched_barrier(0);
        });
        // Keep this step's P^T operands and sums computed here: without a use at this point
        // the compiler sinks the exponentials past the next step's rescale branch, out of the
        // MFMA slots they are meant to fill.
#pragma unroll
        for (int j = 0; j < kNBlk; ++j) {
#pragma unroll
            for (int ks = 0; ks < Tr::NKS; ++ks) asm volatile("" ::"v"(pc[j][ks]));
            asm volatile("" ::"v"(Tr::kRoundedP ? w_run[j] : l_run[j]));
        }
    };

    // Prologue: tiles 0 and 1 in flight, wait for tile 0, S(0) of both blocks.
    if (N > 0) issue(0);
    if (N > 1) {
        issue(1);
        if (wave == kCW - 1) wait_loads_but<PER_WAVE + 1>();
        else if (cw) wait_loads_but<PER_WAVE>();
        else wait_loads();
    } else {
        wait_loads();
    }
    wait_lds();   // the cleared V block
    block_barrier();
    if (N > 0) {
        static_for<Tr::NDS>([&](auto nc) __attribute__((always_inline)) {
            constexpr int n = decltype(nc)::value;
            const frag op = Tr::k_frag_at(smem + klane[n] + LD::K_OFF);
#pragma unroll
            for (int j = 0; j < kNBlk; ++j) {
                if constexpr (n == 0) sA[j] = Tr::mfma(op, qf[j][0], zero16());
                else sA[j] = Tr::mfma(op, qf[j][n], sA[j]);
            }
        });
    }
    static_for<kAhead>([&](auto ic) __attribute__((always_inline)) {
        ring[decltype(ic)::value] = load(ic, std::integral_constant<int, 1>{}, koff(0, 0), voff_of(0, 0));
    });
    // NB tiles per iteration (t0 a multiple of NB), so that every buffer slot (t & (NB - 1))
    // is a compile-time constant and the fragment reads take it as an instruction immediate
    // instead of an address add per read.
    for (int t0 = 0; t0 < N; t0 += NB) {
        static_for<NB>([&](auto sc) __attribute__((always_inline)) {
            const int t = t0 + decltype(sc)::value;
            if (t >= N) return;
            // Tile t+1 (read from step 2t+1 on) must have landed, and every wave must be done
            // with tile t-2 (last read in step 2t-2) before its buffer takes tile t+2.
            if (t + 1 < N) wait_loads();
            block_barrier();
            const int ent = __builtin_amdgcn_readfirstlane(lst[t]);
            if (t + 2 < N) issue(t + 2);
            step(std::integral_constant<int, 0>{}, t, ent, sA, sB, pA, pB);
            step(std::integral_constant<int, 1>{}, t, ent, sB, sA, pB, pA);
        });
    }
    // Drain: PV of the last step (block 1 of tile N-1, weights pB).
    if (N > 0) {
        if (pending) rescale();
        const char *vb = smem + ((N - 1) & (NB - 1)) * LD::TILE;
        static_for<Tr::NDB * Tr::NKS>([&](auto nc) __attribute__((always_inline)) {
            constexpr int n = decltype(nc)::value, db = n % Tr::NDB, ks = n / Tr::NDB;
            const frag op = Tr::template v_frag_at<1, ks>(vb + vlane[db]);
#pragma unroll
            for (int j = 0; j < kNBlk; ++j) acc[j][db] = Tr::mfma(op, pB[j][ks], acc[j][db]);
        });
    }

    // Epilogue: combine the two lane halves' partial sums, normalize.
    float lse_v[kNBlk];
#pragma unroll
    for (int j = 0; j < kNBlk; ++j) {
        const float w_tot = xchg_sum(Tr::kRoundedP ? w_run[j] : l_run[j]);
        const float inv = w_tot > 0.f ? 1.f / w_tot : 0.f;
#pragma unroll
        for (int db = 0; db < Tr::NDB; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[j][db][i] *= inv;
        lse_v[j] = w_tot > 0.f ? m_run[j] * a.scale + __logf(w_tot) : -INFINITY;
    }
    // The next item, claimed before this item's stores (so that waiting for the claim does not
    // wait for them).
    int next = 0;
    if (tid == 0) next = n_wg + fetch_add(take);
    wait_lds();
    block_barrier();   // every wave is done reading this item's tiles
    {
        // O goes out through LDS as whole rows: each wave writes its 32 x D block into the K / V
        // regions of slots 0 and 1, reads it back row by row and stores 16 bytes per lane, CH
        // lanes per row.  16-byte chunks are XOR-swizzled by row.
        constexpr int ROWB = D * Tr::kEsz, CH = ROWB / 16, RPI = 64 / CH;
        // Lane index hidden from loop-invariant code motion: the staging addresses are computed
        // here, per item, instead of living (spilled) across the tile loop.
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const int p32 = ln & 31;
#pragma unroll
        for (int j = 0; j < kNBlk; ++j) {
            const int b = kNBlk * wave + j, area = b >> 1;
            char *base = smem + ((area & 1) ? LD::V_OFF : LD::K_OFF) + (area >> 1) * LD::TILE + (b & 1) * 32 * ROWB;
#pragma unroll
            for (int db = 0; db < Tr::NDB; ++db) {
#pragma unroll
                for (int i4 = 0; i4 < 4; ++i4) {
                    const int byte = (32 * db + 8 * i4 + 4 * h) * Tr::kEsz;
                    char *dst = base + p32 * ROWB + ((((byte >> 4) ^ p32) & (CH - 1)) << 4) + (byte & 15);
                    if constexpr (Tr::kEsz == 2) {
                        uint2 w;
                        w.x = uint32_t(__builtin_bit_cast(uint16_t, static_cast<__bf16>(acc[j][db][4 * i4 + 0]))) |
                              (uint32_t(__builtin_bit_cast(uint16_t, static_cast<__bf16>(acc[j][db][4 * i4 + 1]))) << 16);
                        w.y = uint32_t(__builtin_bit_cast(uint16_t, static_cast<__bf16>(acc[j][db][4 * i4 + 2]))) |
                              (uint32_t(__builtin_bit_cast(uint16_t, static_cast<__bf16>(acc[j][db][4 * i4 + 3]))) << 16);
                        *reinterpret_cast<uint2 *>(dst) = w;
                    } else {
                        *reinterpret_cast<float4 *>(dst) = make_float4(acc[j][db][4 * i4 + 0], acc[j][db][4 * i4 + 1],
                                                                       acc[j][db][4 * i4 + 2], acc[j][db][4 * i4 + 3]);
                    }
                }
            }
            asm volatile("" ::: "memory");   // the wave's LDS accesses stay in program order
            const int pos0 = qpos[j] - l32;   // first position of the block
            char *orow = reinterpret_cast<char *>(a.o) + ((int64_t(r) * T + pos0) * a.Hq + head[j]) * ROWB;
            const int64_t pstride = int64_t(a.Hq) * ROWB;
#pragma unroll
            for (int k = 0; k < 32 / RPI; ++k) {
                const int p = k * RPI + ln / CH, c = ln % CH;
                const uint4 v = *reinterpret_cast<const uint4 *>(base + p * ROWB + (((c ^ p) & (CH - 1)) << 4));
                *reinterpret_cast<uint4 *>(orow + p * pstride + c * 16) = v;
            }
            if (h == 0) a.lse[(int64_t(r) * a.Hq + head[j]) * T + qpos[j]] = lse_v[j];
        }
    }
    if (tid == 0) ctrl[0] = next;
    wait_lds();
    block_barrier();   // staged O read back by every wave; the claim visible
    item = __builtin_amdgcn_readfirstlane(ctrl[0]);
    }

    // The lane's last workgroup to finish leaves its counters at zero for the next launch.
    if (tid == 0) {
        if (__hip_atomic_fetch_add(done, 1, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT) == n_wg - 1) {
            __hip_atomic_store(take, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(done, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

template <class Tr>
hipError_t launch_tr(const FwdArgs &args, int n_blocks, hipStream_t s) {
    const int max_list = args.T / kFwdBlockK;
    if (max_list > kFwdMaxKTiles) return hipErrorInvalidValue;
    const int smem = Lds<Tr>::LIST_OFF + 4 * ((max_list + 3) & ~3);
    if (smem > 160 * 1024) return hipErrorInvalidValue;
    auto kern = tree_attn_fwd_kernel<Tr>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, smem);
    if (e != hipSuccess) return e;
    kern<<<n_blocks, kWaves * 64, smem, s>>>(args);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd(const FwdShape &sh, const WsLayout &w, char *ws, const void *q,
                      const void *k, const void *v, void *o, float *lse, hipStream_t s) {
    FwdArgs a;
    a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
    a.qt_ptr = reinterpret_cast<const int32_t *>(ws + w.qt_ptr);
    a.kt_idx = reinterpret_cast<const int32_t *>(ws + w.kt_idx);
    a.kt_kind = reinterpret_cast<const uint8_t *>(ws + w.kt_kind);
    a.kend = reinterpret_cast<const int32_t *>(ws + w.kend);
    a.work = reinterpret_cast<const int32_t *>(ws + w.work);
    a.n_real = reinterpret_cast<const int32_t *>(ws + w.n_real);
    a.status = reinterpret_cast<const int32_t *>(ws + w.status);
    a.T = sh.T; a.Hq = sh.Hq; a.Hkv = sh.Hkv; a.G = sh.G; a.HCH = sh.HCH;
    a.nQ = w.nQ; a.BQ = sh.BQ;
    a.L = sh.Hkv * (sh.G / sh.HCH);
    a.scale = sh.scale;
    a.c = sh.scale * 1.4426950408889634f;
    a.ctr = reinterpret_cast<int32_t *>(ws + w.ctr);
    if (a.L != w.n_lanes) return hipErrorInvalidValue;
    const int64_t n_items = int64_t(sh.R) * w.nQ;
    if (n_items == 0) return hipSuccess;
    if (n_items > INT32_MAX) return hipErrorInvalidValue;
    a.n_items = int32_t(n_items);
    // One workgroup per CU (an item's K/V buffers fill the CU's LDS), rounded down to whole lanes.
    int dev = 0, n_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n_cu <= 0)
        n_cu = 256;
    const int64_t n_blocks = std::min<int64_t>(std::max(1, n_cu / a.L), n_items) * a.L;
    if (n_blocks > INT32_MAX) return hipErrorInvalidValue;
    if (sh.dtype == TREE_DT_BF16) {
        if (sh.D == 128) return launch_tr<Bf16Traits<128>>(a, int(n_blocks), s);
        if (sh.D == 64) return launch_tr<Bf16Traits<64>>(a, int(n_blocks), s);
    } else {
        if (sh.D == 64) return launch_tr<F32Traits<64>>(a, int(n_blocks), s);
    }
    return hipErrorInvalidValue;
}

}  // namespace treeattn
