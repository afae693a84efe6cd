// Tree-masked attention backward for gfx950 (CDNA4): dQ, dK, dV on bf16 MFMA.
//
// What is computed ("Prefix tree packing", furtherai.github.io: the packing serves training,
// so every attention layer is differentiated; the mask is the attention-mask passage's
// ancestor rule, in its pre-order interval form j <= i < kend[j]).  With P the softmax of the
// visible scores (recomputed from Q, K and the forward's LSE), D_i = rowsum(dO_i * O_i):
//   dV = P^T dO,   dP = dO V^T,   dS = P * (dP - D),   dQ = scale dS K,   dK = scale dS^T Q.
//
// Three launches on the caller's stream:
//   * dq_kernel: one workgroup per forward item (row, q-tile, KV head, chunk of its query
//     heads), 8 waves of 32 query rows, walking the q-tile's k-tile list with K/V tiles
//     staged in LDS (direct-to-LDS copies, two tiles ahead); each wave first forms its rows'
//     D = rowsum(dO * O) and log2-domain LSE and writes them for the dK/dV kernel;
//   * dkdv_kernel: one workgroup per (row, group of kKvGroup = 4 k-tiles, KV head, query
//     slice), 8 waves of 32 keys (two per SIMD) whose K fragments stay in registers and whose
//     V rows stay in LDS, walking the slice's run of the group's list of q-tiles (the
//     transposed tile lists) and every query head of the group in blocks of 32 queries; each
//     block's Q, dO, LSE and D are staged in LDS once for all eight waves, three blocks ahead.
//     A wave whose k-tile does not see a block's q-tile skips it.  A group seen by many q-tiles
//     (a shared prefix's keys are seen by every query after them) is split into up to
//     kBwdSlices slices so that its work spreads over several CUs, as long as the bounded pool
//     of partial slots lasts (the plan hands the slots to the longest groups first).  The grid
//     follows the plan's list of (group, slice) units, so no workgroup is launched for a slice
//     that does not exist; only a short surplus at the end of the grid exits at once;
//   * dkdv_reduce (only where a group was split): adds the slices' fp32 partials in slice order.
// Every result is written exactly once (no atomics); gradients of pads are zero.
//
// Orientation (32x32x16 bf16 MFMA, accumulator element i of lane l at row 8(i/4) + 4(l/32) +
// i%4, column l%32):
//   dq_kernel:  S^T = K Q^T and dP^T = V dO^T (keys x queries, a query per lane), then
//               dQ^T += K^T dS^T with dS^T's accumulator registers as the second operand;
//   dkdv_kernel: S = Q K^T and dP = dO V^T (queries x keys, a key per lane), then
//               dV^T += dO^T P and dK^T += Q^T dS.
// The "transposed" operands (K^T, dO^T, Q^T) are LDS transpose reads of row-major tiles.
// The softmax takes the LSE in log2 units (one FMA and one exp per element); the mask of a
// PARTIAL tile is applied in its own uniform branch, so FULL tiles do no mask arithmetic.
#include <algorithm>
#include <type_traits>

#include "internal.h"
#include "tile_ops.h"

namespace treeattn {
namespace {

using tile::bf16x4_t;
using tile::bf16x8_t;
using tile::floatx16;
using tile::int32x4_t;
using tile::shortx4;
using tile::zero16;

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kLdsBytes = 160 * 1024;     // LDS of one CU (one workgroup per CU at most)

struct BwdArgs {
    const void *q, *k, *v, *o, *dout;
    void *dq, *dk, *dv;
    const float *lse;
    float *delta, *lse2;
    const int32_t *qt_ptr, *kt_idx;
    const uint8_t *kt_kind;
    const int32_t *kp_ptr, *kp_list, *kwork;
    float *part;                   // per-slice dK^T / dV^T partials (BwdLayout::part)
    const int2 *pslot;             // per k-tile group: (query slices, first partial slot)
    const int2 *units;             // (group item, slice) of every dK/dV workgroup, work order
    const int32_t *n_units;        // units in use; workgroups past them exit
    const int32_t *kend, *work, *n_real, *status;
    int32_t T, Hq, Hkv, G, HCH, nQ, nK, nP, L, BQ;
    int32_t lcap;  // q-tile list entries the dK/dV kernel stages in LDS at a time
    float c;       // scale * log2(e)
    float scale;
};

// ------------------------------------------------------------------------- tiles and operands
//
// Tiles are row-major [rows][D] bf16 in LDS with XOR-swizzled 16-byte chunks (tile::Tile);
// every fragment address is a per-lane register computed once (tile::LaneOffsets) plus an
// instruction immediate.
using tile::acc_frag;
using tile::block_barrier;
using tile::buf_rsrc;
using tile::buf_to_lds16;
using tile::buf_to_lds4;
using tile::LaneOffsets;
using tile::lds_base;
using tile::mfma;
using tile::static_for;
using tile::Tile;
using tile::wait_loads;
using tile::wait_loads_but;

// A tile copy split over NW waves with the split fixed at compile time: wave w issues the 1 KB
// block copies w, w + NW, ... (ROWS rows of D bf16 in all), an unrolled run of immediates
// instead of a loop with a runtime trip count.
template <int D, int ROWS, int NW>
__device__ __forceinline__ void copy_rows(const char *src, int n_valid, int stride, uint32_t dst, int wave,
                                          int lane) {
    constexpr int NBLK = ROWS / (1024 / (D * 2));
    static_assert(NBLK % NW == 0, "the waves must split the tile evenly");
    const int32x4_t rs = tile::tile_rsrc(src, n_valid, stride);
#pragma unroll
    for (int i = 0; i < NBLK / NW; ++i) tile::copy_block<D>(rs, stride, dst, wave + NW * i, lane);
}

// ------------------------------------------------------------------------------ dq_kernel
constexpr int kDqWaves = 8;
constexpr int kBK = 64;                   // keys per k-tile

template <int D>
struct DqLds {
    static constexpr int TILE = kBK * D * 2;
    static constexpr int NB = 3;                       // k-tile buffers (tile t+2 copied under t)
    static constexpr int K_OFF = 0, V_OFF = NB * TILE, KE_OFF = 2 * NB * TILE;
    static constexpr int LIST_OFF = KE_OFF + NB * 256;
    // K and V copies per copying wave per tile.  One wave per SIMD copies (waves 0-3): a wave
    // that issues direct-to-LDS loads stalls while the CU's memory pipeline is full, and the
    // other wave of its SIMD keeps issuing meanwhile.
    static constexpr int CW = 4;
    static constexpr int PERW = 2 * (TILE / 1024) / CW;
    static_assert((2 * (TILE / 1024)) % CW == 0, "waves must split a tile evenly");
    static_assert(PERW + 1 < 16, "vmcnt field");
};

// One k-tile of the dq pass for a wave's 32 queries: P^T, dS^T of both 32-key blocks, then
// dQ^T += K^T dS^T.  Element i of the score accumulators is key 32 kb + 8(i/4) + 4h + i%4.
template <int D>
__device__ __forceinline__ void dq_tile(const char *Kt, const char *Vt, const int32_t *KEs, const LaneOffsets<D> &lo,
                                        const bf16x8_t (&qf)[D / 16], const bf16x8_t (&dof)[D / 16], float c,
                                        float lse2, float dlt, bool partial, int dq_, int qpos,
                                        floatx16 (&acc)[D / 32]) {
    using TL = Tile<D>;
    // Operand reads run RING MFMAs ahead of use, across the softmax and the two 32-key halves.
    // Operand i of half kb = i / PER: r = i % PER < NA a row read of K (even r) or V (odd) for
    // S^T / dP^T; else the transposed K read of dQ^T's MFMA (ks, db) = ((r - NA) / NDB, % NDB).
    constexpr int NDB = TL::NDB, NA = 2 * TL::NDS, PER = NA + 2 * NDB, TOT = 2 * PER, RING = 3;
    auto operand = [&](auto ic) __attribute__((always_inline)) {
        constexpr int i = decltype(ic)::value, kb = i / PER, r = i % PER;
        if constexpr (r < NA) {
            return TL::row_at((r % 2 == 0 ? Kt : Vt) + lo.row[r / 2] + 32 * kb * TL::ROWB);
        } else {
            constexpr int j = r - NA, ks = j / NDB, db = j % NDB;
            const int rofs = (32 * kb + 16 * ks) * TL::ROWB;
            return TL::tr_at(Kt + lo.tr[db][0] + rofs, Kt + lo.tr[db][1] + rofs);
        }
    };
    bf16x8_t ring[RING];
    static_for<RING>([&](auto ic) __attribute__((always_inline)) { ring[decltype(ic)::value] = operand(ic); });
    auto next = [&](auto ic) __attribute__((always_inline)) {
        constexpr int i = decltype(ic)::value;
        const bf16x8_t op = ring[i % RING];
        if constexpr (i + RING < TOT) ring[i % RING] = operand(std::integral_constant<int, i + RING>{});
        return op;
    };
    static_for<2>([&](auto kbc) __attribute__((always_inline)) {
        constexpr int kb = decltype(kbc)::value;
        // dP^T starts from -D (every element of a lane is its query), so dS = P * that.  The
        // empty asm keeps the splat inside the loop (hoisted, its 16 registers would stay live
        // through the whole tile loop).
        float nd = -dlt;
        asm volatile("" : "+v"(nd));
        floatx16 s = zero16(), dp;
#pragma unroll
        for (int i = 0; i < 16; ++i) dp[i] = nd;
        static_for<NA>([&](auto rc) __attribute__((always_inline)) {
            constexpr int r = decltype(rc)::value;
            const bf16x8_t op = next(std::integral_constant<int, kb * PER + r>{});
            if constexpr (r % 2 == 0) s = mfma(op, qf[r / 2], s);
            else dp = mfma(op, dof[r / 2], dp);
            __builtin_amdgcn_sched_barrier(0);
        });
#pragma unroll
        for (int i = 0; i < 16; ++i) s[i] = __builtin_amdgcn_exp2f(fmaf(s[i], c, -lse2));
        if (partial) {             // uniform: FULL tiles skip the mask
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const int4 ke = *reinterpret_cast<const int4 *>(KEs + 32 * kb + 8 * i4);
                const int kev[4] = {ke.x, ke.y, ke.z, ke.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int cc = 32 * kb + 8 * i4 + e;
                    s[4 * i4 + e] = ((cc <= dq_) & (qpos < kev[e])) ? s[4 * i4 + e] : 0.f;
                }
            }
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) s[i] = s[i] * dp[i];
        const bf16x8_t dsf[2] = {acc_frag(s, 0), acc_frag(s, 1)};
        static_for<2 * NDB>([&](auto jc) __attribute__((always_inline)) {
            constexpr int j = decltype(jc)::value, ks = j / NDB, db = j % NDB;
            const bf16x8_t op = next(std::integral_constant<int, kb * PER + NA + j>{});
            acc[db] = mfma(op, dsf[ks], acc[db]);
            __builtin_amdgcn_sched_barrier(0);
        });
    });
}

template <int D>
__global__ __launch_bounds__(kDqWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void dq_kernel(BwdArgs a) {
    using TL = Tile<D>;
    using LD = DqLds<D>;
    constexpr int NB = LD::NB;
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    if (a.status[0] != 0) return;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, h = lane >> 5;
    const int u = blockIdx.x % a.L, item = blockIdx.x / a.L;
    const int g = u % a.Hkv, chunk = u / a.Hkv;
    const int tile = a.work[item];
    const int r = tile / a.nQ, qt = tile % a.nQ;
    const int T = a.T;
    const int n_real = a.n_real[r];
    const int hl = wave % a.HCH, pb = wave / a.HCH;
    const int head = g * a.G + chunk * a.HCH + hl;
    const int qpos = qt * a.BQ + pb * 32 + l32;
    const bool qreal = qpos < n_real;

    // Q and dO fragments of the wave's 32 queries (dO zero at pad queries: its contents never
    // reach dK / dV / dQ); per-lane log2-domain LSE (+inf at pads so that P = 0) and
    // D = rowsum(dO * O) in fp32 (0 at pads), both also written to the workspace for the dK/dV
    // kernel (every (row, position, head) belongs to exactly one dQ work item).
    bf16x8_t qf[TL::NDS], dof[TL::NDS];
    float dsum = 0.f;
    {
        const int64_t row_off = ((int64_t(r) * T + qpos) * a.Hq + head) * D;
        const bf16x8_t *pq = reinterpret_cast<const bf16x8_t *>(reinterpret_cast<const __bf16 *>(a.q) + row_off);
        const bf16x8_t *pd = reinterpret_cast<const bf16x8_t *>(reinterpret_cast<const __bf16 *>(a.dout) + row_off);
        const bf16x8_t *po = reinterpret_cast<const bf16x8_t *>(reinterpret_cast<const __bf16 *>(a.o) + row_off);
#pragma unroll
        for (int ds = 0; ds < TL::NDS; ++ds) {
            qf[ds] = pq[2 * ds + h];
            const bf16x8_t x = pd[2 * ds + h];
            const bf16x8_t ov = po[2 * ds + h];
            bf16x8_t z;
#pragma unroll
            for (int e = 0; e < 8; ++e) z[e] = qreal ? x[e] : static_cast<__bf16>(0.f);
            dof[ds] = z;
            static_for<4>([&](auto ec) __attribute__((always_inline)) {
                constexpr int e = 2 * decltype(ec)::value;
                dsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(x, x, e, e + 1),
                                                       __builtin_shufflevector(ov, ov, e, e + 1), dsum, false);
            });
        }
    }
    const int64_t term = (int64_t(r) * a.Hq + head) * T + qpos;
    const float lse2_raw = a.lse[term] * kLog2e;
    const float lse2 = (qreal && lse2_raw > -INFINITY) ? lse2_raw : INFINITY;
    {
        // the two lane halves hold the two halves of each 16-column chunk pair
        const auto r2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(dsum), __float_as_uint(dsum), false, false);
        dsum = __uint_as_float(r2[0]) + __uint_as_float(r2[1]);
    }
    const float dlt = qreal ? dsum : 0.f;   // a select: pad O / dO contents (even NaN) stay out
    if (h == 0) {
        a.delta[term] = dlt;
        a.lse2[term] = lse2_raw;
    }
    const LaneOffsets<D> lo(lane);

    floatx16 acc[TL::NDB];
#pragma unroll
    for (int db = 0; db < TL::NDB; ++db) acc[db] = zero16();

    const int32_t t_begin = a.qt_ptr[tile];
    const int N = a.qt_ptr[tile + 1] - t_begin;
    int32_t *const lst = reinterpret_cast<int32_t *>(smem + LD::LIST_OFF);
    for (int i = tid; i < N; i += kDqWaves * 64) lst[i] = a.kt_idx[t_begin + i] * 4 + a.kt_kind[t_begin + i];
    __syncthreads();

    const int row_stride = a.Hkv * D * 2;
    const char *kbase0 = reinterpret_cast<const char *>(a.k) + ((int64_t(r) * T) * a.Hkv + g) * D * 2;
    const char *vbase0 = reinterpret_cast<const char *>(a.v) + ((int64_t(r) * T) * a.Hkv + g) * D * 2;
    const int32_t *kend_row = a.kend + int64_t(r) * T;
    const uint32_t lds0 = lds_base(smem);
    auto issue = [&](int t) __attribute__((always_inline)) {
        const int kt = __builtin_amdgcn_readfirstlane(lst[t]) >> 2;
        const int slot = t % NB;
        const int n_valid = __builtin_amdgcn_readfirstlane(min(max(n_real - kt * kBK, 0), kBK));
        const int64_t tb = int64_t(kt) * kBK * row_stride;
        if (wave < LD::CW) {
            copy_rows<D, kBK, LD::CW>(kbase0 + tb, n_valid, row_stride, lds0 + LD::K_OFF + slot * LD::TILE, wave, lane);
            copy_rows<D, kBK, LD::CW>(vbase0 + tb, n_valid, row_stride, lds0 + LD::V_OFF + slot * LD::TILE, wave, lane);
        }
        if (wave == LD::CW - 1) buf_to_lds4(buf_rsrc(kend_row + kt * kBK, 256), lds0 + LD::KE_OFF + slot * 256, lane * 4);
    };

    if (N > 0) issue(0);
    if (N > 1) issue(1);
    // NB tiles per iteration, one per buffer slot, so that slot offsets are compile-time
    // constants (instruction immediates of the operand reads).
    for (int t0 = 0; t0 < N; t0 += NB) {
        static_for<NB>([&](auto sc) __attribute__((always_inline)) {
            constexpr int slot = decltype(sc)::value;
            const int t = t0 + slot;
            if (t >= N) return;
            // Tile t has landed for every wave once each waited for its own copies of t (only
            // t+1's may still be in flight), and every wave is past tile t-1 before its buffer
            // slot takes tile t+2.
            if (t + 1 < N) {
                // leave tile t+1's copies (the newest) in flight
                if (wave == LD::CW - 1) wait_loads_but<DqLds<D>::PERW + 1>();
                else if (wave < LD::CW) wait_loads_but<DqLds<D>::PERW>();
                else wait_loads();
            } else {
                wait_loads();
            }
            block_barrier();
            if (t + 2 < N) issue(t + 2);
            const int ent = __builtin_amdgcn_readfirstlane(lst[t]);
            const int kt = ent >> 2;
            const char *Kt = smem + LD::K_OFF + slot * LD::TILE;
            const char *Vt = smem + LD::V_OFF + slot * LD::TILE;
            const int32_t *KEs = reinterpret_cast<const int32_t *>(smem + LD::KE_OFF + slot * 256) + 4 * h;
            const int dq_ = qpos - kt * kBK - 4 * h;
            dq_tile<D>(Kt, Vt, KEs, lo, qf, dof, a.c, lse2, dlt, (ent & 3) == kTilePartial, dq_, qpos, acc);
        });
    }

    // dQ = scale * (dQ^T)^T; lane holds query qpos, 4 consecutive d per register group.
    __bf16 *op = reinterpret_cast<__bf16 *>(a.dq) + ((int64_t(r) * T + qpos) * a.Hq + head) * D;
#pragma unroll
    for (int db = 0; db < TL::NDB; ++db)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
            const int d0 = 32 * db + 8 * i4 + 4 * h;
            uint2 w;
            w.x = uint32_t(__builtin_bit_cast(uint16_t, static_cast<__bf16>(acc[db][4 * i4 + 0] * a.scale))) |
                  (uint32_t(__builtin_bit_cast(uint16_t, static_cast<__bf16>(acc[db][4 * i4 + 1] * a.scale))) << 16);
            w.y = uint32_t(__builtin_bit_cast(uint16_t, static_cast<__bf16>(acc[db][4 * i4 + 2] * a.scale))) |
                  (uint32_t(__builtin_bit_cast(uint16_t, static_cast<__bf16>(acc[db][4 * i4 + 3] * a.scale))) << 16);
            *reinterpret_cast<uint2 *>(op + d0) = w;
        }
}

// ---------------------------------------------------------------------------- dkdv_kernel
constexpr int kKvWaves = 2 * kKvGroup;    // 32 keys each: kKvGroup 64-key tiles per workgroup
constexpr int kQBlk = 32;                 // queries per block (one LDS stage)

template <int D>
struct KvLds {
    static constexpr int TILE = kQBlk * D * 2;                  // Q or dO of one block
    static constexpr int BLK = 2 * TILE + 2 * kQBlk * 4;       // Q, dO, LSE2, D of one block
    static constexpr int Q_OFF = 0, DO_OFF = TILE, LSE_OFF = 2 * TILE, DL_OFF = 2 * TILE + kQBlk * 4;
    static constexpr int NS = 4;                                // stages, one block each
    static constexpr int AHEAD = NS - 1;                        // blocks copied ahead of the one in use
    // Copies are issued by one wave per SIMD (waves 0-3): a wave that issues direct-to-LDS
    // loads stalls while the CU's memory pipeline is full, and the other wave of its SIMD keeps
    // issuing meanwhile.  Per block each copying wave issues PERW 1 KB loads of Q and dO; the
    // last one also the LSE2 and D rows.
    static constexpr int CW = 4;
    static constexpr int PERW = 2 * (TILE / 1024) / CW;
    static_assert((2 * (TILE / 1024)) % CW == 0, "copying waves must split a block evenly");
    static_assert(AHEAD == 3 && 2 * (PERW + 2) < 64, "vmcnt field");
    // V of the group's 64 kKvGroup keys (B operand of dP = dO V^T, read like the Q / dO rows),
    // then the slice's q-tile list
    static constexpr int V_OFF = NS * BLK, VTILE = kKvWaves * 32 * D * 2, LIST_OFF = V_OFF + VTILE;
};

// Softmax of one block for a wave's 32 keys: P and dS as bf16 operands (accumulator register
// order), dp holding dP - D (its accumulator started from -D).  Element i is query
// q0 + 8(i/4) + 4h + i%4 of the block (qh = q0 + 4h).
template <int D>
__device__ __forceinline__ void kv_softmax(const floatx16 &s, const floatx16 &dp, const char *blk, int h, float c,
                                           bool partial, int key, int kend_k, int qh, bf16x8_t (&pf)[2],
                                           bf16x8_t (&sf)[2]) {
    using LD = KvLds<D>;
    const float *LS = reinterpret_cast<const float *>(blk + LD::LSE_OFF) + 4 * h;
    floatx16 pm, dsm;
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
        const float4 l4 = *reinterpret_cast<const float4 *>(LS + 8 * i4);
        const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) pm[4 * i4 + e] = __builtin_amdgcn_exp2f(fmaf(s[4 * i4 + e], c, -lv[e]));
    }
    if (partial) {                 // uniform: FULL blocks skip the mask
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int q = qh + 8 * i4 + e;
                pm[4 * i4 + e] = ((key <= q) & (q < kend_k)) ? pm[4 * i4 + e] : 0.f;
            }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) dsm[i] = pm[i] * dp[i];   // dp holds dP - D
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        pf[ks] = acc_frag(pm, ks);
        sf[ks] = acc_frag(dsm, ks);
    }
}

// One block for a wave: S and dP, softmax, then dV^T += dO^T P and dK^T += Q^T dS.
template <int D>
__device__ __forceinline__ void kv_block(const char *blk, const LaneOffsets<D> &lo, const bf16x8_t (&kf)[D / 16],
                                         const char *Vt, float c, int h, int key, int kend_k,
                                         int q0, bool partial, floatx16 (&dk)[D / 32], floatx16 (&dv)[D / 32]) {
    using TL = Tile<D>;
    using LD = KvLds<D>;
    const char *Qt = blk + LD::Q_OFF;
    const char *Ot = blk + LD::DO_OFF;
    // Operand reads run RING reads ahead of their use, from the S / dP products into the dV /
    // dK ones (whose first operands are read before the softmax).  Three: with the stage
    // offsets as immediates (the block loop runs one stage per unrolled copy) a fourth would
    // push the kernel past 256 registers.
    constexpr int NP1 = 3 * TL::NDS, NP2 = 4 * TL::NDB, RING = 3;
    static_assert(NP1 >= RING && NP2 >= RING, "ring deeper than a phase");
    // operand i < NP1: row read of Q (i % 3 == 0, for S), dO (1) and V (2, for dP) at k-step
    // i / 3; NP1 + j: transposed read of dO (j even, for dV) / Q (j odd, for dK),
    // j = (ks NDB + db) 2 + t
    auto operand = [&](auto ic) __attribute__((always_inline)) {
        constexpr int i = decltype(ic)::value;
        if constexpr (i < NP1) {
            constexpr int t = i % 3;
            return TL::row_at((t == 0 ? Qt : t == 1 ? Ot : Vt) + lo.row[i / 3]);
        } else {
            constexpr int j = i - NP1, t = j % 2, db = (j / 2) % TL::NDB, ks = j / 2 / TL::NDB;
            const char *base = (t == 0 ? Ot : Qt) + 16 * ks * TL::ROWB;
            return TL::tr_at(base + lo.tr[db][0], base + lo.tr[db][1]);
        }
    };
    bf16x8_t ring[RING];
    static_for<RING>([&](auto ic) __attribute__((always_inline)) { ring[decltype(ic)::value] = operand(ic); });
    // dP starts from -D of each element's query (staged with the block), so dS = P * dP.
    floatx16 s = zero16(), dp;
    {
        const float *DL = reinterpret_cast<const float *>(blk + LD::DL_OFF) + 4 * h;
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
            const float4 d4 = *reinterpret_cast<const float4 *>(DL + 8 * i4);
            dp[4 * i4 + 0] = -d4.x;
            dp[4 * i4 + 1] = -d4.y;
            dp[4 * i4 + 2] = -d4.z;
            dp[4 * i4 + 3] = -d4.w;
        }
    }
    bf16x8_t dof;                            // the k-step's dO operand, until its V operand
    static_for<NP1>([&](auto ic) __attribute__((always_inline)) {
        constexpr int i = decltype(ic)::value;
        const bf16x8_t op = ring[i % RING];
        ring[i % RING] = operand(std::integral_constant<int, i + RING>{});
        if constexpr (i % 3 == 0) {
            s = mfma(op, kf[i / 3], s);
            __builtin_amdgcn_sched_barrier(0);
        } else if constexpr (i % 3 == 1) {
            dof = op;
        } else {
            dp = mfma(dof, op, dp);
            __builtin_amdgcn_sched_barrier(0);
        }
    });
    bf16x8_t pf[2], sf[2];
    kv_softmax<D>(s, dp, blk, h, c, partial, key, kend_k, q0 + 4 * h, pf, sf);
    static_for<NP2>([&](auto jc) __attribute__((always_inline)) {
        constexpr int j = decltype(jc)::value, t = j % 2, db = (j / 2) % TL::NDB, ks = j / 2 / TL::NDB;
        const bf16x8_t op = ring[j % RING];
        if constexpr (j + RING < NP2) ring[j % RING] = operand(std::integral_constant<int, NP1 + j + RING>{});
        if constexpr (t == 0) dv[db] = mfma(op, pf[ks], dv[db]);
        else dk[db] = mfma(op, sf[ks], dk[db]);
        __builtin_amdgcn_sched_barrier(0);
    });
}

// Position in a k-tile group's sequence of 32-query blocks: list entry, query head of the KV group,
// 32-query chunk of the q-tile.
struct BlockCursor {
    int e = 0, hd = 0, ch = 0;
    __device__ __forceinline__ void next(int G, int CH) {
        if (++ch == CH) {
            ch = 0;
            if (++hd == G) {
                hd = 0;
                ++e;
            }
        }
    }
};

// kKvWaves waves of 32 keys each (two per SIMD); waves 0-3 also issue the copies.
template <int D>
__global__ __launch_bounds__(kKvWaves * 64) void dkdv_kernel(BwdArgs a) {
    using TL = Tile<D>;
    using LD = KvLds<D>;
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    if (a.status[0] != 0) return;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31, h = lane >> 5;
    const int g = blockIdx.x % a.Hkv, unit = blockIdx.x / a.Hkv;
    if (unit >= a.n_units[0]) return;                    // the grid's surplus (end of the grid)
    const int2 us = a.units[unit];
    const int pitem = us.x, slice = us.y;
    const int32_t list_begin = a.kp_ptr[pitem];
    const int NL_pair = a.kp_ptr[pitem + 1] - list_begin;
    const int2 ps = a.pslot[pitem];
    const int n_slices = ps.x;
    const int r = pitem / a.nP, pr = pitem % a.nP;
    const int T = a.T;
    const int n_real = a.n_real[r];
    const bool cw = wave < LD::CW;                       // a copying wave
    const int key0 = kKvGroup * pr * kBK;                // the group's first key
    const int key = key0 + 32 * wave + l32;              // this lane's key (k-tile wave / 2)
    const bool kin = key < T;                            // false only past the row's last k-tile
    const bool kreal = key < n_real;
    const int kend_k = kin ? a.kend[int64_t(r) * T + key] : key;      // == key at pads: never visible
    const int cls_shift = 2 * (kKvGroup - 1 - (wave >> 1));

    // K fragments of the wave's 32 keys (B operand of S = Q K^T): lane holds columns 16 ds +
    // 8h .. +7 of its key; zero at pad keys.  (V is read from LDS, rows past the last real key
    // zero.)
    bf16x8_t kf[TL::NDS];
    {
        const int64_t off = ((int64_t(r) * T + (kin ? key : 0)) * a.Hkv + g) * D;
        const bf16x8_t *pk = reinterpret_cast<const bf16x8_t *>(reinterpret_cast<const __bf16 *>(a.k) + off);
#pragma unroll
        for (int ds = 0; ds < TL::NDS; ++ds) {
            const bf16x8_t x = pk[2 * ds + h];
            bf16x8_t zx;
#pragma unroll
            for (int e = 0; e < 8; ++e) zx[e] = kreal ? x[e] : static_cast<__bf16>(0.f);
            kf[ds] = zx;
        }
    }
    const LaneOffsets<D> lo(lane);
    floatx16 dk[TL::NDB], dv[TL::NDB];       // dK^T, dV^T: rows d, a key per lane
#pragma unroll
    for (int db = 0; db < TL::NDB; ++db) {
        dk[db] = zero16();
        dv[db] = zero16();
    }

    // Blocks: (entry of the group's q-tile list, query head, 32-query chunk), one LDS stage
    // each, copied AHEAD blocks ahead of the one in use.  The slice's entries are staged in LDS
    // (no scalar load inside the block loop), lcap at a time: a longer slice (only on rows of
    // more than lcap q-tiles) runs as several passes, the copies drained between them.
    const int32_t l_begin = list_begin + NL_pair * slice / n_slices;
    const int NL = list_begin + NL_pair * (slice + 1) / n_slices - l_begin;
    int32_t *lst = reinterpret_cast<int32_t *>(smem + LD::LIST_OFF);
    const int CH = a.BQ / kQBlk;
    const int q_stride = a.Hq * D * 2;
    const uint32_t lds0 = lds_base(smem);
    // The group's V rows, before block 0's copies (so they land first).
    if (cw && NL > 0) {
        const int n_valid = __builtin_amdgcn_readfirstlane(min(max(n_real - key0, 0), kKvWaves * 32));
        const int64_t voff = ((int64_t(r) * T + key0) * a.Hkv + g) * D * 2;
        copy_rows<D, kKvWaves * 32, LD::CW>(reinterpret_cast<const char *>(a.v) + voff, n_valid, a.Hkv * D * 2,
                                            lds0 + LD::V_OFF, wave, lane);
    }
    for (int c0 = 0; c0 < NL; c0 += a.lcap) {
        const int nl = min(a.lcap, NL - c0);
        if (c0 > 0) __syncthreads();   // every wave is done with the previous pass's list and stages
        for (int e = tid; e < nl; e += kKvWaves * 64) lst[e] = a.kp_list[l_begin + c0 + e];
        __syncthreads();
        const int NB = nl * a.G * CH;
        BlockCursor ci, cc;            // next block to copy / to compute
        auto issue = [&](int n) __attribute__((always_inline)) {
            if (!cw) return;
            const int ent = __builtin_amdgcn_readfirstlane(lst[ci.e]);
            const int q0 = (ent >> 8) * a.BQ + ci.ch * kQBlk;
            const int head = g * a.G + ci.hd;
            ci.next(a.G, CH);
            const uint32_t bl = lds0 + (n % LD::NS) * LD::BLK;
            const int n_valid = __builtin_amdgcn_readfirstlane(min(max(n_real - q0, 0), kQBlk));
            const int64_t roff = ((int64_t(r) * T + q0) * a.Hq + head) * D * 2;
            copy_rows<D, kQBlk, LD::CW>(reinterpret_cast<const char *>(a.q) + roff, n_valid, q_stride, bl + LD::Q_OFF,
                                        wave, lane);
            copy_rows<D, kQBlk, LD::CW>(reinterpret_cast<const char *>(a.dout) + roff, n_valid, q_stride,
                                        bl + LD::DO_OFF, wave, lane);
            if (wave == LD::CW - 1 && lane < kQBlk) {
                const int64_t loff = (int64_t(r) * a.Hq + head) * T + q0;
                buf_to_lds4(buf_rsrc(a.lse2 + loff, uint32_t(n_valid) * 4), bl + LD::LSE_OFF, lane * 4);
                buf_to_lds4(buf_rsrc(a.delta + loff, uint32_t(n_valid) * 4), bl + LD::DL_OFF, lane * 4);
            }
        };
#pragma unroll
        for (int n = 0; n < LD::AHEAD; ++n)
            if (n < NB) issue(n);
        // The loop runs NS blocks per iteration, one per stage, so that every stage offset is
        // a compile-time constant (an instruction immediate of the operand reads).
        for (int n0 = 0; n0 < NB; n0 += LD::NS) {
            static_for<LD::NS>([&](auto sc) __attribute__((always_inline)) {
                constexpr int st = decltype(sc)::value;
                const int n = n0 + st;
                if (n >= NB) return;
                // Block n has landed once each copying wave has only the newer blocks' copies
                // (at most AHEAD - 1 of them) in flight (loads only: they land in order); the
                // barrier extends that to every wave and also means every wave is done with
                // block n - 1, whose stage block n + AHEAD takes.
                if (cw) {
                    const int newer = min(LD::AHEAD - 1, NB - 1 - n);
                    if (wave == LD::CW - 1) {
                        if (newer >= 2) wait_loads_but<2 * (LD::PERW + 2)>();
                        else if (newer == 1) wait_loads_but<LD::PERW + 2>();
                        else wait_loads();
                    } else {
                        if (newer >= 2) wait_loads_but<2 * LD::PERW>();
                        else if (newer == 1) wait_loads_but<LD::PERW>();
                        else wait_loads();
                    }
                }
                block_barrier();
                if (n + LD::AHEAD < NB) issue(n + LD::AHEAD);
                const int ent = __builtin_amdgcn_readfirstlane(lst[cc.e]);
                const int q0 = (ent >> 8) * a.BQ + cc.ch * kQBlk;
                cc.next(a.G, CH);
                const int cls = (ent >> cls_shift) & 3;
                if (cls != kTileSkip)
                    kv_block<D>(smem + st * LD::BLK, lo, kf, smem + LD::V_OFF + 32 * wave * TL::ROWB, a.c, h, key,
                                kend_k, q0, cls == kTilePartial, dk, dv);
            });
        }
    }

    if (n_slices > 1) {
        // fp32 partial in accumulator order: float4 ((wave NDB + db) 4 + i4) 64 + lane
        float4 *pp = reinterpret_cast<float4 *>(a.part) +
                     (int64_t(ps.y + slice) * a.Hkv + g) * 2 * (kKvWaves * TL::NDB * 4 * 64);
#pragma unroll
        for (int db = 0; db < TL::NDB; ++db)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const int idx = ((wave * TL::NDB + db) * 4 + i4) * 64 + lane;
                pp[idx] = make_float4(dk[db][4 * i4], dk[db][4 * i4 + 1], dk[db][4 * i4 + 2], dk[db][4 * i4 + 3]);
                pp[kKvWaves * TL::NDB * 4 * 64 + idx] =
                    make_float4(dv[db][4 * i4], dv[db][4 * i4 + 1], dv[db][4 * i4 + 2], dv[db][4 * i4 + 3]);
            }
        return;
    }
    // dK = scale dS^T Q, dV = P^T dO: lane holds its key, 4 consecutive d per register group.
    if (!kin) return;
    const int64_t off = ((int64_t(r) * T + key) * a.Hkv + g) * D;
    __bf16 *pk = reinterpret_cast<__bf16 *>(a.dk) + off;
    __bf16 *pv = reinterpret_cast<__bf16 *>(a.dv) + off;
#pragma unroll
    for (int db = 0; db < TL::NDB; ++db)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
            const int d0 = 32 * db + 8 * i4 + 4 * h;
            uint2 wk, wv;
            wk.x = uint32_t(__builtin_bit_cast(uint16_t, static_cast<__bf16>(dk[db][4 * i4 + 0] * a.scale))) |
                   (uint32_t(__builtin_bit_cast(uint16_t, static_cast<__bf16>(dk[db][4 * i4 + 1] * a.scale))) << 16);
            wk.y = uint32_t(__builtin_bit_cast(uint16_t, static_cast<__bf16>(dk[db][4 * i4 + 2] * a.scale))) |
                   (uint32_t(__builtin_bit_cast(uint16_t, static_cast<__bf16>(dk[db][4 * i4 + 3] * a.scale))) << 16);
            wv.x = uint32_t(__builtin_bit_cast(uint16_t, static_cast<__bf16>(dv[db][4 * i4 + 0]))) |
                   (uint32_t(__builtin_bit_cast(uint16_t, static_cast<__bf16>(dv[db][4 * i4 + 1]))) << 16);
            wv.y = uint32_t(__builtin_bit_cast(uint16_t, static_cast<__bf16>(dv[db][4 * i4 + 2]))) |
                   (uint32_t(__builtin_bit_cast(uint16_t, static_cast<__bf16>(dv[db][4 * i4 + 3]))) << 16);
            *reinterpret_cast<uint2 *>(pk + d0) = wk;
            *reinterpret_cast<uint2 *>(pv + d0) = wv;
        }
}

// Sum of a split group's slice partials, in slice order, to bf16 dK (times scale) and dV.
// kRedParts workgroups per (group item, KV head), each over an equal part of the group's
// accumulator elements (a single workgroup per group left most CUs idle); unsplit groups return.
constexpr int kRedParts = 4;
template <int D>
__global__ __launch_bounds__(256) void dkdv_reduce(BwdArgs a) {
    using TL = Tile<D>;
    if (a.status[0] != 0) return;
    const int part = blockIdx.x % kRedParts, gi = blockIdx.x / kRedParts;
    const int g = gi % a.Hkv, item = gi / a.Hkv;
    const int pitem = a.kwork[item];
    const int2 ps = a.pslot[pitem];
    const int n_slices = ps.x;
    if (n_slices == 1) return;
    const int r = pitem / a.nP, pr = pitem % a.nP;
    const int T = a.T;
    constexpr int PER = kKvWaves * TL::NDB * 4 * 64;            // float4 per tensor per slice
    // slot (first + sl) of head g: float4 ((first + sl) Hkv + g) 2 PER, dK then dV
    const float4 *base = reinterpret_cast<const float4 *>(a.part) + (int64_t(ps.y) * a.Hkv + g) * 2 * PER;
    static_assert(PER % (kRedParts * 256) == 0, "parts of whole 256-thread rounds");
    for (int idx = part * (PER / kRedParts) + threadIdx.x; idx < (part + 1) * (PER / kRedParts); idx += blockDim.x) {
        const int lane = idx % 64, i4 = (idx / 64) % 4, db = (idx / 256) % TL::NDB, wave = idx / (256 * TL::NDB);
        float4 sk = base[idx], sv = base[PER + idx];
        for (int sl = 1; sl < n_slices; ++sl) {
            const float4 k4 = base[int64_t(sl) * a.Hkv * 2 * PER + idx];
            const float4 v4 = base[int64_t(sl) * a.Hkv * 2 * PER + PER + idx];
            sk.x += k4.x; sk.y += k4.y; sk.z += k4.z; sk.w += k4.w;
            sv.x += v4.x; sv.y += v4.y; sv.z += v4.z; sv.w += v4.w;
        }
        const int key = kKvGroup * pr * kBK + 32 * wave + (lane & 31);
        if (key >= T) continue;
        const int d0 = 32 * db + 8 * i4 + 4 * (lane >> 5);
        const int64_t off = ((int64_t(r) * T + key) * a.Hkv + g) * D + d0;
        bf16x4_t wk, wv;
        wk[0] = static_cast<__bf16>(sk.x * a.scale); wk[1] = static_cast<__bf16>(sk.y * a.scale);
        wk[2] = static_cast<__bf16>(sk.z * a.scale); wk[3] = static_cast<__bf16>(sk.w * a.scale);
        wv[0] = static_cast<__bf16>(sv.x); wv[1] = static_cast<__bf16>(sv.y);
        wv[2] = static_cast<__bf16>(sv.z); wv[3] = static_cast<__bf16>(sv.w);
        *reinterpret_cast<bf16x4_t *>(reinterpret_cast<__bf16 *>(a.dk) + off) = wk;
        *reinterpret_cast<bf16x4_t *>(reinterpret_cast<__bf16 *>(a.dv) + off) = wv;
    }
}

template <int D>
hipError_t launch_d(const BwdArgs &a, int R, int n_items_q, int n_items_k, int n_units_k, hipStream_t s) {
    if (n_items_q > 0) {
        const int smem = DqLds<D>::LIST_OFF + 4 * ((a.nK + 3) & ~3);
        if (smem > kLdsBytes) return hipErrorInvalidValue;
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(dq_kernel<D>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, smem);
        if (e != hipSuccess) return e;
        dq_kernel<D><<<n_items_q, kDqWaves * 64, smem, s>>>(a);
    }
    if (n_items_k > 0) {
        // stages, the group's V rows, then the list entries of one pass
        const int smem = KvLds<D>::LIST_OFF + 4 * a.lcap;
        if (a.lcap < 1 || smem > kLdsBytes) return hipErrorInvalidValue;
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(dkdv_kernel<D>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, smem);
        if (e != hipSuccess) return e;
        dkdv_kernel<D><<<n_units_k, kKvWaves * 64, smem, s>>>(a);
        dkdv_reduce<D><<<n_items_k * kRedParts, 256, 0, s>>>(a);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd(const FwdShape &sh, const WsLayout &w, const BwdLayout &b, const char *ws, char *bws,
                      const void *q, const void *k, const void *v, const void *o, const float *lse,
                      const void *dout, void *dq, void *dk, void *dv, hipStream_t s) {
    BwdArgs a;
    a.q = q; a.k = k; a.v = v; a.o = o; a.dout = dout;
    a.dq = dq; a.dk = dk; a.dv = dv;
    a.lse = lse;
    a.delta = reinterpret_cast<float *>(bws + b.delta);
    a.lse2 = reinterpret_cast<float *>(bws + b.lse2);
    a.qt_ptr = reinterpret_cast<const int32_t *>(ws + w.qt_ptr);
    a.kt_idx = reinterpret_cast<const int32_t *>(ws + w.kt_idx);
    a.kt_kind = reinterpret_cast<const uint8_t *>(ws + w.kt_kind);
    a.kp_ptr = reinterpret_cast<const int32_t *>(bws + b.kp_ptr);
    a.kp_list = reinterpret_cast<const int32_t *>(bws + b.kp_list);
    a.kwork = reinterpret_cast<const int32_t *>(bws + b.kwork);
    a.part = reinterpret_cast<float *>(bws + b.part);
    a.pslot = reinterpret_cast<const int2 *>(bws + b.pslot);
    a.units = reinterpret_cast<const int2 *>(bws + b.units);
    a.n_units = reinterpret_cast<const int32_t *>(bws + b.n_units);
    a.kend = reinterpret_cast<const int32_t *>(ws + w.kend);
    a.work = reinterpret_cast<const int32_t *>(ws + w.work);
    a.n_real = reinterpret_cast<const int32_t *>(ws + w.n_real);
    a.status = reinterpret_cast<const int32_t *>(ws + w.status);
    a.T = sh.T; a.Hq = sh.Hq; a.Hkv = sh.Hkv; a.G = sh.G; a.HCH = sh.HCH;
    a.nQ = w.nQ; a.nK = w.nK; a.nP = b.nP; a.BQ = sh.BQ;
    a.L = sh.Hkv * (sh.G / sh.HCH);
    {
        // as many list entries as fit beside the stages and V rows (a multiple of 4), at most nQ
        const int room = (kLdsBytes - (sh.D == 128 ? KvLds<128>::LIST_OFF : KvLds<64>::LIST_OFF)) / 4 & ~3;
        a.lcap = std::min(room, (w.nQ + 3) & ~3);
    }
    a.scale = sh.scale;
    a.c = sh.scale * kLog2e;
    const int64_t n_q = int64_t(sh.R) * w.nQ * a.L;
    const int64_t n_k = int64_t(sh.R) * b.nP * sh.Hkv;
    if (n_k * kRedParts > INT32_MAX) return hipErrorInvalidValue;
    const int64_t n_u = b.max_units * sh.Hkv;
    if (n_q > INT32_MAX || n_k > INT32_MAX || n_u > INT32_MAX) return hipErrorInvalidValue;
    if (sh.dtype != TREE_DT_BF16) return hipErrorInvalidValue;
    if (sh.BQ % kQBlk != 0) return hipErrorInvalidValue;
    if (sh.D == 128) return launch_d<128>(a, sh.R, int(n_q), int(n_k), int(n_u), s);
    if (sh.D == 64) return launch_d<64>(a, sh.R, int(n_q), int(n_k), int(n_u), s);
    return hipErrorInvalidValue;
}

}  // namespace treeattn
