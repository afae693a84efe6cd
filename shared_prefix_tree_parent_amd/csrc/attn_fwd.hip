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
//   * K/V tiles (64 keys) are copied HBM -> LDS with direct-to-LDS loads into a double
//     buffer, so the copy of tile t+1 runs under the compute of tile t with no registers.
// MFMA orientation: S^T = K Q^T and O^T = V^T P^T, so each lane owns one query (column) of
// every 32x32 accumulator: row max / row sum are in-lane plus one exchange with lane^32
// (v_permlane32_swap), and the P^T operand of the second product is the first product's
// accumulator, converted in place.  V stays row-major in LDS; its V^T operand comes from
// LDS transpose reads (ds_read_b64_tr_b16).
// Softmax: the reference max only moves when a tile's max exceeds it by more than 2^8 in
// the exponent domain (a wave-uniform branch), so the accumulator rescale is rare; O is
// normalized by the sum of the bf16-rounded weights actually fed to the MFMA, the LSE by the
// fp32 sum.
// Scheduling: items are dispatched longest first (work list from the classifier); the item's
// KV head is blockIdx % n_kv_lanes, so with 8 KV heads every XCD (blockIdx round-robin over
// 8 XCDs) works on one KV head and keeps that head's K/V in its own L2.
#include <type_traits>

#include "internal.h"

namespace treeattn {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

struct FwdArgs {
    const void *q, *k, *v;
    void *o;
    float *lse;
    const int32_t *qt_ptr, *kt_idx;
    const uint8_t *kt_kind;
    const int32_t *kend, *work, *n_real, *status;
    int32_t T, Hq, Hkv, G, HCH, nQ, L, BQ;
    float c;       // scale * log2(e): exponent scale for exp2
    float scale;   // softmax scale (for the natural-log LSE)
};

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

__device__ __forceinline__ floatx16 zero16() {
    floatx16 z;
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = 0.f;
    return z;
}

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

// LDS buffer layout: [K tile][V tile][kend of the tile's 64 keys]; four buffers rotate.
template <class Tr>
struct Lds {
    static constexpr int TILE = 64 * Tr::D * Tr::kEsz;
    static constexpr int K_OFF = 0, V_OFF = TILE, KE_OFF = 2 * TILE;
    static constexpr int BUF = 2 * TILE + 256;
    static constexpr int NBUF = 4;
};

constexpr int kWaves = 8;           // 256 rows = 8 blocks of 32, one per wave
constexpr int kBufFlags = 0x00020000;

// Wait until this wave's loads (including the ones into LDS) have landed, or all but the
// newest n of them (vmcnt(n); the counter's low 4 bits, lgkmcnt / expcnt not waited for).
__device__ __forceinline__ void wait_loads() { __builtin_amdgcn_s_waitcnt(0x0f70); }
template <int N>
__device__ __forceinline__ void wait_loads_but() { __builtin_amdgcn_s_waitcnt(0x0f70 | N); }

__device__ __forceinline__ void buf_to_lds16(__amdgpu_buffer_rsrc_t r, char *lds, int voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 16, voff, 0, 0, 0);
}
__device__ __forceinline__ void buf_to_lds4(__amdgpu_buffer_rsrc_t r, char *lds, int voff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 4, voff, 0, 0, 0);
}

__device__ __forceinline__ float xchg_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xchg_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ------------------------------------------------------------------------------------ kernel
//
// Each wave's work on tile t is split into a softmax phase V(t) (VALU: mask, max, exp, sums,
// P^T operands) and a matrix phase M(t) = { O^T += V^T P^T for tile t ; S^T = K Q^T for tile
// t+1 } (MFMA).  Waves 0-3 (group 0) run the sequence S(0), V(0), M(0), V(1), M(1), ... and
// waves 4-7 (group 1, one per SIMD beside a group-0 wave) run the same sequence one phase
// later.  Every phase ends with a workgroup barrier, so at any time one wave of each SIMD is
// in a matrix phase and the other in a softmax phase: the VALU work hides under the MFMAs.
// K/V tiles rotate through three LDS buffers: tile t is copied during step 2t-1 (ready at the
// barrier that ends it), first read by group 0 in step 2t and last read by group 1 in step
// 2t+3; tile t+3 reuses the buffer from step 2t+5.
template <class Tr>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void tree_attn_fwd_kernel(FwdArgs a) {
    using elem = typename Tr::elem;
    using frag = typename Tr::frag;
    constexpr int D = Tr::D;
    // Grow the reference max only when a tile's max exceeds it by more than 2^8 in the
    // exponent domain; otherwise keep the stale reference (exp2 values stay <= 256), which
    // keeps O and the sums exactly consistent and skips the accumulator rescale.
    constexpr float kGrow = 8.0f;

    extern __shared__ __attribute__((aligned(1024))) char smem[];

    if (a.status[0] != 0) return;   // invalid segment table: write nothing

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: phases branch per wave
    const int l32 = lane & 31, h = lane >> 5;
    const int grp = wave >> 2;
    const int bid = blockIdx.x;
    const int u = bid % a.L, item = bid / a.L;
    const int g = u % a.Hkv, chunk = u / a.Hkv;
    const int tile = a.work[item];
    const int r = tile / a.nQ, qt = tile % a.nQ;
    const int T = a.T;
    const int n_real = a.n_real[r];

    const int hl = wave % a.HCH, pb = wave / a.HCH;
    const int head = g * a.G + chunk * a.HCH + hl;
    const int qpos = qt * a.BQ + pb * 32 + l32;

    // Q fragments (B operand of S^T = K Q^T): lane holds query l32, head_dim chunk (2ds + h).
    frag qf[Tr::NDS];
    {
        const elem *qrow = reinterpret_cast<const elem *>(a.q) + ((int64_t(r) * T + qpos) * a.Hq + head) * D;
#pragma unroll
        for (int ds = 0; ds < Tr::NDS; ++ds) qf[ds] = Tr::q_frag(qrow, ds, h);
    }

    floatx16 acc[Tr::NDB];
#pragma unroll
    for (int db = 0; db < Tr::NDB; ++db) acc[db] = zero16();
    // m_run: reference max (raw score units); l_run: fp32 sum of the exponentials (for LSE);
    // w_run: sum of the weights as rounded for the PV product (normalizes O, so the weights
    // applied to V sum to one exactly as used).
    float m_run = -INFINITY, l_run = 0.f, w_run = 0.f;

    const int32_t t_begin = a.qt_ptr[tile];
    const int N = a.qt_ptr[tile + 1] - t_begin;
    const int row_stride = a.Hkv * D * Tr::kEsz;   // bytes between keys
    const char *kbase0 = reinterpret_cast<const char *>(a.k) + ((int64_t(r) * T) * a.Hkv + g) * D * Tr::kEsz;
    const char *vbase0 = reinterpret_cast<const char *>(a.v) + ((int64_t(r) * T) * a.Hkv + g) * D * Tr::kEsz;
    const int32_t *kend_row = a.kend + int64_t(r) * T;

    // Copy plan of one 64-key tile: one wave instruction moves 64 chunks of 16 bytes into 1 KB
    // of consecutive LDS (lane l at byte 16 l); each lane's source is the chunk that belongs
    // there after swizzling.  The per-lane source offsets never change; the tile base lives in
    // the buffer descriptor, whose size stops at the row's last real key, so pad keys read as
    // zeros (NaN pads cannot reach PV).
    constexpr int ROWS = 64 / Tr::CPR, INSTR = Tr::CPR, PER_WAVE = 2 * INSTR / kWaves;
    static_assert((2 * INSTR) % kWaves == 0, "waves must split the tile evenly");
    int voff[PER_WAVE], loff[PER_WAVE];
#pragma unroll
    for (int jj = 0; jj < PER_WAVE; ++jj) {
        const int i = wave + kWaves * jj;
        const bool isv = jj >= INSTR / kWaves;
        const int blk = isv ? i - INSTR : i;
        const int row = blk * ROWS + lane / Tr::CPR;
        const int c = (lane % Tr::CPR) ^ (isv ? Tr::vsw(row) : Tr::ksw(row));
        voff[jj] = row * row_stride + c * 16;
        loff[jj] = (isv ? Lds<Tr>::V_OFF : Lds<Tr>::K_OFF) + blk * 1024;
    }
    auto issue = [&](int t) __attribute__((always_inline)) {
        const int kt = __builtin_amdgcn_readfirstlane(a.kt_idx[t_begin + t]);
        char *bb = smem + (t % Lds<Tr>::NBUF) * Lds<Tr>::BUF;
        const int n_valid = __builtin_amdgcn_readfirstlane(min(max(n_real - kt * 64, 0), 64));
        const int64_t tb = int64_t(kt) * 64 * row_stride;
        const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<char *>(kbase0 + tb), 0, n_valid * row_stride, kBufFlags);
        const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<char *>(vbase0 + tb), 0, n_valid * row_stride, kBufFlags);
#pragma unroll
        for (int jj = 0; jj < PER_WAVE; ++jj)
            buf_to_lds16(jj >= INSTR / kWaves ? rv : rk, bb + loff[jj], voff[jj]);
        if (wave == kWaves - 1) {
            const __amdgpu_buffer_rsrc_t re = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<int32_t *>(kend_row + kt * 64), 0, 256, kBufFlags);
            buf_to_lds4(re, bb + Lds<Tr>::KE_OFF, lane * 4);
        }
    };

    floatx16 s[2];                  // S^T of the tile the wave works on (two 32-key blocks)
    frag pf[2][Tr::NKS];            // its P^T operands

    // Lane-dependent byte offsets of the K / V fragments inside a tile (loop invariant).
    int klane[Tr::NDS], vlane[Tr::NDB];
#pragma unroll
    for (int ds = 0; ds < Tr::NDS; ++ds) klane[ds] = Tr::k_lane(ds, l32, h);
#pragma unroll
    for (int db = 0; db < Tr::NDB; ++db) vlane[db] = Tr::v_lane(db, lane);

    // Matrix phase as a fixed pipeline of MFMA slots: S^T = K Q^T for tile ts (16 slots) and/or
    // O^T += V^T P^T for tile tpv (16 slots), interleaved S, PV, S, PV, ...  Each slot's LDS
    // operand is read kAhead slots earlier into a small ring; scheduling fences keep this
    // order, so few fragments are in flight (no register pressure from hoisted reads).
    constexpr int kAhead = 4;
    auto matrix_ops = [&](auto with_pv, auto with_s, int tpv, int ts) __attribute__((always_inline)) {
        constexpr bool PV = decltype(with_pv)::value, S = decltype(with_s)::value;
        // S op n: 32-key block n % 2, head_dim step n / 2 (the two accumulator chains alternate);
        // PV op n: d-block n % NDB, key step (n / NDB) % NKS, 32-key block n / (NDB * NKS).
        constexpr int NS_ALL = 2 * Tr::NDS, NPV_ALL = 2 * Tr::NKS * Tr::NDB;
        static_assert(!(PV && S) || NS_ALL == NPV_ALL, "interleave needs equal slot counts");
        constexpr int NPV = PV ? NPV_ALL : 0, NS = S ? NS_ALL : 0, NSLOT = NPV + NS;
        const int bpv = (tpv % Lds<Tr>::NBUF) * Lds<Tr>::BUF, bs = (ts % Lds<Tr>::NBUF) * Lds<Tr>::BUF;
        // slot i -> (is S op, index within its kind): S, PV, S, PV, ... when both
        constexpr auto is_s = [](int i) { return (PV && S) ? (i % 2 == 0) : S; };
        constexpr auto idx = [](int i) { return (PV && S) ? i / 2 : i; };
        auto load = [&](auto ic) __attribute__((always_inline)) -> frag {
            constexpr int i = decltype(ic)::value, n = idx(i);
            if constexpr (is_s(i)) {
                return Tr::k_frag_at(smem + (bs + klane[n / 2]) + Lds<Tr>::K_OFF + Tr::K_KB_BYTES * (n % 2));
            } else {
                constexpr int db = n % Tr::NDB, kb = n / (Tr::NDB * Tr::NKS), ks = (n / Tr::NDB) % Tr::NKS;
                return Tr::template v_frag_at<kb, ks>(smem + (bpv + vlane[db]) + Lds<Tr>::V_OFF);
            }
        };
        if constexpr (S) {
            s[0] = zero16();
            s[1] = zero16();
        }
        frag ring[kAhead];
        static_for<(kAhead < NSLOT ? kAhead : NSLOT)>([&](auto ic) __attribute__((always_inline)) {
            constexpr int i = decltype(ic)::value;
            ring[i] = load(ic);
        });
        static_for<NSLOT>([&](auto ic) __attribute__((always_inline)) {
            constexpr int i = decltype(ic)::value, n = idx(i);
            const frag op = ring[i % kAhead];
            if constexpr (i + kAhead < NSLOT) ring[i % kAhead] = load(std::integral_constant<int, i + kAhead>{});
            if constexpr (is_s(i)) s[n % 2] = Tr::mfma(op, qf[n / 2], s[n % 2]);
            else acc[n % Tr::NDB] = Tr::mfma(op, pf[n / (Tr::NDB * Tr::NKS)][(n / Tr::NDB) % Tr::NKS], acc[n % Tr::NDB]);
            __builtin_amdgcn_sched_barrier(0);
        });
    };
    using yes = std::integral_constant<bool, true>;
    using no = std::integral_constant<bool, false>;
    auto softmax = [&](int t) __attribute__((always_inline)) {     // online softmax of tile t -> pf
        if (a.kt_kind[t_begin + t] == kTilePartial) {
            // Interval mask: key j visible to query i iff j <= i < kend[j].  Register i of block
            // kb holds key kbase + 4h + c with c = 32kb + 8(i/4) + i%4, so the first test is
            // c <= qpos - kbase - 4h against an immediate; kend comes four keys at a time.
            const int32_t *KEs = reinterpret_cast<const int32_t *>(
                smem + (t % Lds<Tr>::NBUF) * Lds<Tr>::BUF + Lds<Tr>::KE_OFF) + 4 * h;
            const int dq = qpos - a.kt_idx[t_begin + t] * 64 - 4 * h;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i4 = 0; i4 < 4; ++i4) {
                    const int4 ke = *reinterpret_cast<const int4 *>(KEs + 32 * kb + 8 * i4);
                    const int kev[4] = {ke.x, ke.y, ke.z, ke.w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int c = 32 * kb + 8 * i4 + e;
                        const bool vis = (c <= dq) & (qpos < kev[e]);
                        s[kb][4 * i4 + e] = vis ? s[kb][4 * i4 + e] : -INFINITY;
                    }
                }
        }
        float mx = s[0][0];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
        mx = xchg_max(mx);
        const bool grow = mx * a.c > m_run * a.c + kGrow;
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {
            const float m_new = grow ? mx : m_run;
            const float alpha = grow ? __builtin_amdgcn_exp2f((m_run - m_new) * a.c) : 1.f;
            l_run *= alpha;
            w_run *= alpha;
#pragma unroll
            for (int db = 0; db < Tr::NDB; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[db][i] *= alpha;
            m_run = m_new;
        }
        const float mc = (m_run == -INFINITY ? 0.f : m_run) * a.c;
        float ls = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float e = __builtin_amdgcn_exp2f(fmaf(s[kb][i], a.c, -mc));
                s[kb][i] = e;
                ls += e;
            }
#pragma unroll
            for (int ks = 0; ks < Tr::NKS; ++ks) {
                pf[kb][ks] = Tr::p_frag(s[kb], ks);
                if constexpr (Tr::kRoundedP) w_run = Tr::wsum(pf[kb][ks], w_run);
            }
        }
        l_run += ls;
    };

    auto matrix_phase = [&](int t) __attribute__((always_inline)) {   // M(t): PV of tile t and S of tile t+1
        __builtin_amdgcn_s_setprio(1);
        // One code path for every tile (two variants in the loop cost ~70 spilled registers);
        // on the last tile the S slots recompute S of the same tile, which is never used.
        matrix_ops(yes{}, yes{}, t, t + 1 < N ? t + 1 : t);
        __builtin_amdgcn_s_setprio(0);
    };
    auto first_s = [&]() __attribute__((always_inline)) {
        __builtin_amdgcn_s_setprio(1);
        matrix_ops(no{}, yes{}, 0, 0);
        __builtin_amdgcn_s_setprio(0);
    };

    // Steps are numbered globally; barrier #n ends step n.  Group 0: step 1 S(0), step 2t+2
    // V(t), step 2t+3 M(t); group 1 runs one step later.  Tile s is copied in two halves:
    // group 1's waves issue theirs in step 2s-3, group 0's in step 2s-2 (tiles 0 and 1 in the
    // prologue), each at the start of a softmax phase.  Tile s is first read in step 2s+1, so
    // at the end of step 2s every wave waits for its copies of tile s only (the next tile's
    // may stay in flight: two steps of lead time).  Tile s+4 reuses tile s's buffer from step
    // 2s+5; tile s is last read in step 2s+4.  Both groups pass 2N+3 barriers.
    int step = 0, issued = -1;
    auto issue_tile = [&](int t) __attribute__((always_inline)) {
        issue(t);
        issued = t;
    };
    auto step_end = [&]() __attribute__((always_inline)) {
        if ((step & 1) == 0 && (step >> 1) < N) {
            if (issued <= (step >> 1)) wait_loads_but<0>();
            else if (wave == kWaves - 1) wait_loads_but<PER_WAVE + 1>();
            else wait_loads_but<PER_WAVE>();
        }
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        ++step;
    };

    if (N > 0) issue_tile(0);
    if (N > 1) issue_tile(1);
    step_end();                                   // step 0
    if (grp == 1) {
        if (N > 2) issue_tile(2);                 // step 1
        step_end();
    }
    if (N > 0) first_s();                         // step 1 (group 0) / 2 (group 1)
    step_end();
    for (int t = 0; t < N; ++t) {
        if (t + 2 + grp < N) issue_tile(t + 2 + grp);
        softmax(t);
        step_end();
        matrix_phase(t);
        step_end();
    }
    if (grp == 0) step_end();                     // step 2N+2

    // Epilogue: combine the two lane halves' partial sums, normalize, write O and LSE.
    const float l_tot = xchg_sum(l_run);
    const float w_tot = Tr::kRoundedP ? xchg_sum(w_run) : l_tot;
    const float inv = w_tot > 0.f ? 1.f / w_tot : 0.f;
    elem *op = reinterpret_cast<elem *>(a.o) + ((int64_t(r) * T + qpos) * a.Hq + head) * D;
#pragma unroll
    for (int db = 0; db < Tr::NDB; ++db) {
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
            const int d0 = 32 * db + 8 * i4 + 4 * h;
            float vals[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) vals[e] = acc[db][4 * i4 + e] * inv;
            if constexpr (Tr::kEsz == 2) {
                uint2 w;
                w.x = uint32_t(__builtin_bit_cast(uint16_t, static_cast<__bf16>(vals[0]))) |
                      (uint32_t(__builtin_bit_cast(uint16_t, static_cast<__bf16>(vals[1]))) << 16);
                w.y = uint32_t(__builtin_bit_cast(uint16_t, static_cast<__bf16>(vals[2]))) |
                      (uint32_t(__builtin_bit_cast(uint16_t, static_cast<__bf16>(vals[3]))) << 16);
                *reinterpret_cast<uint2 *>(op + d0) = w;
            } else {
                *reinterpret_cast<float4 *>(op + d0) = make_float4(vals[0], vals[1], vals[2], vals[3]);
            }
        }
    }
    if (h == 0) {
        const float lse = l_tot > 0.f ? m_run * a.scale + __logf(l_tot) : -INFINITY;
        a.lse[(int64_t(r) * a.Hq + head) * T + qpos] = lse;
    }
}

template <class Tr>
hipError_t launch_tr(const FwdArgs &args, int n_blocks, hipStream_t s) {
    constexpr int smem = Lds<Tr>::NBUF * Lds<Tr>::BUF;
    auto kern = tree_attn_fwd_kernel<Tr>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, smem);
    if (e != hipSuccess) return e;
    kern<<<n_blocks, kWaves * 64, smem, s>>>(args);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd(const FwdShape &sh, const WsLayout &w, const char *ws, const void *q,
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
    const int64_t n_blocks = int64_t(sh.R) * w.nQ * a.L;
    if (n_blocks == 0) return hipSuccess;
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
