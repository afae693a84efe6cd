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
    const char *zeros;     // >= 512 zero bytes (source of pad rows)
    int32_t T, Hq, Hkv, G, HCH, nQ, L, BQ;
    float c;       // scale * log2(e): exponent scale for exp2
    float scale;   // softmax scale (for the natural-log LSE)
};

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
    static __device__ __forceinline__ frag p_frag(const floatx16 &p, int ks) { return p[ks]; }
    static __device__ __forceinline__ float wsum(frag f, float acc) { return acc + f; }
    static constexpr bool kRoundedP = false;
};

// LDS buffer layout: [K tile][V tile][kend of the tile's 64 keys].
template <class Tr>
struct Lds {
    static constexpr int TILE = 64 * Tr::D * Tr::kEsz;
    static constexpr int K_OFF = 0, V_OFF = TILE, KE_OFF = 2 * TILE;
    static constexpr int BUF = 2 * TILE + 256;
};

__device__ __forceinline__ void lds_dma16(const void *src, void *lds_dst) {
    __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1))) *)src,
                                     (void __attribute__((address_space(3))) *)lds_dst, 16, 0, 0);
}
__device__ __forceinline__ void lds_dma4(const void *src, void *lds_dst) {
    __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1))) *)src,
                                     (void __attribute__((address_space(3))) *)lds_dst, 4, 0, 0);
}
// Wait until this wave's loads (including direct-to-LDS ones) have landed.
__device__ __forceinline__ void wait_loads() { __builtin_amdgcn_s_waitcnt(0x0f70); }

// Copy one 64-key tile (K, V, kend) HBM -> LDS buffer.  One wave instruction moves 64 chunks of
// 16 bytes into 1 KB of consecutive LDS, lane l landing at byte 16 l; the lane's source is the
// chunk that belongs there after swizzling.  Keys at or past the row's last real token read a
// zero block instead, so pad rows of K and V are zero in LDS (NaN pads cannot reach PV).
template <class Tr, int NW>
__device__ __forceinline__ void issue_tile(char *buf, const char *kbase, const char *vbase, const char *zeros,
                                           const int32_t *kend_t, int64_t row_stride, int n_valid,
                                           int wave, int lane) {
    constexpr int ROWS = 64 / Tr::CPR;          // rows per instruction
    constexpr int INSTR = Tr::CPR;              // instructions per tensor
    static_assert((2 * INSTR) % NW == 0, "waves must split the tile evenly");
    const int pc = lane % Tr::CPR;
#pragma unroll
    for (int jj = 0; jj < 2 * INSTR / NW; ++jj) {
        const int i = wave + NW * jj;
        const bool isv = jj >= INSTR / NW;      // i >= INSTR
        const int blk = isv ? i - INSTR : i;
        const int row = blk * ROWS + lane / Tr::CPR;
        const int c = pc ^ (isv ? Tr::vsw(row) : Tr::ksw(row));
        const char *src = row < n_valid ? (isv ? vbase : kbase) + row * row_stride + c * 16 : zeros + c * 16;
        lds_dma16(src, buf + (isv ? Lds<Tr>::V_OFF : Lds<Tr>::K_OFF) + blk * 1024);
    }
    if (wave == NW - 1) lds_dma4(kend_t + lane, buf + Lds<Tr>::KE_OFF);
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

// RB 32-row blocks per wave, NW waves per workgroup, RB * NW * 32 = 256 rows per workgroup.
template <class Tr, int RB, int NW, bool kSamePos>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4)))
void tree_attn_fwd_kernel(FwdArgs a) {
    static_assert(RB * NW == 8, "a workgroup owns 8 row blocks of 32");
    using elem = typename Tr::elem;
    using frag = typename Tr::frag;
    constexpr int D = Tr::D;
    // Grow the running max only when a tile's max exceeds it by more than 2^8 in the
    // exponent domain; otherwise keep the stale reference (exp2 values stay <= 256), which
    // leaves O and l exactly consistent and skips the rescale of the accumulators.
    constexpr float kGrow = 8.0f;

    extern __shared__ __attribute__((aligned(1024))) char smem[];

    if (a.status[0] != 0) return;   // invalid segment table: write nothing

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int l32 = lane & 31, h = lane >> 5;
    const int bid = blockIdx.x;
    const int u = bid % a.L, item = bid / a.L;
    const int g = u % a.Hkv, chunk = u / a.Hkv;
    const int tile = a.work[item];
    const int r = tile / a.nQ, qt = tile % a.nQ;
    const int T = a.T;
    const int n_real = a.n_real[r];

    int head[RB], qpos[RB];
#pragma unroll
    for (int b = 0; b < RB; ++b) {
        const int rb = RB * wave + b;
        const int hl = rb % a.HCH, pb = rb / a.HCH;
        head[b] = g * a.G + chunk * a.HCH + hl;
        qpos[b] = qt * a.BQ + pb * 32 + l32;
    }

    // Q fragments (B operand of S^T = K Q^T): lane holds query l32, head_dim chunk (2ds + h).
    frag qf[RB][Tr::NDS];
#pragma unroll
    for (int b = 0; b < RB; ++b) {
        const elem *qrow = reinterpret_cast<const elem *>(a.q) + ((int64_t(r) * T + qpos[b]) * a.Hq + head[b]) * D;
#pragma unroll
        for (int ds = 0; ds < Tr::NDS; ++ds) qf[b][ds] = Tr::q_frag(qrow, ds, h);
    }

    floatx16 acc[RB][Tr::NDB];
#pragma unroll
    for (int b = 0; b < RB; ++b)
#pragma unroll
        for (int db = 0; db < Tr::NDB; ++db) acc[b][db] = zero16();
    // m_run: reference max (raw score units); l_run: fp32 sum of the exponentials (for LSE);
    // w_run: sum of the weights as rounded for the PV product (normalizes O, so the weights
    // applied to V sum to one exactly as used).
    float m_run[RB], l_run[RB], w_run[RB];
#pragma unroll
    for (int b = 0; b < RB; ++b) { m_run[b] = -INFINITY; l_run[b] = 0.f; w_run[b] = 0.f; }

    const int32_t t_begin = a.qt_ptr[tile], t_end = a.qt_ptr[tile + 1];
    const int64_t row_stride = int64_t(a.Hkv) * D * Tr::kEsz;   // bytes between keys
    const char *kbase0 = reinterpret_cast<const char *>(a.k) + ((int64_t(r) * T) * a.Hkv + g) * D * Tr::kEsz;
    const char *vbase0 = reinterpret_cast<const char *>(a.v) + ((int64_t(r) * T) * a.Hkv + g) * D * Tr::kEsz;
    const int32_t *kend_row = a.kend + int64_t(r) * T;
    const int64_t tile_bytes = 64 * row_stride;

    int buf = 0;
    if (t_begin < t_end) {
        const int kt = a.kt_idx[t_begin];
        issue_tile<Tr, NW>(smem, kbase0 + kt * tile_bytes, vbase0 + kt * tile_bytes, a.zeros, kend_row + kt * 64,
                           row_stride, n_real - kt * 64, wave, lane);
    }
    wait_loads();
    __syncthreads();

    for (int32_t t = t_begin; t < t_end; ++t) {
        const int kt = a.kt_idx[t];
        const bool partial = a.kt_kind[t] == kTilePartial;
        if (t + 1 < t_end) {
            const int kn = a.kt_idx[t + 1];
            issue_tile<Tr, NW>(smem + (buf ^ 1) * Lds<Tr>::BUF, kbase0 + kn * tile_bytes, vbase0 + kn * tile_bytes,
                               a.zeros, kend_row + kn * 64, row_stride, n_real - kn * 64, wave, lane);
        }
        const char *bb = smem + buf * Lds<Tr>::BUF;
        const elem *Ks = reinterpret_cast<const elem *>(bb + Lds<Tr>::K_OFF);
        const elem *Vs = reinterpret_cast<const elem *>(bb + Lds<Tr>::V_OFF);
        const int32_t *KEs = reinterpret_cast<const int32_t *>(bb + Lds<Tr>::KE_OFF);

        // S^T = K Q^T for the two 32-key blocks of the tile.
        floatx16 s[RB][2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int b = 0; b < RB; ++b) s[b][kb] = zero16();
#pragma unroll
            for (int ds = 0; ds < Tr::NDS; ++ds) {
                const frag kf = Tr::k_frag(Ks, 32 * kb + l32, ds, h);
#pragma unroll
                for (int b = 0; b < RB; ++b) s[b][kb] = Tr::mfma(kf, qf[b][ds], s[b][kb]);
            }
        }

        // Interval mask on PARTIAL tiles: key j visible to query i iff j <= i < kend[j].
        if (partial) {
            const int kbase = kt * 64;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int kl = 32 * kb + 8 * (i >> 2) + 4 * h + (i & 3);
                    const int key = kbase + kl, ke = KEs[kl];
                    const bool v0 = key <= qpos[0] && qpos[0] < ke;
#pragma unroll
                    for (int b = 0; b < RB; ++b) {
                        const bool vb = (b == 0 || kSamePos) ? v0 : (key <= qpos[b] && qpos[b] < ke);
                        s[b][kb][i] = vb ? s[b][kb][i] : -INFINITY;
                    }
                }
            }
        }

        // Online softmax on raw scores; exp2 with the scale folded into the FMA.
        frag pf[RB][2][Tr::NKS];
#pragma unroll
        for (int b = 0; b < RB; ++b) {
            float mx = s[b][0][0];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[b][kb][i]);
            mx = xchg_max(mx);
            const bool grow = mx * a.c > m_run[b] * a.c + kGrow;
            if (__builtin_amdgcn_ballot_w64(grow) != 0) {
                const float m_new = grow ? mx : m_run[b];
                const float alpha = grow ? __builtin_amdgcn_exp2f((m_run[b] - m_new) * a.c) : 1.f;
                l_run[b] *= alpha;
                w_run[b] *= alpha;
#pragma unroll
                for (int db = 0; db < Tr::NDB; ++db)
#pragma unroll
                    for (int i = 0; i < 16; ++i) acc[b][db][i] *= alpha;
                m_run[b] = m_new;
            }
            const float mc = (m_run[b] == -INFINITY ? 0.f : m_run[b]) * a.c;
            float ls = 0.f;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float e = __builtin_amdgcn_exp2f(fmaf(s[b][kb][i], a.c, -mc));
                    s[b][kb][i] = e;
                    ls += e;
                }
#pragma unroll
                for (int ks = 0; ks < Tr::NKS; ++ks) {
                    pf[b][kb][ks] = Tr::p_frag(s[b][kb], ks);
                    if constexpr (Tr::kRoundedP) w_run[b] = Tr::wsum(pf[b][kb][ks], w_run[b]);
                }
            }
            l_run[b] += ls;
        }

        // O^T += V^T P^T.
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int ks = 0; ks < Tr::NKS; ++ks) {
#pragma unroll
                for (int db = 0; db < Tr::NDB; ++db) {
                    const frag vf = Tr::v_frag(Vs, lane, db, kb, ks);
#pragma unroll
                    for (int b = 0; b < RB; ++b) acc[b][db] = Tr::mfma(vf, pf[b][kb][ks], acc[b][db]);
                }
            }
        }

        wait_loads();
        __syncthreads();
        buf ^= 1;
    }

    // Epilogue: combine the two lane halves' partial sums, normalize, write O and LSE.
#pragma unroll
    for (int b = 0; b < RB; ++b) {
        const float l_tot = xchg_sum(l_run[b]);
        const float w_tot = Tr::kRoundedP ? xchg_sum(w_run[b]) : l_tot;
        const float inv = w_tot > 0.f ? 1.f / w_tot : 0.f;
        const int64_t orow = (int64_t(r) * T + qpos[b]) * a.Hq + head[b];
        elem *op = reinterpret_cast<elem *>(a.o) + orow * D;
#pragma unroll
        for (int db = 0; db < Tr::NDB; ++db) {
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const int d0 = 32 * db + 8 * i4 + 4 * h;
                float vals[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) vals[e] = acc[b][db][4 * i4 + e] * inv;
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
            const float lse = l_tot > 0.f ? m_run[b] * a.scale + __logf(l_tot) : -INFINITY;
            a.lse[(int64_t(r) * a.Hq + head[b]) * T + qpos[b]] = lse;
        }
    }
}

template <class Tr, int RB, int NW>
hipError_t launch_cfg(const FwdArgs &args, int n_blocks, bool same_pos, hipStream_t s) {
    constexpr int smem = 2 * Lds<Tr>::BUF;
    auto k1 = tree_attn_fwd_kernel<Tr, RB, NW, true>;
    auto k0 = tree_attn_fwd_kernel<Tr, RB, NW, false>;
    auto kern = same_pos ? k1 : k0;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, smem);
    if (e != hipSuccess) return e;
    kern<<<n_blocks, NW * 64, smem, s>>>(args);
    return hipGetLastError();
}

// Eight waves of one 32-row block each: two waves per SIMD, so one wave's softmax (VALU) runs
// while the other's MFMAs issue.  (Four waves of two row blocks each, one wave per SIMD,
// measured 774 against 953 TFLOP/s on the long-prefix row.)
template <class Tr>
hipError_t launch_tr(const FwdArgs &args, int n_blocks, bool same_pos, hipStream_t s) {
    return launch_cfg<Tr, 1, 8>(args, n_blocks, same_pos, s);
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
    a.zeros = ws + w.zeros;
    a.T = sh.T; a.Hq = sh.Hq; a.Hkv = sh.Hkv; a.G = sh.G; a.HCH = sh.HCH;
    a.nQ = w.nQ; a.BQ = sh.BQ;
    a.L = sh.Hkv * (sh.G / sh.HCH);
    a.scale = sh.scale;
    a.c = sh.scale * 1.4426950408889634f;
    const int64_t n_blocks = int64_t(sh.R) * w.nQ * a.L;
    if (n_blocks == 0) return hipSuccess;
    if (n_blocks > INT32_MAX) return hipErrorInvalidValue;
    const bool same_pos = sh.HCH >= 2;
    if (sh.dtype == TREE_DT_BF16) {
        if (sh.D == 128) return launch_tr<Bf16Traits<128>>(a, int(n_blocks), same_pos, s);
        if (sh.D == 64) return launch_tr<Bf16Traits<64>>(a, int(n_blocks), same_pos, s);
    } else {
        if (sh.D == 64) return launch_tr<F32Traits<64>>(a, int(n_blocks), same_pos, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace treeattn
