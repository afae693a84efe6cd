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
// Work decomposition (one workgroup = 4 waves = 256 (query head, position) rows):
//   * item = (row, q-tile of BQ positions, KV head g, chunk of HCH query heads of group g);
//     BQ * HCH = 256, so every item owns the same number of rows and each staged K/V tile is
//     shared by all HCH heads of the group (grouped-query reuse);
//   * wave w owns two 32-row blocks; with HCH >= 2 they are two heads at the same 32
//     positions (one mask evaluation serves both), with HCH == 1 two position blocks;
//   * every K or V fragment read from LDS feeds two MFMAs (one per row block).
// MFMA orientation: S^T = K Q^T and O^T = V^T P^T, so each lane owns one query (column) of
// every 32x32 accumulator: row max / row sum are in-lane plus one exchange with lane^32, and
// the P^T operand of the second product is the first product's accumulator, converted in
// place with no data movement.  V is stored transposed in LDS so its fragments are
// contiguous 16-byte reads.
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

template <int D_>
struct Bf16Traits {
    static constexpr int D = D_;
    static constexpr int kEsz = 2;
    static constexpr int NDS = D / 16;        // MFMA k-steps over head_dim for S^T
    static constexpr int NKS = 2;             // MFMA k-steps per 32-key block for O^T
    static constexpr int NDB = D / 32;        // 32-row blocks of O^T
    static constexpr int CPR = D / 8;         // 16-byte chunks per K/V row
    static constexpr int K_LDS = 64 * D;      // elements
    static constexpr int V_LDS = D * 64;
    using frag = bf16x8_t;
    using elem = uint16_t;

    static __device__ __forceinline__ floatx16 mfma(frag a, frag b, floatx16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    // K tile: [64 keys][D], 16-byte chunk index XOR-swizzled by the key so the 32 lanes of a
    // half-wave (32 consecutive keys, one chunk) hit distinct banks.
    static __device__ __forceinline__ int k_off(int key, int chunk) {
        return key * D + ((chunk ^ (key & (CPR - 1))) << 3);
    }
    static __device__ __forceinline__ frag k_frag(const elem *K, int key, int ds, int h) {
        return *reinterpret_cast<const frag *>(K + k_off(key, 2 * ds + h));
    }
    // V^T tile: [D rows][64 key positions]; 16-byte pair index swizzled by the row.
    static __device__ __forceinline__ int v_sw(int d) { return ((d >> 1) & 7) ^ ((d >> 4) & 7); }
    static __device__ __forceinline__ frag v_frag(const elem *V, int d, int kb, int ks, int h) {
        const int pair = 4 * kb + 2 * ks + h;
        return *reinterpret_cast<const frag *>(V + d * 64 + ((pair ^ v_sw(d)) << 3));
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
};

template <int D_>
struct F32Traits {
    static constexpr int D = D_;
    static constexpr int kEsz = 4;
    static constexpr int NDS = D / 2;
    static constexpr int NKS = 16;
    static constexpr int NDB = D / 32;
    static constexpr int CPR = D / 4;
    static constexpr int KP = D + 1;          // padded pitches (conflict-free column reads)
    static constexpr int VP = 64 + 1;
    static constexpr int K_LDS = 64 * KP;
    static constexpr int V_LDS = D * VP;
    using frag = float;
    using elem = float;

    static __device__ __forceinline__ floatx16 mfma(frag a, frag b, floatx16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ frag k_frag(const elem *K, int key, int ds, int h) {
        return K[key * KP + 2 * ds + h];
    }
    // key of lane-half h, element of key step ks inside a 32-key block (accumulator layout).
    static __device__ __forceinline__ frag v_frag(const elem *V, int d, int kb, int ks, int h) {
        return V[d * VP + 32 * kb + 8 * (ks >> 2) + 4 * h + (ks & 3)];
    }
    static __device__ __forceinline__ frag q_frag(const elem *q, int ds, int h) { return q[2 * ds + h]; }
    static __device__ __forceinline__ frag p_frag(const floatx16 &p, int ks) { return p[ks]; }
};

// --------------------------------------------------------------------------- K/V tile staging

__device__ __forceinline__ uint32_t word(const uint4 &v, int i) {
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}
__device__ __forceinline__ float fword(const uint4 &v, int i) { return __uint_as_float(word(v, i)); }

// Global -> registers for one 64-key tile; registers -> LDS after the previous tile's last use.
template <class Tr>
struct Stage {
    static constexpr int KCH = 64 * Tr::CPR;                       // 16-byte chunks per K tile
    static constexpr int NK = (KCH + 255) / 256;                   // per thread
    // V: bf16 threads own 4 consecutive keys x one 16-byte chunk (transposed on the way to
    // LDS); f32 uses the K pattern and scatters elements.
    static constexpr int VUNITS = Tr::kEsz == 2 ? 16 * Tr::CPR : KCH;
    static constexpr int NV = Tr::kEsz == 2 ? (VUNITS + 255) / 256 * 4 : (VUNITS + 255) / 256;
    uint4 kr[NK];
    uint4 vr[NV];
    int32_t ke;

    __device__ __forceinline__ void load(const char *kbase, const char *vbase, const int32_t *kend_t,
                                         int64_t row_stride, int tid, int n_valid) {
#pragma unroll
        for (int i = 0; i < NK; ++i) {
            const int cid = tid + 256 * i;
            if (KCH % 256 == 0 || cid < KCH) {
                const int key = cid / Tr::CPR, ch = cid % Tr::CPR;
                kr[i] = *reinterpret_cast<const uint4 *>(kbase + key * row_stride + ch * 16);
            }
        }
        if constexpr (Tr::kEsz == 2) {
#pragma unroll
            for (int i = 0; i < NV / 4; ++i) {
                const int u = tid + 256 * i;
                if (u < VUNITS) {
                    const int kq = u / Tr::CPR, ch = u % Tr::CPR;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        // Every key of a tile lies inside the row, so the load is always in
                        // bounds; pad keys (>= n_valid) are zeroed so NaN pads cannot reach PV.
                        const int key = 4 * kq + j;
                        uint4 x = *reinterpret_cast<const uint4 *>(vbase + key * row_stride + ch * 16);
                        const uint32_t keep = key < n_valid ? ~0u : 0u;
                        x.x &= keep; x.y &= keep; x.z &= keep; x.w &= keep;
                        vr[4 * i + j] = x;
                    }
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                const int cid = tid + 256 * i;
                if (cid < KCH) {
                    const int key = cid / Tr::CPR, ch = cid % Tr::CPR;
                    uint4 x = *reinterpret_cast<const uint4 *>(vbase + key * row_stride + ch * 16);
                    const uint32_t keep = key < n_valid ? ~0u : 0u;
                    x.x &= keep; x.y &= keep; x.z &= keep; x.w &= keep;
                    vr[i] = x;
                }
            }
        }
        if (tid < 64) ke = kend_t[tid];
    }

    __device__ __forceinline__ void store(typename Tr::elem *K, typename Tr::elem *V, int32_t *KE, int tid) {
        if constexpr (Tr::kEsz == 2) {
#pragma unroll
            for (int i = 0; i < NK; ++i) {
                const int cid = tid + 256 * i;
                if (KCH % 256 == 0 || cid < KCH) {
                    const int key = cid / Tr::CPR, ch = cid % Tr::CPR;
                    *reinterpret_cast<uint4 *>(K + Tr::k_off(key, ch)) = kr[i];
                }
            }
#pragma unroll
            for (int i = 0; i < NV / 4; ++i) {
                const int u = tid + 256 * i;
                if (u < VUNITS) {
                    const int kq = u / Tr::CPR, ch = u % Tr::CPR;
                    // keys 4kq..4kq+3 land on 4 consecutive positions of the permuted order
                    // position(key) = 16ks + 8h + 4e_hi + e_lo for key = 16ks + 8e_hi + 4h + e_lo.
                    const int pq = 8 * (kq >> 3) + 4 * ((kq >> 2) & 1) + 2 * (kq & 1) + ((kq >> 1) & 1);
                    const int pair = pq >> 1, half = pq & 1;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int d = ch * 8 + e;
                        const int sh = (e & 1) * 16;
                        const uint32_t a0 = (word(vr[4 * i + 0], e >> 1) >> sh) & 0xffffu;
                        const uint32_t a1 = (word(vr[4 * i + 1], e >> 1) >> sh) & 0xffffu;
                        const uint32_t a2 = (word(vr[4 * i + 2], e >> 1) >> sh) & 0xffffu;
                        const uint32_t a3 = (word(vr[4 * i + 3], e >> 1) >> sh) & 0xffffu;
                        uint2 val;
                        val.x = a0 | (a1 << 16);
                        val.y = a2 | (a3 << 16);
                        *reinterpret_cast<uint2 *>(V + d * 64 + ((pair ^ Tr::v_sw(d)) << 3) + half * 4) = val;
                    }
                }
            }
        } else {
#pragma unroll
            for (int i = 0; i < NK; ++i) {
                const int cid = tid + 256 * i;
                if (cid < KCH) {
                    const int key = cid / Tr::CPR, ch = cid % Tr::CPR;
#pragma unroll
                    for (int e = 0; e < 4; ++e) K[key * Tr::KP + ch * 4 + e] = fword(kr[i], e);
                }
            }
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                const int cid = tid + 256 * i;
                if (cid < KCH) {
                    const int key = cid / Tr::CPR, ch = cid % Tr::CPR;
#pragma unroll
                    for (int e = 0; e < 4; ++e) V[(ch * 4 + e) * Tr::VP + key] = fword(vr[i], e);
                }
            }
        }
        if (tid < 64) KE[tid] = ke;
    }
};

// ------------------------------------------------------------------------------------ kernel

template <class Tr, bool kSamePos>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void tree_attn_fwd_kernel(FwdArgs a) {
    using elem = typename Tr::elem;
    using frag = typename Tr::frag;
    constexpr int D = Tr::D;

    __shared__ __attribute__((aligned(16))) elem Ks[Tr::K_LDS];
    __shared__ __attribute__((aligned(16))) elem Vs[Tr::V_LDS];
    __shared__ int32_t KEs[64];

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

    // The wave's two row blocks.
    int head[2], pos0[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const int rb = 2 * wave + b;
        const int hl = rb % a.HCH, pb = rb / a.HCH;
        head[b] = g * a.G + chunk * a.HCH + hl;
        pos0[b] = qt * a.BQ + pb * 32;
    }
    const int qpos[2] = {pos0[0] + l32, pos0[1] + l32};

    // Q fragments (B operand of S^T = K Q^T): lane holds query l32, head_dim chunk (2ds + h).
    frag qf[2][Tr::NDS];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const elem *qrow = reinterpret_cast<const elem *>(a.q) +
                           ((int64_t(r) * T + qpos[b]) * a.Hq + head[b]) * D;
#pragma unroll
        for (int ds = 0; ds < Tr::NDS; ++ds) qf[b][ds] = Tr::q_frag(qrow, ds, h);
    }

    floatx16 acc[2][Tr::NDB];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int db = 0; db < Tr::NDB; ++db) acc[b][db] = zero16();
    float m_run[2] = {-INFINITY, -INFINITY};
    float l_run[2] = {0.f, 0.f};

    const int32_t t_begin = a.qt_ptr[tile], t_end = a.qt_ptr[tile + 1];
    const int64_t row_stride = int64_t(a.Hkv) * D * Tr::kEsz;   // bytes between keys
    const char *kbase0 = reinterpret_cast<const char *>(a.k) + ((int64_t(r) * T) * a.Hkv + g) * D * Tr::kEsz;
    const char *vbase0 = reinterpret_cast<const char *>(a.v) + ((int64_t(r) * T) * a.Hkv + g) * D * Tr::kEsz;
    const int32_t *kend_row = a.kend + int64_t(r) * T;

    Stage<Tr> stg;
    if (t_begin < t_end) {
        const int kt = a.kt_idx[t_begin];
        stg.load(kbase0 + int64_t(kt) * 64 * row_stride, vbase0 + int64_t(kt) * 64 * row_stride,
                 kend_row + kt * 64, row_stride, tid, n_real - kt * 64);
        stg.store(Ks, Vs, KEs, tid);
    }
    __syncthreads();

    for (int32_t t = t_begin; t < t_end; ++t) {
        const int kt = a.kt_idx[t];
        const bool partial = a.kt_kind[t] == kTilePartial;
        if (t + 1 < t_end) {
            const int kn = a.kt_idx[t + 1];
            stg.load(kbase0 + int64_t(kn) * 64 * row_stride, vbase0 + int64_t(kn) * 64 * row_stride,
                     kend_row + kn * 64, row_stride, tid, n_real - kn * 64);
        }

        // S^T = K Q^T for the two 32-key blocks of the tile, both row blocks.
        floatx16 s[2][2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            s[0][kb] = zero16();
            s[1][kb] = zero16();
#pragma unroll
            for (int ds = 0; ds < Tr::NDS; ++ds) {
                const frag kf = Tr::k_frag(Ks, 32 * kb + l32, ds, h);
                s[0][kb] = Tr::mfma(kf, qf[0][ds], s[0][kb]);
                s[1][kb] = Tr::mfma(kf, qf[1][ds], s[1][kb]);
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
                    const bool v1 = kSamePos ? v0 : (key <= qpos[1] && qpos[1] < ke);
                    s[0][kb][i] = v0 ? s[0][kb][i] : -INFINITY;
                    s[1][kb][i] = v1 ? s[1][kb][i] : -INFINITY;
                }
            }
        }

        // Online softmax (scores kept raw; exp2 with the scale folded into the FMA).  The
        // exponentials overwrite the scores in place and are packed into P^T operands.
        frag pf[2][2][Tr::NKS];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            float mx = s[b][0][0];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[b][kb][i]);
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
            const float m_new = fmaxf(m_run[b], mx);
            const float m_use = m_new == -INFINITY ? 0.f : m_new;
            const float mc = m_use * a.c;
            const float alpha = __builtin_amdgcn_exp2f(m_run[b] * a.c - mc);
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
                for (int ks = 0; ks < Tr::NKS; ++ks) pf[b][kb][ks] = Tr::p_frag(s[b][kb], ks);
            }
            l_run[b] = l_run[b] * alpha + ls;
            m_run[b] = m_new;
#pragma unroll
            for (int db = 0; db < Tr::NDB; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[b][db][i] *= alpha;
        }

        // O^T += V^T P^T.
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
            for (int ks = 0; ks < Tr::NKS; ++ks) {
#pragma unroll
                for (int db = 0; db < Tr::NDB; ++db) {
                    const frag vf = Tr::v_frag(Vs, 32 * db + l32, kb, ks, h);
                    acc[0][db] = Tr::mfma(vf, pf[0][kb][ks], acc[0][db]);
                    acc[1][db] = Tr::mfma(vf, pf[1][kb][ks], acc[1][db]);
                }
            }
        }

        __syncthreads();
        if (t + 1 < t_end) stg.store(Ks, Vs, KEs, tid);
        __syncthreads();
    }

    // Epilogue: combine the two lane halves' partial sums, normalize, write O and LSE.
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const float l_tot = l_run[b] + __shfl_xor(l_run[b], 32, 64);
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
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

template <class Tr>
hipError_t launch_tr(const FwdArgs &args, int n_blocks, bool same_pos, hipStream_t s) {
    if (same_pos)
        tree_attn_fwd_kernel<Tr, true><<<n_blocks, 256, 0, s>>>(args);
    else
        tree_attn_fwd_kernel<Tr, false><<<n_blocks, 256, 0, s>>>(args);
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
