// Gated delta rule over tree-packed rows for gfx950 (CDNA4), head_dim 128, bf16 in and out.
//
// "Prefix tree packing" (furtherai.github.io), GDN passage: the layer is recurrent, so it
// carries a state along each path instead of using a mask: a child segment starts from the
// state its parent segment ended with, and a root starts from zero; the planner takes one tree depth at a time and runs one causal-conv pass and one
// chunked delta-rule pass per depth, a child starting from its parent's final state.  The
// layer itself (not printed on the page) is the published gated delta rule with a width-4
// depthwise causal convolution, per head:
//   y_c(t) = SiLU(sum_j w_c[:, 3-j] x_c(pi^j(t)))      (pi: token parent; zero past a root)
//   q^ = y_q / sqrt(|y_q|^2 + eps) / sqrt(D),  k^ = y_k / sqrt(|y_k|^2 + eps),  v^ = y_v
//   h_t = a_t (h_pi(t) - b_t k^_t (k^_t^T h_pi(t))) + b_t k^_t v^_t^T,  o_t = h_t^T q^_t.
//
// Launches (all on the caller's stream):
//   * gdn_conv: one workgroup per (16 tokens, tensor q / k / v); the conv follows the
//     token-parent chain, so a child's first tokens convolve with its parent's last ones (the
//     context carried across the join), from a window of the three rows before each token
//     that is reloaded only where the chain leaves the previous row.
//   * gdn_prep: one workgroup per (chunk, head), chunk-parallel.  Chunks are 64 tokens of one
//     segment, counted from the segment's start (the last one ragged), so every segment ends
//     on a chunk boundary and its exact final state is available to its children: no tail is
//     replayed.  With G the cumulative log-decay inside the chunk, gamma = exp(G):
//       A_ts = b_t gamma_t/gamma_s k_t.k_s (s < t),  P_ts = gamma_t/gamma_s q_t.k_s (s <= t),
//       U = (I + A)^-1 diag(b) V,  Y = (I + A)^-1 diag(b gamma) K      (forward substitution)
//     Gram and QK^T on MFMA; (I + A)^-1 in fp32 by 16 x 16 blocks over the four waves (the
//     diagonal blocks by forward substitution, the others from them), U and Y on MFMA.  Prep
//     also writes the decay factors gamma_t and gamma_C / gamma_t, and U in the order the
//     scan's accumulators hold it, so the scan computes no exponential and reads U as whole
//     16-byte lanes.
//   * gdn_scan, once per tree depth: one workgroup per (segment of that depth, head), 4 waves,
//     each holding 32 columns of the 128 x 128 state H in fp32 MFMA accumulators, from the
//     parent's final state (zero at roots); per chunk
//       W = U - Y H,   O = diag(gamma) Q H + P W,   H <- gamma_C H + K^T diag(gamma_C/gamma) W
//     with bf16 operands (H rounded for the products only) and fp32 accumulation; the
//     segment's final H is stored for its children.  A chunk's O goes to LDS at its end and
//     leaves as whole 256-byte rows right after the next chunk's barrier, so no chunk waits
//     for its own stores to be acknowledged.
#include <algorithm>
#include <type_traits>
#include <utility>

#include "internal.h"
#include "lane_sum.h"
#include "tile_ops.h"

namespace treeattn {
namespace {

using namespace tile;

constexpr int kGD = 128;                  // head_dim
constexpr int kGW = 4;                    // conv width
constexpr int kGC = 64;                   // chunk length
constexpr float kGLog2e = 1.4426950408889634f;

// ------------------------------------------------------------------------------ gdn_conv
//
// One workgroup (256 threads) per (block of kConvTok tokens, tensor q / k / v); a thread takes
// 8 consecutive channels and keeps their conv weights in registers; 16 threads cover a head
// (the L2 norm is a 16-lane sum, on DPP row moves, so no LDS round trip).  The block's rows are
// loaded at the start, before any output is stored (stores and loads share one counter, so a
// load issued after a store would also wait for the store).  The taps come from a window of
// the three rows before the current token along its parent chain, in fp32 and zero past a
// root: after a token the window shifts by one (its row enters), which stays right as long as
// the next token's parent is this token; at a join or a root start (the parent is not the
// previous row) the window is reloaded from the chain.  Each row is converted once.  The
// parent chains of the block are loaded once, all tokens in parallel (lane k of every wave
// walks token k's chain).
constexpr int kConvTok = 16;

__device__ __forceinline__ void conv_row(const __bf16 *x, int r, int C, int c8, float (&f)[8]) {
    if (r < 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = 0.f;
    } else {
        const bf16x8_t v = *reinterpret_cast<const bf16x8_t *>(x + int64_t(r) * C + c8);
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = float(v[e]);
    }
}

__global__ __launch_bounds__(256) void gdn_conv(int32_t n_tok, int32_t H, const int32_t *__restrict__ pi,
                                                const __bf16 *__restrict__ xq, const __bf16 *__restrict__ xk,
                                                const __bf16 *__restrict__ xv, const float *__restrict__ w,
                                                float eps, __bf16 *__restrict__ qh, __bf16 *__restrict__ kh,
                                                __bf16 *__restrict__ vh) {
    const int C = H * kGD;                                 // channels per tensor
    const int tsr = blockIdx.y;
    const __bf16 *x = tsr == 0 ? xq : (tsr == 1 ? xk : xv);
    __bf16 *out = tsr == 0 ? qh : (tsr == 1 ? kh : vh);
    const float oscale = tsr == 0 ? 0.08838834764831845f : 1.f;   // q: 1 / sqrt(128)
    const int tok_begin = int(blockIdx.x) * kConvTok;
    // chain of token tok_begin + (lane % 16): c0 = pi(tok) (-2: pad or past the end), then
    // pi^1..pi^3 (-1 past a root's first token)
    int c0, c1, c2, c3;
    {
        const int tk = tok_begin + int(threadIdx.x & (kConvTok - 1));
        c0 = tk < n_tok ? pi[tk] : -2;
        c1 = c0 >= 0 ? c0 : -1;
        c2 = c1 >= 0 ? pi[c1] : -1;
        c3 = c2 >= 0 ? pi[c2] : -1;
    }
    for (int c8 = threadIdx.x * 8; c8 < C; c8 += blockDim.x * 8) {
        float wr[8][kGW];                                  // [channel][tap]
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float4 w4 = *reinterpret_cast<const float4 *>(w + ((int64_t(tsr) * C + c8 + e) * kGW));
            wr[e][0] = w4.x; wr[e][1] = w4.y; wr[e][2] = w4.z; wr[e][3] = w4.w;
        }
        // the block's rows (past n_tok clamped: pads, never stored)
        bf16x8_t xr[kConvTok];
#pragma unroll
        for (int k = 0; k < kConvTok; ++k)
            xr[k] = *reinterpret_cast<const bf16x8_t *>(x + int64_t(min(tok_begin + k, n_tok - 1)) * C + c8);
        // window: rows pi^1, pi^2, pi^3 of the current token
        float r1[8], r2[8], r3[8];
        conv_row(x, __builtin_amdgcn_readfirstlane(c1), C, c8, r1);
        conv_row(x, __builtin_amdgcn_readfirstlane(c2), C, c8, r2);
        conv_row(x, __builtin_amdgcn_readfirstlane(c3), C, c8, r3);
#pragma unroll
        for (int k = 0; k < kConvTok; ++k) {
            const int tok = tok_begin + k;
            if (k > 0) {
                const int p = __builtin_amdgcn_readlane(c1, k);
                if (p != tok - 1) {                        // a join or a root start
                    conv_row(x, p, C, c8, r1);
                    conv_row(x, __builtin_amdgcn_readlane(c2, k), C, c8, r2);
                    conv_row(x, __builtin_amdgcn_readlane(c3, k), C, c8, r3);
                }
            }
            float xc[8], y[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                xc[e] = float(xr[k][e]);
                y[e] = fmaf(wr[e][3], xc[e], 0.f);
                y[e] = fmaf(wr[e][2], r1[e], y[e]);
                y[e] = fmaf(wr[e][1], r2[e], y[e]);
                y[e] = fmaf(wr[e][0], r3[e], y[e]);
                y[e] = y[e] * __builtin_amdgcn_rcpf(1.f + __expf(-y[e]));
            }
            float scale = 1.f;
            if (tsr < 2) {
                float ss = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) ss = fmaf(y[e], y[e], ss);
                scale = __builtin_amdgcn_rsqf(lanes::group_sum<16>(ss) + eps) * oscale;
            }
            if (__builtin_amdgcn_readlane(c0, k) >= -1) {  // pads are never written
                bf16x8_t o8;
#pragma unroll
                for (int e = 0; e < 8; ++e) o8[e] = static_cast<__bf16>(y[e] * scale);
                *reinterpret_cast<bf16x8_t *>(out + int64_t(tok) * C + c8) = o8;
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                r3[e] = r2[e];
                r2[e] = r1[e];
                r1[e] = xc[e];
            }
        }
    }
}

// ------------------------------------------------------------------------------ gdn_prep
//
// LDS: Q, K, V chunk tiles (64 x 128 bf16, swizzled); a 64 x 64 fp32 array holding A^T in its
// upper triangle (As[s][t] = A_ts, s < t), then T = (I + A)^-1 (As[t][s] = T_ts); G, beta and
// gamma (64 fp32 each).  Once the Gram products are done
// the Q tile's 16 KB take the bf16 operand tiles of T diag(beta) (then of T diag(beta gamma)),
// high and low parts, and last the -Y tile on its way out.
struct PrepLds {
    static constexpr int TILE = kGC * kGD * 2;
    static constexpr int Q_OFF = 0, K_OFF = TILE, V_OFF = 2 * TILE, A_OFF = 3 * TILE;
    static constexpr int HI_OFF = Q_OFF, LO_OFF = Q_OFF + kGC * kGC * 2, YS_OFF = Q_OFF;
    static constexpr int G_OFF = A_OFF + kGC * kGC * 4, GB_OFF = G_OFF + kGC * 4, GM_OFF = GB_OFF + kGC * 4;
    static constexpr int SIZE = GM_OFF + kGC * 4;
};

template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F &&f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

struct GdnArgs {
    int32_t R, T, H, n_chunks;
    const int4 *chunk_meta;      // (row, t0, n, seg)
    const int4 *seg_meta;        // (row, first chunk, n chunks, parent segment or -1)
    const int32_t *level_ptr, *level_segs;
    const __bf16 *qh, *kh, *vh;
    const float *g, *beta;
    float *U;                    // [n_chunks, H, 64 x 128] in scan accumulator order (below)
    __bf16 *Yn;                  // [n_chunks, H, 64, 128]  (-Y)
    __bf16 *P;                   // [n_chunks, H, 64, 64]
    float *F;                    // [n_chunks, H, 128]: gamma_t (t < 64), gamma_C / gamma_t
    float *states;               // [n_segs, H, 128, 128]
    __bf16 *o;                   // [R, T, H, 128]
    const int32_t *prep_order;   // [n_chunks]: the chunks of depth-0 segments first, then the rest
    int32_t prep_base, prep_end; // the prep launch takes prep_order[prep_base .. prep_end)
    int32_t scan_wgs;            // fused launch: workgroups of the depth-0 scan before the prep's
};

// Chunk c, head h of the prep.  Four waves do the work; a workgroup of more waves (the fused
// scan and prep launch has five) runs the extra ones through the same barriers, idle (act false).
__device__ __forceinline__ void prep_body(const GdnArgs &a, int c, int h) {
    using T128 = Tile<kGD>;
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool act = wave < 4;
    const int4 cm = a.chunk_meta[c];
    const int r = cm.x, t0 = cm.y, n = cm.z;
    const int64_t tok0 = int64_t(r) * a.T + t0;
    const int stride = a.H * kGD * 2;
    const uint32_t lds0 = lds_base(smem);
    const int64_t hoff = (tok0 * a.H + h) * kGD * 2;
    if (act) {
        copy_tile<kGD>(reinterpret_cast<const char *>(a.qh) + hoff, n, stride, lds0 + PrepLds::Q_OFF, kGC, wave, 4, lane);
        copy_tile<kGD>(reinterpret_cast<const char *>(a.kh) + hoff, n, stride, lds0 + PrepLds::K_OFF, kGC, wave, 4, lane);
        copy_tile<kGD>(reinterpret_cast<const char *>(a.vh) + hoff, n, stride, lds0 + PrepLds::V_OFF, kGC, wave, 4, lane);
    }
    float *Gs = reinterpret_cast<float *>(smem + PrepLds::G_OFF);
    float *Bs = reinterpret_cast<float *>(smem + PrepLds::GB_OFF);
    if (wave == 0) {
        // inclusive cumulative log-decay over the chunk; pad rows: g = 0, beta = 0
        const bool on = lane < n;
        float gv = on ? a.g[(tok0 + lane) * a.H + h] : 0.f;
        const float bv = on ? a.beta[(tok0 + lane) * a.H + h] : 0.f;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const float y = __shfl_up(gv, off, 64);
            if (lane >= off) gv += y;
        }
        Gs[lane] = gv;
        Bs[lane] = bv;
        // decay factors for the scan: gamma_t and gamma_C / gamma_t (both <= 1)
        const float gC = __shfl(gv, kGC - 1, 64);
        const float gam = __builtin_amdgcn_exp2f(gv * kGLog2e);
        reinterpret_cast<float *>(smem + PrepLds::GM_OFF)[lane] = gam;
        float *Fo = a.F + (int64_t(c) * a.H + h) * 2 * kGC;
        Fo[lane] = gam;
        Fo[kGC + lane] = __builtin_amdgcn_exp2f((gC - gv) * kGLog2e);
    }
    wait_loads();
    __syncthreads();

    // Gram and Q K^T: wave w takes the 32 x 32 block (t block w/2, s block w%2), both computed
    // transposed (rows s, columns t): A^T is then stored along lanes, and each lane holds four
    // consecutive s of one t of P (one 8-byte store).
    const char *Qt = smem + PrepLds::Q_OFF, *Kt = smem + PrepLds::K_OFF;
    const int bt = (wave >> 1) & 1, bs = wave & 1;
    float *As = reinterpret_cast<float *>(smem + PrepLds::A_OFF);
    if (act) {
    floatx16 kkT = zero16(), qkT = zero16();
#pragma unroll
    for (int ds = 0; ds < kGD / 16; ++ds) {
        const bf16x8_t kb = T128::row_frag(Kt, 32 * bs, lane, ds);
        kkT = mfma(kb, T128::row_frag(Kt, 32 * bt, lane, ds), kkT);
        qkT = mfma(kb, T128::row_frag(Qt, 32 * bt, lane, ds), qkT);
    }
    {
        const int t = 32 * bt + (lane & 31);
        __bf16 *Pout = a.P + ((int64_t(c) * a.H + h) * kGC + t) * kGC + 32 * bs + 4 * (lane >> 5);
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
            bf16x4_t p4;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = 4 * i4 + e, sv = 32 * bs + 8 * i4 + 4 * (lane >> 5) + e;
                const float dec = __builtin_amdgcn_exp2f((Gs[t] - Gs[sv]) * kGLog2e);   // gamma_t / gamma_s
                As[sv * kGC + t] = sv < t ? Bs[t] * dec * kkT[i] : 0.f;                  // A^T[s][t]
                p4[e] = static_cast<__bf16>(sv <= t ? dec * qkT[i] : 0.f);             // P[t][s]
            }
            *reinterpret_cast<bf16x4_t *>(Pout + 8 * i4) = p4;
        }
    }
    }
    __syncthreads();

    // T = (I + A)^-1 in 16 x 16 blocks, all four waves.  As holds A^T in its strict upper
    // triangle (As[s][t] = A[t][s], s < t); T is built in row-major form (As[t][c] = T[t][c]) in
    // the lower triangle, which A^T does not use.
    //  1. Wave b inverts the diagonal block: D_b = (I + A_bb)^-1 by forward substitution (lane
    //     c < 16 takes column c, A^T rows read one ahead) and stores the whole 16 x 16 block
    //     (the block's A^T entries are read by no one else).
    //  2. Below the diagonal, by distance d = i - j = 1, 2, 3 (one barrier each), wave j takes
    //     block (i, j): M = sum_{k=j}^{i-1} A_ik T_kj (T_jj = D_j), staged in the free Q tile,
    //     then T_ij = -D_i M.  Lane (r, q) computes row r, columns 4q .. 4q + 3.
    //  3. The blocks above the diagonal, still A^T, are cleared.
    {
        constexpr int NB16 = kGC / 16;
        if (act && lane < 16) {
            const int b0 = 16 * wave;
            float x[16];
#pragma unroll
            for (int t = 0; t < 16; ++t) x[t] = t == lane ? 1.f : 0.f;
            float ar[2][16];
            auto load_row = [&](auto sc_, float(&dst)[16]) __attribute__((always_inline)) {
                constexpr int s_ = decltype(sc_)::value;
                static_for<(16 - (s_ + 1) / 4 * 4) / 4>([&](auto qc) __attribute__((always_inline)) {
                    constexpr int t4 = (s_ + 1) / 4 * 4 + 4 * decltype(qc)::value;
                    const float4 v = *reinterpret_cast<const float4 *>(As + (b0 + s_) * kGC + b0 + t4);
                    dst[t4] = v.x; dst[t4 + 1] = v.y; dst[t4 + 2] = v.z; dst[t4 + 3] = v.w;
                });
            };
            load_row(std::integral_constant<int, 0>{}, ar[0]);
            static_for<15>([&](auto sc) __attribute__((always_inline)) {
                constexpr int s0 = decltype(sc)::value;
                if constexpr (s0 + 1 < 15) load_row(std::integral_constant<int, s0 + 1>{}, ar[(s0 + 1) & 1]);
                static_for<15 - s0>([&](auto tc) __attribute__((always_inline)) {
                    constexpr int t = s0 + 1 + decltype(tc)::value;
                    x[t] = fmaf(-ar[s0 & 1][t], x[s0], x[t]);
                });
            });
#pragma unroll
            for (int t = 0; t < 16; ++t) As[(b0 + t) * kGC + b0 + lane] = x[t];
        }
        float *Ms = reinterpret_cast<float *>(smem + PrepLds::Q_OFF) + wave * 256;   // 16 x 16 per wave
        const int r = lane >> 2, c0 = 4 * (lane & 3);
        static_for<NB16 - 1>([&](auto dc) __attribute__((always_inline)) {
            constexpr int d = decltype(dc)::value + 1;
            __syncthreads();
            if (wave < NB16 - d) {
                const int j = wave, i = wave + d;
                float m[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < d; ++kk) {
                    const int k = j + kk;
#pragma unroll
                    for (int mm = 0; mm < 16; ++mm) {
                        const float aik = As[(16 * k + mm) * kGC + 16 * i + r];              // A[16i + r][16k + mm]
                        const float4 tk = *reinterpret_cast<const float4 *>(As + (16 * k + mm) * kGC + 16 * j + c0);
                        m[0] = fmaf(aik, tk.x, m[0]); m[1] = fmaf(aik, tk.y, m[1]);
                        m[2] = fmaf(aik, tk.z, m[2]); m[3] = fmaf(aik, tk.w, m[3]);
                    }
                }
                *reinterpret_cast<float4 *>(Ms + r * 16 + c0) = make_float4(m[0], m[1], m[2], m[3]);
                __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                __builtin_amdgcn_wave_barrier();
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                float t4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int mm = 0; mm < 16; ++mm) {
                    const float di = As[(16 * i + r) * kGC + 16 * i + mm];                  // D_i[r][mm]
                    const float4 mr = *reinterpret_cast<const float4 *>(Ms + mm * 16 + c0);
                    t4[0] = fmaf(di, mr.x, t4[0]); t4[1] = fmaf(di, mr.y, t4[1]);
                    t4[2] = fmaf(di, mr.z, t4[2]); t4[3] = fmaf(di, mr.w, t4[3]);
                }
                *reinterpret_cast<float4 *>(As + (16 * i + r) * kGC + 16 * j + c0) =
                    make_float4(-t4[0], -t4[1], -t4[2], -t4[3]);
            }
        });
        __syncthreads();
        // clear the blocks above the diagonal (i < j): 6 blocks x 64 float4
        for (int e = tid; act && e < 6 * 64; e += 256) {
            const int blk = e >> 6, w = e & 63, rr = w >> 2, cc = 4 * (w & 3);
            const int bi = blk < 3 ? 0 : (blk < 5 ? 1 : 2);
            const int bj = blk < 3 ? blk + 1 : (blk < 5 ? blk - 1 : 3);
            *reinterpret_cast<float4 *>(As + (16 * bi + rr) * kGC + 16 * bj + cc) = make_float4(0.f, 0.f, 0.f, 0.f);
        }
    }
    __syncthreads();

    // U = (T diag(beta)) V and Y = (T diag(beta gamma)) K on MFMA.  The left factor is split in
    // bf16 high and low parts (fp32 accuracy); V and K are bf16 already.  Wave w takes value /
    // key columns 32 w .. 32 w + 31, both 32-row blocks.
    using T64 = Tile<kGC>;
    const float *Gm = reinterpret_cast<const float *>(smem + PrepLds::GM_OFF);
    char *hi_t = smem + PrepLds::HI_OFF, *lo_t = smem + PrepLds::LO_OFF;
    auto build_factor = [&](bool with_gamma) __attribute__((always_inline)) {
        const int t = tid >> 2, q4 = tid & 3;                 // row t, columns 16 q4 .. +15
        bf16x8_t hv[2], lv[2];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int sc = 16 * q4 + e;
            const float f = As[t * kGC + sc] * Bs[sc] * (with_gamma ? Gm[sc] : 1.f);
            const __bf16 fh = static_cast<__bf16>(f);
            hv[e / 8][e % 8] = fh;
            lv[e / 8][e % 8] = static_cast<__bf16>(f - float(fh));
        }
#pragma unroll
        for (int hc = 0; hc < 2; ++hc) {
            *reinterpret_cast<bf16x8_t *>(hi_t + T64::chunk_at(t, 2 * q4 + hc)) = hv[hc];
            *reinterpret_cast<bf16x8_t *>(lo_t + T64::chunk_at(t, 2 * q4 + hc)) = lv[hc];
        }
    };
    auto product = [&](const char *rhs, floatx16 (&acc)[2]) __attribute__((always_inline)) {
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) acc[tb] = zero16();
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const bf16x8_t bv = T128::tr_frag(rhs, 0, lane, ks, wave);
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) {
                acc[tb] = mfma(T64::perm_frag(hi_t, 32 * tb, lane, ks), bv, acc[tb]);
                acc[tb] = mfma(T64::perm_frag(lo_t, 32 * tb, lane, ks), bv, acc[tb]);
            }
        }
    };
    const int64_t chh = int64_t(c) * a.H + h;
    floatx16 acc[2];
    if (act) build_factor(false);
    __syncthreads();
    if (act) {
    product(smem + PrepLds::V_OFF, acc);
    {
        // The scan's accumulator order: float4 (4 cb + tb) * 64 + 16 g + j holds rows 16 tb + 4 g
        // + 0..3 of column 16 cb + j.  This lane holds rows 32 tb + 8 q + 4 (lane / 32) + 0..3 of
        // column 32 wave + lane % 32.
        float4 *Uo = reinterpret_cast<float4 *>(a.U + chh * kGC * kGD);
        const int cl = lane & 31, hh = lane >> 5, cb = 2 * wave + (cl >> 4);
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                Uo[(4 * cb + 2 * tb + (q >> 1)) * 64 + 16 * (2 * (q & 1) + hh) + (cl & 15)] =
                    make_float4(acc[tb][4 * q], acc[tb][4 * q + 1], acc[tb][4 * q + 2], acc[tb][4 * q + 3]);
    }
    }
    __syncthreads();
    if (act) build_factor(true);
    __syncthreads();
    if (act) product(smem + PrepLds::K_OFF, acc);
    __syncthreads();
    if (act) {
        // -Y as bf16, row-major [t][128] in the Q tile's space, then out in 16-byte rows
        __bf16 *Ys = reinterpret_cast<__bf16 *>(smem + PrepLds::YS_OFF);
        const int colw = 32 * wave + (lane & 31);
#pragma unroll
        for (int tb = 0; tb < 2; ++tb)
#pragma unroll
            for (int i = 0; i < 16; ++i)
                Ys[(32 * tb + 8 * (i / 4) + 4 * (lane >> 5) + (i % 4)) * kGD + colw] = static_cast<__bf16>(-acc[tb][i]);
    }
    __syncthreads();
    if (act) {
        const bf16x8_t *src = reinterpret_cast<const bf16x8_t *>(smem + PrepLds::YS_OFF);
        bf16x8_t *dst = reinterpret_cast<bf16x8_t *>(a.Yn + chh * kGC * kGD);
#pragma unroll
        for (int k4 = 0; k4 < kGC * kGD / 8 / 256; ++k4) dst[tid + 256 * k4] = src[tid + 256 * k4];
    }
}

__global__ __launch_bounds__(256) void gdn_prep(GdnArgs a) {
    const int h = blockIdx.x % a.H, ord = a.prep_base + int(blockIdx.x / a.H);
    if (ord >= a.prep_end) return;
    prep_body(a, a.prep_order[ord], h);
}

// ------------------------------------------------------------------------------ gdn_scan
//
// 16x16x32 bf16 MFMA: lane l supplies A[m = l%16][k slot (l/16, e)] and B[k slot (l/16, e)]
// [n = l%16], e = 0..7, and accumulator element i of lane l is C[4(l/16) + i][l%16].  A k-step
// of 32 gives slot (g, e) the reduced index 32 s + 4 g + e (e < 4) or 32 s + 16 + 4 g + e - 4
// (e >= 4): exactly the rows that accumulator blocks 2 s and 2 s + 1 hold in lane l, so a
// product's accumulators become the next product's operand by conversion alone (pair_frag),
// and the operand read from a tile supplies the same k order (row16_frag, tr16_frag).
//
// A wave owns 16 value columns of the state: H (128 x 16) in 8 accumulator blocks, W and O^T
// of the chunk in 4 each.  Per chunk, 56 MFMAs: W = U - Y H and O^T = H^T Q^T (32), O^T +=
// W^T P^T (8), H <- gamma_C H + K^T diag(gamma_C / gamma) W (16).  A workgroup of NW waves
// covers 16 NW columns, so a head takes 128 / (16 NW) workgroups: 2 workgroups of 4 waves when
// a depth level has few segments (the chains then run on twice the CUs, each wave on its own
// SIMD), 1 of 8 waves otherwise (the chunk tiles are copied once per head).
//
// LDS: two stages of chunk tiles (Q, K, -Y: 64 x 128 bf16; P: 64 x 64 bf16; the decay
// factors: 128 fp32), the next chunk's stage copied while the current one is used; two
// buffers of the chunk's O (64 tokens x 16 NW columns bf16, 16-byte chunks XOR-swizzled by the
// token).  U goes straight from HBM into registers (prep wrote it in accumulator order), one
// chunk ahead.  Nothing in the chunk loop waits on a scalar load: chunk ci of a segment starts
// at the segment's first token + 64 ci.
typedef float floatx4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ floatx4 mfma16(bf16x8_t a, bf16x8_t b, floatx4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ floatx4 zero4() { return floatx4{0.f, 0.f, 0.f, 0.f}; }
// Operand of one k-step from accumulator blocks 2 s (slots e < 4) and 2 s + 1 (e >= 4).
__device__ __forceinline__ bf16x8_t pair_frag(const floatx4 &lo, const floatx4 &hi) {
    bf16x8_t f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        f[e] = static_cast<__bf16>(lo[e]);
        f[4 + e] = static_cast<__bf16>(hi[e]);
    }
    return f;
}
// Operand from a swizzled row-major tile: tile row `row` (the lane's m or n), k-step s of the
// columns: 32 s + 4 g + 0..3 and 32 s + 16 + 4 g + 0..3 (two 8-byte reads).
template <int D>
__device__ __forceinline__ bf16x8_t row16_frag(const char *tile, int row, int g, int s) {
    using TL = Tile<D>;
    const int c0 = 32 * s + 4 * g, c1 = c0 + 16;
    const bf16x4_t y0 = *reinterpret_cast<const bf16x4_t *>(tile + TL::chunk_at(row, c0 >> 3) + (c0 & 7) * 2);
    const bf16x4_t y1 = *reinterpret_cast<const bf16x4_t *>(tile + TL::chunk_at(row, c1 >> 3) + (c1 & 7) * 2);
    return __builtin_shufflevector(y0, y1, 0, 1, 2, 3, 4, 5, 6, 7);
}
// Transposed operand from a swizzled row-major tile: lane (g = l/16, j = l%16) receives column
// col0 + j of rows 32 s + 4 g + 0..3 and 32 s + 16 + 4 g + 0..3.  Two LDS transpose reads; in
// each 16-lane group lane j points at row base + j/4, columns col0 + 4(j%4) .. +3.
template <int D>
__device__ __forceinline__ bf16x8_t tr16_frag(const char *tile, int col0, int lane, int s) {
    using TL = Tile<D>;
    typedef shortx4 __attribute__((address_space(3))) *lds_p;
    const int g = lane >> 4, j = lane & 15;
    const int col = col0 + 4 * (j & 3);
    bf16x4_t y[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int row = 32 * s + 16 * r + 4 * g + (j >> 2);
        const char *p = tile + TL::chunk_at(row, col >> 3) + (col & 7) * 2;
        y[r] = __builtin_bit_cast(bf16x4_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_p)(p)));
    }
    return __builtin_shufflevector(y[0], y[1], 0, 1, 2, 3, 4, 5, 6, 7);
}

template <int NW>
struct ScanLds {
    static constexpr int TILE = kGC * kGD * 2;                  // 64 x 128 bf16
    static constexpr int Q_OFF = 0, K_OFF = TILE, Y_OFF = 2 * TILE, P_OFF = 3 * TILE;
    static constexpr int F_OFF = P_OFF + kGC * kGC * 2;
    static constexpr int STAGE = F_OFF + 2 * kGC * 4;
    static constexpr int OROW = 32 * NW, OCPR = OROW / 16;      // O staging: bytes, 16-byte chunks per token
    static constexpr int O_OFF = 2 * STAGE, OBUF = kGC * OROW;
    static constexpr int SIZE = O_OFF + 2 * OBUF;
};

// Copy jobs of a stage (1 KB instructions, except the two 256-byte decay-factor rows):
// Q 0-15, K 16-31, -Y 32-47, P 48-55, gamma 56, gamma_C / gamma 57.
constexpr int kStageJobs = 58;

// With 4 compute waves a fifth, memory wave issues every copy of the stages and every store
// of O: a wave that issues a direct-to-LDS copy waits while the CU's memory pipeline is full,
// and that wait no longer holds a compute wave's MFMAs.  (With 8 compute waves the registers
// leave no room for a ninth; the compute waves copy and store themselves.)
template <int NW>
constexpr bool kMemWave = NW == 4;

template <int NW>
__device__ __forceinline__ void scan_body(const GdnArgs &a, int32_t level, int bid) {
    using LD = ScanLds<NW>;
    constexpr bool MW = kMemWave<NW>;
    constexpr int NS = kGD / (16 * NW);                          // workgroups per head
    extern __shared__ __attribute__((aligned(1024))) char smem[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g4 = lane >> 4, j16 = lane & 15;
    const int cs = bid % NS, h = (bid / NS) % a.H, k = bid / (NS * a.H);
    const int lb = a.level_ptr[level], le = a.level_ptr[level + 1];
    if (lb + k >= le) return;
    const int seg = a.level_segs[lb + k];
    const int4 sm = a.seg_meta[seg];
    const int r = sm.x, c_first = sm.y, n_ch = sm.z, parent = sm.w;
    const int seg_t0 = n_ch > 0 ? a.chunk_meta[c_first].y : 0;
    const int last_n = n_ch > 0 ? a.chunk_meta[c_first + n_ch - 1].z : 0;
    const int cw0 = 16 * NW * cs;                                // the workgroup's first value column
    const bool memw = MW && wave == NW;                          // the memory wave
    const int v0 = cw0 + 16 * (memw ? 0 : wave);                 // the wave's first value column

    // H rows 16 kb + 4 g + i, column v0 + j (accumulator layout).
    floatx4 Hs[8];
    if (parent < 0 || memw) {
#pragma unroll
        for (int kb = 0; kb < 8; ++kb) Hs[kb] = zero4();
    } else {
        const float *src = a.states + (int64_t(parent) * a.H + h) * kGD * kGD + v0 + j16;
#pragma unroll
        for (int kb = 0; kb < 8; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) Hs[kb][i] = src[(16 * kb + 4 * g4 + i) * kGD];
    }

    const int stride = a.H * kGD * 2;
    const uint32_t lds0 = lds_base(smem);
    struct StageSrc {
        int32x4_t q, k, y, p, f;
        uint32_t base;
    };
    auto stage_src = [&](int ci) __attribute__((always_inline)) {
        StageSrc ss;
        const int n = ci + 1 < n_ch ? kGC : last_n;
        const int64_t hoff = ((int64_t(r) * a.T + seg_t0 + kGC * ci) * a.H + h) * kGD * 2;
        const int64_t chh = int64_t(c_first + ci) * a.H + h;
        ss.q = tile_rsrc(reinterpret_cast<const char *>(a.qh) + hoff, n, stride);
        ss.k = tile_rsrc(reinterpret_cast<const char *>(a.kh) + hoff, n, stride);
        ss.y = tile_rsrc(reinterpret_cast<const char *>(a.Yn) + chh * kGC * kGD * 2, kGC, kGD * 2);
        ss.p = tile_rsrc(reinterpret_cast<const char *>(a.P) + chh * kGC * kGC * 2, kGC, kGC * 2);
        ss.f = buf_rsrc(a.F + chh * 2 * kGC, 2 * kGC * 4);
        ss.base = lds0 + (ci & 1) * LD::STAGE;
        return ss;
    };
    // The wave's copy job jj of a stage: job wave + NW jj of the list (wave-uniform branches).
    constexpr int kJobs = (kStageJobs + NW - 1) / NW;
    auto stage_job = [&](const StageSrc &ss, int jj) __attribute__((always_inline)) {
        const int jb = wave + NW * jj;
        if (jb < 16) copy_block<kGD>(ss.q, stride, ss.base + LD::Q_OFF, jb, lane);
        else if (jb < 32) copy_block<kGD>(ss.k, stride, ss.base + LD::K_OFF, jb - 16, lane);
        else if (jb < 48) copy_block<kGD>(ss.y, kGD * 2, ss.base + LD::Y_OFF, jb - 32, lane);
        else if (jb < 56) copy_block<kGC>(ss.p, kGC * 2, ss.base + LD::P_OFF, jb - 48, lane);
        else if (jb < kStageJobs) buf_to_lds4(ss.f, ss.base + LD::F_OFF + (jb - 56) * kGC * 4, (jb - 56) * kGC * 4 + lane * 4);
    };
    // U of chunk ci, this wave's 16 columns: un[tb] holds (t = 16 tb + 4 g + 0..3, v0 + j).
    floatx4 un[4];
    auto u_src = [&](int ci) __attribute__((always_inline)) {
        return reinterpret_cast<const float4 *>(a.U + (int64_t(c_first + ci) * a.H + h) * kGC * kGD) +
               (v0 / 16) * 4 * 64 + lane;
    };
    auto load_u = [&](const float4 *us, int tb) __attribute__((always_inline)) {
        const float4 x = us[tb * 64];
        un[tb] = floatx4{x.x, x.y, x.z, x.w};
    };
    // Every copy of a stage (the memory wave).
    auto stage_all = [&](const StageSrc &ss) __attribute__((always_inline)) {
        static_for<16>([&](auto bc) __attribute__((always_inline)) {
            constexpr int b = decltype(bc)::value;
            copy_block<kGD>(ss.q, stride, ss.base + LD::Q_OFF, b, lane);
            copy_block<kGD>(ss.k, stride, ss.base + LD::K_OFF, b, lane);
            copy_block<kGD>(ss.y, kGD * 2, ss.base + LD::Y_OFF, b, lane);
            if constexpr (b < 8) copy_block<kGC>(ss.p, kGC * 2, ss.base + LD::P_OFF, b, lane);
            if constexpr (b < 2) buf_to_lds4(ss.f, ss.base + LD::F_OFF + b * kGC * 4, b * kGC * 4 + lane * 4);
        });
    };
    // Chunk c's O from its LDS buffer to HBM: NI instructions from instruction i0 on, 16 bytes
    // a lane, OCPR lanes a token row (rows of real tokens only).
    auto store_rows = [&](int c, auto i0c, auto nic) __attribute__((always_inline)) {
        constexpr int RPI = 64 / LD::OCPR;                       // rows per instruction
        constexpr int NI = decltype(nic)::value;
        const int i0 = i0c;
        const int n = c + 1 < n_ch ? kGC : last_n;
        const char *ob = smem + LD::O_OFF + (c & 1) * LD::OBUF;
        char *og = reinterpret_cast<char *>(a.o) + ((int64_t(r) * a.T + seg_t0 + kGC * c) * a.H + h) * kGD * 2 + cw0 * 2;
        const int cc = lane % LD::OCPR;
        uint4 v[NI];
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int t = (i0 + i) * RPI + lane / LD::OCPR;
            v[i] = *reinterpret_cast<const uint4 *>(ob + t * LD::OROW + ((cc ^ (t & (LD::OCPR - 1))) << 4));
        }
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int t = (i0 + i) * RPI + lane / LD::OCPR;
            if (t < n) *reinterpret_cast<uint4 *>(og + int64_t(t) * a.H * kGD * 2 + cc * 16) = v[i];
        }
    };
    constexpr int kOInstr = kGC * LD::OCPR / 64;                 // store instructions per chunk
    // The chunk's O stores: all of them by the memory wave, else a share per compute wave.
    auto store_o = [&](int c) __attribute__((always_inline)) {
        if constexpr (MW) store_rows(c, std::integral_constant<int, 0>{}, std::integral_constant<int, kOInstr>{});
        else store_rows(c, wave * (kOInstr / NW), std::integral_constant<int, kOInstr / NW>{});
    };

    if (n_ch > 0) {
        if (memw) {
            stage_all(stage_src(0));
        } else {
            if constexpr (!MW) {
                const StageSrc s0 = stage_src(0);
#pragma unroll
                for (int jj = 0; jj < kJobs; ++jj) stage_job(s0, jj);
            }
            const float4 *us = u_src(0);
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) load_u(us, tb);
        }
    }
    for (int ci = 0; ci < n_ch; ++ci) {
        // Chunk ci's stage and U have landed for every wave; every wave is done with chunk
        // ci-1, whose stage buffer chunk ci+1 takes, and chunk ci-1's O is in LDS.
        wait_loads();
        __syncthreads();
        if (memw) {
            // The next chunk's stage first (the compute waves wait for it), then chunk ci-1's
            // O, which has the whole chunk to be acknowledged.
            if (ci + 1 < n_ch) stage_all(stage_src(ci + 1));
            if (ci > 0) store_o(ci - 1);
            continue;
        }
        // Without a memory wave chunk ci-1's O leaves now, while no copy is queued ahead of it,
        // and has the whole chunk to be acknowledged before the next wait for loads (which
        // counts stores too).
        if (!MW && ci > 0) store_o(ci - 1);
        const bool more = ci + 1 < n_ch;
        const StageSrc nx = stage_src(ci + 1);
        const float4 *nu = u_src(ci + 1);
        const char *st = smem + (ci & 1) * LD::STAGE;
        const char *Qt = st + LD::Q_OFF, *Kt = st + LD::K_OFF;
        const char *Yt = st + LD::Y_OFF, *Pt = st + LD::P_OFF;
        const float *Fs = reinterpret_cast<const float *>(st + LD::F_OFF);
        floatx4 W[4], Ot[4];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
            W[tb] = un[tb];
            Ot[tb] = zero4();
        }

        // W = U - Y H and O^T = H^T Q^T, H as bf16 operands of both; step s covers reduced rows
        // 32 s .. 32 s + 31, the tiles' fragments read one step ahead; the next chunk's stage
        // copies ride along.
        {
            bf16x8_t hb[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) hb[s] = pair_frag(Hs[2 * s], Hs[2 * s + 1]);
            bf16x8_t fy[4], fq[4];
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                fy[tb] = row16_frag<kGD>(Yt, 16 * tb + j16, g4, 0);
                fq[tb] = row16_frag<kGD>(Qt, 16 * tb + j16, g4, 0);
            }
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                bf16x8_t ny[4], nq[4];
                if (s + 1 < 4) {
#pragma unroll
                    for (int tb = 0; tb < 4; ++tb) {
                        ny[tb] = row16_frag<kGD>(Yt, 16 * tb + j16, g4, s + 1);
                        nq[tb] = row16_frag<kGD>(Qt, 16 * tb + j16, g4, s + 1);
                    }
                }
                if (!MW && more) {
#pragma unroll
                    for (int jj = s * kJobs / 4; jj < (s + 1) * kJobs / 4; ++jj) stage_job(nx, jj);
                }
#pragma unroll
                for (int tb = 0; tb < 4; ++tb) {
                    W[tb] = mfma16(fy[tb], hb[s], W[tb]);
                    Ot[tb] = mfma16(hb[s], fq[tb], Ot[tb]);       // (Q H)^T = H^T Q^T
                }
                __builtin_amdgcn_sched_barrier(0);
                if (s + 1 < 4) {
#pragma unroll
                    for (int tb = 0; tb < 4; ++tb) {
                        fy[tb] = ny[tb];
                        fq[tb] = nq[tb];
                    }
                }
            }
        }
        // O^T = (Q H)^T diag(gamma) + W^T P^T: Ot[tb] holds value columns v0 + 4 g + i (rows)
        // of token 16 tb + j (column).  The next chunk's U rides along.
        {
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                const float gm = Fs[16 * tb + j16];
#pragma unroll
                for (int i = 0; i < 4; ++i) Ot[tb][i] *= gm;
            }
            bf16x8_t wb[2];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) wb[ks] = pair_frag(W[2 * ks], W[2 * ks + 1]);
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                bf16x8_t fp[4];
#pragma unroll
                for (int tb = 0; tb < 4; ++tb) fp[tb] = row16_frag<kGC>(Pt, 16 * tb + j16, g4, ks);
                if (more) {
                    load_u(nu, 2 * ks);
                    load_u(nu, 2 * ks + 1);
                }
#pragma unroll
                for (int tb = 0; tb < 4; ++tb) Ot[tb] = mfma16(wb[ks], fp[tb], Ot[tb]);   // (P W)^T = W^T P^T
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // H <- gamma_C H + K^T diag(gamma_C / gamma) W; k-step ks over tokens 32 ks .. +31, the
        // eight state blocks kb interleaved, K^T fragments read one step ahead.
        {
            bf16x8_t wg[2];
#pragma unroll
            for (int sb = 0; sb < 4; ++sb) {
                const float4 dg = *reinterpret_cast<const float4 *>(Fs + kGC + 16 * sb + 4 * g4);
                W[sb][0] *= dg.x;
                W[sb][1] *= dg.y;
                W[sb][2] *= dg.z;
                W[sb][3] *= dg.w;
            }
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) wg[ks] = pair_frag(W[2 * ks], W[2 * ks + 1]);
            const float dC = Fs[kGC - 1];
#pragma unroll
            for (int kb = 0; kb < 8; ++kb)
#pragma unroll
                for (int i = 0; i < 4; ++i) Hs[kb][i] *= dC;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                bf16x8_t fk[8];
#pragma unroll
                for (int kb = 0; kb < 8; ++kb) fk[kb] = tr16_frag<kGD>(Kt, 16 * kb, lane, ks);
#pragma unroll
                for (int kb = 0; kb < 8; ++kb) Hs[kb] = mfma16(fk[kb], wg[ks], Hs[kb]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        {
            // O of the chunk into its LDS buffer: four consecutive value columns of one token
            // per 8-byte write (local columns 16 wave + 4 g .. +3).
            char *ob = smem + LD::O_OFF + (ci & 1) * LD::OBUF;
            const int c16 = 2 * wave + (g4 >> 1);
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) {
                const int t = 16 * tb + j16;
                bf16x4_t v4;
#pragma unroll
                for (int i = 0; i < 4; ++i) v4[i] = static_cast<__bf16>(Ot[tb][i]);
                *reinterpret_cast<bf16x4_t *>(ob + t * LD::OROW + ((c16 ^ (t & (LD::OCPR - 1))) << 4) + 8 * (g4 & 1)) = v4;
            }
        }
    }
    if (n_ch > 0) {
        __syncthreads();   // the last chunk's O is in LDS
        if (memw || !MW) store_o(n_ch - 1);
    }
    if (memw) return;
    float *dst = a.states + (int64_t(seg) * a.H + h) * kGD * kGD + v0 + j16;
#pragma unroll
    for (int kb = 0; kb < 8; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[(16 * kb + 4 * g4 + i) * kGD] = Hs[kb][i];
}

template <int NW>
__global__ __launch_bounds__((NW + (kMemWave<NW> ? 1 : 0)) * 64) void gdn_scan(GdnArgs a, int32_t level) {
    scan_body<NW>(a, level, int(blockIdx.x));
}

// The depth-0 scan (split shape: 4 compute waves and a memory wave) and, in the workgroups after
// it, the prep of every deeper chunk: the root level's chunk chain runs on a few CUs, and the
// rest of the chip preps the chunks the next levels need meanwhile.
__global__ __launch_bounds__(5 * 64) void gdn_scan_prep(GdnArgs a) {
    if (int(blockIdx.x) < a.scan_wgs) {
        scan_body<4>(a, 0, int(blockIdx.x));
        return;
    }
    const int k = int(blockIdx.x) - a.scan_wgs;
    const int h = k % a.H, ord = a.prep_base + k / a.H;
    if (ord >= a.prep_end) return;
    prep_body(a, a.prep_order[ord], h);
}

}  // namespace

hipError_t launch_gdn(const GdnShape &sh, const GdnLayout &L, char *gws, const void *xq, const void *xk,
                      const void *xv, const float *conv_w, const float *g, const float *beta, void *o,
                      hipStream_t s) {
    GdnArgs a;
    a.R = sh.R; a.T = sh.T; a.H = sh.H; a.n_chunks = L.n_chunks;
    a.chunk_meta = reinterpret_cast<const int4 *>(gws + L.chunk_meta);
    a.seg_meta = reinterpret_cast<const int4 *>(gws + L.seg_meta);
    a.level_ptr = reinterpret_cast<const int32_t *>(gws + L.level_ptr);
    a.level_segs = reinterpret_cast<const int32_t *>(gws + L.level_segs);
    a.qh = reinterpret_cast<const __bf16 *>(gws + L.qh);
    a.kh = reinterpret_cast<const __bf16 *>(gws + L.kh);
    a.vh = reinterpret_cast<const __bf16 *>(gws + L.vh);
    a.g = g; a.beta = beta;
    a.U = reinterpret_cast<float *>(gws + L.U);
    a.Yn = reinterpret_cast<__bf16 *>(gws + L.Yn);
    a.P = reinterpret_cast<__bf16 *>(gws + L.P);
    a.F = reinterpret_cast<float *>(gws + L.F);
    a.states = reinterpret_cast<float *>(gws + L.states);
    a.o = static_cast<__bf16 *>(o);
    const int64_t n_tok = int64_t(sh.R) * sh.T;
    if (n_tok > INT32_MAX || int64_t(L.n_chunks) * sh.H > INT32_MAX) return hipErrorInvalidValue;
    if (n_tok > 0)
        gdn_conv<<<dim3(unsigned((n_tok + kConvTok - 1) / kConvTok), 3), 256, 0, s>>>(int32_t(n_tok), sh.H, reinterpret_cast<const int32_t *>(gws + L.pi),
                                            static_cast<const __bf16 *>(xq), static_cast<const __bf16 *>(xk),
                                            static_cast<const __bf16 *>(xv), conv_w, sh.eps,
                                            reinterpret_cast<__bf16 *>(gws + L.qh), reinterpret_cast<__bf16 *>(gws + L.kh),
                                            reinterpret_cast<__bf16 *>(gws + L.vh));
    if (L.n_chunks > 0) {
        a.prep_order = reinterpret_cast<const int32_t *>(gws + L.prep_order);
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(gdn_prep),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, PrepLds::SIZE);
        if (e != hipSuccess) return e;
        e = hipFuncSetAttribute(reinterpret_cast<const void *>(gdn_scan<4>), hipFuncAttributeMaxDynamicSharedMemorySize,
                                ScanLds<4>::SIZE);
        if (e != hipSuccess) return e;
        e = hipFuncSetAttribute(reinterpret_cast<const void *>(gdn_scan<8>), hipFuncAttributeMaxDynamicSharedMemorySize,
                                ScanLds<8>::SIZE);
        if (e != hipSuccess) return e;
        // Narrow levels (few segments): two workgroups of 4 compute waves and a memory wave per
        // (segment, head); the others: one workgroup of 8 waves per (segment, head).  When depth
        // 0 is narrow and deeper levels exist, only its chunks are prepped first; its scan then
        // shares one launch with the prep of as many other chunks as its chain leaves time for
        // (that launch holds one workgroup per CU: the scan's LDS), and the rest are prepped
        // after it at full occupancy.  A chunk of the chain takes ~2.3 us, a prep workgroup
        // alone on a CU ~15 us, so the chain covers 3/20 of its length in prep rounds.
        int dev = 0, n_cu = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n_cu <= 0)
            n_cu = 256;
        const bool narrow0 = (L.narrow_levels & 1u) != 0 && L.narrow_segs > 0;
        const int64_t scan_wgs = int64_t(L.lead_segs) * sh.H * 2;   // the depth-0 scan's workgroups
        int64_t shadow = 0;     // chunks prepped beside the depth-0 scan
        if (narrow0 && L.n_levels >= 2 && L.lead_segs > 0 && L.lead_chunks < L.n_chunks && n_cu > scan_wgs) {
            const int64_t rounds = int64_t(L.lead_chain) * 3 / 20;
            shadow = std::min<int64_t>(L.n_chunks - L.lead_chunks, (int64_t(n_cu - scan_wgs) * rounds) / sh.H);
        }
        a.prep_base = 0;
        a.prep_end = shadow > 0 ? L.lead_chunks : L.n_chunks;
        gdn_prep<<<a.prep_end * sh.H, 256, PrepLds::SIZE, s>>>(a);
        int32_t lev0 = 0;
        if (shadow > 0) {
            constexpr int kFusedLds = ScanLds<4>::SIZE > PrepLds::SIZE ? ScanLds<4>::SIZE : PrepLds::SIZE;
            e = hipFuncSetAttribute(reinterpret_cast<const void *>(gdn_scan_prep),
                                    hipFuncAttributeMaxDynamicSharedMemorySize, kFusedLds);
            if (e != hipSuccess) return e;
            a.scan_wgs = int32_t(scan_wgs);
            a.prep_base = L.lead_chunks;
            a.prep_end = L.lead_chunks + int32_t(shadow);
            gdn_scan_prep<<<unsigned(scan_wgs + shadow * sh.H), 5 * 64, kFusedLds, s>>>(a);
            if (a.prep_end < L.n_chunks) {
                a.prep_base = a.prep_end;
                a.prep_end = L.n_chunks;
                gdn_prep<<<(a.prep_end - a.prep_base) * sh.H, 256, PrepLds::SIZE, s>>>(a);
            }
            lev0 = 1;
        }
        for (int32_t lev = lev0; lev < L.n_levels; ++lev) {
            if (lev < 32 && ((L.narrow_levels >> lev) & 1u) != 0) {
                if (L.narrow_segs > 0)
                    gdn_scan<4><<<unsigned(L.narrow_segs * sh.H * 2), 5 * 64, ScanLds<4>::SIZE, s>>>(a, lev);
            } else if (L.max_level_segs > 0) {
                gdn_scan<8><<<unsigned(L.max_level_segs * sh.H), 8 * 64, ScanLds<8>::SIZE, s>>>(a, lev);
            }
        }
    }
    return hipGetLastError();
}

}  // namespace treeattn
