// Rotary position embedding at tree positions, in place on Q and K, for gfx950.
//
// In a packed row a token's position is its index in its own unpacked sequence ("Prefix tree
// packing", furtherai.github.io: a packed row must reproduce each unpacked sequence exactly;
// the plan's pos_ids carry these positions).  Rotating Q and K at those positions (instead of
// the row offset) is what keeps rotary attention identical to the unpacked runs.
//
// Rotation (rotate-half pairing): for pair index i < D/2, angle a = pos * theta^(-2i/D),
//   x[i]       <- x[i] cos a - x[i + D/2] sin a
//   x[i + D/2] <- x[i + D/2] cos a + x[i] sin a
// and the inverse rotation (a -> -a), which is also the backward of the forward rotation.
//
// One workgroup per token: the D/2 angles are computed once in fp64 (the product pos * freq
// and the range reduction in single precision would be off by up to ~2e-3 rad at position
// 32768) and kept in LDS as fp32 (cos, sin); the rotation then runs over every query and key
// head of the token, each thread taking 4 consecutive pairs (8-byte loads from both halves).
// HBM-bound: reads and writes (h_q + h_kv) * D elements per token.
#include <cmath>

#include "internal.h"

namespace treeattn {
namespace {

constexpr int kRopeThreads = 256;

template <class E>
struct RopeIo;
template <>
struct RopeIo<__bf16> {
    typedef __bf16 v4 __attribute__((ext_vector_type(4)));
};
template <>
struct RopeIo<float> {
    typedef float v4 __attribute__((ext_vector_type(4)));
};

template <class E>
__global__ __launch_bounds__(kRopeThreads) void rope_kernel(int32_t n_tok, int32_t Hq, int32_t Hkv, int32_t D,
                                                            const int32_t *__restrict__ pos_ids, double log_theta,
                                                            int32_t inverse, E *__restrict__ q, E *__restrict__ k) {
    using v4 = typename RopeIo<E>::v4;
    __shared__ float2 cs[512];                  // (cos, sin) per pair index, D / 2 <= 512
    const int64_t tok = blockIdx.x;
    if (tok >= n_tok) return;
    const int half = D / 2;
    const int pos = pos_ids[tok];
    for (int i = threadIdx.x; i < half; i += blockDim.x) {
        const double inv_freq = exp(-log_theta * (2.0 * i) / D);
        double s, c;
        sincos(double(pos) * inv_freq, &s, &c);
        cs[i] = make_float2(float(c), inverse ? float(-s) : float(s));
    }
    __syncthreads();
    const int quads = half / 4;                 // 4 pairs per thread
    const int items = (Hq + Hkv) * quads;
    for (int it = threadIdx.x; it < items; it += blockDim.x) {
        const int hh = it / quads, i0 = (it % quads) * 4;
        E *const base = hh < Hq ? q : k;
        if (base == nullptr) continue;
        E *row = hh < Hq ? base + (tok * Hq + hh) * int64_t(D) : base + (tok * Hkv + (hh - Hq)) * int64_t(D);
        v4 a = *reinterpret_cast<const v4 *>(row + i0);
        v4 b = *reinterpret_cast<const v4 *>(row + half + i0);
        v4 ya, yb;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float2 w = cs[i0 + e];
            const float x1 = float(a[e]), x2 = float(b[e]);
            ya[e] = E(fmaf(x1, w.x, -x2 * w.y));
            yb[e] = E(fmaf(x2, w.x, x1 * w.y));
        }
        *reinterpret_cast<v4 *>(row + i0) = ya;
        *reinterpret_cast<v4 *>(row + half + i0) = yb;
    }
}

}  // namespace

hipError_t launch_rope(int32_t R, int32_t T, int32_t Hq, int32_t Hkv, int32_t D, int32_t dtype,
                       const int32_t *pos_ids, float theta, int32_t inverse, void *q, void *k, hipStream_t s) {
    const int64_t n_tok = int64_t(R) * T;
    if (n_tok == 0) return hipSuccess;
    if (n_tok > INT32_MAX || D % 8 != 0 || D / 2 > 512) return hipErrorInvalidValue;
    const double log_theta = std::log(double(theta));
    if (dtype == TREE_DT_BF16)
        rope_kernel<__bf16><<<int(n_tok), kRopeThreads, 0, s>>>(int32_t(n_tok), Hq, Hkv, D, pos_ids, log_theta,
                                                               inverse, static_cast<__bf16 *>(q),
                                                               static_cast<__bf16 *>(k));
    else
        rope_kernel<float><<<int(n_tok), kRopeThreads, 0, s>>>(int32_t(n_tok), Hq, Hkv, D, pos_ids, log_theta,
                                                              inverse, static_cast<float *>(q),
                                                              static_cast<float *>(k));
    return hipGetLastError();
}

}  // namespace treeattn
