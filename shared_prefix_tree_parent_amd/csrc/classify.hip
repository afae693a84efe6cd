// Tile classifier: segment table -> per-token subtree ends -> FULL / PARTIAL / SKIP class of
// every (q-tile, k-tile) -> per-q-tile CSR lists -> longest-first work list.
//
// "Prefix tree packing" (furtherai.github.io), attention-mask passage: a token's visible set
// is one fully visible block per ancestor segment plus a causal triangle over its own segment,
// and most blocks of a packed row are empty and skipped.  The same page's indexer passage
// tests ancestry with a depth-first [enter, exit] interval; with segments laid out in
// pre-order that interval becomes, in token coordinates:
//     key j is visible to query i  <=>  j <= i < kend[j],
// where kend[j] is the end of the subtree of j's segment (pads: kend[j] = j, never visible).
// "How to Configure Sequence Packing ... in AReaL", "Lazy Block Mask Conversion": the block
// lists are built once per batch, on the device, and reused by every layer.
#include "internal.h"

namespace treeattn {
namespace {

constexpr int kStatusLayout = 1;

// One thread per row: check the table is a pre-order forest laid out from token 0, record the
// row's used length and every segment's subtree end.
__global__ void validate_rows(int32_t R, int32_t T, int32_t n_segs, const int32_t *__restrict__ rp,
                              const int32_t *__restrict__ st, const int32_t *__restrict__ ln,
                              const int32_t *__restrict__ par, int32_t *__restrict__ n_real,
                              int32_t *__restrict__ seg_end, int32_t *__restrict__ status) {
    const int32_t r = blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= R) return;
    const int32_t a = rp[r], b = rp[r + 1];
    bool ok = a >= 0 && a <= b && b <= n_segs;
    if (r == 0 && a != 0) ok = false;
    if (r == R - 1 && b != n_segs) ok = false;
    int64_t off = 0;
    if (ok) {
        for (int32_t s = a; s < b && ok; ++s) {
            const int32_t ls = s - a, n = ln[s], p = par[s];
            if (n < 1 || st[s] != off) { ok = false; break; }
            if (p != -1) {
                if (p < 0 || p >= ls) { ok = false; break; }
                // In pre-order the parent must be on the path from the root to the previous
                // segment: walk up from ls-1 (indices strictly decrease, parents were checked).
                int32_t x = ls - 1;
                while (x > p) x = par[a + x];
                if (x != p) { ok = false; break; }
            }
            off += n;
            if (off > T) { ok = false; break; }
        }
    }
    if (!ok) {
        n_real[r] = -1;
        atomicOr(status, kStatusLayout);
        return;
    }
    n_real[r] = static_cast<int32_t>(off);
    for (int32_t s = a; s < b; ++s) seg_end[s] = st[s] + ln[s];
    for (int32_t s = b - 1; s >= a; --s) {
        const int32_t p = par[s];
        if (p >= 0) seg_end[a + p] = max(seg_end[a + p], seg_end[s]);
    }
}

// kend[j]: subtree end of j's segment for real tokens, j for pads (and for invalid rows).
__global__ void token_kend(int32_t T, const int32_t *__restrict__ rp, const int32_t *__restrict__ st,
                           const int32_t *__restrict__ n_real, const int32_t *__restrict__ seg_end,
                           int32_t *__restrict__ kend) {
    const int32_t r = blockIdx.y;
    const int32_t j = blockIdx.x * blockDim.x + threadIdx.x;
    if (j >= T) return;
    const int32_t nr = n_real[r];
    int32_t out = j;
    if (nr >= 0 && j < nr) {
        int32_t lo = rp[r], hi = rp[r + 1] - 1;   // last segment with start <= j
        while (lo < hi) {
            const int32_t mid = (lo + hi + 1) >> 1;
            if (st[mid] <= j) lo = mid; else hi = mid - 1;
        }
        out = seg_end[lo];
    }
    kend[int64_t(r) * T + j] = out;
}

// One workgroup per (row, q-tile): exact visible-pair count of every k-tile, its class, and
// the number of non-skip tiles (written to qt_ptr[tile + 1] for the scan).
__global__ void classify_tiles(int32_t T, int32_t BQ, int32_t BK, int32_t nQ, int32_t nK,
                               const int32_t *__restrict__ kend, uint8_t *__restrict__ cmap,
                               int32_t *__restrict__ qt_ptr) {
    const int32_t qt = blockIdx.x, r = blockIdx.y;
    const int32_t q0 = qt * BQ, q1 = q0 + BQ;
    const int32_t *kr = kend + int64_t(r) * T;
    uint8_t *cm = cmap + (int64_t(r) * nQ + qt) * nK;
    int32_t nz = 0;
    for (int32_t kt = threadIdx.x; kt < nK; kt += blockDim.x) {
        const int32_t k0 = kt * BK;
        int64_t c = 0;
        if (k0 < q1) {
            for (int32_t j = k0; j < k0 + BK; ++j) {
                const int32_t hi = min(kr[j], q1), lo = max(j, q0);
                if (hi > lo) c += hi - lo;
            }
        }
        const uint8_t cls = c == 0 ? kTileSkip : (c == int64_t(BQ) * BK ? kTileFull : kTilePartial);
        cm[kt] = cls;
        nz += cls != kTileSkip;
    }
    __shared__ int32_t red[1024 / 64];
    for (int off = 32; off > 0; off >>= 1) nz += __shfl_xor(nz, off, 64);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = nz;
    __syncthreads();
    if (threadIdx.x == 0) {
        int32_t t = 0;
        for (int i = 0; i < int(blockDim.x >> 6); ++i) t += red[i];
        qt_ptr[int64_t(r) * nQ + qt + 1] = t;
    }
}

// Single workgroup: in-place inclusive scan of qt_ptr[1..n], qt_ptr[0] = 0.
__global__ void scan_counts(int32_t n, int32_t *__restrict__ qt_ptr) {
    __shared__ int32_t part[1024 / 64];
    __shared__ int32_t carry;
    if (threadIdx.x == 0) { carry = 0; qt_ptr[0] = 0; }
    __syncthreads();
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, nw = blockDim.x >> 6;
    for (int32_t base = 0; base < n; base += blockDim.x) {
        const int32_t i = base + threadIdx.x;
        int32_t x = i < n ? qt_ptr[i + 1] : 0;
        for (int off = 1; off < 64; off <<= 1) {
            const int32_t y = __shfl_up(x, off, 64);
            if (lane >= off) x += y;
        }
        if (lane == 63) part[wv] = x;
        __syncthreads();
        int32_t before = carry;
        for (int w2 = 0; w2 < wv; ++w2) before += part[w2];
        if (i < n) qt_ptr[i + 1] = x + before;
        __syncthreads();
        if (threadIdx.x == 0) {
            int32_t t = 0;
            for (int w2 = 0; w2 < nw; ++w2) t += part[w2];
            carry += t;
        }
        __syncthreads();
    }
}

// One wave per (row, q-tile): compact the non-skip k-tiles in ascending order.
__global__ void fill_lists(int32_t nK, int32_t n_tiles, const uint8_t *__restrict__ cmap,
                           const int32_t *__restrict__ qt_ptr, int32_t *__restrict__ kt_idx,
                           uint8_t *__restrict__ kt_kind) {
    const int32_t tile = blockIdx.x;
    if (tile >= n_tiles) return;
    const int lane = threadIdx.x;
    const uint8_t *cm = cmap + int64_t(tile) * nK;
    int32_t pos = qt_ptr[tile];
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int32_t k0 = 0; k0 < nK; k0 += 64) {
        const int32_t kt = k0 + lane;
        const uint8_t cls = kt < nK ? cm[kt] : kTileSkip;
        const uint64_t m = __ballot(cls != kTileSkip);
        if (cls != kTileSkip) {
            const int32_t at = pos + __popcll(m & below);
            kt_idx[at] = kt;
            kt_kind[at] = cls;
        }
        pos += __popcll(m);
    }
}

// Single workgroup: order q-tiles by their number of non-skip k-tiles, largest first (a
// counting sort; the order among equal counts is unspecified and does not affect results).
__global__ void build_worklist(int32_t n_tiles, int32_t nK, const int32_t *__restrict__ qt_ptr,
                               int32_t *__restrict__ hist, int32_t *__restrict__ work) {
    for (int32_t c = threadIdx.x; c <= nK + 1; c += blockDim.x) hist[c] = 0;
    __threadfence();
    __syncthreads();
    for (int32_t t = threadIdx.x; t < n_tiles; t += blockDim.x) {
        const int32_t c = qt_ptr[t + 1] - qt_ptr[t];
        atomicAdd(&hist[c], 1);
    }
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) {
        int32_t run = 0;
        for (int32_t c = nK; c >= 0; --c) {   // start offset of each count, descending
            const int32_t h = hist[c];
            hist[c] = run;
            run += h;
        }
    }
    __threadfence();
    __syncthreads();
    for (int32_t t = threadIdx.x; t < n_tiles; t += blockDim.x) {
        const int32_t c = qt_ptr[t + 1] - qt_ptr[t];
        work[atomicAdd(&hist[c], 1)] = t;
    }
}

__global__ void zero_words(int32_t *p, int32_t n) {
    const int32_t i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0;
}

}  // namespace

hipError_t launch_plan(const tree_attn_desc &d, const WsLayout &w, char *ws, hipStream_t s) {
    int32_t *status = reinterpret_cast<int32_t *>(ws + w.status);
    int32_t *n_real = reinterpret_cast<int32_t *>(ws + w.n_real);
    int32_t *seg_end = reinterpret_cast<int32_t *>(ws + w.seg_end);
    int32_t *kend = reinterpret_cast<int32_t *>(ws + w.kend);
    uint8_t *cmap = reinterpret_cast<uint8_t *>(ws + w.cmap);
    int32_t *qt_ptr = reinterpret_cast<int32_t *>(ws + w.qt_ptr);
    int32_t *kt_idx = reinterpret_cast<int32_t *>(ws + w.kt_idx);
    uint8_t *kt_kind = reinterpret_cast<uint8_t *>(ws + w.kt_kind);
    int32_t *work = reinterpret_cast<int32_t *>(ws + w.work);
    int32_t *hist = reinterpret_cast<int32_t *>(ws + w.hist);
    const int32_t n_tiles = w.R * w.nQ;

    // Cleared with a kernel (not a memset node) so the sequence can be captured in a graph.
    zero_words<<<1, 64, 0, s>>>(status, 4);
    zero_words<<<1, 128, 0, s>>>(reinterpret_cast<int32_t *>(ws + w.zeros), 128);
    if (w.R == 0) {
        zero_words<<<1, 64, 0, s>>>(qt_ptr, 1);
        return hipGetLastError();
    }
    validate_rows<<<(w.R + 63) / 64, 64, 0, s>>>(w.R, w.T, d.n_segs, d.seg_row_ptr, d.seg_start,
                                                 d.seg_len, d.seg_parent, n_real, seg_end, status);
    token_kend<<<dim3((w.T + 255) / 256, w.R), 256, 0, s>>>(w.T, d.seg_row_ptr, d.seg_start, n_real,
                                                            seg_end, kend);
    classify_tiles<<<dim3(w.nQ, w.R), 256, 0, s>>>(w.T, w.BQ, w.BK, w.nQ, w.nK, kend, cmap, qt_ptr);
    scan_counts<<<1, 1024, 0, s>>>(n_tiles, qt_ptr);
    fill_lists<<<n_tiles, 64, 0, s>>>(w.nK, n_tiles, cmap, qt_ptr, kt_idx, kt_kind);
    build_worklist<<<1, 1024, 0, s>>>(n_tiles, w.nK, qt_ptr, hist, work);
    return hipGetLastError();
}

}  // namespace treeattn
