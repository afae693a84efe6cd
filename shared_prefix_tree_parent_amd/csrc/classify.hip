// Tile classifier: segment table -> per-token subtree ends -> FULL / PARTIAL / SKIP class of
// every (q-tile, k-tile) -> per-q-tile CSR lists -> longest-first work list.
//
// "Prefix tree packing" (furtherai.github.io), attention-mask passage: the keys a token sees
// are whole ancestor segments (every pair visible) and the lower triangle of its own segment,
// so in a packed row the bulk of the (query block, key block) pairs hold no visible pair at all
// and need no work.  The same page's indexer passage
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
constexpr int kMaxLdsSegs = 2048;   // segments of one row kept in LDS while validating

// One workgroup per row: checks that the table is a pre-order forest laid out from token 0 and
// writes every segment's subtree end.  With the row's segments in LDS (up to kMaxLdsSegs),
// every segment is checked by its own thread; otherwise one thread walks them in global
// memory.  A row that fails the check gets n_real = -1 (then kend[j] = j: all skipped).
__global__ void validate_rows(int32_t R, int32_t T, int32_t n_segs, const int32_t *__restrict__ rp,
                              const int32_t *__restrict__ st, const int32_t *__restrict__ ln,
                              const int32_t *__restrict__ par, int32_t *__restrict__ n_real,
                              int32_t *__restrict__ seg_end) {
    __shared__ int32_t s_st[kMaxLdsSegs], s_len[kMaxLdsSegs], s_par[kMaxLdsSegs], s_dep[kMaxLdsSegs];
    __shared__ int32_t s_a, s_n, s_bad;
    const int32_t r = blockIdx.x;
    const int tid = threadIdx.x;
    if (tid == 0) {
        const int32_t a = rp[r], b = rp[r + 1];
        const bool ok = a >= 0 && a <= b && b <= n_segs && (r != 0 || a == 0) && (r != R - 1 || b == n_segs);
        s_a = ok ? a : 0;
        s_n = ok ? b - a : -1;
        s_bad = ok ? 0 : 1;
    }
    __syncthreads();
    const int32_t a = s_a, n = s_n;
    if (n >= 0 && n <= kMaxLdsSegs) {
        // The row's segments in LDS; every segment checked by its own thread.  The checks are
        // the serial ones (positive length, starts that tile the row from token 0, a parent
        // before the child on the path from the root to the previous segment), so a table
        // passes exactly when every segment passes.
        for (int32_t i = tid; i < n; i += blockDim.x) {
            s_st[i] = st[a + i];
            s_len[i] = ln[a + i];
            s_par[i] = par[a + i];
        }
        __syncthreads();
        for (int32_t sg = tid; sg < n; sg += blockDim.x) {
            const int32_t p = s_par[sg];
            // lengths and starts bounded by the row, the sum in 64 bits: no int32 wrap can make
            // a table that overruns the row look contiguous
            const int64_t prev_end = sg == 0 ? 0 : int64_t(s_st[sg - 1]) + s_len[sg - 1];
            bool ok = s_len[sg] >= 1 && s_len[sg] <= T && s_st[sg] >= 0 && int64_t(s_st[sg]) == prev_end;
            if (ok && p != -1) {
                ok = p >= 0 && p < sg;
                if (ok) {
                    // walk up from sg - 1; a parent that does not precede its child ends the
                    // walk (that segment fails its own check)
                    int32_t x = sg - 1;
                    while (x > p) {
                        const int32_t nx = s_par[x];
                        if (nx >= x || nx < -1) break;
                        x = nx;
                    }
                    ok = x == p;
                }
            }
            // depth: number of ancestors (the walk stops early on an invalid parent)
            int32_t d = 0, x = sg;
            while (true) {
                const int32_t nx = s_par[x];
                if (nx < 0 || nx >= x) break;
                x = nx;
                ++d;
            }
            s_dep[sg] = d;
            if (!ok) s_bad = 1;
        }
        __syncthreads();
        const int64_t total64 = n > 0 ? int64_t(s_st[n - 1]) + s_len[n - 1] : 0;
        const bool ok = s_bad == 0 && total64 <= T;
        const int32_t total = static_cast<int32_t>(ok ? total64 : 0);
        if (ok) {
            // pre-order: a segment's subtree is the run of segments after it that are deeper,
            // and the segments tile the row, so the subtree ends where the next segment at its
            // depth or above starts (or at the row's last real token)
            for (int32_t sg = tid; sg < n; sg += blockDim.x) {
                int32_t x = sg + 1;
                while (x < n && s_dep[x] > s_dep[sg]) ++x;
                seg_end[a + sg] = x < n ? s_st[x] : total;
            }
        }
        if (tid == 0) n_real[r] = ok ? total : -1;
        return;
    }
    // More segments than fit in LDS (or a bad row pointer): one thread, reading global memory.
    if (tid != 0) return;
    bool ok = n >= 0;
    int64_t off = 0;
    for (int32_t sg = 0; sg < n && ok; ++sg) {
        const int32_t len = ln[a + sg], start = st[a + sg], p = par[a + sg];
        if (len < 1 || start != off) { ok = false; break; }
        if (p != -1) {
            if (p < 0 || p >= sg) { ok = false; break; }
            // In pre-order the parent lies on the path from the root to the previous segment:
            // walk up from sg-1 (indices strictly decrease; their parents were checked).
            int32_t x = sg - 1;
            while (x > p) x = par[a + x];
            if (x != p) { ok = false; break; }
        }
        off += len;
        if (off > T) { ok = false; break; }
    }
    if (ok) {
        // subtree ends: children come after their parent, so one reverse sweep suffices
        for (int32_t sg = 0; sg < n; ++sg) seg_end[a + sg] = st[a + sg] + ln[a + sg];
        for (int32_t sg = n - 1; sg >= 0; --sg) {
            const int32_t p = par[a + sg];
            if (p >= 0) seg_end[a + p] = max(seg_end[a + p], seg_end[a + sg]);
        }
    }
    n_real[r] = ok ? static_cast<int32_t>(off) : -1;
}

// Grid (k-tile groups, rows), one wave per k-tile: kend of every token of the tile (its
// segment's subtree end; j itself for pads) and the tile's (min kend, max kend over real keys).
__global__ void kend_stats(int32_t T, int32_t BK, int32_t nK, const int32_t *__restrict__ rp,
                           const int32_t *__restrict__ st, const int32_t *__restrict__ n_real,
                           const int32_t *__restrict__ seg_end, int32_t *__restrict__ kend,
                           int2 *__restrict__ kt_stats) {
    const int32_t r = blockIdx.y;
    const int32_t kt = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    if (kt >= nK) return;
    const int lane = threadIdx.x & 63;
    const int32_t nr = n_real[r];
    const int32_t a = rp[r], n = nr >= 0 ? rp[r + 1] - a : 0;
    int32_t *kr = kend + int64_t(r) * T;
    int32_t mn = INT32_MAX, mx = INT32_MIN;
    for (int32_t o = lane; o < BK; o += 64) {
        const int32_t j = kt * BK + o;
        int32_t ke = j;
        if (j < nr) {
            int32_t lo = 0, hi = n - 1;   // last segment with start <= j
            while (lo < hi) {
                const int32_t mid = (lo + hi + 1) >> 1;
                if (st[a + mid] <= j) lo = mid; else hi = mid - 1;
            }
            ke = seg_end[a + lo];
            mx = max(mx, ke);
        }
        kr[j] = ke;
        mn = min(mn, ke);
    }
    for (int off = 32; off > 0; off >>= 1) {
        mn = min(mn, __shfl_xor(mn, off, 64));
        mx = max(mx, __shfl_xor(mx, off, 64));
    }
    if (lane == 0) kt_stats[int64_t(r) * nK + kt] = make_int2(mn, mx);
}

// One wave per (row, q-tile).  Classes from the k-tile statistics: with segments in pre-order,
// consecutive real keys j, j+1 have kend[j] >= j+1, so the queries that see at least one key
// of a tile form the single interval [first real key, max kend).  Hence, for queries
// [q0, q1) and keys [k0, k0 + BK):
//   SKIP <=> no real key in the tile, or k0 >= q1, or max kend <= q0;
//   FULL <=> k0 + BK - 1 <= q0 and min kend (pads count with kend = j) >= q1;
//   PARTIAL otherwise.
// These are exactly the zero / all-pairs cases of the visible-pair count.  Writes the class
// map and the tile's number of non-skip k-tiles to qt_ptr[tile + 1].
__global__ void classify_tiles(int32_t R, int32_t BQ, int32_t BK, int32_t nQ, int32_t nK,
                               const int32_t *__restrict__ n_real, const int2 *__restrict__ kt_stats,
                               uint8_t *__restrict__ cmap, int32_t *__restrict__ qt_ptr) {
    const int32_t tile = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    if (tile >= R * nQ) return;
    const int lane = threadIdx.x & 63;
    const int32_t r = tile / nQ, qt = tile % nQ;
    const int32_t q0 = qt * BQ, q1 = q0 + BQ, nr = n_real[r];
    const int2 *stats = kt_stats + int64_t(r) * nK;
    uint8_t *cm = cmap + int64_t(tile) * nK;
    int32_t cnt = 0;
    for (int32_t k00 = 0; k00 < nK; k00 += 64) {
        const int32_t kt = k00 + lane;
        uint8_t cls = kTileSkip;
        if (kt < nK) {
            const int32_t k0 = kt * BK;
            const int2 sm = stats[kt];
            const bool skip = !(k0 < nr) || k0 >= q1 || sm.y <= q0;
            const bool full = k0 + BK - 1 <= q0 && sm.x >= q1;
            cls = skip ? kTileSkip : (full ? kTileFull : kTilePartial);
            cm[kt] = cls;
        }
        cnt += __popcll(__ballot(cls != kTileSkip));
    }
    if (lane == 0) qt_ptr[tile + 1] = cnt;
}

// In-place inclusive scan of x[1..n] (x[0] = 0) by one workgroup; `rev` scans x[1..n] as if
// it were reversed (used for descending buckets).
__device__ void block_scan(int32_t n, int32_t *x, int32_t *part, int32_t *carry) {
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, nw = blockDim.x >> 6;
    if (threadIdx.x == 0) *carry = 0;
    __syncthreads();
    for (int32_t base = 0; base < n; base += blockDim.x) {
        const int32_t i = base + threadIdx.x;
        int32_t v = i < n ? x[i + 1] : 0;
        for (int off = 1; off < 64; off <<= 1) {
            const int32_t y = __shfl_up(v, off, 64);
            if (lane >= off) v += y;
        }
        if (lane == 63) part[wv] = v;
        __syncthreads();
        int32_t before = *carry;
        for (int w2 = 0; w2 < wv; ++w2) before += part[w2];
        if (i < n) x[i + 1] = v + before;
        __syncthreads();
        if (threadIdx.x == 0) {
            int32_t t = 0;
            for (int w2 = 0; w2 < nw; ++w2) t += part[w2];
            *carry += t;
        }
        __syncthreads();
    }
}

// One workgroup: CSR offsets (scan of the per-tile counts), the table status word and the
// work list: rows in order, and inside a row its q-tiles by their number of non-skip k-tiles,
// largest first (a counting sort over (row, count) buckets; the order among equal counts does
// not affect any result).  Keeping a row's q-tiles together keeps that row's K/V tiles in the
// L2 of the XCDs that stream them, while the longest-first order inside the row keeps the
// tail short.
__global__ void finish_plan(int32_t R, int32_t nQ, int32_t nK, int32_t n_tiles, const int32_t *__restrict__ n_real,
                            int32_t *__restrict__ qt_ptr, int32_t *__restrict__ hist,
                            int32_t *__restrict__ work, int32_t n_ctr, int32_t *__restrict__ ctr,
                            int32_t *__restrict__ status) {
    __shared__ int32_t part[1024 / 64];
    __shared__ int32_t carry, bad;
    if (threadIdx.x == 0) { bad = 0; qt_ptr[0] = 0; }
    for (int32_t i = threadIdx.x; i < n_ctr; i += blockDim.x) ctr[i] = 0;   // forward item counters
    // tiles of row r and cost c go to bucket b = r (nK + 1) + (nK - c), counted at hist[1 + b],
    // so that an inclusive scan yields at hist[b] the first slot of that bucket.
    const int32_t n_buckets = R * (nK + 1);
    for (int32_t i = threadIdx.x; i < n_buckets + 2; i += blockDim.x) hist[i] = 0;
    __syncthreads();
    for (int32_t r = threadIdx.x; r < R; r += blockDim.x)
        if (n_real[r] < 0) atomicOr(&bad, 1);
    block_scan(n_tiles, qt_ptr, part, &carry);
    __threadfence_block();
    __syncthreads();
    for (int32_t t = threadIdx.x; t < n_tiles; t += blockDim.x)
        atomicAdd(&hist[1 + (t / nQ) * (nK + 1) + nK - (qt_ptr[t + 1] - qt_ptr[t])], 1);
    __threadfence_block();
    __syncthreads();
    block_scan(n_buckets, hist, part, &carry);
    __threadfence_block();
    __syncthreads();
    for (int32_t t = threadIdx.x; t < n_tiles; t += blockDim.x) {
        const int32_t c = qt_ptr[t + 1] - qt_ptr[t];
        work[atomicAdd(&hist[(t / nQ) * (nK + 1) + nK - c], 1)] = t;
    }
    if (threadIdx.x == 0) status[0] = bad ? kStatusLayout : 0;
}

// One wave per (row, q-tile): compact the non-skip k-tiles in ascending order.
__global__ void fill_lists(int32_t nK, int32_t n_tiles, const uint8_t *__restrict__ cmap,
                           const int32_t *__restrict__ qt_ptr, int32_t *__restrict__ kt_idx,
                           uint8_t *__restrict__ kt_kind) {
    const int32_t tile = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    if (tile >= n_tiles) return;
    const int lane = threadIdx.x & 63;
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

// ------------------------------------------------------------ backward (k-tile group) lists
//
// The backward's dK/dV pass walks, for every (row, group of kKvGroup k-tiles kKvGroup p ..),
// called a pair here for short, the q-tiles that see any of them, with every class: the
// transpose of the per-q-tile lists, read from the same class map.  K-tiles past the row's
// last (a tile count that is not a multiple of kKvGroup) count as SKIP.

// Entry of q-tile qt for the group starting at k-tile kt0: qt * 256 + the classes packed two
// bits each, the group's first k-tile in the highest bits; 0 in the class bits means no entry.
__device__ __forceinline__ int32_t group_entry(const uint8_t *cm, int32_t nK, int32_t qt, int32_t kt0, bool &on) {
    static_assert(kKvGroup == 4, "two class bits per k-tile in the low byte");
    int32_t e = 0;
    on = false;
#pragma unroll
    for (int i = 0; i < kKvGroup; ++i) {
        const uint8_t c = kt0 + i < nK ? cm[int64_t(qt) * nK + kt0 + i] : uint8_t(kTileSkip);
        on |= c != kTileSkip;
        e |= int32_t(c) << (2 * (kKvGroup - 1 - i));
    }
    return qt * 256 + e;
}

// One wave per (row, pair): number of q-tiles that see the pair, to kp_ptr[item + 1].
__global__ void count_pairs(int32_t nQ, int32_t nK, int32_t nP, int32_t n_items, const uint8_t *__restrict__ cmap,
                            int32_t *__restrict__ kp_ptr) {
    const int32_t item = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    if (item >= n_items) return;
    const int lane = threadIdx.x & 63;
    const int32_t r = item / nP, p = item % nP;
    const uint8_t *cm = cmap + int64_t(r) * nQ * nK;
    int32_t cnt = 0;
    for (int32_t q0 = 0; q0 < nQ; q0 += 64) {
        const int32_t qt = q0 + lane;
        bool on = false;
        if (qt < nQ) group_entry(cm, nK, qt, kKvGroup * p, on);
        cnt += __popcll(__ballot(on));
    }
    if (lane == 0) kp_ptr[item + 1] = cnt;
}

// One workgroup: scan of the pair counts and the longest-first work list.  The scatter into
// the length buckets is stable (pairs of equal length keep their index order), so the work
// order, and with it the split pairs and their partial slots, is the same on every run.
__global__ void finish_pairs(int32_t nQ, int32_t n_items, int32_t *__restrict__ kp_ptr,
                             int32_t *__restrict__ khist, int32_t *__restrict__ kwork) {
    __shared__ int32_t part[1024 / 64];
    __shared__ int32_t carry;
    if (threadIdx.x == 0) kp_ptr[0] = 0;
    for (int32_t i = threadIdx.x; i < nQ + 2; i += blockDim.x) khist[i] = 0;
    __syncthreads();
    block_scan(n_items, kp_ptr, part, &carry);
    __threadfence_block();
    __syncthreads();
    for (int32_t t = threadIdx.x; t < n_items; t += blockDim.x)
        atomicAdd(&khist[1 + nQ - (kp_ptr[t + 1] - kp_ptr[t])], 1);
    __threadfence_block();
    __syncthreads();
    block_scan(nQ + 1, khist, part, &carry);
    __threadfence_block();
    __syncthreads();
    // khist[b] is now the first position of bucket b = nQ - length.  Chunks of blockDim.x
    // pairs in index order; inside a chunk, a lane's rank among the earlier lanes of its wave
    // with the same bucket comes from ballots, and the waves take their positions one after
    // another.
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, nw = blockDim.x >> 6;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int32_t c0 = 0; c0 < n_items; c0 += blockDim.x) {
        const int32_t t = c0 + threadIdx.x;
        const bool valid = t < n_items;
        const int32_t key = valid ? nQ - (kp_ptr[t + 1] - kp_ptr[t]) : -1;
        int32_t rank = 0, cnt = 0;
        uint64_t left = __ballot(valid);
        while (left) {                                   // one pass per distinct bucket
            const int32_t k = __shfl(key, __ffsll(static_cast<unsigned long long>(left)) - 1, 64);
            const uint64_t m = __ballot(valid && key == k);
            if (valid && key == k) {
                rank = __popcll(m & below);
                cnt = __popcll(m);
            }
            left &= ~m;
        }
        for (int w2 = 0; w2 < nw; ++w2) {
            if (wv == w2 && valid) kwork[khist[key] + rank] = t;
            __threadfence_block();
            __syncthreads();
            if (wv == w2 && valid && rank == cnt - 1) khist[key] += cnt;
            __threadfence_block();
            __syncthreads();
        }
    }
}

// One wave per (row, pair): the q-tiles in ascending order, as group_entry values.
__global__ void fill_pairs(int32_t nQ, int32_t nK, int32_t nP, int32_t n_items, const uint8_t *__restrict__ cmap,
                           const int32_t *__restrict__ kp_ptr, int32_t *__restrict__ kp_list) {
    const int32_t item = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    if (item >= n_items) return;
    const int lane = threadIdx.x & 63;
    const int32_t r = item / nP, p = item % nP;
    const uint8_t *cm = cmap + int64_t(r) * nQ * nK;
    int32_t pos = kp_ptr[item];
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int32_t q0 = 0; q0 < nQ; q0 += 64) {
        const int32_t qt = q0 + lane;
        bool on = false;
        int32_t ent = 0;
        if (qt < nQ) ent = group_entry(cm, nK, qt, kKvGroup * p, on);
        const uint64_t m = __ballot(on);
        if (on) kp_list[pos + __popcll(m & below)] = ent;
        pos += __popcll(m);
    }
}

// Inclusive scan of one value per thread over a workgroup of 1024 threads (LDS array `buf`).
__device__ int32_t scan1024(int32_t v, int32_t *buf) {
    const int tid = threadIdx.x;
    buf[tid] = v;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
        const int32_t add = tid >= off ? buf[tid - off] : 0;
        __syncthreads();
        buf[tid] += add;
        __syncthreads();
    }
    return buf[tid];
}

// One workgroup of 1024 threads: query slices and partial slots of every pair, in the
// longest-first order of kwork.  A pair that splits (bwd_slices > 1) asks for as many slots as
// slices; slots go out in that order while the running total stays within n_slots, so the
// granted ranges are disjoint; a pair past the pool runs unsplit.  pslot[item] = (slices,
// first slot).  units lists (item, slice) for every slice of every pair in the same order, one
// dK/dV workgroup each; n_units[0] = their number (at most max_units: the slices beyond the
// first belong to granted pairs and so fit in the n_slots pool).
__global__ __launch_bounds__(1024) void assign_slices(int32_t n_items, int32_t n_slots, int64_t max_units,
                                                      int32_t slice_entries,
                                                      const int32_t *__restrict__ kp_ptr,
                                                      const int32_t *__restrict__ kwork, int2 *__restrict__ pslot,
                                                      int2 *__restrict__ units, int32_t *__restrict__ n_units) {
    __shared__ int32_t scan[1024];
    __shared__ int32_t s_base, s_extra;
    const int tid = threadIdx.x;
    if (tid == 0) {
        s_base = 0;
        s_extra = 0;
    }
    __syncthreads();
    for (int32_t c0 = 0; c0 < n_items; c0 += 1024) {
        const int32_t t = c0 + tid;
        int32_t item = -1, sl = 1;
        if (t < n_items) {
            item = kwork[t];
            sl = bwd_slices(kp_ptr[item + 1] - kp_ptr[item], slice_entries);
        }
        const int32_t want = sl > 1 ? sl : 0;
        const int32_t req = scan1024(want, scan);            // inclusive scan of the requests
        const int32_t base = s_base + req - want;
        const bool granted = item >= 0 && want > 0 && base + want <= n_slots;
        const int32_t S = granted ? sl : 1;
        const int32_t req_all = scan[1023];
        __syncthreads();
        const int32_t ext = scan1024(S - 1, scan);          // inclusive scan of the extra slices
        const int64_t first = int64_t(t) + s_extra + ext - (S - 1);
        if (item >= 0) {
            pslot[item] = granted ? make_int2(sl, base) : make_int2(1, 0);
            for (int32_t j = 0; j < S; ++j)
                if (first + j < max_units) units[first + j] = make_int2(item, j);
        }
        const int32_t ext_all = scan[1023];
        __syncthreads();
        if (tid == 0) {
            s_base += req_all;
            s_extra += ext_all;
        }
        __syncthreads();
    }
    if (tid == 0) {
        const int64_t n = int64_t(n_items) + s_extra;
        n_units[0] = static_cast<int32_t>(n < max_units ? n : max_units);
    }
}

}  // namespace

hipError_t launch_bwd_plan(const WsLayout &w, const BwdLayout &b, int slice_entries, const char *ws, char *bws,
                           hipStream_t s) {
    const uint8_t *cmap = reinterpret_cast<const uint8_t *>(ws + w.cmap);
    int32_t *kp_ptr = reinterpret_cast<int32_t *>(bws + b.kp_ptr);
    int32_t *kp_list = reinterpret_cast<int32_t *>(bws + b.kp_list);
    int32_t *kwork = reinterpret_cast<int32_t *>(bws + b.kwork);
    int32_t *khist = reinterpret_cast<int32_t *>(bws + b.khist);
    const int32_t n_items = w.R * b.nP;
    if (n_items > 0)
        count_pairs<<<(n_items + 3) / 4, 256, 0, s>>>(w.nQ, w.nK, b.nP, n_items, cmap, kp_ptr);
    finish_pairs<<<1, 1024, 0, s>>>(w.nQ, n_items, kp_ptr, khist, kwork);
    if (n_items > 0) {
        fill_pairs<<<(n_items + 3) / 4, 256, 0, s>>>(w.nQ, w.nK, b.nP, n_items, cmap, kp_ptr, kp_list);
    }
    // Always: an empty batch still needs n_units = 0 for the dK/dV launch.
    assign_slices<<<1, 1024, 0, s>>>(n_items, b.n_slots, b.max_units, slice_entries, kp_ptr, kwork,
                                     reinterpret_cast<int2 *>(bws + b.pslot), reinterpret_cast<int2 *>(bws + b.units),
                                     reinterpret_cast<int32_t *>(bws + b.n_units));
    return hipGetLastError();
}

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
    int2 *kt_stats = reinterpret_cast<int2 *>(ws + w.kt_stats);
    int32_t *ctr = reinterpret_cast<int32_t *>(ws + w.ctr);
    const int32_t n_tiles = w.R * w.nQ;

    // No memset nodes: everything the plan needs cleared is cleared by its own kernels.
    if (w.R > 0) {
        validate_rows<<<w.R, 256, 0, s>>>(w.R, w.T, d.n_segs, d.seg_row_ptr, d.seg_start, d.seg_len,
                                          d.seg_parent, n_real, seg_end);
        kend_stats<<<dim3((w.nK + 3) / 4, w.R), 256, 0, s>>>(w.T, w.BK, w.nK, d.seg_row_ptr, d.seg_start, n_real,
                                                             seg_end, kend, kt_stats);
        classify_tiles<<<(n_tiles + 3) / 4, 256, 0, s>>>(w.R, w.BQ, w.BK, w.nQ, w.nK, n_real, kt_stats, cmap,
                                                         qt_ptr);
    }
    finish_plan<<<1, 1024, 0, s>>>(w.R, w.nQ, w.nK, n_tiles, n_real, qt_ptr, hist, work, 2 * w.n_lanes, ctr, status);
    if (n_tiles > 0)
        fill_lists<<<(n_tiles + 3) / 4, 256, 0, s>>>(w.nK, n_tiles, cmap, qt_ptr, kt_idx, kt_kind);
    return hipGetLastError();
}

}  // namespace treeattn
