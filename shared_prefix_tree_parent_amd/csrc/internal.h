// Internal declarations shared by the C-ABI glue and the HIP kernels of libtreeattn.
#pragma once

#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>

#include "treeattn.h"

namespace treeattn {

constexpr int kTileSkip = 0, kTileFull = 1, kTilePartial = 2;
constexpr int kFwdBlockK = 64;        // keys per k-tile in the forward kernel
constexpr int kFwdRowsPerWG = 256;    // (query head, position) rows one forward workgroup owns
// Longest k-tile list the forward keeps in LDS beside its four 32 KB K/V buffers, their kend
// and 16 bytes of control words (160 KB per workgroup): row_len <= 64 * 7932 = 507648.
constexpr int kFwdMaxKTiles = 7932;

// Device workspace layout: every section 256-byte aligned, offsets from the base pointer.
struct WsLayout {
    int32_t R = 0, T = 0, BQ = 0, BK = 0, nQ = 0, nK = 0, n_segs = 0;
    size_t status = 0;    // int32[4]: [0] layout status (0 = ok), [1..3] scratch counters
    size_t n_real = 0;    // int32[R]   tokens used per row, -1 if the row's table is invalid
    size_t seg_end = 0;   // int32[n_segs] end (exclusive token offset) of each segment's subtree
    size_t kend = 0;      // int32[R*T]
    size_t cmap = 0;      // uint8[R*nQ*nK]
    size_t qt_ptr = 0;    // int32[R*nQ + 1]
    size_t kt_idx = 0;    // int32[R*nQ*nK]
    size_t kt_kind = 0;   // uint8[R*nQ*nK]
    size_t work = 0;      // int32[R*nQ]: (row, q-tile) items, rows in order, longest first in a row
    size_t hist = 0;      // int32[R*(nK + 1) + 2]: work-list buckets (row, k-tile count)
    size_t kt_stats = 0;  // int2[R*nK] per k-tile (min kend, max kend over real keys)
    size_t ctr = 0;       // int32[2*n_lanes]: forward item counters, then finished-workgroup
                          // counters, one per KV lane (zeroed by the plan; each forward leaves
                          // them at zero)
    int32_t n_lanes = 0;  // forward KV lanes: h_q / (query heads per workgroup)
    size_t total = 0;
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

inline WsLayout make_layout(int32_t R, int32_t T, int32_t BQ, int32_t BK, int32_t n_segs, int32_t n_lanes) {
    WsLayout w;
    w.R = R; w.T = T; w.BQ = BQ; w.BK = BK; w.n_segs = n_segs; w.n_lanes = n_lanes;
    w.nQ = T / BQ;
    w.nK = T / BK;
    const size_t tiles = size_t(R) * w.nQ * w.nK;
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off = align256(off + bytes); return o; };
    w.status = take(4 * sizeof(int32_t));
    w.n_real = take(size_t(R) * sizeof(int32_t));
    w.seg_end = take(size_t(n_segs > 0 ? n_segs : 1) * sizeof(int32_t));
    w.kend = take(size_t(R) * T * sizeof(int32_t));
    w.cmap = take(tiles);
    w.qt_ptr = take((size_t(R) * w.nQ + 1) * sizeof(int32_t));
    w.kt_idx = take(tiles * sizeof(int32_t));
    w.kt_kind = take(tiles);
    w.work = take(size_t(R) * w.nQ * sizeof(int32_t));
    w.hist = take((size_t(R) * (w.nK + 1) + 2) * sizeof(int32_t));
    w.kt_stats = take(size_t(R) * w.nK * 2 * sizeof(int32_t));
    w.ctr = take(size_t(2) * n_lanes * sizeof(int32_t));
    w.total = off;
    return w;
}

// Backward workspace layout (caller-allocated, filled by tree_attn_bwd_plan / tree_attn_bwd).
// The dK/dV pass works on groups of kKvGroup consecutive k-tiles (k-tiles 4p .. 4p+3, 256
// keys), called pairs below for short.
// dK/dV query slices: a k-tile group whose q-tile list has n entries is processed as
// min(kBwdSlices, max(1, n / e)) workgroups per KV head (e = kBwdSliceEntries, or
// kBwdSliceEntriesSmall on a batch too small to fill the device), each over an equal
// run of the list; when there is more than one, each writes an fp32 partial and a reduce pass
// adds them in slice order (deterministic).  Partials take slots from a pool of at most
// kBwdMaxSlots (per KV head), handed out to the longest pairs first; a pair that does not fit
// runs unsplit.  The plan lists the (pair, slice) units in work order, so the dK/dV launch
// has one workgroup per unit and KV head (plus a surplus at the end of the grid that exits at
// once): at most R*nP + min((kBwdSlices-1)*R*nP, kBwdMaxSlots) units, since only granted
// pairs have more than one slice and their slices fit in the pool.
constexpr int kKvGroup = 4;        // k-tiles per dK/dV unit
constexpr int kBwdSlices = 4;
constexpr int kBwdSliceEntries = 16;        // list entries per slice ...
constexpr int kBwdSliceEntriesSmall = 8;    // ... where the batch has fewer (group, KV head)
                                            // items than the device has CUs
constexpr int kBwdMaxSlots = 512;
__host__ __device__ inline int bwd_slices(int n, int per) {
    const int k = n / per;
    return k < 1 ? 1 : (k > kBwdSlices ? kBwdSlices : k);
}
inline int bwd_slice_entries(int64_t n_items, int32_t Hkv, int n_cu) {
    return n_items * Hkv < int64_t(n_cu) ? kBwdSliceEntriesSmall : kBwdSliceEntries;
}

struct BwdLayout {
    size_t delta = 0;     // float[R*Hq*T]: rowsum(dO * O) per (row, head, token); 0 at pads
    size_t lse2 = 0;      // float[R*Hq*T]: the forward's LSE times log2(e)
    size_t kp_ptr = 0;    // int32[R*nP + 1]: CSR over (row, k-tile group) of the q-tiles that see it
    size_t kp_list = 0;   // int32[R*nQ*nP]: q-tile*256 + sum_i class(4p+i) << 2(3-i), ascending q-tile
    size_t kwork = 0;     // int32[R*nP]: (row, pair) items, longest list first
    size_t khist = 0;     // int32[nQ + 2]
    size_t pslot = 0;     // int2[R*nP]: per pair (query slices, first partial slot)
    size_t units = 0;     // int2[max_units]: (pair item, slice) in work order
    size_t n_units = 0;   // int32[1]: units in use
    size_t part = 0;      // float[n_slots*Hkv*2*(64 kKvGroup)*D]: per-slice dK^T, dV^T partials
    size_t total = 0;
    int32_t nP = 0;       // k-tile groups per row: ceil(nK / kKvGroup)
    int32_t n_slots = 0;  // partial slots: min(R*nP*kBwdSlices, kBwdMaxSlots)
    int64_t max_units = 0;   // R*nP + min((kBwdSlices-1)*R*nP, kBwdMaxSlots)
};

inline BwdLayout make_bwd_layout(const WsLayout &w, int32_t Hq, int32_t Hkv, int32_t D) {
    BwdLayout b;
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off = align256(off + bytes); return o; };
    b.nP = (w.nK + kKvGroup - 1) / kKvGroup;
    b.delta = take(size_t(w.R) * Hq * w.T * sizeof(float));
    b.lse2 = take(size_t(w.R) * Hq * w.T * sizeof(float));
    b.kp_ptr = take((size_t(w.R) * b.nP + 1) * sizeof(int32_t));
    b.kp_list = take(size_t(w.R) * w.nQ * b.nP * sizeof(int32_t));
    b.kwork = take(size_t(w.R) * b.nP * sizeof(int32_t));
    b.khist = take((size_t(w.nQ) + 2) * sizeof(int32_t));
    const int64_t want = int64_t(w.R) * b.nP * kBwdSlices;
    b.n_slots = static_cast<int32_t>(want < kBwdMaxSlots ? want : kBwdMaxSlots);
    b.pslot = take(size_t(w.R) * b.nP * 2 * sizeof(int32_t));
    const int64_t n_items = int64_t(w.R) * b.nP;
    const int64_t extra = int64_t(kBwdSlices - 1) * n_items;
    b.max_units = n_items + (extra < kBwdMaxSlots ? extra : kBwdMaxSlots);
    b.units = take(size_t(b.max_units) * 2 * sizeof(int32_t));
    b.n_units = take(sizeof(int32_t));
    b.part = take(size_t(b.n_slots) * Hkv * 2 * (64 * kKvGroup) * D * sizeof(float));
    b.total = off;
    return b;
}

// Gated delta rule workspace (caller-allocated; metadata written by tree_gdn_plan).
struct GdnShape {
    int32_t R, T, H;
    float eps;
};
struct GdnLayout {
    size_t pi = 0;           // int32[R*T]: global token parent, -1 at a root's first token, -2 pads
    size_t chunk_meta = 0;   // int4[n_chunks]: (row, first token, tokens, segment)
    size_t seg_meta = 0;     // int4[n_segs]: (row, first chunk, chunks, parent segment or -1)
    size_t level_ptr = 0;    // int32[n_levels + 1] (room for n_segs + 1): segments per depth, CSR
    size_t level_segs = 0;   // int32[n_segs]: segments by depth
    size_t prep_order = 0;   // int32[n_chunks]: chunks of depth-0 segments first, then the rest
    size_t qh = 0, kh = 0, vh = 0;   // bf16[R*T*H*128] each: conv + norm outputs
    size_t U = 0;            // f32[n_chunks*H*64*128], in the scan's accumulator order
    size_t Yn = 0;           // bf16[n_chunks*H*64*128]
    size_t P = 0;            // bf16[n_chunks*H*64*64]
    size_t F = 0;            // f32[n_chunks*H*128]: gamma_t, then gamma_C / gamma_t
    size_t states = 0;       // f32[n_segs*H*128*128]: final state of every segment
    size_t total = 0;
    int32_t n_chunks = 0, n_segs = 0, n_levels = 0, max_level_segs = 0;
    int32_t narrow_segs = 0;      // levels of bit l in narrow_levels: at most this many segments
    uint32_t narrow_levels = 0;
    int32_t lead_chunks = 0;      // chunks of depth-0 segments (the head of prep_order)
    int32_t lead_chain = 0;       // the most chunks of one depth-0 segment
    int32_t lead_segs = 0;        // depth-0 segments
};
inline GdnLayout make_gdn_layout(int32_t R, int32_t T, int32_t H, int32_t n_chunks, int32_t n_segs) {
    GdnLayout g;
    size_t off = 0;
    auto take = [&](size_t bytes) { size_t o = off; off = align256(off + bytes); return o; };
    const size_t tok = size_t(R) * T;
    g.pi = take(tok * 4);
    g.chunk_meta = take(size_t(n_chunks) * 16);
    g.seg_meta = take(size_t(n_segs) * 16);
    g.level_ptr = take((size_t(n_segs) + 1) * 4);
    g.level_segs = take(size_t(n_segs) * 4);
    g.prep_order = take(size_t(n_chunks) * 4);
    g.qh = take(tok * H * 128 * 2);
    g.kh = take(tok * H * 128 * 2);
    g.vh = take(tok * H * 128 * 2);
    g.U = take(size_t(n_chunks) * H * 64 * 128 * 4);
    g.Yn = take(size_t(n_chunks) * H * 64 * 128 * 2);
    g.P = take(size_t(n_chunks) * H * 64 * 64 * 2);
    g.F = take(size_t(n_chunks) * H * 128 * 4);
    g.states = take(size_t(n_segs) * H * 128 * 128 * 4);
    g.total = off;
    g.n_chunks = n_chunks;
    g.n_segs = n_segs;
    return g;
}

// Launchers (defined in classify.hip / attn_fwd.hip / attn_bwd.hip).  Return hipSuccess or the
// first error.
hipError_t launch_plan(const tree_attn_desc &d, const WsLayout &w, char *ws, hipStream_t s);
hipError_t launch_gdn(const GdnShape &sh, const GdnLayout &L, char *gws, const void *xq, const void *xk,
                      const void *xv, const float *conv_w, const float *g, const float *beta, void *o,
                      hipStream_t s);
hipError_t launch_rope(int32_t R, int32_t T, int32_t Hq, int32_t Hkv, int32_t D, int32_t dtype,
                       const int32_t *pos_ids, float theta, int32_t inverse, void *q, void *k, hipStream_t s);
hipError_t launch_bwd_plan(const WsLayout &w, const BwdLayout &b, int slice_entries, const char *ws, char *bws,
                           hipStream_t s);

struct FwdShape {
    int32_t R, T, Hq, Hkv, D, dtype;
    int32_t G;      // h_q / h_kv
    int32_t HCH;    // query heads of one KV group handled by one workgroup (1, 2, 4 or 8)
    int32_t BQ;     // positions per q-tile = kFwdRowsPerWG / HCH
    float scale;
};
hipError_t launch_fwd(const FwdShape &sh, const WsLayout &w, char *ws, const void *q,
                      const void *k, const void *v, void *o, float *lse, hipStream_t s);
hipError_t launch_bwd(const FwdShape &sh, const WsLayout &w, const BwdLayout &b, const char *ws, char *bws,
                      const void *q, const void *k, const void *v, const void *o, const float *lse,
                      const void *dout, void *dq, void *dk, void *dv, hipStream_t s);

}  // namespace treeattn
