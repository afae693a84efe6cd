// C-ABI entry points of the device half of libtreeattn (see include/treeattn.h): argument
// checks, workspace layout, launches.  No device memory is allocated here; the one fixed
// device buffer (tree_attn_fwd_noalloc's scratch) is a file-scope __device__ array.
#include <cmath>
#include <mutex>
#include <vector>

#include "internal.h"

using namespace treeattn;

namespace {

// Largest power of two <= 8 that divides the query-head group size: the number of query
// heads one forward workgroup covers.  block_q = 256 / that.
int32_t heads_per_wg(int32_t G) {
    int32_t h = 1;
    while (h < 8 && G % (2 * h) == 0) h *= 2;
    return h;
}

bool shape_ok(const tree_attn_desc *d) {
    if (d == nullptr) return false;
    if (d->n_rows < 0 || d->row_len <= 0 || d->h_q <= 0 || d->h_kv <= 0 || d->n_segs < 0) return false;
    if (d->h_q % d->h_kv != 0) return false;
    if (d->head_dim != 64 && d->head_dim != 128) return false;
    if (d->dtype != TREE_DT_BF16 && d->dtype != TREE_DT_F32) return false;
    if (!(d->scale >= 0.f) || !std::isfinite(d->scale)) return false;
    if (d->n_rows > 0 && (d->seg_row_ptr == nullptr || (d->n_segs > 0 &&
        (d->seg_start == nullptr || d->seg_len == nullptr || d->seg_parent == nullptr))))
        return false;
    return true;
}

void fwd_blocks(const tree_attn_desc *d, int32_t *bq, int32_t *bk) {
    *bq = kFwdRowsPerWG / heads_per_wg(d->h_q / d->h_kv);
    *bk = kFwdBlockK;
}

// Resolved plan tile sizes: explicit ones must be positive multiples of 16 dividing row_len.
bool plan_blocks(const tree_attn_desc *d, int32_t *bq, int32_t *bk) {
    fwd_blocks(d, bq, bk);
    if (d->block_q != 0) *bq = d->block_q;
    if (d->block_k != 0) *bk = d->block_k;
    for (int32_t b : {*bq, *bk})
        if (b <= 0 || b % 16 != 0 || b > 1024 || d->row_len % b != 0) return false;
    return true;
}

bool layout_of(const tree_attn_desc *d, WsLayout *w) {
    int32_t bq, bk;
    if (!shape_ok(d) || !plan_blocks(d, &bq, &bk)) return false;
    *w = make_layout(d->n_rows, d->row_len, bq, bk, d->n_segs, d->h_q / heads_per_wg(d->h_q / d->h_kv));
    return true;
}

}  // namespace

extern "C" int tree_attn_blocks(const tree_attn_desc *d, int32_t *block_q, int32_t *block_k) {
    if (!shape_ok(d) || block_q == nullptr || block_k == nullptr) return TREE_E_INVAL;
    fwd_blocks(d, block_q, block_k);
    return TREE_OK;
}

extern "C" int tree_attn_workspace_size(const tree_attn_desc *d, size_t *bytes) {
    WsLayout w;
    if (bytes == nullptr || !layout_of(d, &w)) return TREE_E_INVAL;
    *bytes = w.total;
    return TREE_OK;
}

extern "C" int tree_attn_plan(const tree_attn_desc *d, void *ws, void *stream) {
    WsLayout w;
    if (!layout_of(d, &w) || ws == nullptr || (reinterpret_cast<uintptr_t>(ws) & 255) != 0)
        return TREE_E_INVAL;
    const hipError_t e = launch_plan(*d, w, static_cast<char *>(ws), static_cast<hipStream_t>(stream));
    return e == hipSuccess ? TREE_OK : TREE_E_HIP;
}

extern "C" int tree_attn_plan_status(const tree_attn_desc *d, const void *ws, void *stream) {
    WsLayout w;
    if (!layout_of(d, &w) || ws == nullptr) return TREE_E_INVAL;
    int32_t st = 0;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (hipMemcpyAsync(&st, static_cast<const char *>(ws) + w.status, sizeof(st), hipMemcpyDeviceToHost, s) !=
        hipSuccess)
        return TREE_E_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return TREE_E_HIP;
    return st == 0 ? TREE_OK : TREE_E_LAYOUT;
}

extern "C" int tree_attn_tiles(const tree_attn_desc *d, const void *ws, tree_tile_view *out) {
    WsLayout w;
    if (!layout_of(d, &w) || ws == nullptr || out == nullptr) return TREE_E_INVAL;
    const char *b = static_cast<const char *>(ws);
    out->block_q = w.BQ;
    out->block_k = w.BK;
    out->n_qtiles = w.nQ;
    out->n_ktiles = w.nK;
    out->class_map = reinterpret_cast<const uint8_t *>(b + w.cmap);
    out->qt_ptr = reinterpret_cast<const int32_t *>(b + w.qt_ptr);
    out->kt_idx = reinterpret_cast<const int32_t *>(b + w.kt_idx);
    out->kt_kind = reinterpret_cast<const uint8_t *>(b + w.kt_kind);
    out->kend = reinterpret_cast<const int32_t *>(b + w.kend);
    out->work = reinterpret_cast<const int32_t *>(b + w.work);
    out->status = reinterpret_cast<const int32_t *>(b + w.status);
    return TREE_OK;
}

extern "C" int tree_attn_fwd(const tree_attn_desc *d, void *ws, const void *q, const void *k,
                             const void *v, void *o, float *lse, void *stream) {
    WsLayout w;
    if (!layout_of(d, &w) || ws == nullptr) return TREE_E_INVAL;
    if (d->n_rows > 0 && (q == nullptr || k == nullptr || v == nullptr || o == nullptr || lse == nullptr))
        return TREE_E_INVAL;
    int32_t bq, bk;
    fwd_blocks(d, &bq, &bk);
    if (w.BQ != bq || w.BK != bk) return TREE_E_UNSUPPORTED;
    if (d->dtype == TREE_DT_F32 && d->head_dim != 64) return TREE_E_UNSUPPORTED;
    if (w.nK > kFwdMaxKTiles) return TREE_E_UNSUPPORTED;
    FwdShape sh;
    sh.R = d->n_rows; sh.T = d->row_len; sh.Hq = d->h_q; sh.Hkv = d->h_kv; sh.D = d->head_dim;
    sh.dtype = d->dtype;
    sh.G = d->h_q / d->h_kv;
    sh.HCH = heads_per_wg(sh.G);
    sh.BQ = bq;
    sh.scale = d->scale > 0.f ? d->scale : 1.0f / std::sqrt(static_cast<float>(d->head_dim));
    const hipError_t e = launch_fwd(sh, w, static_cast<char *>(ws), q, k, v, o, lse,
                                    static_cast<hipStream_t>(stream));
    return e == hipSuccess ? TREE_OK : TREE_E_HIP;
}

// ----------------------------------------------------------------------------- no allocation
//
// tree_attn_fwd_noalloc keeps the tile plan in this fixed device buffer instead of a caller
// workspace.  In host code `scratch` names a host-side stand-in, not the device array: its
// device address is taken once per device with hipGetSymbolAddress (with that device
// current) and only that address is passed to kernels.  Every call on a device shares the
// device's copy; the plan kernels rewrite every part of it the forward reads, so nothing
// needs clearing between calls, and calls that overlap on one device race.
namespace {
__device__ __align__(256) char scratch[TREE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char *g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (nullptr on failure).
char *scratch_on_current_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
        g_scratch_ptr[dev] = static_cast<char *>(p);
    }
    return g_scratch_ptr[dev];
}
}  // namespace

extern "C" int tree_attn_fwd_noalloc(const tree_attn_desc *d, const void *q, const void *k, const void *v,
                                     void *o, float *lse, void *stream) {
    WsLayout w;
    if (!layout_of(d, &w)) return TREE_E_INVAL;
    if (d->n_rows > 0 && (q == nullptr || k == nullptr || v == nullptr || o == nullptr || lse == nullptr))
        return TREE_E_INVAL;
    int32_t bq, bk;
    fwd_blocks(d, &bq, &bk);
    if (w.BQ != bq || w.BK != bk) return TREE_E_UNSUPPORTED;
    if (d->dtype == TREE_DT_F32 && d->head_dim != 64) return TREE_E_UNSUPPORTED;
    if (w.nK > kFwdMaxKTiles) return TREE_E_UNSUPPORTED;
    if (w.total > TREE_NOALLOC_SCRATCH_BYTES) return TREE_E_UNSUPPORTED;
    char *ws = scratch_on_current_device();
    if (ws == nullptr) return TREE_E_HIP;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (launch_plan(*d, w, ws, s) != hipSuccess) return TREE_E_HIP;
    FwdShape sh;
    sh.R = d->n_rows; sh.T = d->row_len; sh.Hq = d->h_q; sh.Hkv = d->h_kv; sh.D = d->head_dim;
    sh.dtype = d->dtype;
    sh.G = d->h_q / d->h_kv;
    sh.HCH = heads_per_wg(sh.G);
    sh.BQ = bq;
    sh.scale = d->scale > 0.f ? d->scale : 1.0f / std::sqrt(static_cast<float>(d->head_dim));
    return launch_fwd(sh, w, ws, q, k, v, o, lse, s) == hipSuccess ? TREE_OK : TREE_E_HIP;
}

// ----------------------------------------------------------------------------- backward

namespace {
// The backward runs on the forward's plan (same tile sizes) and needs bf16.
int bwd_check(const tree_attn_desc *d, WsLayout *w, BwdLayout *b) {
    if (!layout_of(d, w)) return TREE_E_INVAL;
    int32_t bq, bk;
    fwd_blocks(d, &bq, &bk);
    if (w->BQ != bq || w->BK != bk) return TREE_E_UNSUPPORTED;
    if (d->dtype != TREE_DT_BF16) return TREE_E_UNSUPPORTED;
    if (w->nK > kFwdMaxKTiles) return TREE_E_UNSUPPORTED;
    *b = make_bwd_layout(*w, d->h_q, d->h_kv, d->head_dim);
    return TREE_OK;
}
}  // namespace

extern "C" int tree_attn_bwd_workspace_size(const tree_attn_desc *d, size_t *bytes) {
    WsLayout w;
    BwdLayout b;
    if (bytes == nullptr) return TREE_E_INVAL;
    const int rc = bwd_check(d, &w, &b);
    if (rc != TREE_OK) return rc;
    *bytes = b.total;
    return TREE_OK;
}

extern "C" int tree_attn_bwd_plan(const tree_attn_desc *d, const void *ws, void *bws, void *stream) {
    WsLayout w;
    BwdLayout b;
    const int rc = bwd_check(d, &w, &b);
    if (rc != TREE_OK) return rc;
    if (ws == nullptr || bws == nullptr || (reinterpret_cast<uintptr_t>(bws) & 255) != 0) return TREE_E_INVAL;
    int dev = 0, n_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n_cu <= 0)
        n_cu = 256;
    const int per = bwd_slice_entries(int64_t(w.R) * b.nP, d->h_kv, n_cu);
    const hipError_t e = launch_bwd_plan(w, b, per, static_cast<const char *>(ws), static_cast<char *>(bws),
                                         static_cast<hipStream_t>(stream));
    return e == hipSuccess ? TREE_OK : TREE_E_HIP;
}

extern "C" int tree_attn_bwd_tiles(const tree_attn_desc *d, const void *bws, const int32_t **kp_ptr,
                                   const int32_t **kp_list) {
    WsLayout w;
    BwdLayout b;
    const int rc = bwd_check(d, &w, &b);
    if (rc != TREE_OK) return rc;
    if (bws == nullptr || kp_ptr == nullptr || kp_list == nullptr) return TREE_E_INVAL;
    *kp_ptr = reinterpret_cast<const int32_t *>(static_cast<const char *>(bws) + b.kp_ptr);
    *kp_list = reinterpret_cast<const int32_t *>(static_cast<const char *>(bws) + b.kp_list);
    return TREE_OK;
}

extern "C" int tree_attn_bwd(const tree_attn_desc *d, const void *ws, void *bws, const void *q, const void *k,
                             const void *v, const void *o, const float *lse, const void *dout, void *dq,
                             void *dk, void *dv, void *stream) {
    WsLayout w;
    BwdLayout b;
    const int rc = bwd_check(d, &w, &b);
    if (rc != TREE_OK) return rc;
    if (ws == nullptr || bws == nullptr) return TREE_E_INVAL;
    if (d->n_rows > 0 && (q == nullptr || k == nullptr || v == nullptr || o == nullptr || lse == nullptr ||
                          dout == nullptr || dq == nullptr || dk == nullptr || dv == nullptr))
        return TREE_E_INVAL;
    FwdShape sh;
    sh.R = d->n_rows; sh.T = d->row_len; sh.Hq = d->h_q; sh.Hkv = d->h_kv; sh.D = d->head_dim;
    sh.dtype = d->dtype;
    sh.G = d->h_q / d->h_kv;
    sh.HCH = heads_per_wg(sh.G);
    sh.BQ = w.BQ;
    sh.scale = d->scale > 0.f ? d->scale : 1.0f / std::sqrt(static_cast<float>(d->head_dim));
    const hipError_t e = launch_bwd(sh, w, b, static_cast<const char *>(ws), static_cast<char *>(bws), q, k, v,
                                    o, lse, dout, dq, dk, dv, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? TREE_OK : TREE_E_HIP;
}

// ----------------------------------------------------------------------------- gated delta rule

namespace {
bool gdn_shape_ok(const tree_attn_desc *d) {
    return shape_ok(d) && d->h_q == d->h_kv && d->head_dim == 128 && d->dtype == TREE_DT_BF16;
}

int gdn_counts(const tree_attn_desc *d, const int32_t *rp, const int32_t *len, int32_t *n_segs, int32_t *n_chunks) {
    if (!gdn_shape_ok(d)) return TREE_E_INVAL;
    if (d->n_rows > 0 && (rp == nullptr || len == nullptr)) return TREE_E_INVAL;
    if (d->n_rows > 0 && rp[0] != 0) return TREE_E_LAYOUT;
    int64_t chunks = 0;
    for (int32_t r = 0; r < d->n_rows; ++r) {
        if (rp[r + 1] < rp[r]) return TREE_E_LAYOUT;
        for (int32_t s = rp[r]; s < rp[r + 1]; ++s) {
            if (len[s] <= 0 || len[s] > d->row_len) return TREE_E_LAYOUT;
            chunks += (len[s] + 63) / 64;
        }
    }
    if (chunks > INT32_MAX / 64) return TREE_E_INVAL;
    *n_segs = d->n_rows > 0 ? rp[d->n_rows] : 0;
    *n_chunks = static_cast<int32_t>(chunks);
    return TREE_OK;
}
}  // namespace

extern "C" int tree_gdn_workspace_size(const tree_attn_desc *d, const int32_t *h_seg_row_ptr,
                                       const int32_t *h_seg_len, size_t *bytes) {
    int32_t n_segs = 0, n_chunks = 0;
    if (bytes == nullptr) return TREE_E_INVAL;
    const int rc = gdn_counts(d, h_seg_row_ptr, h_seg_len, &n_segs, &n_chunks);
    if (rc != TREE_OK) return rc;
    *bytes = make_gdn_layout(d->n_rows, d->row_len, d->h_q, n_chunks, n_segs).total;
    return TREE_OK;
}

extern "C" int tree_gdn_plan(const tree_attn_desc *d, const int32_t *h_seg_row_ptr, const int32_t *h_seg_start,
                             const int32_t *h_seg_len, const int32_t *h_seg_parent, void *gws,
                             tree_gdn_info *info, void *stream) {
    int32_t n_segs = 0, n_chunks = 0;
    const int rc = gdn_counts(d, h_seg_row_ptr, h_seg_len, &n_segs, &n_chunks);
    if (rc != TREE_OK) return rc;
    if (info == nullptr || gws == nullptr || (d->n_rows > 0 && (h_seg_start == nullptr || h_seg_parent == nullptr)))
        return TREE_E_INVAL;
    const int32_t R = d->n_rows, T = d->row_len;
    // Validate the table (segments back to back from token 0, parents before children) and
    // build token parents, chunks, segment records and depth levels.
    std::vector<int32_t> pi(size_t(R) * T, -2), chunk_meta, seg_meta(size_t(n_segs) * 4), depth(n_segs, 0);
    chunk_meta.reserve(size_t(n_chunks) * 4);
    for (int32_t r = 0; r < R; ++r) {
        const int32_t a = h_seg_row_ptr[r], b = h_seg_row_ptr[r + 1];
        int64_t off = 0;
        for (int32_t g = a; g < b; ++g) {
            const int32_t st = h_seg_start[g], n = h_seg_len[g], p = h_seg_parent[g];
            if (st != off || off + n > T || p < -1 || p >= g - a) return TREE_E_LAYOUT;
            off += n;
            const int64_t base = int64_t(r) * T;
            pi[base + st] = p < 0 ? -1 : int32_t(base + h_seg_start[a + p] + h_seg_len[a + p] - 1);
            for (int32_t i = 1; i < n; ++i) pi[base + st + i] = int32_t(base + st + i - 1);
            depth[g] = p < 0 ? 0 : depth[a + p] + 1;
            seg_meta[size_t(g) * 4 + 0] = r;
            seg_meta[size_t(g) * 4 + 1] = static_cast<int32_t>(chunk_meta.size() / 4);
            seg_meta[size_t(g) * 4 + 2] = (n + 63) / 64;
            seg_meta[size_t(g) * 4 + 3] = p < 0 ? -1 : a + p;
            for (int32_t c0 = 0; c0 < n; c0 += 64) {
                chunk_meta.push_back(r);
                chunk_meta.push_back(st + c0);
                chunk_meta.push_back(std::min(64, n - c0));
                chunk_meta.push_back(g);
            }
        }
    }
    int32_t n_levels = 0;
    for (int32_t g = 0; g < n_segs; ++g) n_levels = std::max(n_levels, depth[g] + 1);
    std::vector<int32_t> level_ptr(size_t(n_levels) + 1, 0), level_segs(n_segs);
    for (int32_t g = 0; g < n_segs; ++g) ++level_ptr[depth[g] + 1];
    // Narrow levels: at most (CUs / heads) segments, so that two workgroups per (segment,
    // head) stay within two per CU.
    int dev = 0, n_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n_cu <= 0)
        n_cu = 256;
    const int32_t narrow_max = std::max(1, n_cu / std::max(1, d->h_q));
    int32_t max_level = 0, narrow_segs = 0;
    uint32_t narrow_levels = 0;
    for (int32_t l = 0; l < n_levels; ++l) {
        const int32_t cnt = level_ptr[l + 1];
        max_level = std::max(max_level, cnt);
        if (l < 32 && cnt <= narrow_max) {
            narrow_levels |= 1u << l;
            narrow_segs = std::max(narrow_segs, cnt);
        }
        level_ptr[l + 1] += level_ptr[l];
    }
    {
        std::vector<int32_t> fill(level_ptr.begin(), level_ptr.end() - 1);
        for (int32_t g = 0; g < n_segs; ++g) level_segs[fill[depth[g]]++] = g;
    }
    // Prep order: the chunks of depth-0 segments first (the depth-0 scan needs only these).
    std::vector<int32_t> prep_order;
    prep_order.reserve(size_t(n_chunks));
    for (int pass = 0; pass < 2; ++pass)
        for (int32_t c = 0; c < n_chunks; ++c)
            if ((depth[chunk_meta[size_t(c) * 4 + 3]] == 0) == (pass == 0)) prep_order.push_back(c);
    int32_t lead_chunks = 0, lead_chain = 0, lead_segs = 0;
    for (int32_t c = 0; c < n_chunks; ++c) lead_chunks += depth[chunk_meta[size_t(c) * 4 + 3]] == 0 ? 1 : 0;
    for (int32_t g = 0; g < n_segs; ++g)
        if (depth[g] == 0) {
            lead_chain = std::max(lead_chain, seg_meta[size_t(g) * 4 + 2]);
            ++lead_segs;
        }
    const GdnLayout L = make_gdn_layout(R, T, d->h_q, n_chunks, n_segs);
    char *w = static_cast<char *>(gws);
    hipStream_t s = static_cast<hipStream_t>(stream);
    struct Part { size_t off; const void *src; size_t bytes; };
    const Part parts[] = {{L.pi, pi.data(), pi.size() * 4},
                          {L.chunk_meta, chunk_meta.data(), chunk_meta.size() * 4},
                          {L.seg_meta, seg_meta.data(), seg_meta.size() * 4},
                          {L.level_ptr, level_ptr.data(), level_ptr.size() * 4},
                          {L.level_segs, level_segs.data(), level_segs.size() * 4},
                          {L.prep_order, prep_order.data(), prep_order.size() * 4}};
    for (const Part &pt : parts)
        if (pt.bytes > 0 && hipMemcpyAsync(w + pt.off, pt.src, pt.bytes, hipMemcpyHostToDevice, s) != hipSuccess)
            return TREE_E_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return TREE_E_HIP;   // the host arrays are temporaries
    info->n_chunks = n_chunks;
    info->n_segs = n_segs;
    info->n_levels = n_levels;
    info->max_level_segs = max_level;
    info->narrow_segs = narrow_segs;
    info->narrow_levels = narrow_levels;
    info->lead_chunks = lead_chunks;
    info->lead_chain = lead_chain;
    info->lead_segs = lead_segs;
    return TREE_OK;
}

extern "C" int tree_gdn_fwd(const tree_attn_desc *d, const tree_gdn_info *info, void *gws, const void *x_q,
                            const void *x_k, const void *x_v, const float *conv_w, const float *g, const float *beta,
                            void *o, void *stream) {
    if (!gdn_shape_ok(d) || info == nullptr || gws == nullptr) return TREE_E_INVAL;
    if (info->n_chunks < 0 || info->n_segs < 0 || info->n_levels < 0 || info->n_levels > info->n_segs ||
        info->max_level_segs < 0 || info->max_level_segs > info->n_segs || info->narrow_segs < 0 ||
        info->narrow_segs > info->max_level_segs || info->lead_chunks < 0 || info->lead_chunks > info->n_chunks ||
        info->lead_chain < 0 || info->lead_chain > info->lead_chunks || info->lead_segs < 0 ||
        info->lead_segs > info->n_segs)
        return TREE_E_INVAL;
    if (d->n_rows > 0 && (x_q == nullptr || x_k == nullptr || x_v == nullptr || conv_w == nullptr || g == nullptr ||
                          beta == nullptr || o == nullptr))
        return TREE_E_INVAL;
    GdnLayout L = make_gdn_layout(d->n_rows, d->row_len, d->h_q, info->n_chunks, info->n_segs);
    L.n_levels = info->n_levels;
    L.max_level_segs = info->max_level_segs;
    L.narrow_segs = info->narrow_segs;
    L.narrow_levels = info->narrow_levels;
    L.lead_chunks = info->lead_chunks;
    L.lead_chain = info->lead_chain;
    L.lead_segs = info->lead_segs;
    GdnShape sh{d->n_rows, d->row_len, d->h_q, 1e-6f};
    const hipError_t e = launch_gdn(sh, L, static_cast<char *>(gws), x_q, x_k, x_v, conv_w, g, beta, o,
                                    static_cast<hipStream_t>(stream));
    return e == hipSuccess ? TREE_OK : TREE_E_HIP;
}

extern "C" int tree_rope(const tree_attn_desc *d, const int32_t *pos_ids, float theta, int32_t inverse, void *q,
                         void *k, void *stream) {
    if (!shape_ok(d) || !(theta > 1.0f) || (inverse != 0 && inverse != 1)) return TREE_E_INVAL;
    if (d->n_rows > 0 && (pos_ids == nullptr || (q == nullptr && k == nullptr))) return TREE_E_INVAL;
    const hipError_t e = launch_rope(d->n_rows, d->row_len, d->h_q, d->h_kv, d->head_dim, d->dtype, pos_ids, theta,
                                     inverse, q, k, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? TREE_OK : TREE_E_HIP;
}

extern "C" const char *tree_status_str(int code) {
    switch (code) {
        case TREE_OK: return "ok";
        case TREE_E_INVAL: return "invalid argument";
        case TREE_E_TOOLONG: return "a sequence is longer than the row capacity";
        case TREE_E_LAYOUT: return "segment table is not a valid pre-order forest layout";
        case TREE_E_NOMEM: return "out of host memory";
        case TREE_E_HIP: return "HIP runtime or launch error";
        case TREE_E_UNSUPPORTED: return "no kernel for these arguments (plan tile sizes differ from the forward kernel's, the row is too long, or no backward for this dtype)";
        default: return "unknown status";
    }
}
