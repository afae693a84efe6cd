// C-ABI entry points of the device half of libtreeattn (see include/treeattn.h): argument
// checks, workspace layout, launches.  No device memory is allocated here.
#include <cmath>

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
    *w = make_layout(d->n_rows, d->row_len, bq, bk, d->n_segs);
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

extern "C" int tree_attn_fwd(const tree_attn_desc *d, const void *ws, const void *q, const void *k,
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
    const hipError_t e = launch_fwd(sh, w, static_cast<const char *>(ws), q, k, v, o, lse,
                                    static_cast<hipStream_t>(stream));
    return e == hipSuccess ? TREE_OK : TREE_E_HIP;
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
    *b = make_bwd_layout(*w, d->h_q);
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
    const hipError_t e = launch_bwd_plan(w, b, static_cast<const char *>(ws), static_cast<char *>(bws),
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
