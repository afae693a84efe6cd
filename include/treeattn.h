/*
 * treeattn.h — C ABI of libtreeattn.so: prefix-tree packing and tree-masked attention
 * forward for AMD Instinct MI355X (gfx950).
 *
 * Sources, cited by page title and passage:
 *   [PTP]   "Prefix tree packing", furtherai.github.io/blog/posts/prefix-tree-packing
 *   [AReaL] "How to Configure Sequence Packing for Efficient GPU Utilization in AReaL"
 *   [AOM]   "ART-Optimized Megatron (AOM): 12x higher training throughput" (CoreWeave)
 *
 * Two halves:
 *   1. Host planning over integers only ([PTP] integer-planning passage): tree_pack_plan
 *      builds the radix segment tree, packs its leaves into fixed-length rows and emits
 *      the per-row segment/parent table, position ids and a gather map.
 *   2. Device attention: tree_attn_plan turns a segment table (device copy) into tile
 *      lists once per batch ([PTP] mask passage: in a packed row most key blocks hold no key
 *      a query block sees, and they are not visited; [AReaL] "Lazy Block Mask Conversion"),
 *      and tree_attn_fwd runs the masked attention forward on Q/K/V, reusing that plan for
 *      every layer.
 *
 * Conventions.
 *   - Every call returns int32: TREE_OK (0) or a negative TREE_E_* code;
 *     tree_status_str(code) gives a static text.
 *   - Argument errors are detected and returned synchronously, before any launch.
 *   - The library never allocates device memory; the caller owns every device buffer
 *     (inputs, outputs, workspace).  The one exception to "no global mutable state" is
 *     tree_attn_fwd_noalloc's fixed per-device buffer.  The host plan is library-owned until
 *     tree_plan_free.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Device calls
 *     are asynchronous on that stream unless stated otherwise.
 */
#ifndef TREEATTN_H
#define TREEATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    TREE_OK = 0,
    TREE_E_INVAL = -1,        /* bad argument (null pointer, size, shape, unsupported dtype / head_dim) */
    TREE_E_TOOLONG = -2,      /* a sequence is longer than the row capacity */
    TREE_E_LAYOUT = -3,       /* the segment table is not a valid pre-order forest layout */
    TREE_E_NOMEM = -4,        /* host allocation failed */
    TREE_E_HIP = -5,          /* a HIP runtime call or kernel launch failed */
    TREE_E_UNSUPPORTED = -6   /* valid arguments this build has no kernel for (e.g. block sizes) */
};

enum { TREE_DT_BF16 = 1, TREE_DT_F32 = 2 };
enum { TREE_PLACE_BFD = 0, TREE_PLACE_IN_ORDER = 1 };
enum { TREE_SCOPE_GLOBAL = 0, TREE_SCOPE_PER_GROUP = 1 };

/* ------------------------------------------------------------------------------------ *
 * 1. Host planning
 * ------------------------------------------------------------------------------------ */

typedef struct {
    int32_t row_len;       /* row capacity C in tokens, > 0 */
    int32_t min_shared;    /* minimum shared-segment length, >= 1 ([PTP]: 64 by default) */
    int32_t pad_multiple;  /* 0: every row is row_len long; m > 0: rows are the longest row's
                              used length rounded up to a multiple of m */
    int32_t placement;     /* TREE_PLACE_BFD ([PTP] placement listing) or TREE_PLACE_IN_ORDER
                              ([PTP] historical section: fill the current row, move on for good
                              when the next leaf does not fit) */
    int32_t tree_scope;    /* TREE_SCOPE_GLOBAL ([PTP] scope passage: one tree over every
                              sequence, no group boundary) or TREE_SCOPE_PER_GROUP (the
                              comparison that passage draws: one tree per group of group_ids,
                              groups in order of first appearance; nothing is shared across
                              groups).  Packing is the same either way. */
} tree_pack_params;

typedef struct tree_plan tree_plan;   /* opaque, host memory, owned by the library */

/*
 * tree_pack_plan — radix segment build + row packing + row layout ([PTP] tree-building
 * passage and its refinements, scope passage, bin-packing passage and placement listing,
 * integer-planning passage).
 *
 *   tokens       host int32 [seq_offsets[n_seqs]]: all sequences back to back.
 *   seq_offsets  host int64 [n_seqs + 1], non-decreasing, seq_offsets[0] = 0; every
 *                sequence must hold >= 1 token.
 *   trainable    host uint8 [seq_offsets[n_seqs]] or NULL (nothing trainable).  Trainable
 *                tokens and the token right before one are never shared, so each branch
 *                keeps its own copy of the join token ([PTP] off-by-one note).
 *   group_ids    host int32 [n_seqs] or NULL (each sequence its own group): placement
 *                groups, placed by their longest sequence, descending.
 *   p            packing parameters (see tree_pack_params).
 *   out          receives the plan; free with tree_plan_free.
 *
 * The build runs over one global tree of every sequence ([PTP] scope passage).  Segments
 * are numbered in depth-first pre-order; row r is the r-th bin; inside a row segments are
 * ordered by that number, laid out back to back from token 0, parents row-local.
 * Errors: TREE_E_INVAL, TREE_E_TOOLONG (a sequence longer than row_len), TREE_E_NOMEM.
 * On error *out is set to NULL.  The inputs are only read during the call.
 */
int tree_pack_plan(const int32_t *tokens, const int64_t *seq_offsets, int32_t n_seqs,
                   const uint8_t *trainable, const int32_t *group_ids,
                   const tree_pack_params *p, tree_plan **out);

/* Read-only views into a plan; valid until tree_plan_free.  All arrays are host memory. */
typedef struct {
    int32_t n_rows, row_len, n_segs, n_seqs;
    int64_t real_tokens;       /* tokens laid out in rows (sum of used lengths) */
    int64_t unpacked_tokens;   /* sum of sequence lengths; unpacked / real is the
                                  tree_token_ratio of [AReaL] "Monitoring Packing Efficiency" */
    int64_t tree_walk_ns, bin_pack_ns;   /* host time of the two planning phases */
    const int32_t *seg_row_ptr;          /* [n_rows + 1] CSR over segments */
    const int32_t *seg_start, *seg_len;  /* [n_segs] row-local token offset and length */
    const int32_t *seg_parent;           /* [n_segs] row-local parent index, -1 = root */
    const int32_t *seg_pos0;             /* [n_segs] position id of the segment's first token */
    const int32_t *seg_global_id;        /* [n_segs] global pre-order segment number */
    const int32_t *seg_src_seq;          /* [n_segs] a sequence holding the segment's tokens */
    const int32_t *row_used;             /* [n_rows] real tokens per row */
    const int32_t *pos_ids, *tok_seg;    /* [n_rows * row_len]; pads: 0 and -1 */
    const int32_t *gather_seq, *gather_pos;  /* [n_rows * row_len] token source; pads: -1 */
    const int32_t *seq_row, *seq_leaf_seg;   /* [n_seqs] row and row-local leaf segment */
} tree_plan_view;

int  tree_plan_get(const tree_plan *plan, tree_plan_view *out);
void tree_plan_free(tree_plan *plan);

/* ------------------------------------------------------------------------------------ *
 * 2. Device attention
 * ------------------------------------------------------------------------------------ */

/*
 * Attention problem description.  The segment arrays are DEVICE copies of a plan's (or any)
 * segment table: per row, segments in depth-first pre-order, laid out back to back from
 * token 0 with no gaps, parents row-local and earlier in the row; the rest of the row is
 * padding.  Tensors (all contiguous, caller-owned, device):
 *   q    [n_rows, row_len, h_q,  head_dim]  dtype
 *   k, v [n_rows, row_len, h_kv, head_dim]  dtype
 *   o    [n_rows, row_len, h_q,  head_dim]  dtype
 *   lse  [n_rows, h_q, row_len]             float32, natural log
 * Query head h reads key/value head h / (h_q / h_kv) (grouped-query attention).
 */
typedef struct {
    int32_t n_rows, row_len, h_q, h_kv, head_dim, dtype;
    int32_t block_q, block_k;   /* tile sizes of the plan; 0 = the forward kernel's sizes */
    float   scale;              /* softmax scale; 0 = 1/sqrt(head_dim) */
    int32_t n_segs;
    const int32_t *seg_row_ptr; /* device [n_rows + 1] */
    const int32_t *seg_start, *seg_len, *seg_parent;   /* device [n_segs] */
} tree_attn_desc;

/*
 * tree_attn_blocks — the tile sizes tree_attn_fwd runs with for this description
 * (block_q = 256 / the largest power of two <= 8 dividing h_q / h_kv; block_k = 64).
 * A plan made with other (block_q, block_k) is valid for tree_attn_tiles but not for
 * tree_attn_fwd.  Host only.  Errors: TREE_E_INVAL.
 */
int tree_attn_blocks(const tree_attn_desc *d, int32_t *block_q, int32_t *block_k);

/* Bytes of device workspace tree_attn_plan needs for `d` (resolved tile sizes).  Host only. */
int tree_attn_workspace_size(const tree_attn_desc *d, size_t *bytes);

/*
 * tree_attn_plan — tile classification on the device ([PTP] mask passage: a token sees whole
 * ancestor segments and the lower triangle of its own segment, so a (q-tile, k-tile) block
 * is fully visible, partly visible or empty, and empty blocks are skipped).  Validates the
 * table into a device status word, computes for every token the end of its segment's subtree,
 * classifies every (q-tile, k-tile) by its exact visible-pair count, builds the per-q-tile CSR
 * lists and the work list (rows in order, a row's q-tiles longest list first).
 * `ws` must hold tree_attn_workspace_size bytes (256-byte aligned).  Asynchronous.
 * Errors: TREE_E_INVAL (sizes, tiles not dividing row_len), TREE_E_HIP.
 */
int tree_attn_plan(const tree_attn_desc *d, void *ws, void *stream);

/*
 * tree_attn_plan_status — synchronizes `stream`, then returns TREE_OK or TREE_E_LAYOUT if
 * the device found the segment table invalid (tree_attn_fwd then writes nothing).
 */
int tree_attn_plan_status(const tree_attn_desc *d, const void *ws, void *stream);

/* Device pointers into a planned workspace (for tests and tools). */
typedef struct {
    int32_t block_q, block_k, n_qtiles, n_ktiles;   /* per row */
    const uint8_t *class_map;   /* [n_rows * n_qtiles * n_ktiles] 0 skip, 1 full, 2 partial */
    const int32_t *qt_ptr;      /* [n_rows * n_qtiles + 1] CSR offsets, row-major (row, q-tile) */
    const int32_t *kt_idx;      /* [nnz] ascending k-tiles with class != skip */
    const uint8_t *kt_kind;     /* [nnz] their classes */
    const int32_t *kend;        /* [n_rows * row_len] token j is visible to exactly the queries
                                   i with j <= i < kend[j]; pads: kend[j] = j */
    const int32_t *work;        /* [n_rows * n_qtiles] (row, q-tile) items: rows in order, inside
                                   a row most non-skip tiles first */
    const int32_t *status;      /* [1] 0 = table valid */
} tree_tile_view;

int tree_attn_tiles(const tree_attn_desc *d, const void *ws, tree_tile_view *out);

/*
 * tree_attn_fwd — tree-masked attention forward ([PTP] attention-mask passage; [AOM] "How do
 * we implement shared prefix?"): for every real token i and query head h,
 *   O[i,h] = softmax_j(scale * q[i,h] . k[j,g]) v[j,g] over j in anc*(i)
 * (itself, earlier tokens of its segment, every token of its ancestor segments), and
 * LSE[h,i] = log-sum-exp of those scores.  Pads get O = 0 and LSE = -inf; pad Q/K/V
 * contents never reach a result.  `ws` must come from tree_attn_plan with the same `d`.
 * The call hands the plan's (row, q-tile) items out to its workgroups from counters in `ws`
 * (two int32 per KV lane, zeroed by tree_attn_plan) and leaves them at zero when it ends, so
 * the plan is reusable by any number of forwards in stream order; two forwards on one
 * workspace must not overlap (other streams without ordering, other host threads).
 * bf16: bf16 MFMA with fp32 accumulation, head_dim 64 or 128; f32: fp32 MFMA, head_dim 64.
 * Asynchronous.  Errors: TREE_E_INVAL, TREE_E_UNSUPPORTED (plan tiles differ from
 * tree_attn_blocks, f32 with head_dim 128, or row_len > 507648: a workgroup keeps its q-tile's
 * list of row_len/64 k-tiles in LDS), TREE_E_HIP.
 */
int tree_attn_fwd(const tree_attn_desc *d, void *ws, const void *q, const void *k,
                  const void *v, void *o, float *lse, void *stream);

/*
 * tree_attn_fwd_noalloc — for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): tree_attn_plan followed by
 * tree_attn_fwd on the same stream, with the tile plan kept in a fixed buffer of the library
 * instead of a caller workspace.  Same inputs, outputs, layouts and results as that pair (the
 * same kernels); no workspace argument and no device allocation by the call.
 * The buffer is a file-scope device array of TREE_NOALLOC_SCRATCH_BYTES (64 MiB); every GPU
 * the library runs on holds its own copy until the process ends.  All calls on one GPU share
 * that GPU's copy, so calls that overlap on one GPU (other streams, other host threads) race;
 * calls in order on one stream are safe.  An invalid segment table makes the forward write
 * nothing, as with tree_attn_fwd; its status is not reported.
 * Errors: as tree_attn_fwd, plus TREE_E_UNSUPPORTED when tree_attn_workspace_size exceeds
 * TREE_NOALLOC_SCRATCH_BYTES (e.g. a 131,072-token row with 64/8 heads needs 49 MiB and fits;
 * the 507,648-token row does not), and TREE_E_HIP if the buffer's device address cannot be
 * resolved on the current device.
 */
#define TREE_NOALLOC_SCRATCH_BYTES (64u << 20)
int tree_attn_fwd_noalloc(const tree_attn_desc *d, const void *q, const void *k, const void *v,
                          void *o, float *lse, void *stream);

/*
 * Backward of tree_attn_fwd ([PTP]: the packing serves training, so every attention layer is
 * differentiated).  For an upstream gradient dO of O, with P the softmax of the visible
 * scores and D_i = sum_d dO[i,h,d] O[i,h,d]:
 *   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),  dQ = scale dS K,  dK = scale dS^T Q,
 * dK / dV summed over the query heads of each KV head.  Pads get zero gradients; pad contents
 * of q/k/v/o/dO never reach a result.  bf16 only (TREE_E_UNSUPPORTED otherwise); the plan in
 * `ws` must use the forward's tile sizes (tree_attn_blocks).
 *
 * tree_attn_bwd_workspace_size: bytes of the caller-allocated backward workspace `bws`
 *   (256-byte aligned): per-token row terms D and log2-scaled LSE ([R, Hq, T] fp32 each),
 *   the per-group q-tile lists and unit list below, and a pool of at most 512 fp32 partial
 *   slots of dK and dV per KV head (each 2 x 256 x head_dim x 4 bytes; 128 MiB per KV head at
 *   head_dim 128, whatever the batch size and row length): a k-tile group seen by many
 *   q-tiles is split over up to 4 workgroups along its list, so that the long groups of a
 *   shared prefix do not serialize, as long as slots remain (longest groups first); the
 *   partials are added in a fixed order (results do not depend on timing).
 * tree_attn_bwd_plan: from the forward plan in `ws`, build into `bws`, for every group of four
 *   consecutive k-tiles (4p .. 4p+3) of a row, the list of q-tiles that see any of them
 *   (ascending, entry = q_tile * 256 + sum_i class(4p+i) << 2(3-i), classes as in
 *   tree_tile_view, k-tiles past the row's last counting as SKIP), the order of the group work
 *   (longest list first, equal lengths in group order, so the same on every run), the partial
 *   slots of the split groups and the list of (group, slice) units the dK/dV pass launches
 *   one workgroup for.  Once per batch, like tree_attn_plan; asynchronous.
 * tree_attn_bwd_tiles: device pointers (into bws) of those lists, for tests:
 *   kp_ptr[R * ceil(n_ktiles / 4) + 1] CSR over (row, group), kp_list the entries.
 * tree_attn_bwd: q, k, v as given to tree_attn_fwd; o and lse as it returned them; dout in
 *   q's layout; writes dq (q's layout), dk and dv (k's layout), bf16.  Overwrites the row
 *   terms in bws (the lists are kept).  Asynchronous.  Errors: TREE_E_INVAL,
 *   TREE_E_UNSUPPORTED, TREE_E_HIP.
 */
int tree_attn_bwd_workspace_size(const tree_attn_desc *d, size_t *bytes);
int tree_attn_bwd_plan(const tree_attn_desc *d, const void *ws, void *bws, void *stream);
int tree_attn_bwd_tiles(const tree_attn_desc *d, const void *bws, const int32_t **kp_ptr,
                        const int32_t **kp_list);
int tree_attn_bwd(const tree_attn_desc *d, const void *ws, void *bws, const void *q, const void *k,
                  const void *v, const void *o, const float *lse, const void *dout, void *dq,
                  void *dk, void *dv, void *stream);

/*
 * Gated delta rule (GDN) threaded along the token tree ([PTP] GDN passage: a recurrent layer
 * carries a state along each path instead of a mask; a child segment starts from its parent's
 * final state, a root from zero;
 * the conv context is carried across the join).  Per head (head_dim 128, width-4 conv):
 *   y_c(t) = SiLU(sum_j conv_w[c][ch][3 - j] * x_c(pi^j(t)))   c = q, k, v; pi = token parent,
 *            zero input past a root's first token
 *   q^ = y_q / sqrt(|y_q|^2 + 1e-6) / sqrt(128),  k^ = y_k / sqrt(|y_k|^2 + 1e-6),  v^ = y_v
 *   h_t = exp(g_t) (h_pi(t) - beta_t k^_t (k^_t^T h_pi(t))) + beta_t k^_t v^_t^T  (h = 0 at roots)
 *   o_t = h_t^T q^_t
 * Shapes from the descriptor: h_q = h_kv = heads, head_dim 128, dtype bf16 (else
 * TREE_E_INVAL).  The host planner's segment table (host copies) drives the depth levels.
 *
 * tree_gdn_workspace_size: bytes of the caller-allocated GDN workspace (256-byte aligned):
 *   token parents, chunk / segment / level records, conv outputs (3 x [R, T, H, 128] bf16),
 *   per-(chunk, head) WY factors (~56 KiB each) and one 128 x 128 fp32 state per (segment,
 *   head).
 * tree_gdn_plan: validates the host segment table (segments back to back from token 0, a
 *   parent before its children; else TREE_E_LAYOUT), writes the records into gws (synchronous
 *   on `stream`) and fills *info, which tree_gdn_fwd needs.  Once per batch.
 * tree_gdn_fwd: x_q, x_k, x_v DEVICE [R, T, H, 128] bf16 (before the conv); conv_w DEVICE
 *   float32 [3][H * 128][4] (tap 3 = current token); g, beta DEVICE float32 [R, T, H] (log
 *   decay <= 0, beta in [0, 1]); writes o DEVICE [R, T, H, 128] bf16 at real tokens (pads
 *   untouched).  Asynchronous; overwrites everything in gws after the records.
 */
typedef struct {
    int32_t n_chunks, n_segs, n_levels, max_level_segs;
    /* Depth levels 0..31 with few segments (at most the device's CU count / heads): bit l of
     * narrow_levels; narrow_segs = the most segments of such a level.  tree_gdn_fwd splits a
     * head's state over two workgroups on these levels (launch shape only; results do not
     * depend on it). */
    int32_t narrow_segs;
    uint32_t narrow_levels;
    /* Chunks of depth-0 segments.  When depth 0 is narrow and deeper levels exist, tree_gdn_fwd
     * preps only these before the depth-0 scan and preps the others beside it, as many as the
     * scan's chain (lead_chain) leaves time for, then the rest (launch order only; results do
     * not depend on it). */
    int32_t lead_chunks;
    int32_t lead_chain;   /* the most chunks of one depth-0 segment (its scan's chain length) */
    int32_t lead_segs;    /* depth-0 segments */
} tree_gdn_info;
int tree_gdn_workspace_size(const tree_attn_desc *d, const int32_t *h_seg_row_ptr, const int32_t *h_seg_len,
                            size_t *bytes);
int tree_gdn_plan(const tree_attn_desc *d, const int32_t *h_seg_row_ptr, const int32_t *h_seg_start,
                  const int32_t *h_seg_len, const int32_t *h_seg_parent, void *gws, tree_gdn_info *info,
                  void *stream);
int tree_gdn_fwd(const tree_attn_desc *d, const tree_gdn_info *info, void *gws, const void *x_q,
                 const void *x_k, const void *x_v, const float *conv_w, const float *g, const float *beta,
                 void *o, void *stream);

/*
 * tree_rope — rotary position embedding at tree positions, in place on q and/or k.
 * [PTP]: a packed row must reproduce every unpacked sequence exactly, so a token is rotated
 * at its position in its own sequence (the plan's pos_ids: the segment's pos0 plus the offset
 * in the segment), not at its row offset; with these positions the tree-masked attention of
 * each root-to-leaf path equals rotary causal attention over that path unpacked.
 *
 *   d        shapes and dtype (n_rows, row_len, h_q, h_kv, head_dim, dtype); the segment
 *            arrays are not used.
 *   pos_ids  DEVICE int32 [n_rows * row_len] (tree_plan_view.pos_ids uploaded; pads 0).
 *   theta    rotary base (> 1, e.g. 10000).  Pair i < D/2 (elements i and i + D/2, the
 *            rotate-half pairing) turns by pos * theta^(-2i/D); angles are computed in fp64.
 *   inverse  0: rotate by +angle; 1: by -angle (the backward of the rotation, for dq / dk).
 *   q, k     DEVICE [n_rows, row_len, h_q | h_kv, head_dim] in dtype, rotated in place;
 *            either may be NULL.  Asynchronous on `stream`.
 * Errors: TREE_E_INVAL (shape, theta, inverse, null pos_ids or both q and k null),
 * TREE_E_HIP.
 */
int tree_rope(const tree_attn_desc *d, const int32_t *pos_ids, float theta, int32_t inverse, void *q,
              void *k, void *stream);

const char *tree_status_str(int code);

#ifdef __cplusplus
}
#endif
#endif /* TREEATTN_H */
