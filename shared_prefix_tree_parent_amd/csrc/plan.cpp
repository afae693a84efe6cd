// Host planner: radix segment build, tree-aware row packing and row layout.
//
// Integers only ("Prefix tree packing", furtherai.github.io, integer-planning passage):
// nothing here touches a tensor.  The method, by passage of that page:
//   * tree-building passage: the longest common run of the sequences still in play becomes one
//     segment; the remainder is partitioned by the following token and each part recursed on;
//   * refinements: minimum shared-segment length; trainable tokens are never shared;
//     each branch keeps its own copy of the non-trainable join token;
//   * scope passage: one global tree over every sequence of the batch;
//   * bin-packing passage and placement listing: a leaf's cost in a row is the length of
//     its path segments the row does not hold yet; best fit (strict <, rows in creation
//     order); groups placed by their most expensive leaf, descending;
//   * historical section: the older in-order filler (optional placement);
//   * the per-group trees the scope passage compares against (optional tree scope).
// Readings of open points (same as the design notes): a short common run is pushed down
// into the parts it splits into and rebuilt from the same start; singleton parts (next
// token not shareable) follow the token-keyed parts in input order; a sequence longer than
// the row is an error; inside a row segments are ordered by pre-order number.
#include <algorithm>
#include <chrono>
#include <cstdint>
#include <climits>
#include <cstring>
#include <memory>
#include <new>
#include <utility>
#include <vector>

#include "treeattn.h"

struct tree_plan {
    int32_t n_rows = 0, row_len = 0, n_segs = 0, n_seqs = 0;
    int64_t real_tokens = 0, unpacked_tokens = 0, tree_walk_ns = 0, bin_pack_ns = 0;
    std::vector<int32_t> seg_row_ptr, seg_start, seg_len, seg_parent, seg_pos0, seg_global_id,
        seg_src_seq, row_used, pos_ids, tok_seg, gather_seq, gather_pos, seq_row, seq_leaf_seg;
};

namespace {

struct Input {
    const int32_t *tok;
    const int64_t *off;
    const uint8_t *tr;
    int32_t n;
    int64_t len(int32_t s) const { return off[s + 1] - off[s]; }
    int32_t at(int32_t s, int64_t t) const { return tok[off[s] + t]; }
    bool trainable(int32_t s, int64_t t) const { return tr != nullptr && tr[off[s] + t] != 0; }
    // A position may be shared iff it exists, is not trainable and is not the context token
    // right before a trainable one (that token is the branch's own join token).
    bool shareable(int32_t s, int64_t t) const {
        const int64_t n = len(s);
        if (t >= n || trainable(s, t)) return false;
        if (t + 1 < n && trainable(s, t + 1)) return false;
        return true;
    }
};

struct Seg {
    int64_t start, end;
    int32_t parent;
    int32_t rep;   // first member in input order
};

struct Tree {
    std::vector<Seg> segs;
    std::vector<int32_t> leaf_of;
};

// One pending build(members, start, parent) call of the recursive definition.  An explicit
// stack replaces the recursion; parts are pushed in reverse key order so they are built,
// and their segments numbered, in exactly the recursive depth-first order.
struct Work {
    std::vector<int32_t> members;
    int64_t start;
    int32_t parent;
};

// `scopes`: the member lists of the independent trees (one list for the global tree), built
// one after the other, so segment ids are pre-order within each tree and trees follow in
// list order.
void build_tree(const Input &in, int32_t min_shared, const std::vector<std::vector<int32_t>> &scopes,
                Tree &tree) {
    tree.segs.clear();
    tree.leaf_of.assign(in.n, -1);
    std::vector<Work> stack;
    for (size_t i = scopes.size(); i-- > 0;) {
        Work w;
        w.members = scopes[i];
        w.start = 0;
        w.parent = -1;
        stack.push_back(std::move(w));
    }
    auto emit = [&](const std::vector<int32_t> &m, int64_t a, int64_t b, int32_t parent) {
        const int32_t id = static_cast<int32_t>(tree.segs.size());
        tree.segs.push_back(Seg{a, b, parent, m[0]});
        for (int32_t s : m) tree.leaf_of[s] = id;
        return id;
    };
    // (key class, key value, member): class 0 = shareable next token keyed by its value,
    // class 1 = member on its own keyed by its index.
    std::vector<std::pair<std::pair<int32_t, int64_t>, int32_t>> keyed;
    while (!stack.empty()) {
        Work w = std::move(stack.back());
        stack.pop_back();
        const int64_t start = w.start;
        std::vector<int32_t> act;
        act.reserve(w.members.size());
        for (int32_t s : w.members)
            if (in.len(s) > start) act.push_back(s);
        if (act.empty()) continue;
        if (act.size() == 1) {
            emit(act, start, in.len(act[0]), w.parent);
            continue;
        }
        int64_t end = start;
        for (;;) {
            bool ok = true;
            const int32_t s0 = act[0];
            if (!in.shareable(s0, end)) break;
            const int32_t x = in.at(s0, end);
            for (size_t i = 1; i < act.size() && ok; ++i) {
                const int32_t s = act[i];
                ok = in.shareable(s, end) && in.at(s, end) == x;
            }
            if (!ok) break;
            ++end;
        }
        if (end - start >= min_shared) {
            const int32_t id = emit(act, start, end, w.parent);
            Work next;
            next.members = std::move(act);
            next.start = end;
            next.parent = id;
            stack.push_back(std::move(next));
            continue;
        }
        // Too short to share: split where the members diverge, rebuild each part from start.
        keyed.clear();
        for (int32_t s : act) {
            if (in.shareable(s, end))
                keyed.push_back({{0, static_cast<int64_t>(in.at(s, end))}, s});
            else
                keyed.push_back({{1, static_cast<int64_t>(s)}, s});
        }
        std::stable_sort(keyed.begin(), keyed.end(),
                         [](const auto &a, const auto &b) { return a.first < b.first; });
        std::vector<std::vector<int32_t>> parts;
        for (size_t i = 0; i < keyed.size(); ++i) {
            if (i == 0 || keyed[i].first != keyed[i - 1].first) parts.emplace_back();
            parts.back().push_back(keyed[i].second);
        }
        for (size_t i = parts.size(); i-- > 0;) {
            Work p;
            p.members = std::move(parts[i]);
            p.start = start;
            p.parent = w.parent;
            stack.push_back(std::move(p));
        }
    }
}

struct Bin {
    std::vector<uint64_t> occ;   // bitset over global segment ids
    int64_t token_count = 0;
    bool has(int32_t id) const { return (occ[id >> 6] >> (id & 63)) & 1u; }
};

// Path of a sequence, root first: (segment id, length).
using Path = std::vector<std::pair<int32_t, int64_t>>;

int64_t insertion_delta(const Bin &b, const Path &p) {
    int64_t d = 0;
    for (const auto &e : p)
        if (!b.has(e.first)) d += e.second;
    return d;
}

void add_leaf(Bin &b, const Path &p) {
    b.token_count += insertion_delta(b, p);
    for (const auto &e : p) b.occ[e.first >> 6] |= (uint64_t(1) << (e.first & 63));
}

int fail(tree_plan **out, int code) {
    if (out) *out = nullptr;
    return code;
}

}  // namespace

extern "C" int tree_pack_plan(const int32_t *tokens, const int64_t *seq_offsets, int32_t n_seqs,
                              const uint8_t *trainable, const int32_t *group_ids,
                              const tree_pack_params *p, tree_plan **out) {
    if (out == nullptr) return TREE_E_INVAL;
    *out = nullptr;
    if (p == nullptr || n_seqs < 0 || p->row_len <= 0 || p->min_shared < 1 || p->pad_multiple < 0 ||
        (p->placement != TREE_PLACE_BFD && p->placement != TREE_PLACE_IN_ORDER) ||
        (p->tree_scope != TREE_SCOPE_GLOBAL && p->tree_scope != TREE_SCOPE_PER_GROUP))
        return TREE_E_INVAL;
    if (n_seqs > 0 && (seq_offsets == nullptr || tokens == nullptr)) return TREE_E_INVAL;
    if (n_seqs > 0 && seq_offsets[0] != 0) return TREE_E_INVAL;
    for (int32_t s = 0; s < n_seqs; ++s) {
        const int64_t n = seq_offsets[s + 1] - seq_offsets[s];
        if (n <= 0) return TREE_E_INVAL;
    }
    for (int32_t s = 0; s < n_seqs; ++s)
        if (seq_offsets[s + 1] - seq_offsets[s] > p->row_len) return fail(out, TREE_E_TOOLONG);
    try {
        using clk = std::chrono::steady_clock;
        tree_plan *plan = new tree_plan();
        std::unique_ptr<tree_plan> guard(plan);
        Input in{tokens, seq_offsets, trainable, n_seqs};
        plan->n_seqs = n_seqs;

        // Groups: the caller's ids (else one per sequence), in order of first appearance,
        // members in input order.  They order the placement, and with the per-group scope
        // each is its own tree.
        std::vector<int32_t> gid(n_seqs);
        for (int32_t s = 0; s < n_seqs; ++s) gid[s] = group_ids ? group_ids[s] : s;
        std::vector<std::vector<int32_t>> members;
        {
            std::vector<std::pair<int32_t, int32_t>> idx;   // (group key, slot), sorted by key
            for (int32_t s = 0; s < n_seqs; ++s) {
                auto it = std::lower_bound(idx.begin(), idx.end(), std::make_pair(gid[s], INT32_MIN));
                if (it == idx.end() || it->first != gid[s]) {
                    const int32_t slot = static_cast<int32_t>(members.size());
                    idx.insert(it, {gid[s], slot});
                    members.emplace_back();
                    members[slot].push_back(s);
                } else {
                    members[it->second].push_back(s);
                }
            }
        }

        const auto t0 = clk::now();
        Tree tree;
        if (p->tree_scope == TREE_SCOPE_PER_GROUP) {
            build_tree(in, p->min_shared, members, tree);
        } else {
            std::vector<std::vector<int32_t>> all(1);
            all[0].resize(n_seqs);
            for (int32_t s = 0; s < n_seqs; ++s) all[0][s] = s;
            if (n_seqs == 0) all.clear();
            build_tree(in, p->min_shared, all, tree);
        }
        const int32_t n_segs_total = static_cast<int32_t>(tree.segs.size());
        std::vector<Path> paths(n_seqs);
        std::vector<int64_t> cost(n_seqs, 0);
        for (int32_t s = 0; s < n_seqs; ++s) {
            for (int32_t id = tree.leaf_of[s]; id >= 0; id = tree.segs[id].parent)
                paths[s].push_back({id, tree.segs[id].end - tree.segs[id].start});
            std::reverse(paths[s].begin(), paths[s].end());
            for (const auto &e : paths[s]) cost[s] += e.second;
            if (cost[s] != in.len(s)) return TREE_E_INVAL;   // cannot happen: path covers the sequence
        }
        const auto t1 = clk::now();

        // Placement order: groups by first appearance, stably sorted by their most
        // expensive leaf, descending; leaves of a group in input order.
        std::vector<int32_t> order;
        order.reserve(n_seqs);
        if (p->placement == TREE_PLACE_BFD) {
            std::vector<int64_t> gmax(members.size(), 0);
            std::vector<int32_t> slots(members.size());
            for (size_t g = 0; g < members.size(); ++g) {
                slots[g] = static_cast<int32_t>(g);
                for (int32_t s : members[g]) gmax[g] = std::max(gmax[g], cost[s]);
            }
            std::stable_sort(slots.begin(), slots.end(),
                             [&](int32_t a, int32_t b) { return gmax[a] > gmax[b]; });
            for (int32_t g : slots)
                for (int32_t s : members[g]) order.push_back(s);
        } else {
            for (int32_t s = 0; s < n_seqs; ++s) order.push_back(s);
        }

        const int64_t C = p->row_len;
        const size_t words = (static_cast<size_t>(n_segs_total) + 63) / 64;
        std::vector<Bin> bins;
        std::vector<std::vector<int32_t>> bin_leaves;
        std::vector<int32_t> seq_bin(n_seqs, -1);
        for (int32_t s : order) {
            int32_t best = -1;
            if (p->placement == TREE_PLACE_BFD) {
                int64_t best_rem = C + 1;
                for (size_t b = 0; b < bins.size(); ++b) {
                    const int64_t count = bins[b].token_count + insertion_delta(bins[b], paths[s]);
                    if (count <= C && C - count < best_rem) {
                        best = static_cast<int32_t>(b);
                        best_rem = C - count;
                    }
                }
            } else if (!bins.empty() &&
                       bins.back().token_count + insertion_delta(bins.back(), paths[s]) <= C) {
                best = static_cast<int32_t>(bins.size()) - 1;
            }
            if (best < 0) {
                bins.emplace_back();
                bins.back().occ.assign(words, 0);
                bin_leaves.emplace_back();
                best = static_cast<int32_t>(bins.size()) - 1;
            }
            add_leaf(bins[best], paths[s]);
            bin_leaves[best].push_back(s);
            seq_bin[s] = best;
        }
        const auto t2 = clk::now();

        // Row layout.
        const int32_t R = static_cast<int32_t>(bins.size());
        int64_t max_used = 0;
        for (const Bin &b : bins) max_used = std::max(max_used, b.token_count);
        int64_t T = C;
        if (p->pad_multiple > 0) T = (max_used + p->pad_multiple - 1) / p->pad_multiple * p->pad_multiple;
        if (static_cast<int64_t>(R) * T > INT32_MAX) return TREE_E_INVAL;
        plan->n_rows = R;
        plan->row_len = static_cast<int32_t>(T);
        plan->seg_row_ptr.assign(1, 0);
        const size_t RT = static_cast<size_t>(R) * static_cast<size_t>(T);
        plan->pos_ids.assign(RT, 0);
        plan->tok_seg.assign(RT, -1);
        plan->gather_seq.assign(RT, -1);
        plan->gather_pos.assign(RT, -1);
        plan->seq_row.assign(n_seqs, -1);
        plan->seq_leaf_seg.assign(n_seqs, -1);
        plan->row_used.assign(R, 0);
        std::vector<int32_t> local(n_segs_total, -1);
        for (int32_t r = 0; r < R; ++r) {
            const Bin &b = bins[r];
            std::vector<int32_t> ids;
            for (size_t w = 0; w < words; ++w) {
                uint64_t m = b.occ[w];
                while (m) {
                    const int bit = __builtin_ctzll(m);
                    ids.push_back(static_cast<int32_t>(w * 64 + bit));
                    m &= m - 1;
                }
            }
            for (size_t i = 0; i < ids.size(); ++i) local[ids[i]] = static_cast<int32_t>(i);
            int64_t off = 0;
            for (size_t i = 0; i < ids.size(); ++i) {
                const Seg &sg = tree.segs[ids[i]];
                const int64_t n = sg.end - sg.start;
                plan->seg_start.push_back(static_cast<int32_t>(off));
                plan->seg_len.push_back(static_cast<int32_t>(n));
                plan->seg_parent.push_back(sg.parent >= 0 ? local[sg.parent] : -1);
                plan->seg_pos0.push_back(static_cast<int32_t>(sg.start));
                plan->seg_global_id.push_back(ids[i]);
                plan->seg_src_seq.push_back(sg.rep);
                const size_t base = static_cast<size_t>(r) * T;
                for (int64_t t = 0; t < n; ++t) {
                    plan->pos_ids[base + off + t] = static_cast<int32_t>(sg.start + t);
                    plan->tok_seg[base + off + t] = static_cast<int32_t>(i);
                    plan->gather_seq[base + off + t] = sg.rep;
                    plan->gather_pos[base + off + t] = static_cast<int32_t>(sg.start + t);
                }
                off += n;
            }
            plan->row_used[r] = static_cast<int32_t>(off);
            plan->real_tokens += off;
            plan->seg_row_ptr.push_back(static_cast<int32_t>(plan->seg_start.size()));
            for (int32_t s : bin_leaves[r]) {
                plan->seq_row[s] = r;
                plan->seq_leaf_seg[s] = local[tree.leaf_of[s]];
            }
            for (int32_t id : ids) local[id] = -1;
        }
        plan->n_segs = static_cast<int32_t>(plan->seg_start.size());
        for (int32_t s = 0; s < n_seqs; ++s) plan->unpacked_tokens += in.len(s);
        plan->tree_walk_ns = std::chrono::duration_cast<std::chrono::nanoseconds>(t1 - t0).count();
        plan->bin_pack_ns = std::chrono::duration_cast<std::chrono::nanoseconds>(t2 - t1).count();
        *out = guard.release();
        return TREE_OK;
    } catch (const std::bad_alloc &) {
        return fail(out, TREE_E_NOMEM);
    } catch (...) {
        return fail(out, TREE_E_INVAL);
    }
}

extern "C" int tree_plan_get(const tree_plan *plan, tree_plan_view *v) {
    if (plan == nullptr || v == nullptr) return TREE_E_INVAL;
    std::memset(v, 0, sizeof(*v));
    v->n_rows = plan->n_rows;
    v->row_len = plan->row_len;
    v->n_segs = plan->n_segs;
    v->n_seqs = plan->n_seqs;
    v->real_tokens = plan->real_tokens;
    v->unpacked_tokens = plan->unpacked_tokens;
    v->tree_walk_ns = plan->tree_walk_ns;
    v->bin_pack_ns = plan->bin_pack_ns;
    v->seg_row_ptr = plan->seg_row_ptr.data();
    v->seg_start = plan->seg_start.data();
    v->seg_len = plan->seg_len.data();
    v->seg_parent = plan->seg_parent.data();
    v->seg_pos0 = plan->seg_pos0.data();
    v->seg_global_id = plan->seg_global_id.data();
    v->seg_src_seq = plan->seg_src_seq.data();
    v->row_used = plan->row_used.data();
    v->pos_ids = plan->pos_ids.data();
    v->tok_seg = plan->tok_seg.data();
    v->gather_seq = plan->gather_seq.data();
    v->gather_pos = plan->gather_pos.data();
    v->seq_row = plan->seq_row.data();
    v->seq_leaf_seg = plan->seq_leaf_seg.data();
    return TREE_OK;
}

extern "C" void tree_plan_free(tree_plan *plan) { delete plan; }
