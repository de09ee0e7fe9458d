// Host-side integer work: the trie builder, the DFS layout and argument checks.
//
// Everything here is plain C++ on integers (no device calls): [ART "Metadata
// space first"] keeps the whole packing plan in integer indices and lengths
// and touches real tensors only afterwards.
#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <vector>

#include "common.h"

namespace {
thread_local char g_last_error[512] = "";
}

namespace treeattn {

tree_status fail(tree_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return s;
}

void clear_error() { g_last_error[0] = '\0'; }

}  // namespace treeattn

using treeattn::fail;

extern "C" int tree_abi_version(void) { return 5; }

extern "C" const char* tree_status_string(int s) {
    switch (s) {
        case TREE_OK: return "TREE_OK";
        case TREE_ERR_INVALID_ARG: return "TREE_ERR_INVALID_ARG";
        case TREE_ERR_BAD_TREE: return "TREE_ERR_BAD_TREE";
        case TREE_ERR_CAPACITY: return "TREE_ERR_CAPACITY";
        case TREE_ERR_UNSUPPORTED: return "TREE_ERR_UNSUPPORTED";
        case TREE_ERR_DEVICE: return "TREE_ERR_DEVICE";
        default: return "TREE_ERR_UNKNOWN";
    }
}

extern "C" const char* tree_last_error(void) { return g_last_error; }

// ---------------------------------------------------------------------------
// tree_build_trie
// ---------------------------------------------------------------------------
//
// [ART "The tree"] as an explicit work stack instead of recursion.  A work
// item is (active sequences, start, parent node).  Sub-branches are pushed in
// reverse so the first branch is finished before the second starts, which
// keeps the emission order a depth-first pre-order.

namespace {

struct TrieBuilder {
    const int64_t* off;
    const int32_t* tok;
    const uint8_t* train;  // per token, nonzero = trainable; NULL = no trainable tokens (default mode)
    int32_t min_shared;
    std::vector<int32_t> parent;
    std::vector<int32_t> seq_last;
    const int32_t* ids = nullptr;  // sequence s of this trie is input sequence ids[s] (NULL: s itself)

    int64_t first(int32_t s) const { return off[ids ? ids[s] : s]; }
    int64_t len(int32_t s) const { return off[(ids ? ids[s] : s) + 1] - first(s); }
    int32_t at(int32_t s, int64_t t) const { return tok[first(s) + t]; }
    bool trained(int32_t s, int64_t t) const { return train && train[first(s) + t]; }

    // One node per position in [start, end), shared by every sequence in `act`.
    int32_t emit(const std::vector<int32_t>& act, int64_t start, int64_t end, int32_t par) {
        if (end <= start) return par;
        int32_t last = par;
        for (int64_t t = start; t < end; ++t) {
            int32_t id = (int32_t)parent.size();
            parent.push_back(last);
            last = id;
        }
        for (int32_t s : act)
            if (len(s) == end) seq_last[s] = last;
        return last;
    }

    // Split by the token at `pos`: sequences that end at `pos` first, then
    // ascending token, keeping input order inside a branch.  A sequence whose
    // token at `pos` is trainable is a branch of its own, after the shared
    // branch of the same token.
    void split(std::vector<int32_t>& act, int64_t pos, std::vector<std::vector<int32_t>>& parts) const {
        std::stable_sort(act.begin(), act.end(), [&](int32_t a, int32_t b) {
            bool ea = len(a) == pos, eb = len(b) == pos;
            if (ea != eb) return ea;
            if (ea) return false;
            return at(a, pos) < at(b, pos);
        });
        parts.clear();
        size_t i = 0;
        while (i < act.size()) {
            size_t j = i + 1;
            bool ended = len(act[i]) == pos;
            while (j < act.size()) {
                bool ej = len(act[j]) == pos;
                if (ej != ended) break;
                if (!ended && at(act[j], pos) != at(act[i], pos)) break;
                ++j;
            }
            if (ended || !train) {
                parts.emplace_back(act.begin() + i, act.begin() + j);
            } else {
                std::vector<int32_t> shared;
                for (size_t x = i; x < j; ++x)
                    if (!trained(act[x], pos)) shared.push_back(act[x]);
                if (!shared.empty()) parts.push_back(std::move(shared));
                for (size_t x = i; x < j; ++x)
                    if (trained(act[x], pos)) parts.push_back({act[x]});
            }
            i = j;
        }
    }

    struct Item {
        std::vector<int32_t> act;
        int64_t start;
        int32_t par;
    };

    void run(int32_t n_seqs) {
        std::vector<Item> stack;
        std::vector<int32_t> all(n_seqs);
        for (int32_t s = 0; s < n_seqs; ++s) all[s] = s;
        stack.push_back({std::move(all), 0, -1});
        std::vector<std::vector<int32_t>> parts;
        auto push_parts = [&](int64_t start, int32_t par) {
            for (size_t p = parts.size(); p-- > 0;) stack.push_back({std::move(parts[p]), start, par});
        };
        while (!stack.empty()) {
            Item it = std::move(stack.back());
            stack.pop_back();
            std::vector<int32_t> act;
            act.reserve(it.act.size());
            for (int32_t s : it.act)
                if (len(s) > it.start) act.push_back(s);
            if (act.empty()) continue;
            const int64_t start = it.start;
            if (act.size() == 1) {  // a private leaf
                emit(act, start, len(act[0]), it.par);
                continue;
            }
            int64_t m = len(act[0]);
            for (int32_t s : act) m = std::min(m, len(s));
            int64_t end = start;  // the shared run: equal tokens, none of them trainable
            while (end < m) {
                int32_t t0 = at(act[0], end);
                bool same = !trained(act[0], end);
                for (size_t i = 1; i < act.size() && same; ++i) same = at(act[i], end) == t0 && !trained(act[i], end);
                if (!same) break;
                ++end;
            }
            if (end == start) {  // nothing shared: split by next token
                split(act, start, parts);
                push_parts(start, it.par);
                continue;
            }
            bool all_end = true;
            for (int32_t s : act) all_end = all_end && len(s) == end;
            if (all_end) {  // identical remainders
                emit(act, start, end, it.par);
                continue;
            }
            if (end - start >= min_shared && !train) {  // share the run minus the join token
                int32_t node = emit(act, start, end - 1, it.par);
                split(act, end, parts);
                push_parts(end - 1, node);
            } else if (end - start >= min_shared) {
                // trainable mode: branches whose next token is trainable get a
                // copy of the join token; the others (and sequences ending
                // here) hang off the shared join token
                split(act, end, parts);
                std::vector<char> copy(parts.size());
                bool any = false;
                for (size_t p = 0; p < parts.size(); ++p) {
                    copy[p] = len(parts[p][0]) > end && trained(parts[p][0], end);
                    any = any || copy[p];
                }
                if (!any) {
                    int32_t node = emit(act, start, end, it.par);
                    push_parts(end, node);
                    continue;
                }
                int32_t node = emit(act, start, end - 1, it.par);
                std::vector<int32_t> stay;
                for (size_t p = 0; p < parts.size(); ++p)
                    if (!copy[p]) stay.insert(stay.end(), parts[p].begin(), parts[p].end());
                const int32_t join = stay.empty() ? -1 : emit(stay, end - 1, end, node);
                for (size_t p = parts.size(); p-- > 0;)
                    stack.push_back({std::move(parts[p]), copy[p] ? end - 1 : end, copy[p] ? node : join});
            } else {  // too short: copy it into every branch
                split(act, end, parts);
                push_parts(start, it.par);
            }
        }
    }
};

}  // namespace

extern "C" tree_status tree_build_trie(int32_t n_seqs, const int64_t* seq_offsets,
                                       const int32_t* tokens, const uint8_t* trainable, int32_t min_shared,
                                       int32_t* parent, int64_t parent_cap, int64_t* n_nodes,
                                       int32_t* seq_last) {
    treeattn::clear_error();
    if (n_seqs < 0) return fail(TREE_ERR_INVALID_ARG, "n_seqs = %d < 0", n_seqs);
    if (!n_nodes) return fail(TREE_ERR_INVALID_ARG, "n_nodes is NULL");
    if (min_shared < 1) return fail(TREE_ERR_INVALID_ARG, "min_shared = %d < 1", min_shared);
    if (n_seqs > 0 && !seq_offsets) return fail(TREE_ERR_INVALID_ARG, "seq_offsets is NULL");
    if (n_seqs > 0 && seq_offsets[0] != 0) return fail(TREE_ERR_INVALID_ARG, "seq_offsets[0] != 0");
    for (int32_t s = 0; s < n_seqs; ++s)
        if (seq_offsets[s + 1] < seq_offsets[s])
            return fail(TREE_ERR_INVALID_ARG, "seq_offsets decreases at %d", s);
    int64_t total = n_seqs > 0 ? seq_offsets[n_seqs] : 0;
    if (total > 0 && !tokens) return fail(TREE_ERR_INVALID_ARG, "tokens is NULL");
    if (total > INT32_MAX) return fail(TREE_ERR_UNSUPPORTED, "more than 2^31-1 tokens");
    if (parent && parent_cap < 0) return fail(TREE_ERR_INVALID_ARG, "parent_cap < 0");

    TrieBuilder tb{seq_offsets, tokens, trainable, min_shared, {}, {}};
    tb.parent.reserve((size_t)total);
    tb.seq_last.assign((size_t)n_seqs, -1);
    if (n_seqs > 0) tb.run(n_seqs);
    *n_nodes = (int64_t)tb.parent.size();
    if (seq_last && n_seqs > 0) std::memcpy(seq_last, tb.seq_last.data(), sizeof(int32_t) * n_seqs);
    if (!parent) return TREE_OK;
    if ((int64_t)tb.parent.size() > parent_cap)
        return fail(TREE_ERR_CAPACITY, "parent_cap %lld < %lld nodes", (long long)parent_cap,
                    (long long)tb.parent.size());
    if (!tb.parent.empty()) std::memcpy(parent, tb.parent.data(), sizeof(int32_t) * tb.parent.size());
    return TREE_OK;
}

// ---------------------------------------------------------------------------
// tree_plan_rows
// ---------------------------------------------------------------------------

extern "C" tree_status tree_plan_rows(int32_t n_seqs, const int64_t* seq_offsets, const int32_t* tokens,
                                      int32_t fork_threshold_tokens, int64_t token_budget, int32_t* row_of_seq,
                                      int64_t* row_tokens, int32_t rows_cap, int32_t* n_rows, uint8_t* forked) {
    treeattn::clear_error();
    if (n_seqs < 0) return fail(TREE_ERR_INVALID_ARG, "n_seqs = %d < 0", n_seqs);
    if (!n_rows) return fail(TREE_ERR_INVALID_ARG, "n_rows is NULL");
    if (fork_threshold_tokens < 0) return fail(TREE_ERR_INVALID_ARG, "fork_threshold_tokens = %d < 0",
                                               fork_threshold_tokens);
    if (token_budget < 1) return fail(TREE_ERR_INVALID_ARG, "token_budget = %lld < 1", (long long)token_budget);
    if (rows_cap < 0) return fail(TREE_ERR_INVALID_ARG, "rows_cap < 0");
    if (n_seqs > 0 && (!seq_offsets || !row_of_seq))
        return fail(TREE_ERR_INVALID_ARG, "seq_offsets or row_of_seq is NULL");
    if (n_seqs > 0 && seq_offsets[0] != 0) return fail(TREE_ERR_INVALID_ARG, "seq_offsets[0] != 0");
    for (int32_t s = 0; s < n_seqs; ++s)
        if (seq_offsets[s + 1] < seq_offsets[s])
            return fail(TREE_ERR_INVALID_ARG, "seq_offsets decreases at %d", s);
    const int64_t total = n_seqs > 0 ? seq_offsets[n_seqs] : 0;
    if (total > 0 && !tokens) return fail(TREE_ERR_INVALID_ARG, "tokens is NULL");
    if (total > INT32_MAX) return fail(TREE_ERR_UNSUPPORTED, "more than 2^31-1 tokens");
    for (int32_t s = 0; s < n_seqs; ++s)
        if (seq_offsets[s + 1] - seq_offsets[s] > token_budget)
            return fail(TREE_ERR_CAPACITY, "sample %d has %lld tokens, more than token_budget %lld", s,
                        (long long)(seq_offsets[s + 1] - seq_offsets[s]), (long long)token_budget);

    // Forwarded tokens of the trie over `members` (node count), and, when
    // wanted, which members share a node with another member.
    const int32_t thr = std::max<int32_t>(1, fork_threshold_tokens);
    auto trie_of = [&](const std::vector<int32_t>& members, std::vector<uint8_t>* shares) -> int64_t {
        TrieBuilder tb{seq_offsets, tokens, nullptr, thr, {}, {}};
        tb.ids = members.data();
        tb.seq_last.assign(members.size(), -1);
        tb.run((int32_t)members.size());
        if (shares) {
            std::vector<int32_t> users(tb.parent.size(), 0);
            for (int32_t v : tb.seq_last)
                for (int32_t x = v; x >= 0; x = tb.parent[x]) ++users[x];
            shares->assign(members.size(), 0);
            for (size_t i = 0; i < members.size(); ++i)
                for (int32_t x = tb.seq_last[i]; x >= 0; x = tb.parent[x])
                    if (users[x] > 1) {
                        (*shares)[i] = 1;
                        break;
                    }
        }
        return (int64_t)tb.parent.size();
    };

    int32_t rows = 0;
    std::vector<int32_t> cur;
    int64_t cur_tokens = 0;
    auto close_row = [&]() {
        if (cur.empty()) return;
        if (rows < rows_cap && row_tokens) row_tokens[rows] = cur_tokens;
        if (forked) {
            std::vector<uint8_t> sh;
            trie_of(cur, &sh);
            for (size_t i = 0; i < cur.size(); ++i) forked[cur[i]] = sh[i];
        }
        for (int32_t s : cur) row_of_seq[s] = rows;
        ++rows;
        cur.clear();
    };
    for (int32_t s = 0; s < n_seqs; ++s) {
        cur.push_back(s);
        const int64_t t = trie_of(cur, nullptr);
        if (t <= token_budget) {
            cur_tokens = t;
            continue;
        }
        cur.pop_back();
        close_row();
        cur.push_back(s);
        cur_tokens = seq_offsets[s + 1] - seq_offsets[s];
    }
    close_row();
    *n_rows = rows;
    if (rows > rows_cap && row_tokens)
        return fail(TREE_ERR_CAPACITY, "rows_cap %d < %d rows", rows_cap, rows);
    return TREE_OK;
}

// ---------------------------------------------------------------------------
// tree_pack_layout
// ---------------------------------------------------------------------------

extern "C" tree_status tree_pack_layout(int32_t n_nodes, const int32_t* parent, int32_t n_seqs,
                                        const int32_t* seq_last, int32_t row_len,
                                        int32_t* slot_node, int32_t* pos_ids,
                                        int32_t* subtree_end, int64_t* seq_offsets,
                                        int32_t* token_index, int64_t token_index_cap) {
    treeattn::clear_error();
    if (n_nodes < 0 || n_seqs < 0 || row_len < 0)
        return fail(TREE_ERR_INVALID_ARG, "negative size (n_nodes %d, n_seqs %d, row_len %d)",
                    n_nodes, n_seqs, row_len);
    if (n_nodes > row_len)
        return fail(TREE_ERR_CAPACITY, "row_len %d < n_nodes %d", row_len, n_nodes);
    if ((n_nodes > 0 && !parent) || (n_seqs > 0 && !seq_last) || !seq_offsets ||
        (row_len > 0 && (!slot_node || !pos_ids || !subtree_end)))
        return fail(TREE_ERR_INVALID_ARG, "null pointer argument");
    for (int32_t v = 0; v < n_nodes; ++v)
        if (parent[v] < -1 || parent[v] >= n_nodes || parent[v] == v)
            return fail(TREE_ERR_BAD_TREE, "parent[%d] = %d out of range", v, parent[v]);
    for (int32_t s = 0; s < n_seqs; ++s)
        if (seq_last[s] < -1 || seq_last[s] >= n_nodes)
            return fail(TREE_ERR_BAD_TREE, "seq_last[%d] = %d out of range", s, seq_last[s]);

    // children lists in CSR form; filling in ascending v keeps them sorted
    std::vector<int32_t> cstart((size_t)n_nodes + 1, 0), child((size_t)n_nodes), roots;
    for (int32_t v = 0; v < n_nodes; ++v)
        if (parent[v] >= 0) ++cstart[parent[v] + 1];
    for (int32_t v = 0; v < n_nodes; ++v) cstart[v + 1] += cstart[v];
    {
        std::vector<int32_t> fill(cstart.begin(), cstart.end() - 1);
        for (int32_t v = 0; v < n_nodes; ++v) {
            if (parent[v] >= 0) child[fill[parent[v]]++] = v;
            else roots.push_back(v);
        }
    }
    // iterative pre-order
    std::vector<int32_t> node_slot((size_t)n_nodes, -1), depth((size_t)n_nodes, 0), stack;
    stack.reserve(64);
    for (size_t r = roots.size(); r-- > 0;) stack.push_back(roots[r]);
    int32_t next = 0;
    while (!stack.empty()) {
        int32_t v = stack.back();
        stack.pop_back();
        node_slot[v] = next;
        slot_node[next] = v;
        depth[v] = parent[v] < 0 ? 0 : depth[parent[v]] + 1;
        ++next;
        for (int32_t c = cstart[v + 1]; c-- > cstart[v];) stack.push_back(child[c]);
    }
    if (next != n_nodes)
        return fail(TREE_ERR_BAD_TREE, "parent array has a cycle (%d of %d nodes reachable)", next,
                    n_nodes);
    // subtree sizes, children before parents (reverse pre-order)
    std::vector<int32_t> size((size_t)n_nodes, 1);
    for (int32_t s = n_nodes; s-- > 0;) {
        int32_t v = slot_node[s];
        if (parent[v] >= 0) size[parent[v]] += size[v];
    }
    for (int32_t s = 0; s < n_nodes; ++s) {
        int32_t v = slot_node[s];
        pos_ids[s] = depth[v];
        subtree_end[s] = s + size[v] - 1;
    }
    for (int32_t s = n_nodes; s < row_len; ++s) {
        slot_node[s] = -1;
        pos_ids[s] = 0;
        subtree_end[s] = s;
    }
    seq_offsets[0] = 0;
    for (int32_t s = 0; s < n_seqs; ++s)
        seq_offsets[s + 1] = seq_offsets[s] + (seq_last[s] < 0 ? 0 : depth[seq_last[s]] + 1);
    if (!token_index) return TREE_OK;
    if (token_index_cap < seq_offsets[n_seqs])
        return fail(TREE_ERR_CAPACITY, "token_index_cap %lld < %lld", (long long)token_index_cap,
                    (long long)seq_offsets[n_seqs]);
    for (int32_t s = 0; s < n_seqs; ++s) {
        int64_t p = seq_offsets[s + 1];
        for (int32_t v = seq_last[s]; v >= 0; v = parent[v]) token_index[--p] = node_slot[v];
    }
    return TREE_OK;
}

// ---------------------------------------------------------------------------
// tree_validate_subtree_end
// ---------------------------------------------------------------------------

extern "C" tree_status tree_validate_subtree_end(const int32_t* se, int64_t n) {
    treeattn::clear_error();
    if (n < 0) return fail(TREE_ERR_INVALID_ARG, "n < 0");
    if (n > 0 && !se) return fail(TREE_ERR_INVALID_ARG, "subtree_end is NULL");
    // open intervals on a stack; each new one must close before its enclosing one
    std::vector<int64_t> open;
    for (int64_t j = 0; j < n; ++j) {
        if (se[j] < j || se[j] >= n)
            return fail(TREE_ERR_BAD_TREE, "subtree_end[%lld] = %d outside [%lld, %lld)",
                        (long long)j, se[j], (long long)j, (long long)n);
        while (!open.empty() && open.back() < j) open.pop_back();
        if (!open.empty() && se[j] > open.back())
            return fail(TREE_ERR_BAD_TREE, "interval of slot %lld crosses its enclosing interval",
                        (long long)j);
        open.push_back(se[j]);
    }
    return TREE_OK;
}

// ---------------------------------------------------------------------------
// tree_place_leaves
// ---------------------------------------------------------------------------

extern "C" tree_status tree_place_leaves(int32_t n_nodes, const int32_t* parent, int32_t n_seqs,
                                         const int32_t* seq_last, const int32_t* group, int32_t seq_len,
                                         int32_t mode, int32_t* bin_of_seq, int32_t* bin_tokens,
                                         int32_t bins_cap, int32_t* n_bins) {
    treeattn::clear_error();
    if (n_nodes < 0 || n_seqs < 0) return fail(TREE_ERR_INVALID_ARG, "negative size");
    if (seq_len < 1) return fail(TREE_ERR_INVALID_ARG, "seq_len = %d < 1", seq_len);
    if (mode != TREE_PLACE_GLOBAL && mode != TREE_PLACE_IN_ORDER)
        return fail(TREE_ERR_INVALID_ARG, "unknown placement mode %d", mode);
    if (!n_bins || (n_nodes > 0 && !parent) || (n_seqs > 0 && (!seq_last || !bin_of_seq)) ||
        (mode == TREE_PLACE_GLOBAL && n_seqs > 0 && !group) || (bins_cap > 0 && !bin_tokens))
        return fail(TREE_ERR_INVALID_ARG, "null pointer argument");
    for (int32_t v = 0; v < n_nodes; ++v)
        if (parent[v] < -1 || parent[v] >= v)
            return fail(TREE_ERR_BAD_TREE, "parent[%d] = %d: nodes must follow their parent", v, parent[v]);
    for (int32_t s = 0; s < n_seqs; ++s)
        if (seq_last[s] < -1 || seq_last[s] >= n_nodes)
            return fail(TREE_ERR_BAD_TREE, "seq_last[%d] = %d out of range", s, seq_last[s]);

    // segments: maximal chains; a node starts one at a root, below a fork, or
    // below the last token of a sequence [ART "Bin packing, with a twist"]
    // per node: bit 0-1 child count saturated at 2, bit 2 = last token of a sequence
    std::vector<uint8_t> flag((size_t)n_nodes, 0);
    std::vector<int32_t> seg_of((size_t)n_nodes);
    for (int32_t v = 0; v < n_nodes; ++v)
        if (parent[v] >= 0 && (flag[parent[v]] & 3) < 2) ++flag[parent[v]];
    for (int32_t s = 0; s < n_seqs; ++s)
        if (seq_last[s] >= 0) flag[seq_last[s]] |= 4;
    std::vector<int64_t> seg_len;
    std::vector<int32_t> seg_up;  // segment of the parent of the segment's first node, -1 at a root
    for (int32_t v = 0; v < n_nodes; ++v) {
        const int32_t p = parent[v];
        if (p < 0 || (flag[p] & 3) > 1 || (flag[p] & 4)) {
            seg_of[v] = (int32_t)seg_len.size();
            seg_len.push_back(0);
            seg_up.push_back(p < 0 ? -1 : seg_of[p]);
        } else {
            seg_of[v] = seg_of[p];
        }
        ++seg_len[seg_of[v]];
    }
    // each sequence's segments (root first) and standalone cost
    std::vector<int64_t> poff((size_t)n_seqs + 1, 0), cost((size_t)n_seqs, 0);
    std::vector<int32_t> path;
    for (int32_t s = 0; s < n_seqs; ++s) {
        int32_t d = 0;
        for (int32_t x = seq_last[s] < 0 ? -1 : seg_of[seq_last[s]]; x >= 0; x = seg_up[x]) ++d;
        poff[s + 1] = poff[s] + d;
    }
    path.resize((size_t)poff[n_seqs]);
    for (int32_t s = 0; s < n_seqs; ++s) {
        int64_t p = poff[s + 1];
        for (int32_t x = seq_last[s] < 0 ? -1 : seg_of[seq_last[s]]; x >= 0; x = seg_up[x]) {
            path[--p] = x;
            cost[s] += seg_len[x];
        }
        if (cost[s] > seq_len)
            return fail(TREE_ERR_CAPACITY, "sequence %d needs %lld tokens, more than a row of %d", s,
                        (long long)cost[s], seq_len);
    }

    // rows: tokens held, and for each segment the rows that hold it
    std::vector<int64_t> tokens;
    std::vector<std::vector<int32_t>> rows_of(seg_len.size());
    std::vector<int64_t> shared;  // per row: tokens of the current leaf it already holds
    std::vector<int32_t> touched;
    auto gather = [&](int32_t s) {  // shared[b] for every row b touching leaf s
        for (int32_t b : touched) shared[b] = 0;
        touched.clear();
        for (int64_t i = poff[s]; i < poff[s + 1]; ++i)
            for (int32_t b : rows_of[path[i]]) {
                if (shared[b] == 0) touched.push_back(b);
                shared[b] += seg_len[path[i]];
            }
    };
    auto add = [&](int32_t b, int32_t s) {
        tokens[b] += cost[s] - shared[b];
        for (int64_t i = poff[s]; i < poff[s + 1]; ++i) {
            std::vector<int32_t>& r = rows_of[path[i]];
            if (r.empty() || r.back() != b) {
                if (std::find(r.begin(), r.end(), b) == r.end()) r.push_back(b);
            }
        }
        bin_of_seq[s] = b;
    };
    auto new_row = [&]() {
        tokens.push_back(0);
        shared.push_back(0);
        return (int32_t)tokens.size() - 1;
    };

    if (mode == TREE_PLACE_IN_ORDER) {
        // [ART "Does it actually help?"]: fill one row at a time in arrival
        // order, moving on for good when the next sequence does not fit
        int32_t cur = -1;
        for (int32_t s = 0; s < n_seqs; ++s) {
            gather(s);
            if (cur < 0 || tokens[cur] + cost[s] - shared[cur] > seq_len) {
                cur = new_row();
                gather(s);
            }
            add(cur, s);
        }
    } else {
        // [ART "Bin packing, with a twist"]: groups in decreasing order of their
        // most expensive leaf (stable), leaves in input order; each leaf into
        // the row left with the least free space, a new row if none fits
        std::vector<int32_t> gid;                // distinct group ids, first-appearance order
        std::vector<std::vector<int32_t>> members;
        {
            std::vector<std::pair<int32_t, int32_t>> key((size_t)n_seqs);
            for (int32_t s = 0; s < n_seqs; ++s) key[s] = {group[s], s};
            std::stable_sort(key.begin(), key.end());
            std::vector<std::pair<int32_t, int32_t>> first;  // (first sequence, group index)
            for (size_t i = 0; i < key.size();) {
                size_t j = i;
                members.emplace_back();
                while (j < key.size() && key[j].first == key[i].first) members.back().push_back(key[j++].second);
                first.push_back({members.back()[0], (int32_t)members.size() - 1});
                i = j;
            }
            std::sort(first.begin(), first.end());
            for (auto& f : first) gid.push_back(f.second);
        }
        std::vector<int64_t> gmax(members.size(), 0);
        for (size_t g = 0; g < members.size(); ++g)
            for (int32_t s : members[g]) gmax[g] = std::max(gmax[g], cost[s]);
        std::stable_sort(gid.begin(), gid.end(), [&](int32_t a, int32_t b) { return gmax[a] > gmax[b]; });
        for (int32_t g : gid)
            for (int32_t s : members[g]) {
                gather(s);
                int32_t best = -1;
                int64_t best_free = (int64_t)seq_len + 1;
                for (int32_t b = 0; b < (int32_t)tokens.size(); ++b) {
                    const int64_t c = tokens[b] + cost[s] - shared[b];
                    if (c <= seq_len && seq_len - c < best_free) {
                        best = b;
                        best_free = seq_len - c;
                    }
                }
                if (best < 0) {
                    best = new_row();
                    gather(s);
                }
                add(best, s);
            }
    }
    *n_bins = (int32_t)tokens.size();
    if ((int64_t)tokens.size() > bins_cap)
        return fail(TREE_ERR_CAPACITY, "bins_cap %d < %zu rows", bins_cap, tokens.size());
    for (size_t b = 0; b < tokens.size(); ++b) bin_tokens[b] = (int32_t)tokens[b];
    return TREE_OK;
}

// ---------------------------------------------------------------------------
// tree_gdn_plan
//
// A recurrent layer threads its state along each root-to-leaf path, forks it
// at branch points and starts from zero at roots [ART "Token-mixing layers"].
// In a DFS row the state passes from slot t-1 to slot t exactly when t-1 is
// t's parent and has no other child, so the row splits into maximal runs of
// consecutive slots (chains) that each start from one known state: zero at a
// root, the final state of the chain ending at the parent otherwise.  Chains
// are grouped by depth (number of chains above them): all chains of one depth
// run together once every shallower chain is done, as the pages' planner
// does with one pair of calls per depth.  Each chain is cut into chunks of up
// to 64 slots starting at the chain's first slot.
// ---------------------------------------------------------------------------

extern "C" tree_status tree_gdn_plan(int64_t n, const int32_t* subtree_end, int32_t* parent_slot,
                                     int32_t* segments, int64_t seg_cap, int64_t* n_segments,
                                     int32_t* chunks, int64_t chunk_cap, int64_t* n_chunks,
                                     int32_t* depth_offsets, int64_t depth_cap, int64_t* n_depths,
                                     int64_t* n_states) {
    treeattn::clear_error();
    if (n < 0 || n > INT32_MAX) return fail(TREE_ERR_INVALID_ARG, "n = %lld", (long long)n);
    if (n > 0 && !subtree_end) return fail(TREE_ERR_INVALID_ARG, "subtree_end is NULL");
    if (!n_segments || !n_chunks || !n_depths || !n_states)
        return fail(TREE_ERR_INVALID_ARG, "count outputs are NULL");
    const tree_status vs = tree_validate_subtree_end(subtree_end, n);
    if (vs != TREE_OK) return vs;
    // parent of every slot: the innermost interval still open
    std::vector<int32_t> par(n), nchild(n, 0);
    {
        std::vector<int32_t> open;
        for (int32_t t = 0; t < (int32_t)n; ++t) {
            while (!open.empty() && subtree_end[open.back()] < t) open.pop_back();
            par[t] = open.empty() ? -1 : open.back();
            if (par[t] >= 0) ++nchild[par[t]];
            open.push_back(t);
        }
    }
    // chains in slot order: start, length, parent chain, depth
    std::vector<int32_t> seg_of(n), s_start, s_len, s_par, s_depth;
    for (int32_t t = 0; t < (int32_t)n; ++t) {
        const int32_t p = par[t];
        if (p < 0 || p != t - 1 || nchild[p] > 1) {
            const int32_t ps = p < 0 ? -1 : seg_of[p];
            s_start.push_back(t);
            s_len.push_back(0);
            s_par.push_back(ps);
            s_depth.push_back(ps < 0 ? 0 : s_depth[ps] + 1);
        }
        seg_of[t] = (int32_t)s_start.size() - 1;
        ++s_len.back();
    }
    const int64_t ns = (int64_t)s_start.size();
    int32_t max_depth = -1;
    for (int32_t d : s_depth) max_depth = std::max(max_depth, d);
    const int64_t nd = max_depth + 1;
    // stable bucket sort by depth
    std::vector<int64_t> off(nd + 1, 0);
    for (int32_t d : s_depth) ++off[d + 1];
    for (int64_t d = 0; d < nd; ++d) off[d + 1] += off[d];
    std::vector<int32_t> order(ns);
    {
        std::vector<int64_t> fill(off.begin(), off.end() - 1);
        for (int64_t s = 0; s < ns; ++s) order[fill[s_depth[s]]++] = (int32_t)s;
    }
    int64_t nc = 0;
    for (int32_t L : s_len) nc += (L + 63) / 64;
    // a saved final state only for chains with children, numbered in plan order
    std::vector<uint8_t> has_kids(ns, 0);
    for (int64_t s = 0; s < ns; ++s)
        if (s_par[s] >= 0) has_kids[s_par[s]] = 1;
    std::vector<int32_t> state_of(ns, -1);
    int32_t nst = 0;
    for (int64_t r = 0; r < ns; ++r)
        if (has_kids[order[r]]) state_of[order[r]] = nst++;
    *n_segments = ns;
    *n_chunks = nc;
    *n_depths = nd;
    *n_states = nst;
    if (!parent_slot && !segments && !chunks && !depth_offsets) return TREE_OK;  // size query
    if (!parent_slot || !segments || !chunks || !depth_offsets)
        return fail(TREE_ERR_INVALID_ARG, "some plan outputs are NULL");
    if (ns > seg_cap || nc > chunk_cap || nd > depth_cap)
        return fail(TREE_ERR_CAPACITY, "plan needs %lld chains, %lld chunks, %lld depths", (long long)ns,
                    (long long)nc, (long long)nd);
    std::copy(par.begin(), par.end(), parent_slot);
    int64_t c = 0;
    for (int64_t r = 0; r < ns; ++r) {
        const int32_t s = order[r];
        const int32_t k = (s_len[s] + 63) / 64;
        segments[4 * r + 0] = (int32_t)c;
        segments[4 * r + 1] = k;
        segments[4 * r + 2] = s_par[s] < 0 ? -1 : state_of[s_par[s]];
        segments[4 * r + 3] = state_of[s];
        for (int32_t j = 0; j < k; ++j, ++c) {
            chunks[2 * c + 0] = s_start[s] + 64 * j;
            chunks[2 * c + 1] = std::min(64, s_len[s] - 64 * j);
        }
    }
    for (int64_t d = 0; d <= nd; ++d) depth_offsets[d] = (int32_t)off[d];
    return TREE_OK;
}
