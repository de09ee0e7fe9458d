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

extern "C" int tree_abi_version(void) { return 1; }

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
    int32_t min_shared;
    std::vector<int32_t> parent;
    std::vector<int32_t> seq_last;

    int64_t len(int32_t s) const { return off[s + 1] - off[s]; }
    int32_t at(int32_t s, int64_t t) const { return tok[off[s] + t]; }

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
    // ascending token, keeping input order inside a branch.
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
            parts.emplace_back(act.begin() + i, act.begin() + j);
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
            int64_t end = start;
            while (end < m) {
                int32_t t0 = at(act[0], end);
                bool same = true;
                for (size_t i = 1; i < act.size() && same; ++i) same = at(act[i], end) == t0;
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
            if (end - start >= min_shared) {  // share the run minus the join token
                int32_t node = emit(act, start, end - 1, it.par);
                split(act, end, parts);
                push_parts(end - 1, node);
            } else {  // too short: copy it into every branch
                split(act, end, parts);
                push_parts(start, it.par);
            }
        }
    }
};

}  // namespace

extern "C" tree_status tree_build_trie(int32_t n_seqs, const int64_t* seq_offsets,
                                       const int32_t* tokens, int32_t min_shared, int32_t* parent,
                                       int64_t parent_cap, int64_t* n_nodes, int32_t* seq_last) {
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

    TrieBuilder tb{seq_offsets, tokens, min_shared, {}, {}};
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
