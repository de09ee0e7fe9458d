// Host entry points of the library under AddressSanitizer and
// UndefinedBehaviorSanitizer: the integer path (trie builder, layout, subtree_end
// validation, leaf placement, row planner, GDN chain plan) on random forests
// and on rows of the workloads' sizes, with the size-query and capacity paths.
// Built and run by tests/test_host_sanitized.py; exits non-zero on a failed
// check, and the sanitizers abort on an invalid access or undefined behaviour.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "../../include/tree_attn.h"

namespace {

int g_failures = 0;

#define CHECK(cond)                                                            \
    do {                                                                       \
        if (!(cond)) {                                                         \
            std::fprintf(stderr, "check failed: %s (line %d)\n", #cond, __LINE__); \
            ++g_failures;                                                      \
        }                                                                      \
    } while (0)

struct Batch {
    std::vector<int64_t> off{0};
    std::vector<int32_t> tok;
    std::vector<uint8_t> train;
    void add(const std::vector<int32_t>& s, int trainable_from = -1) {
        for (size_t t = 0; t < s.size(); ++t) {
            tok.push_back(s[t]);
            train.push_back(trainable_from >= 0 && (int)t >= trainable_from);
        }
        off.push_back((int64_t)tok.size());
    }
    int32_t n() const { return (int32_t)off.size() - 1; }
};

// Runs of a small alphabet: many forks, short and long shared runs, empty sequences.
Batch random_batch(std::mt19937& rng, int n_seqs, int max_len, int vocab, bool with_train) {
    Batch b;
    std::uniform_int_distribution<int> len(0, max_len), sym(0, vocab - 1), run(1, 12), coin(0, 1);
    for (int s = 0; s < n_seqs; ++s) {
        std::vector<int32_t> seq;
        const int L = len(rng);
        while ((int)seq.size() < L) {
            const int r = run(rng), x = sym(rng);
            for (int i = 0; i < r && (int)seq.size() < L; ++i) seq.push_back(x);
        }
        b.add(seq, with_train && coin(rng) ? (int)(seq.size() / 2) : -1);
    }
    return b;
}

// Trie, layout, validation, GDN plan and placement of one batch, with invariants.
void exercise(const Batch& b, int32_t min_shared, bool trainable, std::mt19937& rng) {
    const int32_t ns = b.n();
    const int64_t total = b.off.back();
    int64_t n_nodes = -1;
    const uint8_t* tr = trainable ? b.train.data() : nullptr;
    // size query, then a too-small buffer, then the real call
    CHECK(tree_build_trie(ns, b.off.data(), b.tok.data(), tr, min_shared, nullptr, 0, &n_nodes, nullptr) == TREE_OK);
    CHECK(n_nodes >= 0 && n_nodes <= total);
    std::vector<int32_t> parent((size_t)std::max<int64_t>(n_nodes, 1)), seq_last((size_t)std::max(ns, 1));
    if (n_nodes > 1) {
        int64_t m = -1;
        CHECK(tree_build_trie(ns, b.off.data(), b.tok.data(), tr, min_shared, parent.data(), n_nodes - 1, &m,
                              seq_last.data()) == TREE_ERR_CAPACITY);
        CHECK(m == n_nodes);
    }
    CHECK(tree_build_trie(ns, b.off.data(), b.tok.data(), tr, min_shared, parent.data(), n_nodes, &n_nodes,
                          seq_last.data()) == TREE_OK);
    for (int64_t v = 0; v < n_nodes; ++v) CHECK(parent[v] < v && parent[v] >= -1);
    // layout with padding, in the builder's numbering and in a shuffled one
    const int32_t R = (int32_t)n_nodes + 7;
    for (int shuffled = 0; shuffled < 2; ++shuffled) {
        std::vector<int32_t> perm((size_t)n_nodes), par2((size_t)std::max<int64_t>(n_nodes, 1)),
            last2((size_t)std::max(ns, 1));
        for (int64_t v = 0; v < n_nodes; ++v) perm[v] = (int32_t)v;
        if (shuffled) std::shuffle(perm.begin(), perm.end(), rng);
        for (int64_t v = 0; v < n_nodes; ++v) par2[perm[v]] = parent[v] < 0 ? -1 : perm[parent[v]];
        for (int32_t s = 0; s < ns; ++s) last2[s] = seq_last[s] < 0 ? -1 : perm[seq_last[s]];
        std::vector<int32_t> slot(R), pos(R), se(R);
        std::vector<int64_t> offs((size_t)ns + 1);
        CHECK(tree_pack_layout((int32_t)n_nodes, par2.data(), ns, last2.data(), R, slot.data(), pos.data(), se.data(),
                               offs.data(), nullptr, 0) == TREE_OK);
        const int64_t ti_n = offs[ns];
        std::vector<int32_t> ti((size_t)std::max<int64_t>(ti_n, 1));
        if (ti_n > 0)
            CHECK(tree_pack_layout((int32_t)n_nodes, par2.data(), ns, last2.data(), R, slot.data(), pos.data(),
                                   se.data(), offs.data(), ti.data(), ti_n - 1) == TREE_ERR_CAPACITY);
        CHECK(tree_pack_layout((int32_t)n_nodes, par2.data(), ns, last2.data(), R, slot.data(), pos.data(), se.data(),
                               offs.data(), ti.data(), ti_n) == TREE_OK);
        CHECK(tree_validate_subtree_end(se.data(), R) == TREE_OK);
        for (int32_t j = 0; j < R; ++j) CHECK(j <= se[j] && se[j] < R);
        for (int32_t s = 0; s < ns; ++s) {  // token_index spells the sequence: consecutive depths 0, 1, ...
            for (int64_t t = offs[s]; t < offs[s + 1]; ++t) CHECK(pos[ti[t]] == (int32_t)(t - offs[s]));
        }
        // GDN chain plan of the real slots
        const int64_t n = n_nodes;
        if (n > 0) {
            int64_t nseg = 0, nch = 0, nd = 0, nst = 0;
            CHECK(tree_gdn_plan(n, se.data(), nullptr, nullptr, 0, &nseg, nullptr, 0, &nch, nullptr, 0, &nd, &nst) ==
                  TREE_OK);
            std::vector<int32_t> ps((size_t)n), segs((size_t)nseg * 4 + 4), chunks((size_t)nch * 2 + 2),
                dofs((size_t)nd + 2);
            CHECK(tree_gdn_plan(n, se.data(), ps.data(), segs.data(), nseg, &nseg, chunks.data(), nch, &nch, dofs.data(),
                                nd, &nd, &nst) == TREE_OK);
            int64_t covered = 0;
            for (int64_t c = 0; c < nch; ++c) {
                CHECK(chunks[2 * c + 1] >= 1 && chunks[2 * c + 1] <= 64);
                covered += chunks[2 * c + 1];
            }
            CHECK(covered == n);
            if (nseg > 1) CHECK(tree_gdn_plan(n, se.data(), ps.data(), segs.data(), nseg - 1, &nseg, chunks.data(), nch,
                                              &nch, dofs.data(), nd, &nd, &nst) == TREE_ERR_CAPACITY);
        }
    }
    // placement, both modes, and the row planner
    std::vector<int32_t> grp((size_t)std::max(ns, 1));
    for (int32_t s = 0; s < ns; ++s) grp[s] = s % 3;
    int64_t longest = 1;
    for (int32_t s = 0; s < ns; ++s) longest = std::max<int64_t>(longest, b.off[s + 1] - b.off[s]);
    const int32_t cap = (int32_t)longest + 13;
    for (int mode = 0; mode < 2; ++mode) {
        std::vector<int32_t> bin((size_t)std::max(ns, 1)), tok((size_t)std::max(ns, 1));
        int32_t nb = -1;
        CHECK(tree_place_leaves((int32_t)n_nodes, parent.data(), ns, seq_last.data(), grp.data(), cap, mode, bin.data(),
                                tok.data(), std::max(ns, 1), &nb) == TREE_OK);
        for (int32_t r = 0; r < nb; ++r) CHECK(tok[r] <= cap);
        if (nb > 1) {
            int32_t nb2 = -1;
            CHECK(tree_place_leaves((int32_t)n_nodes, parent.data(), ns, seq_last.data(), grp.data(), cap, mode,
                                    bin.data(), tok.data(), nb - 1, &nb2) == TREE_ERR_CAPACITY);
            CHECK(nb2 == nb);
        }
    }
    if (!trainable) {
        std::vector<int32_t> row((size_t)std::max(ns, 1));
        std::vector<int64_t> rtok((size_t)std::max(ns, 1));
        std::vector<uint8_t> forked((size_t)std::max(ns, 1));
        int32_t nr = -1;
        CHECK(tree_plan_rows(ns, b.off.data(), b.tok.data(), min_shared, cap, row.data(), rtok.data(), std::max(ns, 1),
                             &nr, forked.data()) == TREE_OK);
        for (int32_t r = 0; r < nr; ++r) CHECK(rtok[r] <= cap);
        if (nr > 1) CHECK(tree_plan_rows(ns, b.off.data(), b.tok.data(), min_shared, cap, row.data(), rtok.data(), 1,
                                         &nr, nullptr) == TREE_ERR_CAPACITY);
    }
}

}  // namespace

int main() {
    std::mt19937 rng(12345);
    for (int it = 0; it < 300; ++it) {
        std::uniform_int_distribution<int> ns(0, 14), ml(0, 90), vocab(2, 4), ms(1, 8);
        const bool trainable = it % 3 == 0;
        const Batch b = random_batch(rng, ns(rng), ml(rng), vocab(rng), trainable);
        exercise(b, it % 5 == 0 ? 64 : ms(rng), trainable, rng);
    }
    {  // rows of the workloads' sizes: a group of 16 rollouts on a 2,048-token prompt, a 40,000-token chain
        Batch g;
        std::vector<int32_t> prompt(2048);
        for (int i = 0; i < 2048; ++i) prompt[i] = 7 + i;
        for (int r = 0; r < 16; ++r) {
            std::vector<int32_t> s = prompt;
            for (int i = 0; i < 1024; ++i) s.push_back(100000 + 5000 * r + i);
            g.add(s);
        }
        exercise(g, 64, false, rng);
        Batch chain;
        std::vector<int32_t> c(40000);
        for (int i = 0; i < 40000; ++i) c[i] = i;
        chain.add(c);
        exercise(chain, 64, false, rng);
    }
    // malformed inputs: errors, never an access out of bounds
    {
        std::vector<int32_t> par = {1, 0}, last = {0};
        std::vector<int32_t> slot(2), pos(2), se(2);
        std::vector<int64_t> offs(2);
        CHECK(tree_pack_layout(2, par.data(), 1, last.data(), 2, slot.data(), pos.data(), se.data(), offs.data(),
                               nullptr, 0) == TREE_ERR_BAD_TREE);
        std::vector<int32_t> bad = {2, 3, 2, 3};
        CHECK(tree_validate_subtree_end(bad.data(), 4) == TREE_ERR_BAD_TREE);
        std::vector<int32_t> beyond = {0, 9};
        CHECK(tree_validate_subtree_end(beyond.data(), 2) == TREE_ERR_BAD_TREE);
    }
    if (g_failures) {
        std::fprintf(stderr, "%d checks failed\n", g_failures);
        return 1;
    }
    std::printf("host entry points: all checks passed under the sanitizers\n");
    return 0;
}
