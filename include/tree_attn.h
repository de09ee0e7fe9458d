/*
 * tree_attn.h - attention over prefix-tree-packed rows on AMD Instinct MI355X (gfx950).
 *
 * A batch of token sequences that share prefixes is packed as a trie: a
 * shared prefix is stored once, laid out depth-first, each token takes its
 * tree depth as position id, and each token attends only to itself and its
 * root-to-leaf ancestors.  This library is the data-parallel hot path of
 * that method, as a plain C ABI:
 *
 *   tree_build_trie      token sequences -> token-level parent array (host)
 *   tree_place_leaves    sequences of a trie -> fixed-length rows (host)
 *   tree_plan_rows       samples -> rows grown in order under a forwarded-token budget (host)
 *   tree_pack_layout     parent array -> DFS slots, depth, subtree end, token_index (host)
 *   tree_rope            rotary embedding at depth, in place (device)
 *   tree_rope_qk         the same on q and k in one launch (device)
 *   tree_attn_fwd        masked attention forward (device)
 *   tree_attn_fwd_noalloc  the same without a workspace, for callers that cannot allocate (device)
 *   tree_attn_bwd        its exact gradient (device)
 *   tree_gdn_plan        DFS row -> chains, 64-token chunks, depth buckets (host)
 *   tree_gdn_fwd         gated-delta-rule mixing over the row (device)
 *
 * Sources (web pages, cited by title and section):
 *   [ART] "Prefix Tree Packing in ART" (FurtherAI blog)
 *   [DAG] "DAG packing" (sudakov.site)
 *   [TRL] "TRL Tree Packing for AsyncGRPO: The 26x Claim vs. the 3x the Pull
 *         Request Measures" (explainx.ai)
 *
 * Conventions shared by every entry point
 *   - Every call returns a tree_status; TREE_OK (0) on success.  On failure
 *     tree_last_error() returns a thread-local message naming the problem.
 *   - Argument checks run before any device work: a call that fails them
 *     enqueues nothing.  A failed kernel launch returns TREE_ERR_DEVICE.
 *   - The caller owns and allocates every buffer.  Host entry points take
 *     host pointers; device entry points take device pointers and enqueue
 *     asynchronously on `stream` (a hipStream_t; NULL = the default stream).
 *     The library keeps no state between calls beyond a per-device count of
 *     compute units (read once) and the per-device scratch array of
 *     tree_attn_fwd_noalloc (below), and is thread-safe (that one entry
 *     point excepted, as it says).
 *   - Device tensors are contiguous:
 *       q, out, dout, dq : [B, N, Hq, D]      k, v, dk, dv : [B, N, Hkv, D]
 *       lse              : [B, Hq, N] fp32, natural log
 *       subtree_end, pos_ids : [B, N] int32
 *     Query head h reads KV head h / (Hq / Hkv).  D is 64 or 128.
 *   - Buffer sizes cannot be checked through plain pointers: each device
 *     buffer must hold its shape above in the element type `dt` names
 *     (lse and the index rows keep theirs).  A dtype code that does not
 *     match the buffers (TREE_F32 for bf16 tensors, say) makes the kernels
 *     read and write past the buffers' ends.
 *   - Integers are int32 for token ids, node ids and slots, int64 for CSR
 *     offsets into flattened arrays.
 */
#ifndef TREE_ATTN_H
#define TREE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum tree_status {
    TREE_OK = 0,
    TREE_ERR_INVALID_ARG = 1, /* null pointer, negative or inconsistent size, bad dtype */
    TREE_ERR_BAD_TREE = 2,    /* parent array is not a forest; subtree_end not nested */
    TREE_ERR_CAPACITY = 3,    /* an output buffer is too small (required size still reported) */
    TREE_ERR_UNSUPPORTED = 4, /* head dim, head ratio or dtype this build has no kernel for */
    TREE_ERR_DEVICE = 5       /* a HIP call or kernel launch failed */
} tree_status;

typedef enum tree_dtype { TREE_F32 = 0, TREE_BF16 = 1 } tree_dtype;

/* Version of this ABI (bumped on any signature change). */
int tree_abi_version(void);
/* Static name of a status code. */
const char* tree_status_string(int status);
/* Message for the last failed call on this thread ("" if none). */
const char* tree_last_error(void);

/*
 * tree_build_trie - pack token sequences into a token-level trie (host, synchronous).
 *
 * [ART "The tree"]: take the longest run that every active sequence agrees
 * on, emit it once, split the rest by their next token and recurse.  A run
 * shorter than `min_shared` tokens is not shared but copied into each
 * next-token branch (sharing resumes deeper where a branch agrees longer).
 * At every fork each branch keeps its own copy of the join token, the last
 * shared token [ART "The tree"; DAG "The walk"].  The run length compared
 * with `min_shared` is measured before the join token is split off.
 * Branches are taken in ascending next-token order; sequences that end where
 * the others fork come first; identical sequences share one path.  Nodes are
 * numbered in emission order, a depth-first pre-order, so
 * tree_pack_layout() of the result keeps node i in slot i.
 *
 * Trainable mode (`trainable` not NULL), [ART "The tree"]: trainable tokens
 * are never shared (a shared run stops at the first trainable token of any
 * active sequence, and a sequence whose next token is trainable is a branch
 * of its own), and the join token is copied only into branches whose next
 * token is trainable, so that first trainable token has its own prediction
 * position; other branches, and sequences ending at the fork, hang off the
 * shared join token.  This is the accounting of [ART "Does it actually
 * help?"]: a system prompt shared whole, then 11,999 shared group-prefix
 * tokens and completion + 1 tokens per rollout.
 *
 *   n_seqs       number of sequences (>= 0)
 *   seq_offsets  [n_seqs + 1] CSR offsets into `tokens`, non-decreasing, seq_offsets[0] == 0
 *   tokens       [seq_offsets[n_seqs]] token ids (any int32 values)
 *   trainable    [seq_offsets[n_seqs]] per token, nonzero = trainable; NULL = default mode
 *   min_shared   minimum shared run length (>= 1; 64 is the pages' default)
 *   parent       out [parent_cap] parent node of each node, -1 for a root; NULL = size query
 *   parent_cap   capacity of `parent` in elements; seq_offsets[n_seqs] always suffices
 *   n_nodes      out: number of nodes (written also on TREE_ERR_CAPACITY)
 *   seq_last     out [n_seqs] node of each sequence's last token, -1 for an empty sequence;
 *                may be NULL
 */
tree_status tree_build_trie(int32_t n_seqs, const int64_t* seq_offsets, const int32_t* tokens,
                            const uint8_t* trainable, int32_t min_shared, int32_t* parent,
                            int64_t parent_cap, int64_t* n_nodes, int32_t* seq_last);

/* Row placement modes of tree_place_leaves(). */
typedef enum tree_place_mode {
    TREE_PLACE_GLOBAL = 0,    /* best-fit decreasing over every leaf of the batch */
    TREE_PLACE_IN_ORDER = 1   /* one row at a time, in arrival order */
} tree_place_mode;

/*
 * tree_place_leaves - assign the sequences of a packed trie to fixed-length
 * rows (host, synchronous).
 *
 * [ART "Bin packing, with a twist"]: a leaf (one sequence) is the list of
 * segments on its root-to-leaf path; its cost of joining a row is the length
 * of the segments that row does not hold yet, so a row holds the union of
 * its leaves' segments.  TREE_PLACE_GLOBAL is best-fit decreasing over that
 * cost: groups in decreasing order of their most expensive leaf (a leaf's
 * standalone cost is its path length; equal groups keep the order of their
 * first sequence), leaves in input order inside a group, each leaf into the
 * row left with the least free space (the earliest row on a tie), a new row
 * when none fits.  TREE_PLACE_IN_ORDER is the packer [ART "Does it actually
 * help?"] compares against: rows filled one at a time in input order, moving
 * on for good when the next sequence does not fit.
 *
 * A segment is a maximal chain of nodes: a node starts one when it is a root,
 * when its parent has several children, or when its parent is the last
 * token of a sequence.  A row's token count is therefore the node count of
 * the sub-forest its sequences span (what a trie rebuilt for the row alone
 * would hold).
 *
 *   n_nodes      nodes of the trie
 *   parent       [n_nodes] parent node, -1 for a root; every node after its parent
 *                (the numbering tree_build_trie() produces), else TREE_ERR_BAD_TREE
 *   n_seqs       number of sequences
 *   seq_last     [n_seqs] node of each sequence's last token (-1: empty sequence, cost 0)
 *   group        [n_seqs] group id of each sequence (any int32); may be NULL in
 *                TREE_PLACE_IN_ORDER mode
 *   seq_len      row capacity in tokens (>= 1); a sequence longer than a row is
 *                TREE_ERR_CAPACITY
 *   mode         a tree_place_mode
 *   bin_of_seq   out [n_seqs] row of each sequence
 *   bin_tokens   out [bins_cap] tokens held by each row
 *   bins_cap     capacity of bin_tokens; fewer rows than needed is TREE_ERR_CAPACITY
 *                (n_bins and bin_of_seq are still written)
 *   n_bins       out: number of rows
 */
tree_status tree_place_leaves(int32_t n_nodes, const int32_t* parent, int32_t n_seqs,
                              const int32_t* seq_last, const int32_t* group, int32_t seq_len,
                              int32_t mode, int32_t* bin_of_seq, int32_t* bin_tokens,
                              int32_t bins_cap, int32_t* n_bins);

/*
 * tree_plan_rows - grow packed rows sample by sample under a budget of
 * forwarded tokens (host, synchronous).
 *
 * [TRL "How tree packing works"]: the planner grows the trie sample by
 * sample and its token_budget bounds unique (forwarded) tokens, not raw ones;
 * [TRL "Limits and caveats to know before you switch"]: fork_threshold_tokens
 * (1024 by default) sets how much prefix samples must have in common before
 * they share it.  Samples are taken in input order; a sample joins the open
 * row when the trie of the row plus the sample (tree_build_trie() with the
 * fork threshold as its minimum shared run, default mode) holds at most
 * token_budget nodes, else the open row is closed for good and the sample
 * opens the next row.
 *
 *   n_seqs, seq_offsets, tokens   the samples, as for tree_build_trie()
 *   fork_threshold_tokens  minimum common run that is shared (>= 0; 0 and 1 share any run)
 *   token_budget  forwarded tokens a row may hold (>= 1); a sample longer than this is
 *                 TREE_ERR_CAPACITY
 *   row_of_seq    out [n_seqs] row of each sample
 *   row_tokens    out [rows_cap] forwarded tokens of each row (NULL: not wanted)
 *   n_rows        out: number of rows (written also on TREE_ERR_CAPACITY)
 *   forked        out [n_seqs] 1 if the sample shares a slot with another sample of its row,
 *                 else 0 (the per-sample flag behind [TRL "How to evaluate it on your own
 *                 workload"]'s fork fraction); may be NULL
 * TREE_ERR_CAPACITY when rows_cap < n_rows (row_of_seq is complete).
 */
tree_status tree_plan_rows(int32_t n_seqs, const int64_t* seq_offsets, const int32_t* tokens,
                           int32_t fork_threshold_tokens, int64_t token_budget, int32_t* row_of_seq,
                           int64_t* row_tokens, int32_t rows_cap, int32_t* n_rows, uint8_t* forked);

/*
 * tree_pack_layout - lay one packed row out depth-first (host, synchronous).
 *
 * [TRL "How tree packing works"]: the collator lays tokens out depth-first,
 * uses depth as position ids and keeps a token_index from each trained token
 * back to its packed slot.  [DAG "Positions"]: depth is the number of steps
 * from the root (roots are at depth 0).  [ART "Token-mixing layers"]: the
 * pre-order/exit-order interval decides ancestry; subtree_end[j] is the
 * exit half: slot j is an ancestor-or-self of slot i iff
 * j <= i <= subtree_end[j].
 *
 *   n_nodes      nodes in the row's forest (0 <= n_nodes <= row_len)
 *   parent       [n_nodes] parent node id, -1 for a root; any numbering
 *   n_seqs       number of sequences whose paths are wanted in token_index
 *   seq_last     [n_seqs] node of each sequence's last token (-1: empty sequence)
 *   row_len      slots in the row; slots >= n_nodes are padding
 *   slot_node    out [row_len] node in each slot, -1 for padding
 *   pos_ids      out [row_len] depth of each slot (0 for padding)
 *   subtree_end  out [row_len] last slot of each slot's subtree (padding: its own slot)
 *   seq_offsets  out [n_seqs + 1] CSR offsets into token_index
 *   token_index  out [token_index_cap] slot of every token of every sequence, root first;
 *                NULL = size query (seq_offsets is still written)
 *
 * Children are visited in ascending node id.  The walk is iterative (rows of
 * tens of thousands of tokens are chains that deep).  Returns
 * TREE_ERR_BAD_TREE for a parent out of range or a cycle, TREE_ERR_CAPACITY
 * when token_index_cap < seq_offsets[n_seqs].
 */
tree_status tree_pack_layout(int32_t n_nodes, const int32_t* parent, int32_t n_seqs,
                             const int32_t* seq_last, int32_t row_len, int32_t* slot_node,
                             int32_t* pos_ids, int32_t* subtree_end, int64_t* seq_offsets,
                             int32_t* token_index, int64_t token_index_cap);

/*
 * tree_validate_subtree_end - check a subtree_end row (host, synchronous).
 *
 * [ART "Token-mixing layers"]: in a depth-first layout a node's subtree is
 * the contiguous run from its pre-order position to its exit position, so
 * the intervals [j, subtree_end[j]] of a tree are nested or disjoint.
 * TREE_OK iff j <= subtree_end[j] < n for every j and the intervals are
 * nested or disjoint; TREE_ERR_BAD_TREE otherwise.  The device entry points
 * trust their subtree_end; call this on input that did not come from
 * tree_pack_layout().
 */
tree_status tree_validate_subtree_end(const int32_t* subtree_end, int64_t n);

/*
 * tree_rope - rotary position embedding at tree depth, in place (device).
 *
 * [DAG "Positions"]: positions are graph depth, so along every root-to-leaf
 * path neighbouring tokens are one position apart.  Rotate-half pairing:
 * dimensions i and i + D/2 rotate by pos * theta^(-2i/D), i < D/2.  Angles
 * are formed in fp64 (for fp32 storage the sines and the rotation too; for
 * bf16 the sines of the fp64-reduced angle in fp32, errors near 1e-7) and
 * the result is rounded once to `dt`.  Slots at depth 0 are the identity
 * and are left untouched.
 *
 *   x        [B, N, H, D] of dtype dt, rotated in place
 *   pos_ids  [B, N] int32 (tree_pack_layout's pos_ids per row)
 *   theta    base (> 0), e.g. 10000
 * Errors: TREE_ERR_INVALID_ARG (negative sizes, null pointers, bad dtype or
 * theta), TREE_ERR_UNSUPPORTED (D other than 64 or 128), TREE_ERR_DEVICE.
 */
tree_status tree_rope(tree_dtype dt, void* x, int64_t B, int64_t N, int64_t H, int64_t D,
                      const int32_t* pos_ids, float theta, void* stream);

/*
 * tree_rope_qk - tree_rope on q [B, N, Hq, D] and k [B, N, Hkv, D] in one
 * launch (same dtype, head dim, positions and theta; each slot's sines are
 * computed once for both).  The results are those of tree_rope(q) followed
 * by tree_rope(k), bit for bit.  q and k must not overlap
 * (TREE_ERR_INVALID_ARG when they are the same buffer); either head count
 * may be 0.  Other errors as tree_rope.
 */
tree_status tree_rope_qk(tree_dtype dt, void* q, void* k, int64_t B, int64_t N, int64_t Hq, int64_t Hkv,
                         int64_t D, const int32_t* pos_ids, float theta, void* stream);

/*
 * tree_attn_workspace_bytes - device workspace tree_attn_fwd (bwd = 0) or
 * tree_attn_bwd (bwd = 1) needs for these sizes, whatever the tree.  Returns
 * 0 on bad sizes.  The workspace holds per-call tables and work-queue
 * counters that each call re-initialises on its stream: calls that may run at
 * the same time on the GPU need workspaces of their own.
 *
 * For the backward this is the largest workspace a call can use: a fixed
 * part (delta, lse, tile tables, the dK/dV work plan) plus the most fp32
 * partial-sum slots the plan ever takes (1,536 slots of 256 keys x D x 2;
 * 384 MiB at D = 128).  The plan cuts key tiles whose visible query range is
 * long into chunks that write partial sums; tree_attn_bwd() takes as many
 * slots as the workspace it is given holds beyond the fixed part (down to
 * none, when no tile is cut), and tree_attn_bwd_workspace_bytes_for() gives
 * the exact size a row's plan uses.
 */
size_t tree_attn_workspace_bytes(tree_dtype dt, int64_t B, int64_t N, int64_t Hq, int64_t Hkv,
                                 int64_t D, int bwd);

/*
 * tree_attn_bwd_workspace_bytes_for - backward workspace these rows' dK/dV
 * plan uses (host, synchronous): the fixed part plus the partial-sum slots the
 * plan takes at its first chunk budget (at most the 1,536 of
 * tree_attn_workspace_bytes).  With at least this much, tree_attn_bwd() runs
 * the same plan as with the largest workspace (bitwise the same results).
 *
 *   subtree_end  [B, N] int32 in HOST memory (the rows tree_attn_bwd() will get)
 * Returns 0 on bad sizes or a NULL subtree_end with B * N > 0.  For shapes the
 * vector path serves it returns its fixed workspace.
 */
size_t tree_attn_bwd_workspace_bytes_for(tree_dtype dt, const int32_t* subtree_end, int64_t B, int64_t N,
                                         int64_t Hq, int64_t Hkv, int64_t D);

/*
 * tree_attn_fwd - attention forward over packed rows (device).
 *
 * [ART "Token-mixing layers"; DAG "The mask"]: query i attends to key j iff
 * j is i or an ancestor of i, i.e. j <= i <= subtree_end[j].  The row's
 * visible set splits into fully visible blocks (ancestor segments) and a
 * causal block on its own segment; blocks with no visible pair are skipped.
 *
 *   out[b,i,h,:] = sum_j P[i,j] v[b,j,h/(Hq/Hkv),:],  P = softmax_j(softmax_scale * q_i . k_j)
 *   lse[b,h,i]   = log sum_j exp(softmax_scale * q_i . k_j)     (visible j only)
 *
 *   dt           TREE_BF16 (MFMA, fp32 accumulation and softmax) or TREE_F32
 *   q, k, v      inputs in dt (see layouts above); typically after tree_rope
 *   subtree_end  [B, N] int32 from tree_pack_layout (not checked on device)
 *   softmax_scale  usually 1/sqrt(D); finite and > 0, else TREE_ERR_INVALID_ARG
 *                (the matrix-core path masks scores before scaling them)
 *   out          out [B, N, Hq, D] in dt
 *   lse          out [B, Hq, N] fp32
 *   ws, ws_bytes device workspace of at least tree_attn_workspace_bytes(dt, ..., 0) bytes
 *
 * Padding slots (subtree_end[j] == j, no descendants) attend to themselves only:
 * out = v, lse = softmax_scale * q . k.
 */
tree_status tree_attn_fwd(tree_dtype dt, const void* q, const void* k, const void* v,
                          const int32_t* subtree_end, int64_t B, int64_t N, int64_t Hq,
                          int64_t Hkv, int64_t D, float softmax_scale, void* out, float* lse,
                          void* ws, size_t ws_bytes, void* stream);

/*
 * tree_attn_fwd_noalloc - tree_attn_fwd without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * serving loops, harnesses that forbid hipMalloc).  Same arguments, kernels
 * and results as tree_attn_fwd; its per-call tables live in a fixed
 * 1,114,112-byte array of the library's device code (one per GPU, held until
 * the process ends), so the call itself allocates nothing.
 *
 * Limit: B x ceil(N / 64) <= 65,536 (e.g. one row of 4M slots, or 128 rows
 * of 32K); beyond it TREE_ERR_CAPACITY, before any device call.  The array's
 * device address is looked up on the first call on each device
 * (hipGetSymbolAddress; TREE_ERR_DEVICE if that fails).  Every call on one
 * GPU shares that GPU's array: calls that may run at the same time on one
 * GPU (other streams, other threads) race and must be serialised by the
 * caller; a call re-initialises the tables it reads, so nothing carries over
 * from the previous call.
 */
tree_status tree_attn_fwd_noalloc(tree_dtype dt, const void* q, const void* k, const void* v,
                                  const int32_t* subtree_end, int64_t B, int64_t N, int64_t Hq, int64_t Hkv,
                                  int64_t D, float softmax_scale, void* out, float* lse, void* stream);

/*
 * tree_attn_bwd - exact gradient of tree_attn_fwd (device).
 *
 * The pages give no backward pass; this is the exact gradient of the
 * forward above for L = sum <dout, out>, each packed slot counted once
 * (a shared token is forwarded once, so its gradient arrives once).
 * dk and dv sum over the query heads that share a KV head.
 *
 *   out, lse     the forward's outputs for these inputs
 *   softmax_scale  the forward's; finite and > 0, else TREE_ERR_INVALID_ARG
 *   dout         [B, N, Hq, D] in dt
 *   dq           out [B, N, Hq, D] in dt
 *   dk, dv       out [B, N, Hkv, D] in dt
 *   ws, ws_bytes device workspace: tree_attn_bwd_workspace_bytes_for() of these rows
 *                (or tree_attn_workspace_bytes(dt, ..., 1), which fits any rows).  Less
 *                is accepted down to the fixed part (the size for rows without cut
 *                tiles); the plan then cuts long key tiles into fewer chunks (same
 *                results up to the order of summation).  Below that: TREE_ERR_CAPACITY.
 */
tree_status tree_attn_bwd(tree_dtype dt, const void* q, const void* k, const void* v,
                          const int32_t* subtree_end, const void* out, const float* lse,
                          const void* dout, int64_t B, int64_t N, int64_t Hq, int64_t Hkv,
                          int64_t D, float softmax_scale, void* dq, void* dk, void* dv, void* ws,
                          size_t ws_bytes, void* stream);

/*
 * Gated-delta-rule (GDN) token mixing over a packed row.
 *
 * [ART "Token-mixing layers"]: a recurrent layer has no mask; its state runs
 * token by token along each root-to-leaf path, is forked at every branch
 * point and starts from zero at every tree root.  Its pages run it depth by
 * depth over the tree's segments, a causal convolution and a chunked (64
 * token) delta-rule call per depth, a child starting from its parent's final
 * state.  The layer is Gated DeltaNet (Yang, Kautz and Hatamizadeh, 2024):
 * per slot t, x_t holds C = 2 Hk dk + Hv dv channels, ordered q | k | v; a
 * depthwise causal convolution of width W over the slot and its W-1 nearest
 * ancestors (zeros above a root; tap W-1 weighs the slot itself), then SiLU;
 * q and k divided by their L2 norm per head (zero stays zero), q scaled by
 * dk^-1/2; then per value head h (key head h / (Hv / Hk)), with state
 * S in R^{dv x dk}:
 *     S_t = exp(g_t) S_parent (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
 *     o_t = S_t q_t,
 * S_parent the state after the slot's parent (zero for a root).
 */

/*
 * tree_gdn_plan - the work plan of tree_gdn_fwd for one packed row (host).
 *
 * The parent of each slot is the innermost interval [j, subtree_end[j]]
 * containing it.  A chain is a maximal run of consecutive slots each of which
 * is the only child of the one before; every chain starts from one state (zero
 * at a root, else the final state of the chain ending at its parent).  Chains
 * are bucketed by depth (the number of chains above them) and cut into chunks
 * of up to 64 slots from the chain's first slot.  A chunk that ends a chain
 * short of 64 slots is run as it is (its final state is exact), so no tail is
 * replayed per child.
 *
 *   n              real slots of the row (padding slots after them are not given)
 *   subtree_end    [n] the row's subtree_end (tree_pack_layout), validated here
 *   parent_slot    out [n] parent slot, -1 at roots
 *   segments       out [seg_cap][4] per chain, depth-major: first chunk, chunk count,
 *                  state slot of the parent chain (-1 at a root: zero state), own
 *                  state slot (-1 for a chain without children: its final state is
 *                  not kept); slots number the chains with children in plan order
 *   chunks         out [chunk_cap][2] per chunk, chain by chain: first slot, length (1..64)
 *   depth_offsets  out [depth_cap + 1] chains of depth d are segments[depth_offsets[d] ..
 *                  depth_offsets[d+1])
 *   n_segments, n_chunks, n_depths, n_states   out: counts (written also on TREE_ERR_CAPACITY)
 * All four arrays NULL: size query.  TREE_ERR_BAD_TREE for a subtree_end that
 * is not a nested interval set.
 */
tree_status tree_gdn_plan(int64_t n, const int32_t* subtree_end, int32_t* parent_slot, int32_t* segments,
                          int64_t seg_cap, int64_t* n_segments, int32_t* chunks, int64_t chunk_cap,
                          int64_t* n_chunks, int32_t* depth_offsets, int64_t depth_cap, int64_t* n_depths,
                          int64_t* n_states);

/*
 * tree_gdn_workspace_bytes - device workspace of tree_gdn_fwd (0 for
 * unsupported sizes).  It holds the convolved inputs ([n, C] bf16), the
 * chunk operands (57,856 bytes per chunk and value head) and the final state
 * of every chain with children (fp32 [n_states, Hv, dk, dv]).
 */
size_t tree_gdn_workspace_bytes(int64_t n, int64_t n_states, int64_t n_chunks, int64_t Hk, int64_t Hv,
                                int64_t dk, int64_t dv);

/*
 * tree_gdn_fwd - gated-delta-rule mixing over one packed row (device, async).
 *
 *   dt             TREE_BF16 (x and out bf16; gates fp32; state fp32)
 *   x              [n, C] mixing input, C = 2 Hk dk + Hv dv, channels q | k | v
 *   conv_w         [C, conv_width] fp32 convolution taps, conv_width 1..4
 *   g, beta        [n, Hv] fp32 log decay (<= 0) and write strength per slot and value head
 *   parent_slot, segments, chunks   device copies of tree_gdn_plan's outputs
 *   depth_offsets  HOST array [n_depths + 1] from tree_gdn_plan (launch sizes)
 *   n_states       tree_gdn_plan's state count
 *   n              real slots; Hk, Hv heads (Hv a multiple of Hk); dk = dv = 128
 *   out            [n, Hv, dv] bf16
 *   ws, ws_bytes   device workspace of at least tree_gdn_workspace_bytes() bytes
 * The device tables are trusted: pass tree_gdn_plan's output for this row.
 * Work: one convolution launch, one chunk launch, one state launch per depth.
 */
tree_status tree_gdn_fwd(tree_dtype dt, const void* x, const float* conv_w, int64_t conv_width, const float* g,
                         const float* beta, const int32_t* parent_slot, const int32_t* segments,
                         int64_t n_segments, const int32_t* chunks, int64_t n_chunks, const int32_t* depth_offsets,
                         int64_t n_depths, int64_t n_states, int64_t n, int64_t Hk, int64_t Hv, int64_t dk,
                         int64_t dv, void* out, void* ws, size_t ws_bytes, void* stream);

/*
 * tree_mfma_peak - measurement aid, not part of the path (device, async).
 *
 * Launches `blocks` workgroups of four waves; every wave issues `iters` x 4
 * bf16 32x32x16 matrix products on register operands (four independent
 * accumulators), nothing else.  Timing the call on `stream` gives the
 * matrix-core rate the GPU sustains; the products performed are written to
 * *flops (host) before the launch.  `sink` is a device buffer of at least 256
 * floats that the kernel may write (it never does for these operands; the
 * store only keeps the products live).
 */
tree_status tree_mfma_peak(int64_t blocks, int64_t iters, float* sink, double* flops, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TREE_ATTN_H */
