"""Oracle for attention over a prefix-tree-packed row: plain, slow, CPU, fp64.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
CPU-baseline leg may import this package; the library never does, and this
package imports nothing from the library.  The two share no code: the only
common inputs are the seeded workloads in ``synth``.

Sources (web pages; cited by title and section):
  [ART]  "Prefix Tree Packing in ART" (FurtherAI blog)
  [DAG]  "DAG packing" (sudakov.site)
  [TRL]  "TRL Tree Packing for AsyncGRPO: The 26x Claim vs. the 3x the Pull
         Request Measures" (explainx.ai)

Modules and what pins each one (tests/test_oracle_*.py):
  trie       - trie builder: longest shared run, split by next token [ART "The
               tree"], min shared run, join-token copy per branch [ART "The
               tree"; DAG "The walk"].  Pinned by the worked counts of [TRL
               "How tree packing works" and "A back-of-envelope example"] and
               by a brute-force count over a plain dict trie.
  layout     - DFS pre-order, depth positions, subtree end, token_index
               [ART "Token-mixing layers"; DAG "The walk", "Positions"; TRL
               "How tree packing works"].  Pinned by the 9-token mask figure
               caption of [ART "Token-mixing layers"] and tree invariants.
  counts     - raw / forwarded / packing ratio [TRL "How tree packing works"].
  rope       - rotary embedding at depth [DAG "Positions"].  Pinned by the
               complex-number closed form and the relative-position identity.
  attention  - ordinary causal attention per unpacked sequence, forward and
               exact backward, mapped back through token_index.  Pinned by a
               dense ancestor-masked brute force (brute), by torch's CPU
               scaled_dot_product_attention and autograd, and by central
               finite differences.
  brute      - dense N x N ancestor mask from parent pointers [DAG "The mask"].

Every function is pinned; none is "parity unpinned".
"""
