"""Plain fp64 CPU oracle for one context-parallel rank's ring attention forward.

TEST INFRASTRUCTURE ONLY. Nothing on the product path imports, calls or
executes anything in this package: only the tests, the smoke check and the
benchmark's ``cpu_baseline`` leg use it. It shares no code with the HIP path
(no kernels, headers, helpers, constants or pre/post-processing) and imports
nothing from it. Every input it sees is passed in as an array; the seeded
generators live in a module of their own.

Sources (the pages this oracle restates; cited by title and section):

* "Context Parallelism and Ring Attention" (hs-black.github.io, posts/
  scaling-context-parallel) -- §2 basic CP, §3 blockwise attention with
  online softmax and the log-sum-exp merge, §4 Ring Attention, §5 causal
  imbalance, §6 zig-zag and striped token reassignment, §8 all-gather CP,
  §9 DeepSpeed-Ulysses.
* "Tensor Parallelism" (t6page.pages.dev, LLM parallel communication) -- the
  GQA head table (tbl-tp-gqa).
* "DeepSpeed-Ulysses and hybrids" (t6page.pages.dev, context parallelism) --
  the pre/post all-to-all shapes.

Modules:

* :mod:`oracle.attention` -- the plain definition of softmax attention
  (primary oracle), the per-block statistics and the two-block merge
  (secondary, block-then-merge oracle), and the ring schedule.
* :mod:`oracle.partition` -- contiguous / zig-zag / striped token maps,
  visible-pair counts, tile classification, tile-level work and ring
  efficiency.
* :mod:`oracle.backward` -- the gradients of softmax attention (plain
  definition by the chain rule), one block's contributions with the global
  lse (§3 backward paragraph), and the ring backward (§4).
* :mod:`oracle.documents` -- all-gather CP (§8): the K/V of every rank
  gathered into global order, and the rank's attention under the document
  mask (no attention across documents) combined with the causal rule.

Parity status: every public function here is pinned by ``tests/test_oracle*.py``
against closed forms, brute force, a library special case or numbers the
pages print, and the planted-mistake tests show the pins catch a wrong
sign, term, index or operand in each. The row-subset checkers
(``attention.rows_attention``, ``documents.rows_attention_docs``) are pinned
against brute-force loops on chosen rows; the work counts (``rank_work``,
``tile_work_pairs``, ``tile_work_pairs_increasing``, ``tile_step_work``) against
brute-force tile loops and the per-rank closed forms; the FLOP convention
(``causal_adjusted_flops``) against counted multiply-adds and the
communication-hiding thresholds §4 prints.
"""

from . import attention, backward, documents, partition  # noqa: F401
