"""CPU oracle for the EAGLE tree-verification step.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow, fp64 definition
of what the verification step computes, used to check the GPU library.  Only
the test suite, the smoke check and the benchmark's CPU-baseline leg may
import it; the product path (the C-ABI library and its Python binding) never
does, and shares no code with it.

Sources, cited by page title and section:
  [EAGLE-p2]  "EAGLE: Speculative Sampling Requires Rethinking Feature
              Uncertainty", paperlayer.ai source-linked summary of arXiv
              2401.15077 — §2 Preliminaries, §3 EAGLE, A.1 Tree Structure,
              A.2 Multi-Round Speculative Sampling, B Detailed results.
  [EAGLE-2-blog] EAGLE-2 overview blog (jxzklqfsx.com) — §1 overview (the
              temperature-0 = most-probable-token convention), §3 EAGLE
              (tree-structured verification).

Parts:
  tree       ancestor sets, depths                     (tree mask row)
  attention  tree attention over cache + ancestors     (tree attention row)
  vocab      temperature softmax / argmax              (vocabulary row)
  walk       multi-round acceptance walk, residual,    (acceptance + bonus rows)
             bonus sample
  compact    KV compaction of the accepted path        (compaction row)

Parity status: every function is pinned by CPU tests in tests/test_oracle_*.py
against closed forms, library witnesses, hand-derived fixtures, exact
enumeration of the output law and a chi-square test.  The near-tie window
and the inverse-CDF tie conventions are conventions, not results: parity
unpinned for those conventions themselves.
"""
from .tree import ancestors, ancestor_masks, depths, validate_parents  # noqa: F401
from .attention import bf16_bits_to_f64, tree_attention, tree_attention_one  # noqa: F401
from .vocab import argmax_lowest, target_distribution  # noqa: F401
from .walk import (NEAR_TIE, WalkResult, inverse_cdf, node_round,  # noqa: F401
                   verify_batch, verify_sequence)
from .compact import feature_gather, kv_compact  # noqa: F401
from . import dynamic_tree  # noqa: F401
