"""Plain fp64 CPU oracle for Core Context Aware (CCA) attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  It shares no code
with the GPU library (``sparse_long_context_cca_amd``) and never imports it.

Sources (cited by page and section throughout):
  [card]     Core Context Aware Transformers for Long Context Language Modeling,
             paper card at atlas.scime.ai ("Approach").
  [article]  ICML 2025 news article on CCA-Attention at changsha.jmyizhao.com
             (paragraphs on the global-aware pooling and locality-preserving
             modules; its formulas are stripped and its sentences shuffled).
  [digest]   Core Context Aware Transformers for Long Context Language Modeling,
             digest at digest.lyk-ai.com/posts/2412.12465 ("Method": the pooling
             formula and the fusion formula).
  [rebuttal] Core Context Aware Attention for Long Context Language Modeling,
             OpenReview rebuttal thread at paperhub.cn (answers on 128K context
             and on GQA).

Readings of points the pages leave open, and which functions have no pin from
the pages ("parity unpinned"), are listed in ``cca_oracle``'s module docstring.
"""
from .cca_oracle import (  # noqa: F401
    n_core, win_lo, visibility, visible_pairs_total, cache_tokens,
    pool_core, pool_from_last, attn_prefill, attn_row, attn_decode, attn_rows, attn_rows_q,
)
