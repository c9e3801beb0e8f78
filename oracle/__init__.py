"""Plain, slow, fp64 CPU oracle of the paged MLA latent cache with a DSA-style indexer.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or load
this package: only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` use it. It shares no code, header, table or constant
generator with the HIP library; both sides read only the seeded inputs of
``synth``.

Sources (web pages, cited by title and section):

* [#1313] "GLM-5.3-Flash CUDA at TP=2: --parallel 8 at a 1M window is refused
  ... though KV pages would serve it" (issue 1313): the plan's order, window
  pages, FP8 rows with per-page scale blocks, the owner split.
* [#1732] "TF_GLM_KV_SHARE=n with TF_KV_PAGES=on keeps GLM's prompts as the
  pool's pages" (pull request 1732): marks, lookahead, pages held by reference.
* [#1312] "GLM-5.3-Flash on CUDA cannot keep conversation states on disk"
  (issue 1312): rows by position in a kept state.
* [CPM] "Running CHUNKED_PREFILL_SIZE above 1024 without the long-prompt memory
  problem" (chunked-prefill-memory): the indexer's masked fp32 MQA logits
  (section 1), the adaptive chunk rule (section 2.1), blocked top-k (2.3).
* [#1142] "Proposal: GLM-5.3-Flash on CUDA takes its streams' KV pages from the
  core pool, and kept prompt states copy only their rows" (issue 1142): page
  tables, 512-row pages, a null table as contiguous rows, snapshots of the
  first ``at`` rows, bytes per token.

Each function names the passage it follows. Where the pages are silent the
reading taken is stated in the function's docstring.

Parity status: every function here is pinned by the ``-m "not gpu"`` tests
except the softmax scale (a free call argument: no page fixes it) and the
pooling that produces pooled keys (the pages never define it; keys are inputs).
"""
from .layout import Geom, BlockLayout, block_layout, page_bytes, PoolImage  # noqa: F401
from .plan import bytes_per_token, bytes_per_token_rank, kv_pool_plan, Plan  # noqa: F401
from .schedule import chunk_size, chunk_schedule  # noqa: F401
from .indexer import n_compressed, indexer_logits  # noqa: F401
from .topk import topk_blocks, candidate_groups, topk_in_candidates  # noqa: F401
from .attention import selected_tokens, sparse_mla_row, sparse_mla  # noqa: F401
from .attention import dense_tokens, dense_mla_row, dense_mla  # noqa: F401
from .fp8 import e4m3_decode, e4m3_encode_nearest, quantize_rows  # noqa: F401
