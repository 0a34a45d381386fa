"""CPU oracle for headwise hybrid attention (TEST INFRASTRUCTURE ONLY).

A plain, slow, obviously-correct numpy implementation in fp32 of what the HIP
library computes. It exists to check the GPU path and nothing else: only
``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import it. The product path never calls it and shares no
code, table or helper with it.

Sources (the pages are web articles; cited by title and section):

* "阿里Qwen3 RTPurbo：15%全量Attention长文本5倍压缩方案" (Synced repost),
  section "化繁为简，被低估的 SWA": a small share of heads keep full-range
  attention, the rest use sliding-window attention (scheme one).
* "阿里RTPurboV2：Transformer再次崛起，百步训练实现10倍稀少把稳", paragraphs
  on the low-rank projector (D -> r = 16), on clustering in the low-rank space,
  on K-cache clustering for decode, and on the all-sparse variant
  (``cluster.py``: k-means of the projected keys and the decode step that
  chooses among clusters).
* aitop.news summary of "Full Attention Strikes Back": a 16-dimensional
  indexer guesses which earlier tokens matter, and the real attention then
  runs only on that selected set.

The block rule (64-token blocks; keep the sink block, the diagonal block and
the top-k candidate blocks by max over the block of the block-mean projected
query dotted with projected keys) is this library's reading of the indexer;
the pages leave it open.

Parity status: every function here is pinned by tests under ``tests/``
(closed forms, library special cases, brute force, constructed cases).
"""
from .numerics import bf16_to_f32, f32_to_bf16, round_bf16  # noqa: F401
from .prefill import (  # noqa: F401
    project_keys, query_block_means, block_score_row, select_row,
    retrieval_selection, block_centroids, swa_keys, selected_keys,
    swa_block_keys, retrieval_block_keys, attend,
    hybrid_prefill,
)
from .decode import decode_centroids, decode_select, hybrid_decode  # noqa: F401
from .cluster import (  # noqa: F401
    cluster_count, cluster_keys, lloyd_step, nearest_centroid, group_members,
    clustered_select, kept_tokens, clustered_decode,
)
