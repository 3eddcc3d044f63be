"""CPU oracle for dynamic sparse attention — TEST INFRASTRUCTURE ONLY.

A plain, slow fp64 NumPy statement of what the sparse attention path
computes.  Only the test-suite, the smoke check and the CPU-baseline leg of the
benchmark may import it; the library itself never does, and shares no code,
constant or table with it (the HIP path lives in
``dynamic_sparse_attention_pool_amd``).

Sources (cited by page title and section in each function):
  * "MInference 1.0" article — §方法介紹 (three per-head patterns: A-shape,
    vertical-slash and block-sparse; block-sparse estimate by mean-pooled
    Q and K, vertical-slash estimate from the last queries) and
    §延遲和內核中的稀疏模式, Fig. 4 (verticals in 1x64 pieces, slashes in
    64x64 blocks).
  * "Squeezed Attention：基于语义聚类的长上下文LLM推理加速" — §技术方案
    (offline k-means of the context keys; query-centroid similarity, top-K
    clusters, attention over their keys; the number of clusters adapting to
    the similarity distribution) and
    §部署建议 (K = sqrt(N) clusters, select 1/4 to 1/2 of them).
  * IndexCache article — §长文本的算力困境 (lightning indexer keeps a token
    subset per layer) and §"偷懒"的艺术 (shared layers copy the nearest full
    layer's indices).
  * "稀疏注意力机制解析" explainer — §1.1 (dense attention is the O(n^2)
    baseline) and §1.2 (local-window and global-token patterns).

Readings where the pages are silent are listed next to the code that takes
them.  Functions with no independent pin say "parity unpinned" in their
docstring.
"""
from .select import (candidate_count, forced_set, budget, topk_row, select_rows,
                     certified_row, ratio_budget, mass_weights, mass_count, mass_row, mass_margin)
from .attention import attend_rows, gqa_group
from .blocksparse import mean_pool, block_scores, block_select, block_sparse_attention
from .vslash import vs_estimate, vs_select, vs_block_keys, vs_block_tables, vs_attention
from .cluster import centroid_scores, cluster_select, cluster_select_mass, cluster_pack, cluster_decode
from .indexer import indexer_scores, indexer_select, gathered_attention, index_cache_forward
from .kmeans import assign as kmeans_assign, kmeans, objective as kmeans_objective
from .patterns import A_SHAPE, VERTICAL_SLASH, BLOCK_SPARSE, ashape_blocks, ashape_attention, mixed_layer

__all__ = [
    "candidate_count", "forced_set", "budget", "topk_row", "select_rows", "certified_row",
    "ratio_budget", "mass_weights", "mass_count", "mass_row", "mass_margin", "attend_rows",
    "gqa_group", "mean_pool", "block_scores", "block_select", "block_sparse_attention",
    "vs_estimate", "vs_select", "vs_block_keys", "vs_block_tables", "vs_attention",
    "centroid_scores", "cluster_select", "cluster_select_mass", "cluster_pack", "cluster_decode",
    "indexer_scores", "indexer_select", "gathered_attention", "index_cache_forward",
    "A_SHAPE", "VERTICAL_SLASH", "BLOCK_SPARSE", "ashape_blocks", "ashape_attention", "mixed_layer",
    "kmeans", "kmeans_assign", "kmeans_objective",
]
