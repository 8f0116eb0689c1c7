"""CPU oracle (test infrastructure only).

Plain float64 numpy definitions of the MISA / MISA-dagger / HISA indexer steps,
used by the tests, the smoke check and the benchmark's CPU-baseline leg to
check and time the HIP library.  Nothing in the HIP library's product path may
import or call this package, and it shares no code with that library.
"""
from .indexer import (KDT_BF16, KDT_FP8, QDT_BF16, QDT_FP8, Problem, dequant_queries, block_logits, block_means, block_ranges,
                      decode_bf16, decode_e4m3fn, dense_scores, dense_topk, dequant_keys,
                      block_maxima, first_k, full_block_means, head_logits, hisa_block_scores, hisa_topk,
                      magnitude_terms, misa_hier_topk, misa_hisa_topk, misa_topk, route,
                      routed_block_scores, routed_scores)

__all__ = ["KDT_BF16", "KDT_FP8", "QDT_BF16", "QDT_FP8", "Problem", "dequant_queries", "block_logits", "block_means", "block_ranges",
           "decode_bf16", "decode_e4m3fn", "dense_scores", "dense_topk", "dequant_keys",
           "block_maxima", "first_k", "full_block_means", "head_logits", "hisa_block_scores", "hisa_topk",
           "magnitude_terms", "misa_hier_topk", "misa_hisa_topk", "misa_topk", "route",
           "routed_block_scores", "routed_scores"]
