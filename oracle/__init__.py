"""CPU oracle of the DSA hot path -- TEST INFRASTRUCTURE ONLY.

A plain, slow, fp64 numpy implementation of what the GPU path computes:
dense index scores, exact top-k with ties to the lower index, and softmax
attention over the kept set (MLA in MQA mode).  Only tests/,
__graft_entry__.smoke() and bench.py's cpu_baseline leg may import it; the
product path (long_context_sparse_06_amd) never does, and the two share no code.

Pinning status: every function here is pinned by `-m "not gpu"` tests against
closed forms, exact rational arithmetic, library routines or hand-worked golden
cases (tests/test_oracle.py, tests/golden/).  One reading stays unverifiable from
the pages -- the indexer's formula itself (ReLU of per-head dots, weighted by w
and scaled per token): parity is against this reading only.
"""
from .dsa import (attention_pairs, dense_attention_distribution, dense_causal_mla, encode_e4m3,
                  index_scores, indexer_kl_reverse, indexer_quality, kth_score, logical_rows,
                  quantize_key, sparse_mla, topk)
from .formats import E4M3_TABLE, decode_bf16, decode_e4m3
from . import pipeline

__all__ = [
    "attention_pairs", "dense_attention_distribution", "dense_causal_mla", "encode_e4m3",
    "index_scores", "indexer_kl_reverse", "indexer_quality", "kth_score",
    "logical_rows", "quantize_key", "sparse_mla", "topk", "E4M3_TABLE", "decode_bf16", "decode_e4m3", "pipeline",
]
