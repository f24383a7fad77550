"""Whole-path oracle: index scores -> top-k -> sparse MLA (test infrastructure).

Works on the storage bytes the GPU receives (e4m3 codes + fp32 scales, bf16 bit
patterns) and decodes them with this package's own decoders.  The order of the
steps is the pages' pipeline -- FP8 indexer, then top-k, then core attention over the
kept tokens (MarkTechPost, "DeepSeek V3.2-Exp Cuts Long-Context Costs with
DeepSeek Sparse Attention (DSA) ...").
"""
from __future__ import annotations

import numpy as np

from .dsa import (dense_attention_distribution, index_scores, indexer_kl_reverse, indexer_quality,
                  logical_rows, sparse_mla, topk)
from .formats import decode_bf16, decode_e4m3


def _dec_idx(x):
    return decode_e4m3(x) if x.dtype == np.uint8 else np.asarray(x, dtype=np.float64)


def _dec_lat(x):
    return decode_bf16(x) if x.dtype == np.uint16 else np.asarray(x, dtype=np.float64)


# ------------------------------------------------------------------ decode
def decode_keys(inp, b: int, positions=None):
    """Decoded indexer keys and scales of sequence b at logical positions."""
    L = int(inp.lengths[b])
    if positions is None:
        positions = np.arange(L)
    if inp.block_table is not None:
        k = logical_rows(inp.keys, inp.block_table[b], inp.page_size, positions)
        sc = logical_rows(inp.k_scale, inp.block_table[b], inp.page_size, positions)
    else:
        k = inp.keys[b][positions]
        sc = inp.k_scale[b][positions]
    return _dec_idx(k), np.asarray(sc, dtype=np.float64)


def decode_kv_rows(inp, b: int, positions):
    positions = np.asarray(positions, dtype=np.int64)
    if inp.block_table is not None:
        rows = logical_rows(inp.kv, inp.block_table[b], inp.page_size, positions)
    else:
        rows = inp.kv[b][positions]
    return _dec_lat(rows)


def decode_scores(inp, b: int) -> np.ndarray:
    """Index scores of sequence b's query (its last token) against all L_b tokens."""
    keys, ks = decode_keys(inp, b)
    return index_scores(_dec_idx(inp.q_idx[b]), float(inp.q_scale[b]), inp.w[b], keys, ks)


def decode_attention(inp, b: int, idx, scale: float):
    """Sparse MLA of sequence b over the logical positions `idx` (entries < 0 ignored)."""
    idx = np.asarray(idx)
    idx = idx[idx >= 0]
    rows = decode_kv_rows(inp, b, idx)
    return sparse_mla(_dec_lat(inp.q[b]), rows, inp.shapes.Dv, scale)


def decode_step(inp, scale: float, k: int = None, rows=None):
    """Full decode step for the listed sequences (default: all).

    Returns dict with per-sequence lists: scores, idx (sorted), o [H,Dv], lse [H].
    """
    k = inp.shapes.k if k is None else k
    rows = range(inp.B) if rows is None else rows
    out = {"scores": [], "idx": [], "o": [], "lse": []}
    for b in rows:
        s = decode_scores(inp, b)
        sel = topk(s, k)
        o, lse = decode_attention(inp, b, sel, scale)
        out["scores"].append(s)
        out["idx"].append(sel)
        out["o"].append(o)
        out["lse"].append(lse)
    return out


# ------------------------------------------------------------------ prefill
def prefill_scores(inp, t: int) -> np.ndarray:
    """Index scores of query token t against tokens 0..t of the same sequence."""
    keys = _dec_idx(inp.keys[: t + 1])
    return index_scores(_dec_idx(inp.q_idx[t]), float(inp.q_scale[t]), inp.w[t], keys,
                        np.asarray(inp.k_scale[: t + 1], dtype=np.float64))


def prefill_attention(inp, t: int, idx, scale: float):
    idx = np.asarray(idx)
    idx = idx[idx >= 0]
    return sparse_mla(_dec_lat(inp.q[t]), _dec_lat(inp.kv[idx]), inp.shapes.Dv, scale)


def prefill(inp, scale: float, k: int = None, rows=None):
    """Causal prefill for the listed query tokens (default: all)."""
    k = inp.shapes.k if k is None else k
    rows = range(inp.T) if rows is None else rows
    out = {"scores": [], "idx": [], "o": [], "lse": []}
    for t in rows:
        s = prefill_scores(inp, t)
        sel = topk(s, k)
        o, lse = prefill_attention(inp, t, sel, scale)
        out["scores"].append(s)
        out["idx"].append(sel)
        out["o"].append(o)
        out["lse"].append(lse)
    return out


def decode_indexer_quality(inp, b: int, scale: float, kept, scores=None, reverse=False):
    """KL(dense head-summed attention || softmax(index scores)) and the kept set's attention
    mass for sequence b's query (all L_b cached tokens are candidates); with `reverse`, also
    KL(softmax(index scores) || dense), returned third."""
    L = int(inp.lengths[b])
    rows = decode_kv_rows(inp, b, np.arange(L))
    p = dense_attention_distribution(_dec_lat(inp.q[b]), rows, scale)
    s = decode_scores(inp, b) if scores is None else np.asarray(scores, dtype=np.float64)
    kl, recall = indexer_quality(p, s, kept)
    return (kl, recall, indexer_kl_reverse(p, s)) if reverse else (kl, recall)

