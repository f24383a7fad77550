"""Plain fp64 CPU oracle of the DSA hot path (test infrastructure).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may use
this module.  It shares no code with the HIP path.

Sources (the pages):
  [MTP] MarkTechPost, "DeepSeek V3.2-Exp Cuts Long-Context Costs with DeepSeek
        Sparse Attention (DSA) While Maintaining Benchmark Parity": the two-tier
        pipeline (FP8 indexer, then top-k, then core attention on the kept tokens); the
        "Training signal" paragraph (top-k = 2048); the "Instantiation"
        paragraph (MLA in MQA mode, one latent KV entry shared by all heads).
  [MV]  maplevalley.com.cn news 1594152, section "1. 细粒度稀疏架构" (Lightning
        Indexer + Top-k Token Selection; each query keeps k key/value pairs;
        O(L^2) -> O(Lk)).
  [TW]  tellworld.net, "DeepSeek debuts sparse attention in DeepSeek-V3.2-Exp and
        halves API prices", "What happened" (token-level, not block, selection).

Readings where the pages are silent (each is listed with its reason in the
design notes):
  * index score  I[t,s] = k_scale[s] * q_scale[t] * sum_j w[t,j] * ReLU(q[t,j,:] . k[s,:])
    (the pages only say a lightweight FP8 indexer scores context tokens);
  * candidates of query t are s <= t (self included);
  * top-k ties go to the lower index; fewer than k candidates -> keep all;
  * softmax scale is an explicit argument; V is the first Dv columns of the
    same latent row; lse is the natural-log log-sum-exp of the scaled logits;
  * an empty selection gives o = 0 and lse = -inf.
"""
from __future__ import annotations

import numpy as np

from .formats import E4M3_TABLE


# ----------------------------------------------------------------------------
# tier 1: lightning indexer  ([MTP] pipeline, [MV] section 1)
# ----------------------------------------------------------------------------
def index_scores(q: np.ndarray, q_scale: float, w: np.ndarray, keys: np.ndarray,
                 k_scale: np.ndarray) -> np.ndarray:
    """Index scores of one query row against n keys.

    q [H_I, d_I] (decoded values), q_scale scalar, w [H_I], keys [n, d_I]
    (decoded), k_scale [n]  ->  scores [n] float64.

    For e4m3 inputs every head's dot product is exact in fp64: each product of
    two e4m3 values is a multiple of 2^-18 below 448^2, and 128 of them stay far
    inside fp64's 53-bit significand.
    """
    q = np.asarray(q, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    acc = np.zeros(keys.shape[0], dtype=np.float64)
    for j in range(q.shape[0]):
        dot = keys @ q[j]
        acc += w[j] * np.maximum(dot, 0.0)
    return acc * np.asarray(k_scale, dtype=np.float64) * float(q_scale)


def logical_rows(pool: np.ndarray, table_row: np.ndarray, page_size: int,
                 positions: np.ndarray) -> np.ndarray:
    """Rows of a paged pool [P, page_size, ...] at logical token positions.

    Physical row of logical position s is table_row[s // page_size] * page_size
    + s % page_size.
    """
    positions = np.asarray(positions, dtype=np.int64)
    flat = pool.reshape((-1,) + pool.shape[2:])
    phys = table_row[positions // page_size].astype(np.int64) * page_size + positions % page_size
    return flat[phys]


# ----------------------------------------------------------------------------
# top-k selection ([MV] section 1: per query keep k key/value pairs; [TW]: token level)
# ----------------------------------------------------------------------------
def topk(scores: np.ndarray, k: int) -> np.ndarray:
    """Indices of the min(k, n) largest scores, ties to the lower index, sorted ascending.

    -0.0 and +0.0 compare equal (IEEE ordering), so they tie.
    """
    scores = np.asarray(scores, dtype=np.float64)
    n = scores.shape[0]
    if n <= k:
        return np.arange(n, dtype=np.int64)
    order = np.lexsort((np.arange(n), -scores))  # primary: score descending, then index ascending
    return np.sort(order[:k])


def kth_score(scores: np.ndarray, k: int) -> float:
    """Score of the k-th ranked candidate (the selection threshold tau)."""
    scores = np.asarray(scores, dtype=np.float64)
    if scores.shape[0] <= k:
        return float(scores.min()) if scores.shape[0] else float("nan")
    return float(-np.sort(-scores)[k - 1])


# ----------------------------------------------------------------------------
# tier 2: sparse core attention, MLA in MQA mode ([MTP] "Instantiation")
# ----------------------------------------------------------------------------
def sparse_mla(q: np.ndarray, kv_rows: np.ndarray, dv: int, scale: float):
    """Softmax attention of H query heads over m shared latent rows.

    q [H, Dqk], kv_rows [m, Dqk]  ->  (o [H, dv], lse [H]).
    logits z = scale * q . row; o = softmax(z) @ rows[:, :dv]; lse = log sum exp z.
    """
    q = np.asarray(q, dtype=np.float64)
    kv_rows = np.asarray(kv_rows, dtype=np.float64)
    H = q.shape[0]
    if kv_rows.shape[0] == 0:
        return np.zeros((H, dv)), np.full(H, -np.inf)
    z = scale * (q @ kv_rows.T)
    zmax = z.max(axis=1, keepdims=True)
    e = np.exp(z - zmax)
    den = e.sum(axis=1)
    o = (e @ kv_rows[:, :dv]) / den[:, None]
    lse = zmax[:, 0] + np.log(den)
    return o, lse


def dense_causal_mla(q: np.ndarray, kv: np.ndarray, dv: int, scale: float):
    """Dense causal MLA over one sequence: query t attends to rows 0..t.

    q [T, H, Dqk], kv [T, Dqk] -> (o [T, H, dv], lse [T, H]).
    """
    T, H, _ = q.shape
    o = np.zeros((T, H, dv))
    lse = np.zeros((T, H))
    for t in range(T):
        o[t], lse[t] = sparse_mla(q[t], kv[: t + 1], dv, scale)
    return o, lse


def attention_pairs(idx_sets) -> int:
    """Number of (query, key) pairs core attention touches."""
    return int(sum(len(s) for s in idx_sets))


# ----------------------------------------------------------------------------
# cache append: the new token's indexer key stored as FP8 ([MTP]: the indexer runs in FP8)
# ----------------------------------------------------------------------------
E4M3_MAX = 448.0


def encode_e4m3(y: np.ndarray) -> np.ndarray:
    """Finite values with |y| <= 448 -> e4m3fn codes, rounding to nearest, ties to even.

    The positive finite codes 0x00..0x7E are the magnitudes in increasing order, so the
    two neighbours of |y| are adjacent codes; on a tie the even code (even mantissa) wins.
    The sign goes to bit 7 (so -0.0 encodes as 0x80).
    """
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    if np.any(a > E4M3_MAX) or np.any(np.isnan(y)):
        raise ValueError("encode_e4m3 takes finite values with |y| <= 448")
    mags = E4M3_TABLE[:0x7F]                       # codes 0x00 .. 0x7E, increasing
    hi = np.searchsorted(mags, a, side="left")     # first code with value >= a
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - mags[lo]
    d_hi = mags[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(a == mags[hi], hi, np.where(pick_hi, hi, lo)).astype(np.uint8)
    neg = np.signbit(y)
    return (code | np.where(neg, 0x80, 0).astype(np.uint8)).astype(np.uint8)


def quantize_key(x: np.ndarray):
    """Per-token e4m3 quantisation of indexer keys x [..., d] (float32).

    scale = amax / 448 (1 when the row is all zero), y = clamp(x / scale, -448, 448),
    codes = e4m3(y) rounded to nearest even.  The scale and the division are float32,
    the precision the stored scale has and the kernel computes in, so both sides take
    the same rounding decisions.  Returns (codes uint8 [..., d], scale float32 [...]).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    amax = np.max(np.abs(x), axis=-1)
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    y = (x / scale[..., None]).astype(np.float32)
    y = np.clip(y, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
    return encode_e4m3(y), scale


# ----------------------------------------------------------------------------
# indexer-quality diagnostic ([MTP] "Training signal": a KL loss pulls the indexer's
# distribution towards the dense attention summed over heads)
# ----------------------------------------------------------------------------
def dense_attention_distribution(q: np.ndarray, kv_rows: np.ndarray, scale: float) -> np.ndarray:
    """Head-summed dense attention over n candidate rows, normalised to a distribution.

    q [H, Dqk], kv_rows [n, Dqk] -> p [n] = (1/H) sum_h softmax_s(scale * q_h . row_s).
    """
    q = np.asarray(q, dtype=np.float64)
    kv_rows = np.asarray(kv_rows, dtype=np.float64)
    z = scale * (q @ kv_rows.T)                     # [H, n]
    z = z - z.max(axis=1, keepdims=True)
    e = np.exp(z)
    return (e / e.sum(axis=1, keepdims=True)).mean(axis=0)


def indexer_quality(p_attn: np.ndarray, scores: np.ndarray, kept) -> tuple:
    """(KL(p_attn || softmax(scores)), attention mass of the kept set) for one query row.

    p_attn [n] the dense distribution (the imitation target), scores [n] the index scores,
    kept the selected positions.  KL in nats; terms with p_attn = 0 contribute 0.
    """
    p = np.asarray(p_attn, dtype=np.float64)
    i = np.asarray(scores, dtype=np.float64)
    log_q = i - i.max()
    log_q = log_q - np.log(np.exp(log_q).sum())
    nz = p > 0
    kl = float(np.sum(p[nz] * (np.log(p[nz]) - log_q[nz])))
    kept = np.asarray(kept, dtype=np.int64)
    kept = kept[kept >= 0]
    recall = float(p[kept].sum())
    return kl, recall


def indexer_kl_reverse(p_attn: np.ndarray, scores: np.ndarray) -> float:
    """KL(softmax(scores) || p_attn) in nats: the other direction of the diagnostic's KL (the
    pages name a KL term without fixing its order).  Infinite where p_attn = 0 < softmax."""
    p = np.asarray(p_attn, dtype=np.float64)
    i = np.asarray(scores, dtype=np.float64)
    log_q = i - i.max()
    log_q = log_q - np.log(np.exp(log_q).sum())
    q = np.exp(log_q)
    with np.errstate(divide="ignore"):
        return float(np.sum(q * (log_q - np.log(p))))

