"""Pins of the CPU oracle against things other than itself (CPU only).

Each pin is chosen so that a plausible mistake in the oracle fails it:
  * decoders vs torch's own float8_e4m3fn / bfloat16 casts (all codes) and closed forms;
  * index scores vs a hand-worked golden case, a closed form (one-hot queries
    select positive parts of key coordinates), exact rational arithmetic, sign
    and scale special cases, and paged == contiguous addressing;
  * top-k vs brute force over all subsets, torch.topk on distinct values, a
    hand-ranked tie case, and structural invariants;
  * sparse MLA vs a hand-worked golden case, closed forms (single row, zero
    query, two rows), torch's scaled_dot_product_attention for the dense
    causal case (k >= L), and permutation invariance;
  * the O(Lk) pair count vs its closed form;
  * the e4m3 encoder vs the decoder on every code, hand-worked ties (to even) and
    subnormals, and torch's float8_e4m3fn cast; the key quantiser vs its closed-form
    consequences (the largest magnitude maps to +-448, zero rows keep scale 1, the
    dequantised value is within half an e4m3 step of the input).
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import datagen
import oracle
from oracle import pipeline
from oracle.dsa import dense_causal_mla, index_scores, kth_score, sparse_mla, topk
from oracle.formats import decode_bf16, decode_e4m3


# ----------------------------------------------------------------------------- formats
def test_e4m3_decoder_matches_torch_on_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    got = decode_e4m3(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.signbit(got[0x80]) and got[0x80] == 0.0


def test_e4m3_closed_forms():
    d = decode_e4m3(np.array([0x7E, 0x01, 0x08, 0x38, 0xB8, 0x00, 0x07], dtype=np.uint8))
    assert d[0] == 448.0                 # 1.75 * 2^8, largest finite
    assert d[1] == 2.0 ** -9             # smallest subnormal
    assert d[2] == 2.0 ** -6             # smallest normal
    assert d[3] == 1.0 and d[4] == -1.0 and d[5] == 0.0
    assert d[6] == 7 / 8 * 2.0 ** -6     # largest subnormal


def test_e4m3_encoder_inverts_the_decoder_on_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(oracle.encode_e4m3(decode_e4m3(codes)), codes)


def test_e4m3_encoder_ties_go_to_even_and_subnormals_by_hand():
    # midpoints between neighbouring codes, worked by hand from the format definition
    cases = {1.0625: 0x38,          # between 1.0 (0x38) and 1.125 (0x39): even 0x38
             1.1875: 0x3A,          # between 1.125 (0x39) and 1.25 (0x3A): even 0x3A
             1.5 * 2.0 ** -9: 0x02,  # between subnormals 1 and 2 (x 2^-9): even 2
             2.5 * 2.0 ** -9: 0x02,  # between 2 and 3: even 2
             7.5 * 2.0 ** -9: 0x08,  # between the largest subnormal and 2^-6: 0x08
             432.0: 0x7E,           # between 416 (0x7D) and 448 (0x7E): even 0x7E
             0.3 * 2.0 ** -9: 0x00,  # below half the smallest subnormal: zero
             -1.0625: 0xB8}
    got = oracle.encode_e4m3(np.array(list(cases.keys())))
    assert got.tolist() == list(cases.values())


def test_e4m3_encoder_matches_torch_cast():
    rng = np.random.default_rng(5)
    y = np.concatenate([rng.uniform(-448, 448, 20000), rng.standard_normal(20000) * 0.01,
                        rng.standard_normal(2000) * 2.0 ** -8]).astype(np.float32)
    ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.encode_e4m3(y), ref)


def test_quantize_key_closed_forms():
    rng = np.random.default_rng(6)
    x = rng.standard_normal((50, 128)).astype(np.float32)
    x[3] = 0.0
    x[4] = 1e-30
    codes, scale = oracle.quantize_key(x)
    assert scale.dtype == np.float32 and scale[3] == 1.0 and (codes[3] == 0).all()
    amax_at = np.argmax(np.abs(x), axis=1)
    top = codes[np.arange(50), amax_at]
    assert ((top & 0x7F) == 0x7E)[np.arange(50) != 3].all()          # +-448
    back = decode_e4m3(codes) * scale[:, None].astype(np.float64)
    err = np.abs(back - x)
    step = np.maximum(np.abs(x) * 2.0 ** -4, scale[:, None] * 2.0 ** -10)  # half an e4m3 step
    assert (err <= step * (1 + 1e-6)).all()


def test_bf16_decoder_matches_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    got = decode_bf16(bits)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert decode_bf16(np.array([0x3F80, 0xC000], dtype=np.uint16)).tolist() == [1.0, -2.0]


# ----------------------------------------------------------------------------- index scores
def test_index_scores_golden(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "index_scores_small.json")))
    s = index_scores(np.array(g["q"]), g["q_scale"], np.array(g["w"]), np.array(g["keys"]),
                     np.array(g["k_scale"]))
    assert s.tolist() == g["expected"]
    assert topk(s, 2).tolist() == g["expected_top2"]
    assert topk(s, 3).tolist() == g["expected_top3"]


def test_index_scores_one_hot_queries_closed_form():
    # q_j = e_j (unit vector on coordinate j), w = 1: score = ks*qs*sum_{j<H} max(k[s,j], 0).
    rng = np.random.default_rng(1)
    H, d, n = 5, 9, 40
    q = np.eye(d)[:H]
    keys = rng.standard_normal((n, d))
    ks = rng.uniform(0.5, 2.0, n)
    s = index_scores(q, 1.5, np.ones(H), keys, ks)
    expect = ks * 1.5 * np.clip(keys[:, :H], 0, None).sum(axis=1)
    np.testing.assert_allclose(s, expect, rtol=1e-14, atol=0)
    # one-hot w at head j with q_j = c * e_m: ks*qs*max(c*k[s,m], 0)
    w = np.zeros(H); w[3] = 1.0
    q2 = np.zeros((H, d)); q2[3, 7] = -2.0
    s2 = index_scores(q2, 1.0, w, keys, ks)
    np.testing.assert_allclose(s2, ks * np.maximum(-2.0 * keys[:, 7], 0), rtol=1e-14, atol=0)


def test_index_scores_signs_and_scales():
    rng = np.random.default_rng(2)
    H, d, n = 4, 16, 64
    q = rng.standard_normal((H, d)); keys = rng.standard_normal((n, d))
    w = rng.uniform(0, 1, H); ks = rng.uniform(0.1, 1, n)
    s = index_scores(q, 1.0, w, keys, ks)
    assert (s >= 0).all()                                    # ReLU and w >= 0
    np.testing.assert_allclose(index_scores(q, 1.0, -w, keys, ks), -s, rtol=0, atol=0)
    np.testing.assert_allclose(index_scores(q, 3.0, w, keys, 2 * ks), 6 * s, rtol=1e-15)
    assert np.all(index_scores(np.zeros((H, d)), 1.0, w, keys, ks) == 0)
    # ReLU is applied per head before weighting: with q_1 = -q_0 and equal w, every
    # key contributes |q_0 . k| (a linear head sum would give exactly 0).
    q2 = np.stack([q[0], -q[0]])
    s2 = index_scores(q2, 1.0, np.ones(2), keys, np.ones(n))
    np.testing.assert_allclose(s2, np.abs(keys @ q[0]), rtol=1e-14)


def test_index_scores_exact_rational_on_e4m3_inputs():
    rng = np.random.default_rng(3)
    H, d, n = 3, 8, 6
    qc = rng.integers(0, 256, (H, d)).astype(np.uint8)
    kc = rng.integers(0, 256, (n, d)).astype(np.uint8)
    qc[(qc & 0x7F) == 0x7F] = 0x38
    kc[(kc & 0x7F) == 0x7F] = 0x38
    q = decode_e4m3(qc); k = decode_e4m3(kc)
    w = rng.uniform(0, 1, H).astype(np.float32); ks = rng.uniform(0.01, 1, n).astype(np.float32)
    qs = np.float32(0.37)
    got = index_scores(q, float(qs), w.astype(np.float64), k, ks.astype(np.float64))
    for s in range(n):
        acc = Fraction(0)
        for j in range(H):
            dot = sum(Fraction(float(q[j, e])) * Fraction(float(k[s, e])) for e in range(d))
            # each per-head dot is exact in fp64 (products are multiples of 2^-18 below 448^2)
            assert Fraction(float(k[s] @ q[j])) == dot
            acc += Fraction(float(w[j])) * max(dot, Fraction(0))
        exact = acc * Fraction(float(ks[s])) * Fraction(float(qs))
        assert abs(Fraction(got[s]) - exact) <= abs(exact) * Fraction(1, 2 ** 50)


def test_paged_equals_contiguous_addressing():
    sh = datagen.Shapes(H=2, Dqk=24, Dv=16, HI=2, dI=8, k=8)
    lengths = np.array([70, 5, 130, 64])
    a = datagen.make_decode(4, None, sh, seed=5, lengths=lengths)
    b = datagen.make_decode(4, None, sh, seed=5, lengths=lengths, paged=True, page_size=16)
    assert b.block_table.shape == (4, 9)
    # physical pages are a permutation: each used exactly once
    used = b.block_table[b.block_table >= 0]
    assert sorted(used.tolist()) == list(range(b.keys.shape[0]))
    for i in range(4):
        np.testing.assert_array_equal(pipeline.decode_scores(a, i), pipeline.decode_scores(b, i))
        idx = np.arange(0, lengths[i], 3)
        np.testing.assert_array_equal(pipeline.decode_kv_rows(a, i, idx), pipeline.decode_kv_rows(b, i, idx))


def test_logical_rows_formula_by_hand():
    pool = np.arange(4 * 2 * 1).reshape(4, 2, 1)   # 4 pages of 2 rows; row value = physical row
    table = np.array([2, 0, 3])
    got = oracle.logical_rows(pool, table, 2, np.array([0, 1, 2, 3, 4, 5]))[:, 0]
    assert got.tolist() == [4, 5, 0, 1, 6, 7]


# ----------------------------------------------------------------------------- top-k
def _brute_force_topk(scores, k):
    """The unique k-subset whose every member outranks every non-member."""
    n = len(scores)
    if n <= k:
        return list(range(n))

    def beats(a, b):
        return scores[a] > scores[b] or (scores[a] == scores[b] and a < b)

    found = [S for S in itertools.combinations(range(n), k)
             if all(beats(a, b) for a in S for b in set(range(n)) - set(S))]
    assert len(found) == 1
    return list(found[0])


def test_topk_golden_ties(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "topk_ties.json")))
    s = np.array([float(x) for x in g["scores"]])
    assert np.signbit(s[6]) and not np.signbit(s[7])
    for k, exp in g["expected"].items():
        assert topk(s, int(k)).tolist() == exp


@pytest.mark.parametrize("seed", range(12))
def test_topk_brute_force_with_ties(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 10))
    vals = np.array([-1.0, -0.0, 0.0, 0.5, 2.0])
    s = vals[rng.integers(0, len(vals), n)]
    for k in range(1, n + 2):
        assert topk(s, k).tolist() == _brute_force_topk(s, k)


def test_topk_matches_torch_on_distinct_values():
    rng = np.random.default_rng(7)
    s = rng.permutation(5000).astype(np.float64) * 0.25 - 100
    for k in (1, 17, 2048, 4999):
        ref = torch.topk(torch.from_numpy(s), k).indices.numpy()
        assert topk(s, k).tolist() == sorted(ref.tolist())


def test_topk_structure():
    rng = np.random.default_rng(8)
    s = np.round(rng.standard_normal(300), 1)          # many ties
    prev = set()
    for k in range(1, 320):
        cur = topk(s, k)
        assert len(cur) == min(k, 300)
        assert set(prev) <= set(cur)                  # nested in k
        assert cur.min() >= 0 and cur.max() < 300
        prev = cur.tolist()
    assert topk(np.full(50, 3.0), 20).tolist() == list(range(20))
    assert topk(np.arange(50.0), 5).tolist() == [45, 46, 47, 48, 49]
    assert topk(np.zeros(0), 4).tolist() == []
    assert kth_score(np.array([3.0, 1.0, 2.0]), 2) == 2.0


# ----------------------------------------------------------------------------- sparse MLA
def test_sparse_mla_golden(golden_dir):
    g = json.load(open(os.path.join(golden_dir, "sparse_mla_small.json")))
    o, lse = sparse_mla(np.array(g["q"]), np.array(g["rows"]), g["dv"], g["scale"])
    env = {"e": math.e, "log": math.log}
    cf = g["expected_closed_form"]
    exp_o = np.array([[eval(x, env) for x in row] for row in cf["o"]])
    exp_lse = np.array([eval(x, env) for x in cf["lse"]])
    np.testing.assert_allclose(o, exp_o, rtol=1e-14)
    np.testing.assert_allclose(lse, exp_lse, rtol=1e-14)


def test_sparse_mla_closed_forms():
    rng = np.random.default_rng(9)
    H, D, dv = 3, 10, 6
    q = rng.standard_normal((H, D)); rows = rng.standard_normal((7, D))
    # one row: o = its value part exactly; lse = scale * q.k
    o, lse = sparse_mla(q, rows[:1], dv, 0.3)
    assert np.array_equal(o, np.broadcast_to(rows[0, :dv], (H, dv)))
    np.testing.assert_allclose(lse, 0.3 * (q @ rows[0]), rtol=1e-15)
    # zero query: uniform weights
    o, lse = sparse_mla(np.zeros((H, D)), rows, dv, 0.3)
    np.testing.assert_allclose(o, np.broadcast_to(rows[:, :dv].mean(0), (H, dv)), rtol=1e-14)
    np.testing.assert_allclose(lse, np.log(7.0), rtol=1e-15)
    # two rows: sigmoid weights
    o, lse = sparse_mla(q, rows[:2], dv, 0.7)
    a = 0.7 * q @ rows[0]; b = 0.7 * q @ rows[1]
    p = 1.0 / (1.0 + np.exp(b - a))
    np.testing.assert_allclose(o, p[:, None] * rows[0, :dv] + (1 - p)[:, None] * rows[1, :dv], rtol=1e-13)
    np.testing.assert_allclose(lse, np.logaddexp(a, b), rtol=1e-14)
    # permutation invariance and the empty set
    perm = rng.permutation(7)
    o1, l1 = sparse_mla(q, rows, dv, 0.5); o2, l2 = sparse_mla(q, rows[perm], dv, 0.5)
    np.testing.assert_allclose(o1, o2, rtol=1e-13); np.testing.assert_allclose(l1, l2, rtol=1e-14)
    o, lse = sparse_mla(q, rows[:0], dv, 0.5)
    assert (o == 0).all() and np.isneginf(lse).all()


def test_dense_causal_matches_torch_sdpa():
    rng = np.random.default_rng(10)
    T, H, D, dv = 24, 3, 20, 12
    q = rng.standard_normal((T, H, D)); kv = rng.standard_normal((T, D))
    o, lse = dense_causal_mla(q, kv, dv, 0.2)
    Q = torch.from_numpy(q).permute(1, 0, 2)[None]                  # [1,H,T,D]
    K = torch.from_numpy(kv)[None, None].expand(1, H, T, D)          # shared by all heads (MQA)
    V = torch.from_numpy(kv[:, :dv].copy())[None, None].expand(1, H, T, dv)
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, is_causal=True, scale=0.2)
    np.testing.assert_allclose(o, ref[0].permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-13)
    # lse against torch.logsumexp of the masked logits
    z = 0.2 * torch.einsum("htd,sd->hts", Q[0], torch.from_numpy(kv))
    z = z.masked_fill(torch.triu(torch.ones(T, T, dtype=torch.bool), 1), float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(z, -1).T.numpy(), rtol=1e-13)


def test_sparse_equals_dense_when_k_covers_context():
    inp = datagen.make_config(1, T=48)
    s = inp.shapes
    scale = 1 / math.sqrt(s.Dqk)
    sp = pipeline.prefill(inp, scale, k=48)
    o_d, lse_d = dense_causal_mla(inp.q.astype(np.float64), inp.kv.astype(np.float64), s.Dv, scale)
    for t in range(48):
        assert sp["idx"][t].tolist() == list(range(t + 1))
        np.testing.assert_allclose(sp["o"][t], o_d[t], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(sp["lse"][t], lse_d[t], rtol=1e-12)


# ----------------------------------------------------------------------------- O(Lk)
def test_pair_count_is_o_lk():
    def closed(T, k):
        return k * (k + 1) // 2 + max(T - k, 0) * k if T >= k else T * (T + 1) // 2
    assert closed(256, 32) == 7696
    assert closed(32768, 2048) == 65_012_736
    inp = datagen.make_config(1)
    res = pipeline.prefill(inp, 1 / math.sqrt(80))
    assert oracle.attention_pairs(res["idx"]) == 7696
    for t, sel in enumerate(res["idx"]):
        assert len(sel) == min(t + 1, 32) and sel.max() <= t
    # dense causal attention touches T(T+1)/2 pairs; a 128K window is 1024x a 4K one
    assert (131072 * 131072) // (4096 * 4096) == 1024


def test_decode_row_equals_last_prefill_row():
    # the decode query of a sequence of length L is prefill row L-1 of the same tokens
    pre = datagen.make_config(1, T=40)
    s_pre = pipeline.prefill_scores(pre, 39)

    class D:  # decode view of the same bytes
        shapes = pre.shapes; lengths = np.array([40]); block_table = None; page_size = 0
        q_idx = pre.q_idx[39:40]; q_scale = pre.q_scale[39:40]; w = pre.w[39:40]
        keys = pre.keys[None]; k_scale = pre.k_scale[None]; q = pre.q[39:40]; kv = pre.kv[None]
    np.testing.assert_array_equal(pipeline.decode_scores(D, 0), s_pre)


# ----------------------------------------------------------------------------- indexer quality
def test_dense_attention_distribution_matches_scipy_softmax_mean():
    from scipy.special import softmax
    rng = np.random.default_rng(61)
    q = rng.standard_normal((5, 12))
    rows = rng.standard_normal((30, 12))
    ref = softmax(0.3 * (q @ rows.T), axis=1).mean(axis=0)
    got = oracle.dense_attention_distribution(q, rows, 0.3)
    assert np.allclose(got, ref, rtol=1e-13, atol=0) and abs(got.sum() - 1) < 1e-13
    # zero queries attend uniformly
    assert np.allclose(oracle.dense_attention_distribution(np.zeros((3, 12)), rows, 0.3), 1 / 30)


def test_indexer_quality_closed_forms_and_scipy_entropy():
    from scipy.special import softmax
    from scipy.stats import entropy
    rng = np.random.default_rng(62)
    p = softmax(rng.standard_normal(40))
    s = rng.standard_normal(40) * 3
    kl, rec = oracle.indexer_quality(p, s, np.arange(40))
    assert abs(kl - entropy(p, softmax(s))) < 1e-12
    assert abs(rec - 1.0) < 1e-12 and kl >= 0
    kl0, _ = oracle.indexer_quality(p, np.log(p) + 7.0, [])
    assert abs(kl0) < 1e-12                                   # scores = log target (+ const)
    kl_u, rec_u = oracle.indexer_quality(np.full(8, 1 / 8), np.zeros(8), [1, 3, -1])
    assert abs(kl_u) < 1e-15 and abs(rec_u - 0.25) < 1e-15   # uniform: mass 2/8
    # one head, two rows, worked by hand: z = (0, ln 3) -> p = (1/4, 3/4); scores (0, 0)
    p2 = oracle.dense_attention_distribution(np.array([[1.0]]), np.array([[0.0], [np.log(3)]]), 1.0)
    assert np.allclose(p2, [0.25, 0.75], atol=1e-15)
    kl2, rec2 = oracle.indexer_quality(p2, np.zeros(2), [1])
    assert abs(kl2 - (0.25 * np.log(0.5) + 0.75 * np.log(1.5))) < 1e-15 and abs(rec2 - 0.75) < 1e-15



def test_indexer_kl_reverse_pins():
    """The other KL direction, KL(softmax(scores) || p): scipy's relative entropy with the
    arguments swapped, zero for scores = log p + c, a two-token case by hand, and infinity
    where the target has a zero the indexer does not."""
    from scipy.special import softmax
    from scipy.stats import entropy
    rng = np.random.default_rng(63)
    p = softmax(rng.standard_normal(40))
    s = rng.standard_normal(40) * 3
    klr = oracle.indexer_kl_reverse(p, s)
    assert abs(klr - entropy(softmax(s), p)) < 1e-12 and klr >= 0
    assert abs(klr - oracle.indexer_quality(p, s, [])[0]) > 1e-3       # not the forward KL
    assert abs(oracle.indexer_kl_reverse(p, np.log(p) - 2.5)) < 1e-12
    # q = softmax(0, ln 3) = (1/4, 3/4) against p = (1/2, 1/2): (1/4) ln(1/2) + (3/4) ln(3/2)
    klr2 = oracle.indexer_kl_reverse(np.array([0.5, 0.5]), np.array([0.0, np.log(3.0)]))
    assert abs(klr2 - (0.25 * np.log(0.5) + 0.75 * np.log(1.5))) < 1e-15
    assert np.isinf(oracle.indexer_kl_reverse(np.array([1.0, 0.0]), np.zeros(2)))
