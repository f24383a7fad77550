"""The host-side validators dsa_check_indices and dsa_check_block_table (CPU only: they read host
memory and launch nothing).

Each rule is checked on hand-built cases, then randomly drawn lists and tables with planted
faults are compared against a plain statement of the rules, and the oracle's own top-k output
(the form dsa_topk writes) must pass the strict check.
"""
import ctypes

import numpy as np
import pytest
from hypothesis import HealthCheck, Phase, given, settings
from hypothesis import strategies as st

import long_context_sparse_06_amd as dsa
import oracle

RANGE = 7  # DSA_ERR_RANGE


@pytest.fixture(scope="module", autouse=True)
def _lib():
    dsa.lib()


def _status(fn, *args):
    try:
        fn(*args)
        return 0, -1
    except dsa.DSAError as e:
        return e.status, getattr(e, "first_bad", None)


# ---------------------------------------------------------------- the rules, stated plainly
def rule_indices(idx, n_valid, strict):
    R, k = idx.shape
    for r in range(R):
        n = int(n_valid[r])
        if n < 0:
            return r * k
        seen_pad, prev = False, -1
        for j in range(k):
            v = int(idx[r, j])
            if v < -1 or v >= n:
                return r * k + j
            if strict and v >= 0 and (seen_pad or v <= prev):
                return r * k + j
            if v < 0:
                seen_pad = True
            else:
                prev = v
    return -1


def rule_table(table, lengths, page_size, pool):
    B, P = table.shape
    for b in range(B):
        L = int(lengths[b])
        if L < 0 or L > P * page_size:
            return -1 - b
        for p in range((L + page_size - 1) // page_size):
            e = int(table[b, p])
            if e < 0 or e >= pool:
                return b * P + p
    return None


# ---------------------------------------------------------------- hand-built cases
def test_indices_hand_cases():
    n = np.array([5, 3], np.int32)
    ok = np.array([[0, 2, 4, -1], [1, -1, -1, -1]], np.int32)
    assert _status(dsa.dsa_check_indices, ok, n, True) == (0, -1)
    bad = ok.copy(); bad[1, 0] = 3                       # index == n_valid
    assert _status(dsa.dsa_check_indices, bad, n, False) == (RANGE, 4)
    bad = ok.copy(); bad[0, 3] = -2                      # below -1
    assert _status(dsa.dsa_check_indices, bad, n, False) == (RANGE, 3)
    loose = np.array([[4, 0, 4, -1], [-1, 2, -1, 1]], np.int32)   # unsorted, repeat, gaps
    assert _status(dsa.dsa_check_indices, loose, n, False) == (0, -1)
    assert _status(dsa.dsa_check_indices, loose, n, True) == (RANGE, 1)
    gap = np.array([[0, -1, 3, -1], [0, 1, 2, -1]], np.int32)     # a kept index after padding
    assert _status(dsa.dsa_check_indices, gap, n, True) == (RANGE, 2)
    rep = np.array([[0, 1, 1, -1], [0, 1, 2, -1]], np.int32)      # a repeat
    assert _status(dsa.dsa_check_indices, rep, n, True) == (RANGE, 2)
    assert _status(dsa.dsa_check_indices, ok, np.array([5, -1], np.int32), False) == (RANGE, 4)


def test_block_table_hand_cases():
    t = np.array([[3, 0, 7, 9], [1, 2, 5, 6]], np.int32)
    assert _status(dsa.dsa_check_block_table, t, np.array([40, 17], np.int32), 16, 8) == (0, -1)
    # page 2 of sequence 1 (tokens 32..47) is used once its length passes 32
    assert _status(dsa.dsa_check_block_table, t, np.array([32, 33], np.int32), 16, 5) == (RANGE, 6)
    # unused pages may hold anything
    t2 = t.copy(); t2[1, 3] = -5
    assert _status(dsa.dsa_check_block_table, t2, np.array([40, 48], np.int32), 16, 8) == (0, -1)
    assert _status(dsa.dsa_check_block_table, t2, np.array([40, 49], np.int32), 16, 8) == (RANGE, 7)
    # a length beyond the table's pages, and a negative one
    assert _status(dsa.dsa_check_block_table, t, np.array([65, 1], np.int32), 16, 10) == (RANGE, -1)
    assert _status(dsa.dsa_check_block_table, t, np.array([0, -1], np.int32), 16, 10) == (RANGE, -2)
    # the first used page out of the pool
    assert _status(dsa.dsa_check_block_table, t, np.array([1, 0], np.int32), 16, 3) == (RANGE, 0)


def test_validators_reject_bad_arguments():
    L = dsa.lib()
    bad = ctypes.c_int64(0)
    a = np.zeros((2, 2), np.int32)
    assert L.dsa_check_indices(None, 2, 2, a.ctypes.data, 0, ctypes.byref(bad)) == 1
    assert L.dsa_check_indices(a.ctypes.data, 0, 2, a.ctypes.data, 0, ctypes.byref(bad)) == 2
    assert L.dsa_check_block_table(a.ctypes.data, 2, 2, a.ctypes.data, 0, 4, ctypes.byref(bad)) == 2
    assert L.dsa_check_block_table(a.ctypes.data, 2, 2, None, 16, 4, ctypes.byref(bad)) == 1


# ---------------------------------------------------------------- drawn cases
_SET = settings(max_examples=200, deadline=None, derandomize=True, database=None,
                phases=[Phase.explicit, Phase.generate],
                suppress_health_check=[HealthCheck.too_slow, HealthCheck.data_too_large])


@_SET
@given(st.integers(0, 2**32 - 1), st.integers(1, 6), st.integers(1, 40), st.booleans(),
       st.integers(0, 3))
def test_indices_against_the_rules(seed, R, k, strict, faults):
    rng = np.random.default_rng(seed)
    n = rng.integers(0, 60, R).astype(np.int32)
    idx = np.full((R, k), -1, np.int32)
    for r in range(R):  # the form dsa_topk writes: ascending, repeat-free, -1 padded
        m = min(k, int(n[r]))
        idx[r, :m] = np.sort(rng.choice(int(n[r]), m, replace=False)) if m else []
    for _ in range(faults):  # plant faults of every kind
        r, j = int(rng.integers(R)), int(rng.integers(k))
        kind = int(rng.integers(4))
        idx[r, j] = [int(n[r]) + int(rng.integers(0, 3)), -2 - int(rng.integers(0, 5)),
                     int(rng.integers(0, max(int(n[r]), 1))), -1][kind]
    exp = rule_indices(idx, n, strict)
    got = _status(dsa.dsa_check_indices, idx, n, strict)
    assert got == ((0, -1) if exp < 0 else (RANGE, exp))


@_SET
@given(st.integers(0, 2**32 - 1), st.integers(1, 5), st.integers(1, 12), st.sampled_from([1, 7, 16, 64]),
       st.integers(0, 3))
def test_block_tables_against_the_rules(seed, B, P, ps, faults):
    rng = np.random.default_rng(seed)
    pool = int(rng.integers(1, B * P + 4))
    table = rng.integers(0, pool, (B, P)).astype(np.int32)
    lengths = rng.integers(0, P * ps + 1, B).astype(np.int32)
    for _ in range(faults):
        b, p = int(rng.integers(B)), int(rng.integers(P))
        kind = int(rng.integers(3))
        if kind == 0:
            table[b, p] = pool + int(rng.integers(0, 3))
        elif kind == 1:
            table[b, p] = -1 - int(rng.integers(0, 3))
        else:
            lengths[b] = P * ps + 1 + int(rng.integers(0, 5))
    exp = rule_table(table, lengths, ps, pool)
    got = _status(dsa.dsa_check_block_table, table, lengths, ps, pool)
    assert got == ((0, -1) if exp is None else (RANGE, exp))


@_SET
@given(st.integers(0, 2**32 - 1), st.integers(1, 300), st.integers(1, 64), st.integers(0, 3))
def test_oracle_topk_output_passes_the_strict_check(seed, n, k, alphabet):
    rng = np.random.default_rng(seed)
    s = [rng.standard_normal(n), rng.integers(0, 3, n).astype(float), np.zeros(n),
         np.where(rng.random(n) < 0.5, -0.0, 0.0)][alphabet]
    kept = oracle.topk(s, k)
    idx = np.full((1, k), -1, np.int32)
    idx[0, : len(kept)] = kept
    assert _status(dsa.dsa_check_indices, idx, np.array([n], np.int32), True) == (0, -1)
