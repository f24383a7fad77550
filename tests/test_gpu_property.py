"""Randomised GPU parity of the top-k and of the fused index + top-k, drawn by hypothesis.

Rows are generated on the CPU from a drawn seed over lengths and value alphabets chosen so that
every selection route runs: trivial rows (n <= k), rows selected in registers by one workgroup
(n <= 32768, or <= 8192 when the call's leading dimension passes 32768), the sampled compaction
with its three resolves (survivors in LDS; a threshold that is the k-th key itself, as on tied
rows; the full-row fallback when the sample keeps fewer than k or too many), and the boundary-
bin ranking.  dsa_topk must equal the oracle's top-k exactly (same float32 scores on both
sides, ties to the lower index, ascending, -1 padded) and pass the strict index check;
dsa_index_topk must equal the two separate calls exactly.  Examples are bounded (200 and 40),
derandomised, and the run stops at the first failure (no shrinking on the GPU).
"""
import dataclasses
import sys

import numpy as np
import pytest
import torch
from hypothesis import HealthCheck, Phase, given, settings
from hypothesis import strategies as st

import datagen
import oracle
from datagen.device import tensor, upload_decode

pytestmark = pytest.mark.gpu

FULL = datagen.FULL
_SET = dict(deadline=None, derandomize=True, database=None, phases=[Phase.explicit, Phase.generate],
            suppress_health_check=[HealthCheck.too_slow, HealthCheck.data_too_large,
                                   HealthCheck.function_scoped_fixture])


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import long_context_sparse_06_amd as dsa
    dsa.lib()


ALPHABETS = ["normal", "few", "equal", "signed_zero", "wide", "sorted", "planted_high", "planted_low",
             "narrow", "quantised"]


def _row(rng, n, ld, alphabet):
    if alphabet == "normal":
        return rng.standard_normal(n)
    if alphabet == "few":
        return rng.integers(0, 3, n).astype(np.float64)
    if alphabet == "equal":
        return np.full(n, float(rng.standard_normal()))
    if alphabet == "signed_zero":
        return np.where(rng.random(n) < 0.5, -0.0, 0.0) + np.where(rng.random(n) < 0.01, 1.0, 0.0)
    if alphabet == "wide":
        return rng.standard_normal(n) * np.exp2(rng.integers(-60, 60, n))
    if alphabet == "sorted":
        return np.sort(rng.standard_normal(n))[:: (1 if rng.random() < 0.5 else -1)]
    if alphabet == "narrow":
        return 7.0 + rng.standard_normal(n) * 1e-4
    if alphabet == "quantised":
        return np.round(rng.standard_normal(n) * int(rng.integers(2, 64))) / 8
    s = rng.uniform(0, 1, n)
    pos = (np.arange(2048, dtype=np.int64) * n) // 2048   # the sample positions of the compaction
    if alphabet == "planted_high":                         # the sample over-estimates: few survivors
        s[pos[: int(rng.integers(1, 2048))]] = 10.0 + rng.random()
    else:                                                  # the sample under-estimates: too many
        s[pos] = -10.0
    return s


@settings(max_examples=200, **_SET)
@given(seed=st.integers(0, 2**32 - 1), R=st.integers(1, 4),
       ld=st.sampled_from([300, 3000, 9000, 32768, 40000, 65536, 131072]),
       k=st.sampled_from([1, 7, 64, 300, 2048, 4096]),
       alphabets=st.lists(st.sampled_from(ALPHABETS), min_size=4, max_size=4))
def test_topk_matches_oracle(seed, R, ld, k, alphabets):
    import long_context_sparse_06_amd as dsa
    rng = np.random.default_rng(seed)
    s = np.zeros((R, ld), np.float32)
    n_valid = np.zeros(R, np.int32)
    for r in range(R):
        # lengths around every cut: n <= k, <= 8192, <= 32768, beyond
        choices = [int(rng.integers(0, min(k, ld) + 1)), int(rng.integers(1, ld + 1)), ld,
                   min(ld, 8192 + int(rng.integers(-2, 3))), min(ld, k + 1)]
        n_valid[r] = max(0, min(ld, choices[int(rng.integers(len(choices)))]))
        n = int(n_valid[r])
        if n:
            s[r, :n] = _row(rng, n, ld, alphabets[r]).astype(np.float32)
        s[r, n:] = rng.standard_normal(ld - n).astype(np.float32) * 100  # beyond n: must be ignored
    print(f"[case] topk seed={seed} R={R} ld={ld} k={k} n={n_valid.tolist()} {alphabets[:R]}", flush=True)
    sys.stdout.flush()
    idx = torch.full((R, k), -7, dtype=torch.int32, device="cuda")
    wsb = dsa.dsa_topk_workspace_size(R, ld, k)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
    dsa.dsa_topk(tensor(s), ld, tensor(n_valid), R, k, idx, ws, wsb)
    got = idx.cpu().numpy()
    for r in range(R):
        n = int(n_valid[r])
        ref = oracle.topk(s[r, :n].astype(np.float64), k)
        exp = np.full(k, -1, np.int64)
        exp[: len(ref)] = ref
        assert np.array_equal(got[r], exp), f"row {r} (n={n}, {alphabets[r]}): first diff at {np.nonzero(got[r] != exp)[0][:5]}"
    dsa.dsa_check_indices(got, n_valid, strict=True)


@settings(max_examples=40, **_SET)
@given(seed=st.integers(0, 2**32 - 1), B=st.integers(1, 3), paged=st.booleans(),
       page_size=st.sampled_from([16, 48, 64]), cap=st.sampled_from([20000, 40000, 70000]),
       k=st.sampled_from([16, 2048]), zero_rows=st.integers(0, 1), regime=st.sampled_from(["gaussian", "peaked"]))
def test_index_topk_fused_equals_two_calls(seed, B, paged, page_size, cap, k, zero_rows, regime):
    import long_context_sparse_06_amd as dsa
    rng = np.random.default_rng(seed)
    lengths = rng.integers(1, cap + 1, B)
    lengths[0] = cap
    print(f"[case] index_topk seed={seed} B={B} paged={paged} ps={page_size} n={lengths.tolist()} k={k} "
          f"zero={zero_rows} {regime}", flush=True)
    sys.stdout.flush()
    sh = dataclasses.replace(FULL, H=4, Dqk=64, Dv=32, k=k)  # attention widths unused here
    inp = datagen.make_decode(B, None, sh, seed=int(seed % 2**31), lengths=lengths, paged=paged,
                              page_size=page_size, regime=regime)
    if zero_rows:
        inp.q_idx[B - 1] = 0                                # every score of that row 0: all tied
    d = upload_decode(inp)
    cache = dsa.Cache(d.keys, d.k_scale, d.block_table, d.page_size, d.seq_stride)
    scores = torch.empty((B, d.ld), device="cuda")
    dsa.dsa_index_scores(dsa.E4M3, d.q_idx, d.q_scale, d.w, cache, d.row_seq, d.row_pos, B, FULL.HI,
                         FULL.dI, scores, d.ld)
    two = torch.full((B, k), -7, dtype=torch.int32, device="cuda")
    tw = dsa.dsa_topk_workspace_size(B, d.ld, k)
    dsa.dsa_topk(scores, d.ld, d.n_valid, B, k, two, torch.empty(max(tw, 1), dtype=torch.uint8, device="cuda"), tw)
    fw = dsa.dsa_index_topk_workspace_size(B, d.ld, k)
    fws = torch.full((fw,), int(rng.integers(0, 256)), dtype=torch.uint8, device="cuda")  # any contents
    got = torch.full((B, k), -7, dtype=torch.int32, device="cuda")
    dsa.dsa_index_topk(dsa.E4M3, d.q_idx, d.q_scale, d.w, cache, d.row_seq, d.row_pos, B, FULL.HI, FULL.dI,
                       k, got, fws, fw)
    assert torch.equal(got, two), "fused index + top-k differs from the two calls"
    dsa.dsa_check_indices(got, d.n_valid, strict=True)
    # one row's scores against the oracle's exact top-k of the same float32 scores
    r = int(rng.integers(B))
    n = int(lengths[r])
    ref = oracle.topk(scores[r, :n].cpu().numpy().astype(np.float64), k)
    exp = np.full(k, -1, np.int64)
    exp[: len(ref)] = ref
    assert np.array_equal(got[r].cpu().numpy(), exp)
