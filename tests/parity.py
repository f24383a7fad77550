"""Comparison rules between the GPU path and the CPU oracle.

* Index scores (fp32 on the GPU, fp64 in the oracle): every per-head dot of e4m3
  values is exact in fp32 products but accumulated in fp32, then weighted and summed
  over heads in fp32.  A bound of 2e-5 times the absolute-value score
  (k_scale * q_scale * sum_j |w_j| * sum_d |q_jd| |k_d|) covers 128 + 64 fp32
  accumulation steps (each <= 2^-24 relative, ~1.1e-5 summed) with margin.
* Kept index sets: |G| = |O| and every index in the symmetric difference has an oracle
  score within 1e-3 relative of the oracle's k-th score tau.
* Standalone top-k on identical fp32 inputs: bit-exact.
* Attention output vs the oracle evaluated on the GPU's own kept set: max-abs <= 2e-2
  (bf16 path) or <= 1e-4 (fp32 path); the log-sum-exp to the same bound (its finiteness
  must match exactly).
"""
from __future__ import annotations

import numpy as np

import oracle

SCORE_RTOL = 2e-5
BAND = 1e-3
BF16_ATOL = 2e-2
F32_ATOL = 1e-4


def abs_scores(q, qs, w, keys, ks):
    return oracle.index_scores(np.abs(q), abs(qs), np.abs(w), np.abs(keys), np.abs(ks))


def check_scores(got, ref, ref_abs, what=""):
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - ref)
    tol = SCORE_RTOL * ref_abs + 1e-30
    bad = np.nonzero(err > tol)[0]
    assert bad.size == 0, (f"{what}: {bad.size} scores off, first s={bad[:5]}, "
                           f"got={got[bad[:5]]}, ref={ref[bad[:5]]}")


def check_index_set(gpu_idx, ref_scores, k, what=""):
    """gpu_idx: the GPU's [k] row (-1 padded).  Compares with the oracle's top-k under the band rule."""
    gpu_idx = np.asarray(gpu_idx)
    n = len(ref_scores)
    m = min(k, n)
    valid = gpu_idx[:m]
    assert (gpu_idx[m:] == -1).all(), f"{what}: padding slots not -1"
    assert (valid >= 0).all() and (valid < n).all(), f"{what}: index out of range"
    assert len(np.unique(valid)) == m, f"{what}: duplicate indices"
    assert (np.diff(valid) > 0).all(), f"{what}: not ascending"
    O = set(oracle.topk(ref_scores, k).tolist())
    G = set(valid.tolist())
    diff = G ^ O
    if diff:
        tau = oracle.kth_score(ref_scores, k)
        d = np.array(sorted(diff))
        off = np.abs(ref_scores[d] - tau) > BAND * abs(tau)
        assert not off.any(), (f"{what}: {off.sum()} swaps outside the band, e.g. s={d[off][:5]} "
                               f"score={ref_scores[d[off][:5]]} tau={tau}")
    return len(diff)


def check_attention(o_gpu, lse_gpu, o_ref, lse_ref, atol, what=""):
    o_gpu = np.asarray(o_gpu, dtype=np.float64)
    err = np.abs(o_gpu - o_ref).max() if o_ref.size else 0.0
    assert err <= atol, f"{what}: max-abs {err:.3e} > {atol}"
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lse_gpu), fin), f"{what}: lse finiteness differs"
    if fin.any():
        lerr = np.abs(np.asarray(lse_gpu, dtype=np.float64)[fin] - lse_ref[fin]).max()
        assert lerr <= atol, f"{what}: lse max-abs {lerr:.3e}"
    return err


def rel_l2(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))
