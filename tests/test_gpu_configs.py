"""End-to-end GPU parity on the five workload configurations (and a peaked-attention stress case).

Each case runs the whole path (dsa_index_scores -> dsa_topk -> dsa_sparse_mla_*) in the
launch configuration bench.py times, then checks against the oracle: index scores of
every checked row, the kept set under the band rule, and the attention output computed
by the oracle on the GPU's own kept set.  Full sizes are checked on every row for the
decode configurations and on sampled rows (plus edge rows) for the 32768-token prefill.
"""
import math
import sys

import numpy as np
import pytest
import torch

import datagen
from datagen.device import upload_decode, upload_prefill
from oracle import pipeline
from oracle.formats import decode_e4m3
import parity

pytestmark = pytest.mark.gpu


def _case(name):
    print(f"[case] {name}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import long_context_sparse_06_amd as dsa
    dsa.lib()


def _check_decode(inp, step, rows, rel_l2_max=None):
    scores = step.scores.cpu().numpy()
    idx = step.idx.cpu().numpy()
    out = step.out.float().cpu().numpy()
    lse = step.lse.cpu().numpy()
    k = step.k
    swaps = 0
    worst = 0.0
    for b in rows:
        L = int(inp.lengths[b])
        ref = pipeline.decode_scores(inp, b)
        keys, ks = pipeline.decode_keys(inp, b)
        ref_abs = parity.abs_scores(decode_e4m3(inp.q_idx[b]), float(inp.q_scale[b]), inp.w[b], keys, ks)
        parity.check_scores(scores[b, :L], ref, ref_abs, f"scores b={b}")
        swaps += parity.check_index_set(idx[b], ref, k, f"idx b={b}")
        o_ref, lse_ref = pipeline.decode_attention(inp, b, idx[b], step.scale)
        worst = max(worst, parity.check_attention(out[b], lse[b], o_ref, lse_ref, parity.BF16_ATOL, f"b={b}"))
        if rel_l2_max is not None:
            assert parity.rel_l2(out[b], o_ref) <= rel_l2_max, f"b={b}: rel-L2"
    print(f"  rows={len(rows)} band swaps={swaps} worst max-abs={worst:.3e}", flush=True)


def _decode_case(config, **over):
    from long_context_sparse_06_amd.step import DecodeStep
    inp = datagen.make_config(config, **over)
    d = upload_decode(inp)
    step = DecodeStep.from_inputs(d, inp.shapes.k, 1.0 / math.sqrt(inp.shapes.Dqk), inp.shapes.Dv)
    step.run()  # fused index + top-k: no score row stored
    # the two separate calls, for the scores the checks read; their kept sets must be the same
    step.index()
    two = torch.empty_like(step.idx)
    step.topk(out=two)
    torch.cuda.synchronize()
    assert torch.equal(step.idx, two), "fused index + top-k differs from the two calls"
    return inp, step


def test_config1_tiny_fp32_prefill():
    from long_context_sparse_06_amd.step import Prefill
    _case("config 1: tiny fp32 prefill T=256")
    inp = datagen.make_config(1)
    s = inp.shapes
    d = upload_prefill(inp)
    pf = Prefill.from_inputs(d, s.k, 1.0 / math.sqrt(s.Dqk), s.Dv)
    pf.run()
    pf.index()
    two = torch.empty_like(pf.idx)
    pf.topk(out=two)
    assert torch.equal(pf.idx, two), "fused index + top-k differs from the two calls"
    scores = pf.scores.cpu().numpy(); idx = pf.idx.cpu().numpy()
    out = pf.out.cpu().numpy(); lse = pf.lse.cpu().numpy()
    pairs = 0
    for t in range(inp.T):
        ref = pipeline.prefill_scores(inp, t)
        ref_abs = parity.abs_scores(inp.q_idx[t], 1.0, inp.w[t], inp.keys[: t + 1], np.ones(t + 1))
        parity.check_scores(scores[t, : t + 1], ref, ref_abs, f"t={t}")
        parity.check_index_set(idx[t], ref, s.k, f"t={t}")
        pairs += int((idx[t] >= 0).sum())
        o_ref, lse_ref = pipeline.prefill_attention(inp, t, idx[t], pf.scale)
        parity.check_attention(out[t], lse[t], o_ref, lse_ref, parity.F32_ATOL, f"t={t}")
    assert pairs == 7696  # sum_t min(t+1, k): the O(Lk) pair count


def test_config2_decode_b32_l8192():
    _case("config 2: decode B=32 L=8192")
    inp, step = _decode_case(2)
    _check_decode(inp, step, range(inp.B))


def test_config3_decode_b8_l131072():
    _case("config 3: decode B=8 L=131072")
    inp, step = _decode_case(3)
    _check_decode(inp, step, range(inp.B))


def test_config5_ragged_paged_decode():
    _case("config 5: ragged paged decode B=64")
    inp, step = _decode_case(5)
    assert inp.lengths.min() >= 1024 and inp.lengths.max() <= 131072
    _check_decode(inp, step, range(inp.B))


def test_decode_step_graph_replays():
    """The decode step (fused index + top-k, then the split attention) captured in HIP graphs,
    as bench.py times it, and replayed: every replay must give the eager step's bits (kept
    set, output, lse).  The fused call clears its own hand-off words, so replays start clean;
    eager steps and synchronisations run between the replays, and a second step object's
    graph (its own workspaces, the same kernels) is replayed in between."""
    from long_context_sparse_06_amd.step import DecodeStep
    _case("decode step graph replays B=4 L=40000")
    inp = datagen.make_config(3, B=4, L=40000)
    d = upload_decode(inp)
    scale = 1.0 / math.sqrt(inp.shapes.Dqk)
    st = DecodeStep.from_inputs(d, inp.shapes.k, scale, inp.shapes.Dv)
    st2 = DecodeStep.from_inputs(d, inp.shapes.k, scale, inp.shapes.Dv)
    st.run()
    st2.run()
    torch.cuda.synchronize()
    ref = (st.idx.clone(), st.out.clone(), st.lse.clone())
    g, g2 = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        st.run()
    with torch.cuda.graph(g2):
        st2.run()
    torch.cuda.synchronize()
    for rep in range(3):
        st.idx.fill_(-7); st.out.fill_(3.0); st.lse.fill_(3.0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(st.idx, ref[0]) and torch.equal(st.out, ref[1]) and torch.equal(st.lse, ref[2]), \
            f"graph replay {rep}"
        st2.idx.fill_(-7); st2.out.fill_(3.0)
        st2.run()  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(st2.idx, ref[0]) and torch.equal(st2.out, ref[1])
        g2.replay()
        torch.cuda.synchronize()
        assert torch.equal(st2.idx, ref[0]) and torch.equal(st2.out, ref[1]) and torch.equal(st2.lse, ref[2])
    st.index()  # score rows for the oracle check of the replayed result
    torch.cuda.synchronize()
    _check_decode(inp, st, range(inp.B))


def test_peaked_decode_stress():
    _case("peaked decode B=4 L=50000")
    inp, step = _decode_case(3, B=4, L=50000, regime="peaked")
    _check_decode(inp, step, range(inp.B), rel_l2_max=1e-2)
    # planted needles outrank the Gaussian background and must all be kept
    idx = step.idx.cpu().numpy()
    for b in range(inp.B):
        assert set(inp.needles[b].tolist()) <= set(idx[b].tolist())


def test_config4_prefill_t32768_sampled_rows():
    from long_context_sparse_06_amd.step import Prefill
    _case("config 4: prefill T=32768")
    inp = datagen.make_config(4)
    s = inp.shapes
    d = upload_prefill(inp)
    pf = Prefill.from_inputs(d, s.k, 1.0 / math.sqrt(s.Dqk), s.Dv)
    pf.run()  # blocked fused index + top-k: no T x T buffer
    pf.index()  # the T x T scores, for the checks below
    two = torch.empty_like(pf.idx)
    pf.topk(out=two)
    torch.cuda.synchronize()
    assert torch.equal(pf.idx, two), "blocked fused index + top-k differs from the two calls"
    del two
    T = inp.T
    rng = np.random.default_rng(4)
    rows = sorted(set([0, 1, 2046, 2047, 2048, 2049, T - 1] + rng.integers(0, T, 9).tolist()))
    idx_all = pf.idx.cpu().numpy()
    # every row keeps min(t+1, k) causal indices
    nkept = (idx_all >= 0).sum(axis=1)
    assert np.array_equal(nkept, np.minimum(np.arange(1, T + 1), s.k))
    assert int(nkept.sum()) == 65_012_736
    assert (idx_all.max(axis=1) <= np.arange(T)).all()
    out = pf.out[rows].float().cpu().numpy(); lse = pf.lse[rows].cpu().numpy()
    for i, t in enumerate(rows):
        ref = pipeline.prefill_scores(inp, t)
        got = pf.scores[t, : t + 1].cpu().numpy()
        keys = decode_e4m3(inp.keys[: t + 1])
        ref_abs = parity.abs_scores(decode_e4m3(inp.q_idx[t]), float(inp.q_scale[t]), inp.w[t], keys,
                                    inp.k_scale[: t + 1].astype(np.float64))
        parity.check_scores(got, ref, ref_abs, f"t={t}")
        parity.check_index_set(idx_all[t], ref, s.k, f"t={t}")
        o_ref, lse_ref = pipeline.prefill_attention(inp, t, idx_all[t], pf.scale)
        parity.check_attention(out[i], lse[i], o_ref, lse_ref, parity.BF16_ATOL, f"t={t}")
