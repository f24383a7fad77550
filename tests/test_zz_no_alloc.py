"""dsa_sparse_mla_decode_noalloc (split partials in the library's static per-GPU array) gives
exactly dsa_sparse_mla_decode's output with a caller workspace: on two calls in a row, the
second with a smaller batch and kept-set size, so the array holds the first call's partials
when the second runs; and captured in a HIP graph and replayed."""
import math

import numpy as np
import pytest
import torch

import datagen
from datagen.device import tensor, upload_decode

pytestmark = pytest.mark.gpu

FULL = datagen.FULL


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import long_context_sparse_06_amd as dsa
    dsa.lib()


def _sets(rng, lengths, k):
    idx = np.full((len(lengths), k), -1, dtype=np.int32)
    for b, L in enumerate(lengths):
        m = min(k, int(L))
        idx[b, :m] = np.sort(rng.choice(int(L), size=m, replace=False))
    return idx


def _both(dsa, d, idx, B, k, paged):
    scale = 1.0 / math.sqrt(FULL.Dqk)
    cache = dsa.Cache(d.kv, None, d.block_table, d.page_size, d.seq_stride)
    outs = []
    for noalloc in (False, True):
        out = torch.full((B, FULL.H, FULL.Dv), float("nan"), dtype=torch.bfloat16, device="cuda")
        lse = torch.full((B, FULL.H), float("nan"), device="cuda")
        if noalloc:
            dsa.dsa_sparse_mla_decode_noalloc(dsa.BF16, d.q, cache, idx, B, FULL.H, FULL.Dqk, FULL.Dv, k,
                                              scale, out, lse)
        else:
            wsb = dsa.dsa_sparse_mla_decode_workspace_size(B, FULL.H, FULL.Dv, k)
            ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
            dsa.dsa_sparse_mla_decode(dsa.BF16, d.q, cache, idx, B, FULL.H, FULL.Dqk, FULL.Dv, k, scale,
                                      out, lse, ws, wsb)
        torch.cuda.synchronize()
        outs.append((out.view(torch.int16).cpu().numpy(), lse.cpu().numpy()))
    (o0, l0), (o1, l1) = outs
    assert np.array_equal(o0, o1), "outputs differ"
    assert np.array_equal(l0.view(np.uint32), l1.view(np.uint32)), "lse differ"


def test_noalloc_matches_workspace_call_twice():
    import long_context_sparse_06_amd as dsa
    assert dsa.dsa_noalloc_scratch_bytes() == 32 << 20
    rng = np.random.default_rng(81)
    # first call: batch 6 with k = 2048 (split over many workgroups: partials in the array)
    lengths = np.array([9000, 2048, 5000, 300, 12000, 4097])
    k = 2048
    inp = datagen.make_decode(len(lengths), None, FULL, seed=82, lengths=lengths, regime="peaked")
    d = upload_decode(inp)
    assert dsa.dsa_sparse_mla_decode_workspace_size(len(lengths), FULL.H, FULL.Dv, k) > 0
    _both(dsa, d, tensor(_sets(rng, lengths, k)), len(lengths), k, False)
    # second call, smaller: batch 2, k = 512, paged (fewer partials than the first call wrote)
    lengths2 = np.array([3000, 700])
    k2 = 512
    inp2 = datagen.make_decode(2, None, FULL, seed=83, lengths=lengths2, paged=True, regime="peaked")
    d2 = upload_decode(inp2)
    assert 0 < dsa.dsa_sparse_mla_decode_workspace_size(2, FULL.H, FULL.Dv, k2) < \
        dsa.dsa_sparse_mla_decode_workspace_size(len(lengths), FULL.H, FULL.Dv, k)
    _both(dsa, d2, tensor(_sets(rng, lengths2, k2)), 2, k2, True)


def test_noalloc_under_graph_capture():
    """The entry point's purpose: a call captured in a HIP graph (nothing allocated inside the
    capture) and replayed.  Every replay must give the workspace call's bits; eager calls of
    both entry points and synchronisations run between the replays."""
    import long_context_sparse_06_amd as dsa
    rng = np.random.default_rng(85)
    lengths = np.array([7000, 2100, 40, 5000])
    B, k = len(lengths), 2048
    inp = datagen.make_decode(B, None, FULL, seed=86, lengths=lengths, regime="peaked")
    d = upload_decode(inp)
    idx = tensor(_sets(rng, lengths, k))
    scale = 1.0 / math.sqrt(FULL.Dqk)
    cache = dsa.Cache(d.kv, None, d.block_table, d.page_size, d.seq_stride)
    wsb = dsa.dsa_sparse_mla_decode_workspace_size(B, FULL.H, FULL.Dv, k)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device="cuda")
    ref_o = torch.empty((B, FULL.H, FULL.Dv), dtype=torch.bfloat16, device="cuda")
    ref_l = torch.empty((B, FULL.H), device="cuda")
    dsa.dsa_sparse_mla_decode(dsa.BF16, d.q, cache, idx, B, FULL.H, FULL.Dqk, FULL.Dv, k, scale, ref_o, ref_l,
                              ws, wsb)
    out = torch.empty_like(ref_o)
    lse = torch.empty_like(ref_l)
    # one eager call first (the array's address is looked up on a device's first call)
    dsa.dsa_sparse_mla_decode_noalloc(dsa.BF16, d.q, cache, idx, B, FULL.H, FULL.Dqk, FULL.Dv, k, scale, out, lse)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dsa.dsa_sparse_mla_decode_noalloc(dsa.BF16, d.q, cache, idx, B, FULL.H, FULL.Dqk, FULL.Dv, k, scale, out,
                                          lse)
    for rep in range(3):
        out.fill_(7.0); lse.fill_(7.0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l), f"graph replay {rep}"
        o2, l2 = torch.empty_like(ref_o), torch.empty_like(ref_l)
        dsa.dsa_sparse_mla_decode_noalloc(dsa.BF16, d.q, cache, idx, B, FULL.H, FULL.Dqk, FULL.Dv, k, scale, o2, l2)
        dsa.dsa_sparse_mla_decode(dsa.BF16, d.q, cache, idx, B, FULL.H, FULL.Dqk, FULL.Dv, k, scale, o2, l2, ws, wsb)
        torch.cuda.synchronize()
        assert torch.equal(o2, ref_o) and torch.equal(l2, ref_l)


def test_noalloc_rejects_sets_beyond_the_array():
    import long_context_sparse_06_amd as dsa
    B, k = 128, 16384
    assert dsa.dsa_sparse_mla_decode_workspace_size(B, FULL.H, FULL.Dv, k) > dsa.dsa_noalloc_scratch_bytes()
    q = torch.empty((1,), device="cuda")
    kv = dsa.Cache(q, seq_stride=k)
    with pytest.raises(dsa.DSAError) as e:
        dsa.dsa_sparse_mla_decode_noalloc(dsa.BF16, q, kv, q, B, FULL.H, FULL.Dqk, FULL.Dv, k, 0.04, q, None)
    assert "DSA_ERR_WORKSPACE" in str(e.value)
