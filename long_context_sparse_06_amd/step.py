"""One DSA attention step composed from the three C-ABI calls.

The pages' order -- an FP8 indexer first, then the top-k choice, then core attention over
the chosen tokens only
(MarkTechPost, "DeepSeek V3.2-Exp Cuts Long-Context Costs with DeepSeek Sparse
Attention (DSA) ...") -- run as dsa_index_scores -> dsa_topk -> dsa_sparse_mla_*.
These classes only own the intermediate buffers (kept indices, workspaces, outputs;
allocated once, at construction) and issue the calls in order.  run() issues the first
two as the one call dsa_index_topk (same result as the two calls), which at decode stores
no score row and at prefill scores a bounded block of rows at a time; index() and topk()
issue the two calls separately into a full score buffer, for per-stage timing and
diagnostics -- that buffer ([B, ld] at decode, [T, T] at prefill) is allocated on first use.

With DSA_DEBUG_CHECKS=1 in the environment the classes also run the library's host-side
validators (which copy to the host and so synchronise): the block table against the caches'
page pools at construction, and every step's kept indices before the attention reads them.
"""
from __future__ import annotations

import os

import torch

from . import (BF16, E4M3, F32, Cache, dsa_check_block_table, dsa_check_indices, dsa_index_scores,
               dsa_index_topk,
               dsa_index_topk_workspace_size, dsa_sparse_mla_decode,
               dsa_sparse_mla_decode_workspace_size, dsa_sparse_mla_prefill, dsa_topk,
               dsa_topk_workspace_size)


def debug_checks() -> bool:
    return os.environ.get("DSA_DEBUG_CHECKS", "") not in ("", "0")


class DecodeStep:
    """Decode for B sequences, one new token each (its KV already in the caches).

    Inputs (device tensors): q_idx [B,H_I,d_I] e4m3 codes (uint8), q_scale [B], w [B,H_I],
    key cache (+ per-token scale), q [B,H,Dqk] bf16, latent cache bf16, row_seq/row_pos/
    n_valid [B] int32.  `ld` is the caches' capacity per sequence.
    """

    def __init__(self, *, q_idx, q_scale, w, keys, k_scale, q, kv, row_seq, row_pos, n_valid, ld,
                 k, softmax_scale, Dv, block_table=None, page_size=0, seq_stride=0, fp32=False):
        dev = q.device
        self.B, self.H, self.Dqk = q.shape
        self.Dv = int(Dv)
        self.HI, self.dI = q_idx.shape[1], q_idx.shape[2]
        self.k, self.ld, self.scale = int(k), int(ld), float(softmax_scale)
        self.q_idx, self.q_scale, self.w, self.q = q_idx, q_scale, w, q
        self.row_seq, self.row_pos, self.n_valid = row_seq, row_pos, n_valid
        self.keys = Cache(keys, k_scale, block_table, page_size, seq_stride)
        self.kv = Cache(kv, None, block_table, page_size, seq_stride)
        self.idx_dt = F32 if fp32 else E4M3
        self.mla_dt = F32 if fp32 else BF16
        fw = dsa_index_topk_workspace_size(self.B, self.ld, self.k)
        # zeroed once: the fused call's hand-off words start clear (any contents are correct)
        self.fused_ws = torch.zeros(max(fw, 1), dtype=torch.uint8, device=dev)
        self.fused_ws_bytes = fw
        self.idx = torch.empty(self.B, self.k, dtype=torch.int32, device=dev)
        self._scores = None
        self._topk_ws = None
        odt = torch.float32 if fp32 else torch.bfloat16
        self.out = torch.empty(self.B, self.H, self.Dv, dtype=odt, device=dev)
        self.lse = torch.empty(self.B, self.H, dtype=torch.float32, device=dev)
        mw = dsa_sparse_mla_decode_workspace_size(self.B, self.H, self.Dv, self.k)
        self.mla_ws = torch.empty(max(mw, 1), dtype=torch.uint8, device=dev)
        self.mla_ws_bytes = mw
        self.debug = debug_checks()
        if self.debug and block_table is not None:
            pool = min(keys.numel() // self.dI, kv.numel() // self.Dqk) // int(page_size)
            dsa_check_block_table(block_table, n_valid, page_size, pool)

    @classmethod
    def from_inputs(cls, d, k, softmax_scale, Dv, fp32=False):
        """From an object carrying the device tensors by name (q_idx, q_scale, w, keys, k_scale,
        q, kv, row_seq, row_pos, n_valid, block_table, page_size, seq_stride, ld)."""
        return cls(q_idx=d.q_idx, q_scale=d.q_scale, w=d.w, keys=d.keys, k_scale=d.k_scale, q=d.q,
                   kv=d.kv, row_seq=d.row_seq, row_pos=d.row_pos, n_valid=d.n_valid, ld=d.ld, k=k,
                   softmax_scale=softmax_scale, Dv=Dv, block_table=d.block_table,
                   page_size=d.page_size, seq_stride=d.seq_stride, fp32=fp32)

    @property
    def scores(self):
        """Score rows [B, ld] of index() (allocated on first use; run() never touches them)."""
        if self._scores is None:
            self._scores = torch.empty(self.B, self.ld, dtype=torch.float32, device=self.q.device)
        return self._scores

    @property
    def topk_ws(self):
        if self._topk_ws is None:
            tw = dsa_topk_workspace_size(self.B, self.ld, self.k)
            self._topk_ws = (torch.empty(max(tw, 1), dtype=torch.uint8, device=self.q.device), tw)
        return self._topk_ws

    def index(self, stream=None):
        dsa_index_scores(self.idx_dt, self.q_idx, self.q_scale, self.w, self.keys, self.row_seq,
                         self.row_pos, self.B, self.HI, self.dI, self.scores, self.ld, stream)

    def topk(self, stream=None, out=None):
        ws, wb = self.topk_ws
        dsa_topk(self.scores, self.ld, self.n_valid, self.B, self.k, self.idx if out is None else out,
                 ws, wb, stream)

    def index_topk(self, stream=None):
        dsa_index_topk(self.idx_dt, self.q_idx, self.q_scale, self.w, self.keys, self.row_seq,
                       self.row_pos, self.B, self.HI, self.dI, self.k, self.idx, self.fused_ws,
                       self.fused_ws_bytes, stream)

    def attend(self, stream=None):
        dsa_sparse_mla_decode(self.mla_dt, self.q, self.kv, self.idx, self.B, self.H, self.Dqk,
                              self.Dv, self.k, self.scale, self.out, self.lse, self.mla_ws,
                              self.mla_ws_bytes, stream)

    def run(self, stream=None):
        self.index_topk(stream)
        if self.debug:
            dsa_check_indices(self.idx, self.n_valid, strict=True)
        self.attend(stream)
        return self.out, self.lse, self.idx


class Prefill:
    """Causal prefill of one sequence of T tokens: row t scores tokens 0..t."""

    @classmethod
    def from_inputs(cls, d, k, softmax_scale, Dv):
        return cls(q_idx=d.q_idx, q_scale=d.q_scale, w=d.w, keys=d.keys, k_scale=d.k_scale, q=d.q,
                   kv=d.kv, row_seq=d.row_seq, row_pos=d.row_pos, n_valid=d.n_valid, k=k,
                   softmax_scale=softmax_scale, Dv=Dv, fp32=d.fp32)

    def __init__(self, *, q_idx, q_scale, w, keys, k_scale, q, kv, row_seq, row_pos, n_valid, k,
                 softmax_scale, Dv, fp32=False):
        dev = q.device
        self.T, self.H, self.Dqk = q.shape
        self.Dv = int(Dv)
        self.HI, self.dI = q_idx.shape[1], q_idx.shape[2]
        self.k, self.scale = int(k), float(softmax_scale)
        self.q_idx, self.q_scale, self.w, self.q, self.kvt = q_idx, q_scale, w, q, kv
        self.row_seq, self.row_pos, self.n_valid = row_seq, row_pos, n_valid
        self.keys = Cache(keys, k_scale, None, 0, self.T)
        self.idx_dt = F32 if fp32 else E4M3
        self.mla_dt = F32 if fp32 else BF16
        self.idx = torch.empty(self.T, self.k, dtype=torch.int32, device=dev)
        fw = dsa_index_topk_workspace_size(self.T, self.T, self.k)
        self.fused_ws = torch.zeros(max(fw, 1), dtype=torch.uint8, device=dev)
        self.fused_ws_bytes = fw
        self._scores = None
        self._topk_ws = None
        odt = torch.float32 if fp32 else torch.bfloat16
        self.out = torch.empty(self.T, self.H, self.Dv, dtype=odt, device=dev)
        self.lse = torch.empty(self.T, self.H, dtype=torch.float32, device=dev)
        self.debug = debug_checks()

    @property
    def scores(self):
        """The [T, T] score matrix of index() (allocated on first use; run() never needs it)."""
        if self._scores is None:
            self._scores = torch.empty(self.T, self.T, dtype=torch.float32, device=self.q.device)
        return self._scores

    @property
    def topk_ws(self):
        if self._topk_ws is None:
            tw = dsa_topk_workspace_size(self.T, self.T, self.k)
            self._topk_ws = (torch.empty(max(tw, 1), dtype=torch.uint8, device=self.q.device), tw)
        return self._topk_ws

    def index(self, stream=None):
        dsa_index_scores(self.idx_dt, self.q_idx, self.q_scale, self.w, self.keys, self.row_seq,
                         self.row_pos, self.T, self.HI, self.dI, self.scores, self.T, stream)

    def topk(self, stream=None, out=None):
        ws, wb = self.topk_ws
        dsa_topk(self.scores, self.T, self.n_valid, self.T, self.k, self.idx if out is None else out,
                 ws, wb, stream)

    def index_topk(self, stream=None):
        dsa_index_topk(self.idx_dt, self.q_idx, self.q_scale, self.w, self.keys, self.row_seq,
                       self.row_pos, self.T, self.HI, self.dI, self.k, self.idx, self.fused_ws,
                       self.fused_ws_bytes, stream)

    def attend(self, stream=None):
        dsa_sparse_mla_prefill(self.mla_dt, self.q, self.kvt, self.idx, self.T, self.H, self.Dqk,
                               self.Dv, self.k, self.scale, self.out, self.lse, stream)

    def run(self, stream=None):
        self.index_topk(stream)
        if self.debug:
            dsa_check_indices(self.idx, self.n_valid, strict=True)
        self.attend(stream)
        return self.out, self.lse, self.idx
