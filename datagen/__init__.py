"""Seeded synthetic inputs for the DSA hot path.

This module is shared by the CPU oracle's tests and by the GPU path's tests and
benchmark.  It only *makes input bytes*: random tensors, their storage encodings
(e4m3 codes with a per-token fp32 scale, bf16 bit patterns) and cache layouts
(contiguous or 64-token pages behind a shuffled block table).  It holds none of
the method's arithmetic (no scoring, no selection, no attention).

Encodings use torch's own casts (round-to-nearest-even); the e4m3 quantiser
clamps to +-448 first because torch maps out-of-range values to NaN.

Workload shapes follow the five synthetic configurations of the DSA build:
  tiny   : fp32 prefill, T=256, H=4, Dqk=80 (64+16), Dv=64, H_I=2, d_I=32, k=32
  decode : B=32, L=8192, H=128, Dqk=576, Dv=512, H_I=64, d_I=128, k=2048
  long   : B=8,  L=131072, same shapes
  prefill: T=32768, same shapes
  ragged : B=64, L_i log-uniform in [1024, 131072], 64-token pages, shuffled table
All activations are N(0,1)/sqrt(d) with d the last dimension; indexer weights
w ~ U(0,1).  Seeds are 1000 + configuration number.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

E4M3_MAX = 448.0


@dataclasses.dataclass(frozen=True)
class Shapes:
    H: int = 128        # query heads
    Dqk: int = 576      # latent row width (512 value + 64 rope)
    Dv: int = 512       # value width
    HI: int = 64        # indexer heads
    dI: int = 128       # indexer head dim
    k: int = 2048       # kept tokens per query


FULL = Shapes()
TINY = Shapes(H=4, Dqk=80, Dv=64, HI=2, dI=32, k=32)

CONFIGS = {
    1: dict(name="tiny_fp32_prefill", kind="prefill", T=256, shapes=TINY, dtype="f32"),
    2: dict(name="decode_b32_l8192", kind="decode", B=32, L=8192, shapes=FULL),
    3: dict(name="decode_b8_l131072", kind="decode", B=8, L=131072, shapes=FULL),
    4: dict(name="prefill_t32768", kind="prefill", T=32768, shapes=FULL),
    5: dict(name="ragged_paged_decode_b64", kind="decode", B=64, L=None, shapes=FULL,
            paged=True, page_size=64, Lmin=1024, Lmax=131072),
}


def seed_for(config: int) -> int:
    return 1000 + config


# ----------------------------------------------------------------------------
# encodings (storage formats of the inputs)
# ----------------------------------------------------------------------------
def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 array -> uint16 bf16 bit patterns (torch cast, RNE)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def quantize_e4m3_per_token(x: np.ndarray):
    """Per-token (last axis) e4m3 quantisation of an fp32 array.

    scale = amax/448 (1 where amax == 0); codes = e4m3(clamp(x/scale, +-448)).
    Returns (codes uint8 same shape, scale float32 shape[:-1]).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    amax = np.abs(x).max(axis=-1)
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
    y = np.clip(x / scale[..., None], -E4M3_MAX, E4M3_MAX).astype(np.float32)
    codes = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, scale


def gaussian(rng: np.random.Generator, shape, d: Optional[int] = None, unscaled=False) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if not unscaled:
        x *= np.float32(1.0 / math.sqrt(d if d is not None else shape[-1]))
    return x


# ----------------------------------------------------------------------------
# paged layout
# ----------------------------------------------------------------------------
def make_block_table(rng: np.random.Generator, lengths, page_size: int):
    """Shuffled physical page assignment.  Returns (table int32 [B, max_pages], n_pages).

    Logical page p of sequence b lives in physical page table[b, p]; unused
    entries are -1.  Physical ids are a random permutation of 0..n_pages-1.
    """
    lengths = np.asarray(lengths, dtype=np.int64)
    pages = (lengths + page_size - 1) // page_size
    n_pages = int(pages.sum())
    max_pages = int(pages.max())
    perm = rng.permutation(n_pages).astype(np.int32)
    table = np.full((len(lengths), max_pages), -1, dtype=np.int32)
    off = 0
    for b, p in enumerate(pages):
        table[b, :p] = perm[off:off + p]
        off += p
    return table, n_pages


def to_pages(per_seq, lengths, table, page_size: int, n_pages: int, width: int, dtype):
    """Scatter per-sequence rows [L_b, width] into a paged pool [n_pages, page_size, width]."""
    pool = np.zeros((n_pages, page_size, width), dtype=dtype)
    for b, L in enumerate(lengths):
        rows = per_seq[b]
        for p in range((L + page_size - 1) // page_size):
            s0 = p * page_size
            s1 = min(L, s0 + page_size)
            pool[table[b, p], : s1 - s0] = rows[s0:s1]
    return pool


def ragged_lengths(rng: np.random.Generator, B: int, Lmin: int, Lmax: int) -> np.ndarray:
    u = rng.uniform(math.log(Lmin), math.log(Lmax), size=B)
    return np.clip(np.floor(np.exp(u)).astype(np.int64), Lmin, Lmax)


# ----------------------------------------------------------------------------
# workloads
# ----------------------------------------------------------------------------
@dataclasses.dataclass
class DecodeInputs:
    """One decode step for B sequences (all arrays host numpy, storage encodings).

    Indexer:  q_idx [B,HI,dI] e4m3 codes, q_scale [B] f32, w [B,HI] f32,
              keys  [B,L,dI] e4m3 codes (contiguous) or [P,ps,dI] (paged),
              k_scale [B,L] f32 or [P,ps].
    MLA:      q [B,H,Dqk] bf16 bits, kv [B,L,Dqk] bf16 bits or [P,ps,Dqk].
    lengths [B] int64: context length per sequence (the query is the last token).
    """
    shapes: Shapes
    lengths: np.ndarray
    q_idx: np.ndarray
    q_scale: np.ndarray
    w: np.ndarray
    keys: np.ndarray
    k_scale: np.ndarray
    q: np.ndarray
    kv: np.ndarray
    block_table: Optional[np.ndarray] = None
    page_size: int = 0
    needles: Optional[np.ndarray] = None

    @property
    def B(self):
        return len(self.lengths)

    @property
    def paged(self):
        return self.block_table is not None


def make_decode(B: int, L, shapes: Shapes = FULL, seed: int = 0, paged: bool = False,
                page_size: int = 64, lengths=None, regime: str = "gaussian",
                n_needles: int = 16) -> DecodeInputs:
    """Synthetic decode-step inputs.

    regime="gaussian": the configurations' N(0,1)/sqrt(d) activations.
    regime="peaked": unscaled N(0,1) q and kv plus `n_needles` planted tokens per
    sequence whose indexer key and latent row are aligned with that sequence's
    queries, so both the index scores and the attention weights are far from
    uniform.
    """
    rng = np.random.default_rng(seed)
    s = shapes
    if lengths is None:
        lengths = np.full(B, int(L), dtype=np.int64)
    lengths = np.asarray(lengths, dtype=np.int64)
    Lmax = int(lengths.max())
    unscaled = regime == "peaked"
    qi = gaussian(rng, (B, s.HI, s.dI))
    w = rng.uniform(0.0, 1.0, size=(B, s.HI)).astype(np.float32)
    q = gaussian(rng, (B, s.H, s.Dqk), unscaled=unscaled)
    ki = np.empty((B, Lmax, s.dI), dtype=np.float32)
    kv = np.empty((B, Lmax, s.Dqk), dtype=np.float32)
    for b in range(B):  # per sequence keeps peak host memory bounded
        ki[b] = gaussian(rng, (Lmax, s.dI))
        kv[b] = gaussian(rng, (Lmax, s.Dqk), unscaled=unscaled)
    needles = None
    if regime == "peaked":
        needles = np.zeros((B, n_needles), dtype=np.int64)
        for b in range(B):
            pos = rng.choice(int(lengths[b]), size=min(n_needles, int(lengths[b])), replace=False)
            needles[b, : len(pos)] = pos
            ki[b, pos] = np.maximum(qi[b], 0).sum(axis=0) * 4.0 / math.sqrt(s.dI) + ki[b, pos]
            kv[b, pos] = q[b].mean(axis=0) * 3.0 + kv[b, pos]
    q_codes, q_scale = quantize_e4m3_per_token(qi.reshape(B, -1))
    q_codes = q_codes.reshape(B, s.HI, s.dI)
    k_codes, k_scale = quantize_e4m3_per_token(ki)
    q_bits = to_bf16_bits(q)
    kv_bits = to_bf16_bits(kv)
    del ki, kv
    out = DecodeInputs(shapes=s, lengths=lengths, q_idx=q_codes, q_scale=q_scale, w=w,
                       keys=k_codes, k_scale=k_scale, q=q_bits, kv=kv_bits, needles=needles)
    if paged:
        table, n_pages = make_block_table(rng, lengths, page_size)
        out.keys = to_pages(k_codes, lengths, table, page_size, n_pages, s.dI, np.uint8)
        sc = to_pages(k_scale[..., None], lengths, table, page_size, n_pages, 1, np.float32)
        out.k_scale = sc[..., 0].copy()
        out.kv = to_pages(kv_bits, lengths, table, page_size, n_pages, s.Dqk, np.uint16)
        out.block_table = table
        out.page_size = page_size
    return out


@dataclasses.dataclass
class PrefillInputs:
    """One causal prefill of T tokens of a single sequence.

    fp32 ("f32"): q_idx [T,HI,dI] f32, keys [T,dI] f32, q [T,H,Dqk] f32, kv [T,Dqk] f32;
                  q_scale / k_scale are all ones.
    fp8/bf16 ("mixed"): q_idx e4m3 codes with per-token scale [T], keys e4m3 codes
                  with per-token scale [T], q / kv bf16 bits.
    needles [n] (peaked regime only): the planted token positions.
    """
    shapes: Shapes
    T: int
    dtype: str
    q_idx: np.ndarray
    q_scale: np.ndarray
    w: np.ndarray
    keys: np.ndarray
    k_scale: np.ndarray
    q: np.ndarray
    kv: np.ndarray
    needles: Optional[np.ndarray] = None


def make_prefill(T: int, shapes: Shapes = FULL, seed: int = 0, dtype: str = "mixed",
                 regime: str = "gaussian", n_needles: int = 16) -> PrefillInputs:
    """Synthetic causal-prefill inputs.

    regime="gaussian": the configurations' N(0,1)/sqrt(d) activations.
    regime="peaked": unscaled N(0,1) q and latent rows, and `n_needles` planted token
    positions.  Every indexer query head gets 0.5 * a added and each needle key 4 * a (a a
    random unit vector), so a needle's per-head dots are about 2 against ~0.1 for other
    tokens and every row at or after a needle keeps it; every query head gets 0.3 * c added
    and each needle latent row 0.7 * c (c with N(0,1) coordinates), which lifts a needle's
    logit by about 0.21 * 576 / 24 = 5 at the 1/sqrt(576) scale, so attention is far from
    uniform.
    """
    rng = np.random.default_rng(seed)
    s = shapes
    unscaled = regime == "peaked"
    qi = gaussian(rng, (T, s.HI, s.dI))
    w = rng.uniform(0.0, 1.0, size=(T, s.HI)).astype(np.float32)
    ki = gaussian(rng, (T, s.dI))
    q = gaussian(rng, (T, s.H, s.Dqk), unscaled=unscaled)
    kv = gaussian(rng, (T, s.Dqk), unscaled=unscaled)
    needles = None
    if regime == "peaked":
        needles = np.sort(rng.choice(T, size=min(n_needles, T), replace=False)).astype(np.int64)
        a = rng.standard_normal(s.dI).astype(np.float32)
        a /= np.float32(np.linalg.norm(a))
        c = rng.standard_normal(s.Dqk).astype(np.float32)
        qi += np.float32(0.5) * a
        ki[needles] += np.float32(4.0) * a
        q += np.float32(0.3) * c
        kv[needles] += np.float32(0.7) * c
    if dtype == "f32":
        ones = np.ones(T, dtype=np.float32)
        return PrefillInputs(s, T, "f32", qi, ones, w, ki, ones.copy(), q, kv, needles)
    q_codes, q_scale = quantize_e4m3_per_token(qi.reshape(T, -1))
    k_codes, k_scale = quantize_e4m3_per_token(ki)
    return PrefillInputs(s, T, "mixed", q_codes.reshape(T, s.HI, s.dI), q_scale, w,
                         k_codes, k_scale, to_bf16_bits(q), to_bf16_bits(kv), needles)


def make_config(config: int, **over):
    """Inputs of one of the five workload configurations (seed 1000 + config)."""
    c = CONFIGS[config]
    seed = over.pop("seed", seed_for(config))
    if c["kind"] == "prefill":
        return make_prefill(over.pop("T", c["T"]), c["shapes"], seed,
                            "f32" if c.get("dtype") == "f32" else "mixed", **over)
    if c.get("paged"):
        rng = np.random.default_rng(seed + 7)
        B = over.pop("B", c["B"])
        lengths = over.pop("lengths", None)
        if lengths is None:
            lengths = ragged_lengths(rng, B, c["Lmin"], c["Lmax"])
        return make_decode(B, None, c["shapes"], seed, paged=True, page_size=c["page_size"],
                           lengths=lengths, **over)
    return make_decode(over.pop("B", c["B"]), over.pop("L", c["L"]), c["shapes"], seed, **over)
