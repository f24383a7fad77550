"""Seeded input generator: determinism, shapes and encodings (CPU only)."""
import numpy as np

import datagen
from oracle.formats import decode_bf16, decode_e4m3


def test_decode_inputs_are_seeded_and_shaped():
    sh = datagen.Shapes(H=4, Dqk=24, Dv=16, HI=2, dI=8, k=8)
    a = datagen.make_decode(3, 50, sh, seed=11)
    b = datagen.make_decode(3, 50, sh, seed=11)
    c = datagen.make_decode(3, 50, sh, seed=12)
    assert a.q_idx.shape == (3, 2, 8) and a.q_idx.dtype == np.uint8
    assert a.keys.shape == (3, 50, 8) and a.k_scale.shape == (3, 50)
    assert a.q.shape == (3, 4, 24) and a.q.dtype == np.uint16 and a.kv.shape == (3, 50, 24)
    assert np.array_equal(a.keys, b.keys) and np.array_equal(a.kv, b.kv)
    assert not np.array_equal(a.keys, c.keys)
    assert (a.w >= 0).all() and (a.w < 1).all()


def test_e4m3_quantiser_round_trip():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((100, 128)).astype(np.float32) / np.sqrt(128)
    x[3] = 0.0
    codes, scale = datagen.quantize_e4m3_per_token(x)
    assert scale[3] == 1.0
    y = decode_e4m3(codes) * scale[:, None]
    assert np.isfinite(y).all()
    # e4m3 has 3 mantissa bits: relative error <= 2^-4 for normals; the row max maps to 448 exactly
    amax = np.abs(x).max(1)
    assert np.all(np.abs(decode_e4m3(codes)).max(1)[amax > 0] == 448.0)
    err = np.abs(y - x)
    assert np.all(err <= np.maximum(np.abs(x) * 2.0 ** -4, scale[:, None] * 2.0 ** -10) + 1e-12)


def test_bf16_encoding_round_trip():
    x = np.array([1.0, -2.5, 3.14159, 1e-30], dtype=np.float32)
    y = decode_bf16(datagen.to_bf16_bits(x))
    assert np.all(np.abs(y - x) <= np.abs(x) * 2.0 ** -8)


def test_ragged_lengths_and_table():
    rng = np.random.default_rng(4)
    L = datagen.ragged_lengths(rng, 64, 1024, 131072)
    assert L.min() >= 1024 and L.max() <= 131072
    table, n_pages = datagen.make_block_table(rng, L, 64)
    assert n_pages == int(((L + 63) // 64).sum())
    used = table[table >= 0]
    assert sorted(used.tolist()) == list(range(n_pages))


def test_config_seeds():
    assert [datagen.seed_for(c) for c in range(1, 6)] == [1001, 1002, 1003, 1004, 1005]
    t = datagen.make_config(1, T=16)
    assert t.dtype == "f32" and t.q.shape == (16, 4, 80) and t.keys.shape == (16, 32)
