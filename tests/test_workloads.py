"""Seeded input generator: determinism, shapes, layout conventions (CPU only)."""
import numpy as np
import torch

import workloads as W


def test_same_seed_same_bytes():
    a = W.make("1")
    b = W.make("1")
    for f in ("q", "k_new", "v_new", "k_cache", "v_cache", "lens", "pos"):
        assert np.array_equal(getattr(a, f), getattr(b, f)), f
    c = W.make("1", seed=99)
    assert not np.array_equal(a.k_cache, c.k_cache)


def test_cache_draws_independent_of_thread_count(monkeypatch):
    monkeypatch.setattr(W, "_CHUNK", 1000)
    monkeypatch.setattr(W, "_THREADS", 1)
    one = W.make("2a", L=100)
    monkeypatch.setattr(W, "_THREADS", 7)
    many = W.make("2a", L=100)
    assert np.array_equal(one.k_cache, many.k_cache)
    assert np.array_equal(one.v_cache, many.v_cache)
    assert not np.array_equal(one.k_cache, one.v_cache)
    assert np.array_equal(one.w_k, many.w_k)


def test_bf16_rounding_of_draws_matches_torch():
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    assert np.array_equal(W.fp32_to_bf16_bits(x), ref)


def test_layouts_and_shapes():
    w1 = W.make("1")
    assert (w1.B, w1.Hq, w1.Hkv, w1.D, w1.T) == (1, 8, 2, 64, 128)
    assert w1.pos.tolist() == [127] and w1.lens.tolist() == [128]
    assert w1.q.shape == (1, 8, 64) and w1.k_cache.shape == (1, 2, 128, 64)
    assert w1.w_q is None and w1.theta == 1e4 and w1.out_dtype == "f32"
    w2 = W.make("2b")
    assert (w2.T, int(w2.pos[0]), int(w2.lens[0])) == (2048 + 64, 2048, 2049)
    assert w2.w_q.dtype == np.float32 and w2.w_q.shape == (128,)
    assert abs(float(w2.w_q.mean()) - 1.0) < 0.05
    w5 = W.make("5", B=2, L=1024, window=256)
    assert w5.window == 256 and w5.pos.tolist() == [1023, 1023]
    w4 = W.make("4", L=4096)
    assert w4.pos is None and w4.k_new is None


def test_ragged_lens_independent_of_sizes():
    # lens are drawn first, so reduced D/T variants keep config 3's lengths
    a = W.make("3", D=8, Hq=4, Hkv=1)
    b = W.make("3", D=16, Hq=8, Hkv=2)
    assert np.array_equal(a.lens, b.lens)
    assert a.lens.min() >= 128 and a.lens.max() <= 4096
    assert np.array_equal(a.pos, a.lens - 1)


def test_peaky_rows_scaled_by_four():
    w = W.make("4", L=2048)
    plain = W.make("4", L=2048, peaky=0.0)
    m = int(round(0.01 * 2048))
    assert w.peaky_rows.shape == (1, 8, m)
    for g in range(8):
        rows = w.peaky_rows[0, g]
        assert len(set(rows.tolist())) == m
        a = w.k_cache[0, g, rows].astype(np.uint32) << 16
        b = plain.k_cache[0, g, rows].astype(np.uint32) << 16
        assert np.array_equal(a.view(np.float32), 4 * b.view(np.float32))
        other = np.setdiff1d(np.arange(2048), rows)
        assert np.array_equal(w.k_cache[0, g, other], plain.k_cache[0, g, other])


def test_kv_bytes():
    w = W.make("5", B=2, L=1024, window=256)
    assert W.kv_bytes(w) == 2 * 8 * 256 * 128 * 4
    w = W.make("3", D=8, Hq=4, Hkv=1)
    assert W.kv_bytes(w) == int(w.lens.sum()) * 1 * 8 * 4
