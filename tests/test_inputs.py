"""The seeded input generator: determinism, shapes, and the stated recipe."""

import numpy as np
import pytest

from exact_tiled_attention_14_amd import inputs as I


def test_bf16_rounding_ties_to_even_and_specials():
    x = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -9, -3.3, np.inf, -np.inf, 3.4e38, 0.0, -0.0],
                 dtype=np.float32)
    bits = I.bf16_bits(x)
    assert list(bits[:3]) == [0x3F80, 0x3F80, 0x3F81]     # tie goes to even, above-tie rounds up
    assert bits[4] == 0x7F80 and bits[5] == 0xFF80 and bits[6] == 0x7F80
    assert bits[7] == 0 and bits[8] == 0x8000
    assert np.isnan(I.bf16_to_f32(I.bf16_bits(np.array([np.nan], np.float32))))[0]


def test_bf16_rounding_is_nearest():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(20000) * 10).astype(np.float32)
    r = I.round_to_bf16(x).astype(np.float64)
    up = I.bf16_to_f32(I.bf16_bits(x) + 1).astype(np.float64)
    dn = I.bf16_to_f32(I.bf16_bits(x) - 1).astype(np.float64)
    err = np.abs(r - x)
    assert (err <= np.abs(up - x)).all() and (err <= np.abs(dn - x)).all()
    y = x.copy()
    I._round_bf16_inplace(y)
    np.testing.assert_array_equal(y, I.round_to_bf16(x))


def test_prefill_is_deterministic_and_bf16_exact():
    a = I.make_prefill(1, 4, 2, 33, 40, 16, causal=True, seed=5)
    b = I.make_prefill(1, 4, 2, 33, 40, 16, causal=True, seed=5)
    c = I.make_prefill(1, 4, 2, 33, 40, 16, causal=True, seed=6)
    for t in "qkv":
        np.testing.assert_array_equal(getattr(a, t), getattr(b, t))
        assert not np.array_equal(getattr(a, t), getattr(c, t))
        np.testing.assert_array_equal(I.round_to_bf16(getattr(a, t)), getattr(a, t))
    assert a.q.shape == (1, 4, 33, 16) and a.k.shape == (1, 2, 40, 16)
    assert a.scale == pytest.approx(0.25)


def test_outliers_count_and_size():
    base = I.make_prefill(1, 2, 2, 64, 64, 32, causal=True, seed=3)
    out = I.make_prefill(1, 2, 2, 64, 64, 32, causal=True, seed=3, outlier_frac=0.001 * 10)
    n = int(round(0.01 * out.k.size))
    assert out.meta["outliers"] == n
    changed = out.k != base.k
    assert changed.sum() <= n          # a scaled exact zero would stay equal
    ratio = out.k[changed] / base.k[changed]
    assert np.allclose(ratio, 20.0, rtol=2 ** -7)
    np.testing.assert_array_equal(out.q, base.q)


def test_checked_rows_are_distinct_and_sorted():
    c = I.make_prefill(1, 3, 1, 100, 100, 8, causal=True, seed=1, check_rows=20)
    assert c.rows.shape == (1, 3, 20)
    for r in c.rows.reshape(-1, 20):
        assert (np.diff(r) > 0).all() and r.min() >= 0 and r.max() < 100


def test_decode_block_table_is_a_permutation():
    d = I.make_decode(6, 8, 2, 16, len_lo=1, len_hi=70, block_size=16, seed=2)
    pages = -(-d.seqlens.astype(int) // 16)
    ids = np.concatenate([d.block_table[s, :p] for s, p in enumerate(pages)])
    assert sorted(ids.tolist()) == list(range(d.kcache_bits.shape[0]))
    for s, p in enumerate(pages):
        assert (d.block_table[s, p:] == -1).all()
    assert d.seqlens.min() >= 1 and d.seqlens.max() <= 70


def test_decode_poisoned_tails_only_past_length():
    d = I.make_decode(5, 4, 1, 8, len_lo=1, len_hi=40, seed=4, poison_tail=True)
    kc = d.kcache
    for s in range(5):
        n = int(d.seqlens[s])
        p = -(-n // 16)
        toks = kc[d.block_table[s, :p], 0].reshape(-1, 8)
        assert np.isfinite(toks[:n]).all()
        assert np.isnan(toks[n:]).all()


def test_decode_subset_keeps_the_logical_sequence():
    d = I.make_decode(4, 4, 2, 8, len_lo=10, len_hi=50, seed=9)
    sub = d.subset([2, 0])
    for i, s in enumerate([2, 0]):
        n = int(d.seqlens[s])
        p = -(-n // 16)
        full = d.kcache[d.block_table[s, :p]]
        mine = sub.kcache[sub.block_table[i, :p]]
        np.testing.assert_array_equal(full, mine)
        assert sub.seqlens[i] == n


def test_rotation_is_seeded_orthogonal_and_bf16_exact():
    R = I.make_rotation(128, seed=3)
    assert R.dtype == np.float32 and R.shape == (128, 128)
    np.testing.assert_array_equal(R, I.make_rotation(128, seed=3))
    assert not np.array_equal(R, I.make_rotation(128, seed=4))
    np.testing.assert_array_equal(R, I.round_to_bf16(R))
    # orthogonal up to the bf16 rounding of its entries (relative 2^-9)
    assert np.abs(R.astype(np.float64) @ R.T - np.eye(128)).max() < 8e-3
