"""Pins of the FP8 oracle (oracle/fp8.py) against what the definitions fix:
landmark values of the E4M3 encoding, brute-force nearest-value rounding with
ties to even, the power-of-two block scale rule checked by exhaustive search,
lossless round trips, and attention of exactly representable inputs.  Planted
mistakes (ties away from zero, the bias-8 variant of the format, a floor in
the scale rule, subnormals flushed) must each fail one of them."""

import numpy as np
import pytest

import oracle
from oracle import fp8 as F


def _finite_table():
    t = F.e4m3_values()
    codes = np.array([c for c in range(256) if np.isfinite(t[c])])
    return codes, t[codes]


def _nearest_even_brute(x):
    """Nearest finite E4M3 value by exhaustive search; on a tie, the code
    with an even mantissa (last bit 0)."""
    codes, vals = _finite_table()
    out = np.empty_like(x)
    for n, xi in enumerate(x):
        dist = np.abs(vals - xi)
        best = np.flatnonzero(dist == dist.min())
        if len(best) > 1:
            # ties between two neighbours (or +0/-0 for xi == 0)
            even = [b for b in best if codes[b] % 2 == 0]
            best = even if even else best
        pick = vals[best]
        # keep the sign of x on zero
        out[n] = np.copysign(pick[0], xi) if pick[0] == 0 else pick[0]
    return out


# --- the encoding -----------------------------------------------------------

def test_e4m3_landmarks():
    v = F.e4m3_values()
    assert v[0x00] == 0.0 and np.signbit(v[0x80])
    assert v[0x01] == 2.0 ** -9            # smallest subnormal
    assert v[0x07] == 7 * 2.0 ** -9        # largest subnormal
    assert v[0x08] == 2.0 ** -6            # smallest normal
    assert v[0x38] == 1.0                  # exponent field 7 = bias
    assert v[0x7E] == 448.0 == F.E4M3_MAX  # largest finite (1.75 * 2^8)
    assert v[0xFE] == -448.0
    assert np.isnan(v[0x7F]) and np.isnan(v[0xFF])
    assert np.isfinite(v).sum() == 254     # no infinities, two NaN codes


def test_positive_codes_increase():
    v = F.e4m3_values()[:0x7F]
    assert np.all(np.diff(v) > 0)
    assert np.array_equal(F.e4m3_values()[0x80:0xFF], -v)


def test_round_is_nearest_with_ties_to_even():
    rng = np.random.default_rng(11)
    mag = np.ldexp(rng.uniform(1, 2, 4000), rng.integers(-12, 9, 4000))
    x = np.where(rng.random(4000) < 0.5, -mag, mag)
    x = x[np.abs(x) < 448 + 16]
    codes, vals = _finite_table()
    pos = vals[vals > 0]
    ties = (pos[:-1] + pos[1:]) / 2           # every midpoint between neighbours
    x = np.concatenate([x, ties[ties < 448], -ties[ties < 448], [0.0, -0.0, 2.0 ** -11, -2.0 ** -11]])
    got = F.e4m3_round(x)
    want = _nearest_even_brute(x)
    assert np.array_equal(got, want)
    assert np.array_equal(np.signbit(got), np.signbit(want))


@pytest.mark.parametrize("x,code", [
    (2.0 ** -10, 0x00), (3 * 2.0 ** -10, 0x02), (1.0625, 0x38), (1.1875, 0x3A), (7.5 * 2.0 ** -9, 0x08),
    (2.5 * 2.0 ** -9, 0x02), (3.375, 0x46), (432.0, 0x7E), (300.0, 0x79), (-0.0, 0x80), (-2.5, 0xC2),
])
def test_encode_examples(x, code):
    assert int(F.e4m3_encode(x)) == code


def test_encode_decode_round_trip():
    codes, vals = _finite_table()
    assert np.array_equal(F.e4m3_encode(vals), codes.astype(np.uint8))


def test_out_of_range_is_an_error():
    assert F.e4m3_round(455.9) == 448.0
    assert F.e4m3_round(464.0) == 448.0  # tie with the missing 480 goes to the even mantissa
    with pytest.raises(ValueError):
        F.e4m3_round(470.0)              # nearest grid point 480 is not finite


# --- the block scale --------------------------------------------------------

def _scale_exp_brute(a):
    if a == 0:
        return 0
    e = -160
    while a > 448.0 * 2.0 ** e:
        e += 1
    return max(e, -127)          # E8M0 range


def test_block_scale_rule_by_search():
    rng = np.random.default_rng(12)
    a = np.ldexp(rng.uniform(1, 2, 500), rng.integers(-40, 40, 500))
    special = [448.0, 448.0 * 2 ** -5, 448.0 * (1 + 2 ** -20), 224.0, 224.0 * (1 + 2 ** -20), 1.75, 1.76, 0.0,
               2.0 ** -130]
    a = np.concatenate([a, special])
    e = F.block_scale_exponent(a)
    assert [int(x) for x in e] == [_scale_exp_brute(float(x)) for x in a]
    pos = a > 448.0 * 2.0 ** -128            # below that the E8M0 floor 2^-127 applies
    r = a[pos] / np.ldexp(1.0, e[pos])
    assert np.all(r <= 448) and np.all(r > 224)
    assert e[a == 2.0 ** -130][0] == -127


def test_quantize_blocks_invariants():
    rng = np.random.default_rng(13)
    x = rng.standard_normal((2, 3, 150, 16)) * np.ldexp(1.0, rng.integers(-6, 6, (2, 3, 1, 1)))
    codes, ex = F.quantize_blocks(x, 64)
    assert codes.shape == x.shape and ex.shape == (2, 3, 3)
    deq = F.dequantize_blocks(codes, ex, 64)
    t = F.e4m3_values()
    _, vals = _finite_table()
    pos = np.unique(np.abs(vals))
    for blk in range(3):
        sl = slice(64 * blk, min(64 * blk + 64, 150))
        s = np.ldexp(1.0, ex[..., blk])[..., None, None]
        xs, ds = x[..., sl, :] / s, deq[..., sl, :] / s
        assert np.isin(np.abs(ds), pos).all()              # every value is an E4M3 value
        # within half the local spacing of the grid around x / s
        hi = np.searchsorted(pos, np.abs(xs))
        lo_v, hi_v = pos[np.maximum(hi - 1, 0)], pos[np.minimum(hi, len(pos) - 1)]
        assert (np.abs(xs - ds) <= (hi_v - lo_v) / 2 + 1e-300).all()
        # the block maximum lands in the top binade (224 itself when a value
        # just above 224 rounds down)
        amax_code = np.abs(t[codes[..., sl, :]]).max(axis=(-2, -1))
        assert ((amax_code >= 224) & (amax_code <= 448)).all()


def test_representable_inputs_are_lossless():
    """Entries that are E4M3 values with each block's maximum in (224, 448]
    quantize with scale 1 and no rounding, so the FP8 attention equals the
    plain definition exactly."""
    rng = np.random.default_rng(14)
    _, vals = _finite_table()

    def draw(shape, rows):
        x = rng.choice(vals[np.abs(vals) <= 64], size=shape)
        x[..., ::rows, 0] = 256.0                       # a maximum in every block
        return x * 2.0 ** -6

    q, k, v = draw((1, 2, 100, 8), 32), draw((1, 1, 70, 8), 16), draw((1, 1, 70, 8), 16)
    q8, qe = F.quantize_blocks(q, 32)
    k8, ke = F.quantize_blocks(k, 16)
    v8, ve = F.quantize_blocks(v, 16)
    assert np.array_equal(F.dequantize_blocks(q8, qe, 32), q)
    O, L = F.sdpa_fp8(q8, qe, k8, ke, v8, ve, True, 0.3, q_rows=32, kv_rows=16)
    O2, L2 = oracle.sdpa(q, k, v, True, 0.3)
    assert np.array_equal(O, O2) and np.array_equal(L, L2)


def test_rotation_leaves_scores_unchanged():
    """Incoherent processing: (Q R)(K R)^T = Q K^T for orthogonal R, so the
    attention of the rotated, unquantized inputs is the original one; and an
    outlier coordinate is spread over the head dimension."""
    rng = np.random.default_rng(15)
    d = 16
    R, _ = np.linalg.qr(rng.standard_normal((d, d)))
    q, k, v = rng.standard_normal((1, 2, 40, d)), rng.standard_normal((1, 2, 40, d)), rng.standard_normal((1, 2, 40, d))
    k[0, 0, 5, 3] = 200.0
    O1, L1 = oracle.sdpa(q @ R, k @ R, v, True, 0.25)
    O2, L2 = oracle.sdpa(q, k, v, True, 0.25)
    np.testing.assert_allclose(O1, O2, atol=1e-12)
    np.testing.assert_allclose(L1, L2, atol=1e-10)
    kr = k[0, 0, 5] @ R
    assert np.abs(kr).max() < 0.9 * 200.0
    # quantize with the rotation = quantize the rotated rows (each row x -> R x)
    c1, e1 = F.quantize_blocks(k, 8, rot=R)
    c2, e2 = F.quantize_blocks(k @ R.T, 8)
    assert np.array_equal(c1, c2) and np.array_equal(e1, e2)


# --- planted mistakes ---------------------------------------------------------

def _run_fp8_pins():
    checks = {
        "landmarks": test_e4m3_landmarks,
        "nearest_even": test_round_is_nearest_with_ties_to_even,
        "round_trip": test_encode_decode_round_trip,
        "scale": test_block_scale_rule_by_search,
        "blocks": test_quantize_blocks_invariants,
        "lossless": test_representable_inputs_are_lossless,
    }
    failed = []
    for name, fn in checks.items():
        try:
            fn()
        except (AssertionError, ValueError, IndexError):
            failed.append(name)
    return failed


def test_fp8_pins_pass_on_the_oracle():
    assert _run_fp8_pins() == []


_orig_round = F.e4m3_round


def _round_ties_away(x):
    x = np.asarray(x, dtype=np.float64)
    a = np.abs(x)
    _, e = np.frexp(a)
    step = np.ldexp(1.0, np.maximum(e - 1, -6) - 3)
    return np.copysign(np.floor(a / step + 0.5) * step, x)


def _round_flush_subnormals(x):
    r = _orig_round(x)
    return np.where(np.abs(r) < 2.0 ** -6, np.copysign(0.0, r), r)


def _decode_bias8(code):
    s, e, m = code >> 7, (code >> 3) & 15, code & 7
    if e == 15 and m == 7:
        return float("nan")
    v = (m / 8.0) * 2.0 ** -7 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 8)
    return -v if s else v


def _scale_floor(amax):
    a = np.asarray(amax, dtype=np.float64)
    f, e2 = np.frexp(a)
    return np.where(a > 0, (e2 - 1) - 8, 0).astype(np.int64)


@pytest.mark.parametrize("name", ["ties_away", "flush_subnormals", "bias8", "scale_floor"])
def test_fp8_planted_mistakes_are_caught(monkeypatch, name):
    if name == "ties_away":
        monkeypatch.setattr(F, "e4m3_round", _round_ties_away)
    elif name == "flush_subnormals":
        monkeypatch.setattr(F, "e4m3_round", _round_flush_subnormals)
    elif name == "bias8":
        monkeypatch.setattr(F, "_decode_one", _decode_bias8)
        monkeypatch.setattr(F, "_TABLE", np.array([_decode_bias8(c) for c in range(256)]))
    else:
        monkeypatch.setattr(F, "block_scale_exponent", _scale_floor)
    assert _run_fp8_pins(), f"no FP8 pin caught {name}"
