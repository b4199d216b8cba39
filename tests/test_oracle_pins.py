"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each test names what fixes the expected value: a hand-derived worked example,
a closed form, an invariant of the mathematics, a library routine, or brute
force on tiny inputs.  ``test_planted_mistakes_are_caught`` plants plausible
mistakes into the oracle (on the CPU) and checks that some pin fails for each.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import attention as oa

RNG = np.random.default_rng(1234)


def _rand(*shape, rng=RNG):
    return rng.standard_normal(shape)


def _num(x):
    if isinstance(x, str) and x.startswith("ln"):
        return math.log(float(x[2:]))
    return float(x)


def _arr(x):
    return np.array([[_num(e) for e in row] for row in x]) if isinstance(x[0], list) \
        else np.array([_num(e) for e in x])


# --- 1. hand-derived worked example ---------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_worked_example(golden_dir, causal):
    g = json.load(open(os.path.join(golden_dir, "worked_example_2q2k.json")))
    q, k, v = _arr(g["q"]), _arr(g["k"]), _arr(g["v"])
    O, lse = oracle.sdpa(q[None, None], k[None, None], v[None, None], causal, g["scale"])
    want = g["causal" if causal else "non_causal"]
    np.testing.assert_allclose(O[0, 0], _arr(want["o"]), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[0, 0], _arr(want["lse"]), rtol=0, atol=1e-12)


# --- 2. brute force with pure-Python loops --------------------------------

def _brute(q, k, v, causal, scale):
    """Softmax straight from its definition: e^s / sum e^s, no max shift."""
    B, Hq, Sq, d = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    O = [[[[0.0] * d for _ in range(Sq)] for _ in range(Hq)] for _ in range(B)]
    L = [[[0.0] * Sq for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        for h in range(Hq):
            kv = h * Hkv // Hq
            for i in range(Sq):
                ws = []
                for j in range(Sk):
                    if causal and j > i + Sk - Sq:
                        ws.append(0.0)
                        continue
                    s = sum(q[b, h, i, t] * k[b, kv, j, t] for t in range(d)) * scale
                    ws.append(math.exp(s))
                tot = sum(ws)
                if tot == 0.0:
                    L[b][h][i] = -math.inf
                    continue
                L[b][h][i] = math.log(tot)
                for c in range(d):
                    O[b][h][i][c] = sum(ws[j] * v[b, kv, j, c] for j in range(Sk)) / tot
    return np.array(O), np.array(L)


@pytest.mark.parametrize("B,Hq,Hkv,Sq,Sk,d", [(1, 1, 1, 5, 5, 3), (2, 4, 2, 4, 6, 2),
                                               (1, 3, 1, 6, 4, 4), (1, 2, 2, 1, 7, 3)])
@pytest.mark.parametrize("causal", [False, True])
def test_brute_force_tiny(B, Hq, Hkv, Sq, Sk, d, causal):
    rng = np.random.default_rng(B * 100 + Sq * 10 + Sk)
    q, k, v = (rng.standard_normal(s) for s in [(B, Hq, Sq, d), (B, Hkv, Sk, d), (B, Hkv, Sk, d)])
    scale = 0.7
    O, lse = oracle.sdpa(q, k, v, causal, scale)
    Ob, Lb = _brute(q, k, v, causal, scale)
    np.testing.assert_allclose(O, Ob, rtol=0, atol=1e-12)
    np.testing.assert_array_equal(np.isinf(lse), np.isinf(Lb))
    fin = np.isfinite(Lb)
    np.testing.assert_allclose(lse[fin], Lb[fin], rtol=0, atol=1e-12)


# --- 3. library routines --------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Sq,Sk", [(16, 16), (8, 24)])
def test_matches_torch_sdpa_and_scipy_logsumexp(causal, Sq, Sk):
    torch = pytest.importorskip("torch")
    from scipy.special import logsumexp
    B, Hq, Hkv, d = 2, 4, 2, 8
    q, k, v = _rand(B, Hq, Sq, d), _rand(B, Hkv, Sk, d), _rand(B, Hkv, Sk, d)
    scale = 1 / math.sqrt(d)
    O, lse = oracle.sdpa(q, k, v, causal, scale)
    g = Hq // Hkv
    kr, vr = np.repeat(k, g, axis=1), np.repeat(v, g, axis=1)
    mask = None
    if causal:
        i, j = np.arange(Sq)[:, None], np.arange(Sk)[None, :]
        mask = torch.from_numpy(j <= i + (Sk - Sq))
    To = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(kr), torch.from_numpy(vr),
        attn_mask=mask, scale=scale).numpy()
    np.testing.assert_allclose(O, To, rtol=0, atol=1e-12)
    S = scale * np.einsum("bhid,bhjd->bhij", q, kr)
    if causal:
        S = np.where(mask.numpy(), S, -np.inf)
    np.testing.assert_allclose(lse, logsumexp(S, axis=-1), rtol=0, atol=1e-12)


# --- 4. closed forms ------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_probability_rows_sum_to_one(causal):
    q, k, v = _rand(1, 2, 9, 4), _rand(1, 2, 9, 4), _rand(1, 2, 9, 4)
    _, _, P = oracle.sdpa(q, k, v, causal, 0.5, return_probs=True)
    np.testing.assert_allclose(P.sum(-1), 1.0, rtol=0, atol=1e-12)
    assert (P >= 0).all()
    if causal:
        assert (P[..., np.triu_indices(9, 1)[0], np.triu_indices(9, 1)[1]] == 0).all()


@pytest.mark.parametrize("causal", [False, True])
def test_all_ones_values_give_all_ones(causal):
    q, k = _rand(2, 4, 11, 8) * 3, _rand(2, 2, 11, 8) * 3
    O, _ = oracle.sdpa(q, k, np.ones((2, 2, 11, 8)), causal, 0.4)
    np.testing.assert_allclose(O, 1.0, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_zero_query_gives_mean_of_visible_values(causal):
    Sq = Sk = 13
    v = _rand(1, 1, Sk, 5)
    O, lse = oracle.sdpa(np.zeros((1, 1, Sq, 5)), _rand(1, 1, Sk, 5), v, causal, 1.0)
    if causal:
        counts = np.arange(1, Sq + 1)
        want = np.cumsum(v[0, 0], axis=0) / counts[:, None]
    else:
        counts = np.full(Sq, Sk)
        want = np.broadcast_to(v[0, 0].mean(0), (Sq, 5))
    np.testing.assert_allclose(O[0, 0], want, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[0, 0], np.log(counts), rtol=0, atol=1e-12)


def test_causal_first_row_is_first_value():
    q, k, v = _rand(2, 3, 7, 6), _rand(2, 3, 7, 6), _rand(2, 3, 7, 6)
    O, lse = oracle.sdpa(q, k, v, True, 0.3)
    np.testing.assert_array_equal(O[:, :, 0], v[:, :, 0])
    np.testing.assert_allclose(lse[:, :, 0], 0.3 * np.einsum("bhd,bhd->bh", q[:, :, 0], k[:, :, 0]),
                               rtol=0, atol=1e-12)


def test_dominant_key_returns_its_value_within_bound():
    Sk, d = 20, 8
    q, k, v = _rand(1, 1, 4, d), _rand(1, 1, Sk, d), _rand(1, 1, Sk, d)
    i, jstar, scale = 2, 13, 1.0
    k[0, 0, jstar] = 12.0 * q[0, 0, i]
    O, _ = oracle.sdpa(q, k, v, False, scale)
    s = scale * k[0, 0] @ q[0, 0, i]
    gaps = s[jstar] - np.delete(s, jstar)
    assert gaps.min() > 10
    bound = 2 * np.abs(v).max() * np.exp(-gaps).sum()
    assert np.abs(O[0, 0, i] - v[0, 0, jstar]).max() <= bound


@pytest.mark.parametrize("causal", [False, True])
def test_common_key_shift_moves_only_lse(causal):
    """Adding u to every key adds scale*q.u to a row's scores: O is unchanged."""
    q, k, v = _rand(1, 2, 10, 6), _rand(1, 2, 10, 6), _rand(1, 2, 10, 6)
    u = 150.0 * _rand(6)                      # scores of order 1e3
    O0, l0 = oracle.sdpa(q, k, v, causal, 1.0)
    O1, l1 = oracle.sdpa(q, k + u, v, causal, 1.0)
    np.testing.assert_allclose(O1, O0, rtol=0, atol=1e-9)
    np.testing.assert_allclose(l1, l0 + q @ u, rtol=1e-12, atol=1e-9)


# --- 5. grouped-query attention -------------------------------------------

def test_kv_head_mapping_table():
    assert [oracle.kv_head_of(h, 32, 8) for h in range(32)] == [h // 4 for h in range(32)]
    assert [oracle.kv_head_of(h, 6, 6) for h in range(6)] == list(range(6))      # MHA
    assert [oracle.kv_head_of(h, 6, 1) for h in range(6)] == [0] * 6              # MQA
    with pytest.raises(ValueError):
        oracle.kv_head_of(0, 6, 4)


@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (8, 8), (8, 1)])
def test_gqa_groups_read_their_own_kv_head(Hq, Hkv):
    """V constant per K/V head: each query head's output names its K/V head."""
    v = np.broadcast_to(np.arange(1, Hkv + 1, dtype=float)[None, :, None, None], (1, Hkv, 9, 4)).copy()
    O, _ = oracle.sdpa(_rand(1, Hq, 9, 4), _rand(1, Hkv, 9, 4), v, True, 0.5)
    want = np.array([h // (Hq // Hkv) + 1 for h in range(Hq)], dtype=float)
    np.testing.assert_allclose(O, np.broadcast_to(want[None, :, None, None], O.shape), rtol=0, atol=1e-12)


def test_gqa_equals_mha_on_repeated_heads():
    q, k, v = _rand(2, 8, 6, 4), _rand(2, 2, 6, 4), _rand(2, 2, 6, 4)
    O, l = oracle.sdpa(q, k, v, True, 0.5)
    O2, l2 = oracle.sdpa(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1), True, 0.5)
    np.testing.assert_array_equal(O, O2)
    np.testing.assert_array_equal(l, l2)


# --- 6. online softmax twins (block size must not matter) ------------------

@pytest.mark.parametrize("fn", [oracle.online_softmax_normalised, oracle.online_softmax_deferred])
@pytest.mark.parametrize("block", [1, 3, 7, 32])
@pytest.mark.parametrize("Sq,Sk,causal", [(17, 17, True), (17, 17, False), (20, 12, True), (9, 25, True)])
def test_online_softmax_equals_definition(fn, block, Sq, Sk, causal):
    q, k, v = _rand(Sq, 5), _rand(Sk, 5), _rand(Sk, 5)
    O, lse = fn(q, k, v, block, causal, 0.6)
    Od, ld = oracle.sdpa(q[None, None], k[None, None], v[None, None], causal, 0.6)
    np.testing.assert_allclose(O, Od[0, 0], rtol=0, atol=1e-12)
    np.testing.assert_array_equal(np.isinf(lse), np.isinf(ld[0, 0]))
    f = np.isfinite(lse)
    np.testing.assert_allclose(lse[f], ld[0, 0][f], rtol=0, atol=1e-12)


@pytest.mark.parametrize("fn", [oracle.online_softmax_normalised, oracle.online_softmax_deferred])
@pytest.mark.parametrize("dtype", [np.float64, np.float32])
def test_online_softmax_handles_large_logits(fn, dtype):
    """Scores near 1e3 would overflow e^s in either precision without the max shift."""
    q, k, v = (_rand(8, 4) * 40).astype(dtype), (_rand(8, 4) * 40).astype(dtype), _rand(8, 4)
    O, lse = fn(q, k, v, 3, True, 1.0)
    assert np.isfinite(O).all() and np.isfinite(lse).all()
    s = np.where(np.tril(np.ones((8, 8), bool)), q.astype(float) @ k.astype(float).T, -np.inf)
    assert np.abs(s[np.isfinite(s)]).max() > 500
    from scipy.special import logsumexp, softmax
    np.testing.assert_allclose(lse, logsumexp(s, axis=1), rtol=1e-12, atol=1e-9)
    np.testing.assert_allclose(O, softmax(s, axis=1) @ v, rtol=0, atol=1e-9)


def test_fully_masked_rows_are_zero_with_minus_inf_lse():
    q, k, v = _rand(1, 1, 6, 3), _rand(1, 1, 2, 3), _rand(1, 1, 2, 3)
    O, lse = oracle.sdpa(q, k, v, True, 1.0)           # rows 0..3 see no key
    assert not np.isnan(O).any() and not np.isnan(lse).any()
    np.testing.assert_array_equal(O[0, 0, :4], 0.0)
    assert np.isneginf(lse[0, 0, :4]).all() and np.isfinite(lse[0, 0, 4:]).all()
    np.testing.assert_array_equal(O[0, 0, 4], v[0, 0, 0])


def test_sdpa_rows_match_brute_force():
    q, k, v = _rand(1, 2, 12, 3), _rand(1, 1, 12, 3), _rand(1, 1, 12, 3)
    rows = np.array([[[0, 5, 11], [2, 3, 7]]])
    O, lse = oracle.sdpa_rows(q, k, v, rows, True, 0.8)
    Ob, Lb = _brute(q, k, v, True, 0.8)
    for h in range(2):
        np.testing.assert_allclose(O[0, h], Ob[0, h, rows[0, h]], rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[0, h], Lb[0, h, rows[0, h]], rtol=0, atol=1e-12)


# --- 7. split ranges and their merge --------------------------------------

@pytest.mark.parametrize("bounds", [[(0, 40)], [(0, 13), (13, 14), (14, 40)],
                                    [(0, 0), (0, 20), (20, 20), (20, 40)]])
def test_merge_of_split_ranges_equals_whole(bounds):
    q, k, v = _rand(3, 6), _rand(40, 6), _rand(40, 6)
    o, lse = oracle.merge_partials(oracle.split_partials(q, k, v, bounds, 0.4))
    Od, ld = oracle.sdpa(q[None, None], k[None, None], v[None, None], False, 0.4)
    np.testing.assert_allclose(o, Od[0, 0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, ld[0, 0], rtol=0, atol=1e-12)


def test_merge_of_empty_ranges_is_zero():
    q, k, v = _rand(2, 4), _rand(5, 4), _rand(5, 4)
    o, lse = oracle.merge_partials(oracle.split_partials(q, k, v, [(0, 0), (3, 3)], 1.0))
    np.testing.assert_array_equal(o, 0.0)
    assert np.isneginf(lse).all()


# --- 8. paged decode ------------------------------------------------------

def _paged(n_lens, Hkv, d, bs, rng):
    """A small paged cache plus the contiguous K/V it stores."""
    pages = [-(-n // bs) for n in n_lens]
    nb = sum(pages)
    perm = rng.permutation(nb)
    table = np.full((len(n_lens), max(pages)), -1, dtype=np.int32)
    kc, vc = rng.standard_normal((nb, Hkv, bs, d)), rng.standard_normal((nb, Hkv, bs, d))
    c = 0
    for s, p in enumerate(pages):
        table[s, :p] = perm[c:c + p]
        c += p
    return kc, vc, table


def test_paged_decode_equals_contiguous_attention():
    rng = np.random.default_rng(7)
    lens, Hq, Hkv, d, bs = [37, 16, 1, 50], 6, 2, 4, 16
    kc, vc, table = _paged(lens, Hkv, d, bs, rng)
    q = rng.standard_normal((len(lens), Hq, d))
    o, lse = oracle.paged_decode(q, kc, vc, table, np.array(lens), 0.5)
    for s, n in enumerate(lens):
        p = -(-n // bs)
        K = kc[table[s, :p]].transpose(1, 0, 2, 3).reshape(Hkv, p * bs, d)[:, :n]
        V = vc[table[s, :p]].transpose(1, 0, 2, 3).reshape(Hkv, p * bs, d)[:, :n]
        Od, ld = oracle.sdpa(q[s][None, :, None], K[None], V[None], False, 0.5)
        np.testing.assert_allclose(o[s], Od[0, :, 0], rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[s], ld[0, :, 0], rtol=0, atol=1e-12)


def test_paged_decode_ignores_physical_placement():
    rng = np.random.default_rng(8)
    lens = [33, 70]
    kc, vc, table = _paged(lens, 1, 3, 16, rng)
    q = rng.standard_normal((2, 2, 3))
    o, lse = oracle.paged_decode(q, kc, vc, table, np.array(lens), 1.0)
    perm = rng.permutation(kc.shape[0])                  # new home of block b is perm[b]
    kc2, vc2 = np.empty_like(kc), np.empty_like(vc)
    kc2[perm], vc2[perm] = kc, vc
    table2 = np.where(table >= 0, perm[np.maximum(table, 0)], -1)
    o2, lse2 = oracle.paged_decode(q, kc2, vc2, table2, np.array(lens), 1.0)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, lse2)


def test_paged_decode_is_last_row_of_causal_prefill():
    rng = np.random.default_rng(9)
    n, Hq, Hkv, d, bs = 45, 4, 2, 4, 16
    kc, vc, table = _paged([n], Hkv, d, bs, rng)
    p = -(-n // bs)
    K = kc[table[0, :p]].transpose(1, 0, 2, 3).reshape(Hkv, p * bs, d)[:, :n]
    V = vc[table[0, :p]].transpose(1, 0, 2, 3).reshape(Hkv, p * bs, d)[:, :n]
    Q = rng.standard_normal((1, Hq, n, d))
    O, L = oracle.sdpa(Q, K[None], V[None], True, 0.5)
    o, lse = oracle.paged_decode(Q[:, :, -1], kc, vc, table, np.array([n]), 0.5)
    np.testing.assert_allclose(o[0], O[0, :, -1], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[0], L[0, :, -1], rtol=0, atol=1e-12)


def test_paged_decode_dominant_key_finds_its_logical_position():
    """A marker key at logical token 21 (page 1, slot 5) must return V at token 21."""
    rng = np.random.default_rng(10)
    n, bs, d = 40, 16, 4
    kc, vc, table = _paged([n], 1, d, bs, rng)
    q = rng.standard_normal((1, 1, d))
    kc[table[0, 1], 0, 5] = 60.0 * q[0, 0] / (q[0, 0] @ q[0, 0])     # score exactly 60
    o, _ = oracle.paged_decode(q, kc, vc, table, np.array([n]), 1.0)
    K = kc[table[0, :3], 0].reshape(-1, d)[:n]
    s = K @ q[0, 0]
    gaps = 60.0 - np.delete(s, 21)
    assert gaps.min() > 20
    bound = 2 * np.abs(vc).max() * np.exp(-gaps).sum()
    assert np.abs(o[0, 0] - vc[table[0, 1], 0, 5]).max() <= bound


def test_paged_decode_empty_sequence():
    rng = np.random.default_rng(11)
    kc, vc, table = _paged([16], 1, 3, 16, rng)
    o, lse = oracle.paged_decode(rng.standard_normal((2, 1, 3)), kc, vc,
                                 np.vstack([table, table]), np.array([16, 0]), 1.0)
    np.testing.assert_array_equal(o[1], 0.0)
    assert np.isneginf(lse[1]).all() and np.isfinite(lse[0]).all()


# --- 8b. multi-query paged attention (verify / chunked steps) -------------

def test_paged_multi_query_is_last_rows_of_causal_prefill():
    """The Sq new tokens of a sequence get exactly the last Sq rows of a causal
    prefill over the whole gathered sequence (their K, V are the last Sq
    cached tokens)."""
    rng = np.random.default_rng(12)
    n, Sq, Hq, Hkv, d, bs = 45, 5, 4, 2, 4, 16
    kc, vc, table = _paged([n], Hkv, d, bs, rng)
    p = -(-n // bs)
    K = kc[table[0, :p]].transpose(1, 0, 2, 3).reshape(Hkv, p * bs, d)[:, :n]
    V = vc[table[0, :p]].transpose(1, 0, 2, 3).reshape(Hkv, p * bs, d)[:, :n]
    Q = rng.standard_normal((1, Hq, n, d))
    O, L = oracle.sdpa(Q, K[None], V[None], True, 0.5)
    q = Q[0, :, n - Sq:].transpose(1, 0, 2)[None]              # [1, Sq, Hq, d]
    o, lse = oracle.paged_multi_query(q, kc, vc, table, np.array([n]), 0.5)
    np.testing.assert_allclose(o[0], O[0, :, n - Sq:].transpose(1, 0, 2), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[0], L[0, :, n - Sq:].T, rtol=0, atol=1e-12)


def test_paged_multi_query_with_one_token_is_decode():
    rng = np.random.default_rng(13)
    lens, Hq, Hkv, d, bs = [37, 16, 1, 50], 6, 2, 4, 16
    kc, vc, table = _paged(lens, Hkv, d, bs, rng)
    q = rng.standard_normal((len(lens), Hq, d))
    o1, l1 = oracle.paged_decode(q, kc, vc, table, np.array(lens), 0.7)
    o2, l2 = oracle.paged_multi_query(q[:, None], kc, vc, table, np.array(lens), 0.7)
    np.testing.assert_allclose(o2[:, 0], o1, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l2[:, 0], l1, rtol=0, atol=1e-12)


def test_paged_multi_query_first_token_sees_all_but_the_new():
    """Closed form of the mask: new token 0 sees the n - Sq + 1 first keys,
    so with equal scores (q = 0) its output is the mean of those values."""
    rng = np.random.default_rng(14)
    n, Sq, d, bs = 40, 6, 3, 16
    kc, vc, table = _paged([n], 1, d, bs, rng)
    o, lse = oracle.paged_multi_query(np.zeros((1, Sq, 1, d)), kc, vc, table, np.array([n]), 1.0)
    V = vc[table[0, :3], 0].reshape(-1, d)[:n]
    for t in range(Sq):
        seen = n - Sq + t + 1
        np.testing.assert_allclose(o[0, t, 0], V[:seen].mean(axis=0), atol=1e-12)
        np.testing.assert_allclose(lse[0, t, 0], np.log(seen), atol=1e-12)


def test_paged_multi_query_short_sequence_rows_see_nothing():
    rng = np.random.default_rng(15)
    kc, vc, table = _paged([3], 1, 3, 16, rng)
    o, lse = oracle.paged_multi_query(rng.standard_normal((1, 5, 2, 3)), kc, vc, table, np.array([3]), 1.0)
    # positions 3 - 5 + t < 0 for t < 2
    assert np.isneginf(lse[0, :2]).all() and np.isfinite(lse[0, 2:]).all()
    np.testing.assert_array_equal(o[0, :2], 0.0)


def test_multi_query_planted_mistakes_are_caught(monkeypatch):
    """A verify step computed without the causal mask among the new tokens,
    or with the new tokens aligned to the start of the cache, fails a pin."""
    orig = oa.sdpa
    for mutant in (lambda q, k, v, causal, scale, **kw: orig(q, k, v, False, scale, **kw),
                   lambda q, k, v, causal, scale, **kw: orig(q, k[:, :, :q.shape[2]], v[:, :, :q.shape[2]], causal,
                                                             scale, **kw)):
        monkeypatch.setattr(oa, "sdpa", mutant)
        caught = 0
        for fn in (test_paged_multi_query_is_last_rows_of_causal_prefill,
                   test_paged_multi_query_first_token_sees_all_but_the_new):
            try:
                fn()
            except AssertionError:
                caught += 1
        monkeypatch.setattr(oa, "sdpa", orig)
        assert caught, "no multi-query pin caught the planted mistake"


# --- 8c. latent-cache (MLA) decode -----------------------------------------

def _mla_case(rng, lens, H=3, dh=4, dc=6, bs=16):
    kc, _, table = _paged(lens, 1, dc, bs, rng)
    cc = kc[:, 0]                                             # [nb, bs, d_c]
    q = rng.standard_normal((len(lens), H, dh))
    wk = rng.standard_normal((H, dc, dh)) / np.sqrt(dc)
    wv = rng.standard_normal((H, dh, dc)) / np.sqrt(dc)
    return q, wk, wv, cc, table


def test_mla_with_selecting_projections_is_mqa_decode():
    """W_K = W_V = [I; 0] pick the first d_h latent values as key and value:
    MLA is then single-K/V-head decode over those values."""
    rng = np.random.default_rng(16)
    lens = [37, 16, 50]
    q, wk, wv, cc, table = _mla_case(rng, lens)
    H, dh, dc = 3, 4, 6
    sel = np.zeros((dc, dh))
    sel[:dh] = np.eye(dh)
    wk[:] = sel
    wv[:] = sel.T
    o, lse = oracle.mla_decode(q, wk, wv, cc, table, np.array(lens), 0.7)
    c4 = cc[..., :dh][:, None]                                # [nb, 1, bs, d_h]
    o2, l2 = oracle.paged_decode(q, c4, c4, table, np.array(lens), 0.7)
    np.testing.assert_allclose(o, o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, l2, rtol=0, atol=1e-12)


def test_mla_absorbed_form_is_the_same_attention():
    """Scores q . (c W_K) = (W_K q) . c and sum_j p_j c_j W_V = (sum_j p_j c_j) W_V:
    attention over the latent values with the absorbed query, then the
    up-projection, gives the same output (the form the kernels compute)."""
    rng = np.random.default_rng(17)
    lens = [40, 23]
    q, wk, wv, cc, table = _mla_case(rng, lens)
    o, lse = oracle.mla_decode(q, wk, wv, cc, table, np.array(lens), 0.5)
    for s, n in enumerate(lens):
        C = cc[table[s, :-(-n // 16)]].reshape(-1, cc.shape[-1])[:n]
        for h in range(q.shape[1]):
            qa = wk[h] @ q[s, h]                              # [d_c]
            sc = 0.5 * (C @ qa)
            m = sc.max()
            p = np.exp(sc - m)
            lat = (p @ C) / p.sum()
            np.testing.assert_allclose(lat @ wv[h].T, o[s, h], atol=1e-12)
            np.testing.assert_allclose(m + np.log(p.sum()), lse[s, h], atol=1e-12)


def test_mla_heads_use_their_own_projections():
    rng = np.random.default_rng(18)
    lens = [30]
    q, wk, wv, cc, table = _mla_case(rng, lens)
    o, lse = oracle.mla_decode(q, wk, wv, cc, table, np.array(lens), 0.5)
    perm = [2, 0, 1]
    o2, l2 = oracle.mla_decode(q[:, perm], wk[perm], wv[perm], cc, table, np.array(lens), 0.5)
    np.testing.assert_allclose(o2, o[:, perm], atol=1e-12)
    np.testing.assert_allclose(l2, lse[:, perm], atol=1e-12)
    # scaling W_V scales the output only; scaling W_K against q changes nothing
    o3, l3 = oracle.mla_decode(q / 2, wk * 2, wv * 3, cc, table, np.array(lens), 0.5)
    np.testing.assert_allclose(o3, 3 * o, atol=1e-12)
    np.testing.assert_allclose(l3, lse, atol=1e-12)


def test_mla_planted_mistakes_are_caught(monkeypatch):
    """Keys from W_V, or values from the untransposed W_V layout, fail a pin."""
    orig = oa.mla_decode

    def swapped(q, w_uk, w_uv_t, *a, **k):
        return orig(q, np.swapaxes(w_uv_t, 1, 2), np.swapaxes(w_uk, 1, 2), *a, **k)

    def no_transpose(q, w_uk, w_uv_t, ccache, *a, **k):
        return orig(q, w_uk, np.swapaxes(w_uk, 1, 2), ccache, *a, **k)

    for mutant in (swapped, no_transpose):
        monkeypatch.setattr(oracle, "mla_decode", mutant)
        caught = 0
        for fn in (test_mla_with_selecting_projections_is_mqa_decode, test_mla_absorbed_form_is_the_same_attention):
            try:
                fn()
            except (AssertionError, ValueError):
                caught += 1
        monkeypatch.setattr(oracle, "mla_decode", orig)
        assert caught, "no MLA pin caught the planted mistake"


# --- 9. the pins catch planted mistakes -----------------------------------

def _run_pins(golden_dir):
    """Run a representative set of pins; return the names of those that fail."""
    failed = []
    checks = {
        "worked_nc": lambda: test_worked_example(golden_dir, False),
        "worked_c": lambda: test_worked_example(golden_dir, True),
        "first_row": test_causal_first_row_is_first_value,
        "gqa": lambda: test_gqa_groups_read_their_own_kv_head(8, 2),
        "zero_q": lambda: test_zero_query_gives_mean_of_visible_values(True),
        "shift": lambda: test_common_key_shift_moves_only_lse(True),
        "decode": test_paged_decode_equals_contiguous_attention,
        "marker": test_paged_decode_dominant_key_finds_its_logical_position,
        "multi_query": test_paged_multi_query_is_last_rows_of_causal_prefill,
        "mq_mask": test_paged_multi_query_first_token_sees_all_but_the_new,
        "brute": lambda: test_brute_force_tiny(1, 3, 1, 6, 4, 4, True),
    }
    for name, fn in checks.items():
        try:
            fn()
        except (AssertionError, ValueError, IndexError):
            failed.append(name)
    return failed


def test_pins_pass_on_the_oracle(golden_dir):
    assert _run_pins(golden_dir) == []


def _attend_no_scale(q, k, v, vis, scale):
    return _orig_attend(q, k, v, vis, 1.0)


def _attend_transposed_mask(q, k, v, vis, scale):
    if vis.shape[0] == vis.shape[1] and not vis.all():
        vis = vis.T
    return _orig_attend(q, k, v, vis, scale)


def _attend_kv_swapped(q, k, v, vis, scale):
    return _orig_attend(q, v, k, vis, scale)


def _attend_lse_log2(q, k, v, vis, scale):
    O, lse, P = _orig_attend(q, k, v, vis, scale)
    return O, lse / math.log(2.0), P


_orig_attend = oa._attend


@pytest.mark.parametrize("mutant,attr", [
    (_attend_no_scale, "_attend"),
    (_attend_transposed_mask, "_attend"),
    (_attend_kv_swapped, "_attend"),
    (_attend_lse_log2, "_attend"),
    (lambda hq, Hq, Hkv: hq % Hkv, "kv_head_of"),
    (lambda rows, Sq, Sk, causal: oa._orig_visible(rows, Sk, Sq, causal), "_visible"),
    (lambda rows, Sq, Sk, causal: np.arange(Sk)[None, :] <= np.asarray(rows)[:, None] if causal
     else np.ones((len(rows), Sk), bool), "_visible"),
])
def test_planted_mistakes_are_caught(monkeypatch, golden_dir, mutant, attr):
    oa._orig_visible = _orig_visible
    monkeypatch.setattr(oa, attr, mutant)
    if attr == "kv_head_of":
        monkeypatch.setattr(oracle, "kv_head_of", mutant)
    assert _run_pins(golden_dir), f"no pin caught the planted mistake in {attr}"


_orig_visible = oa._visible


# --- 10. backward: gradients of the definition -----------------------------

def _loss_and_grads(q, k, v, w, causal, scale):
    """L = sum(W * O) and the oracle's gradients for dO = W."""
    O, _ = oracle.sdpa(q, k, v, causal, scale)
    return float((w * O).sum()), oracle.sdpa_backward(q, k, v, w, causal, scale)


@pytest.mark.parametrize("Hq,Hkv,Sq,Sk,causal", [(2, 1, 5, 7, True), (2, 2, 6, 6, False), (3, 1, 7, 4, True),
                                                 (1, 1, 4, 9, True)])
def test_backward_matches_finite_differences(Hq, Hkv, Sq, Sk, causal):
    """Central differences of L = sum(W * O) in fp64 (no use of the gradient
    formulas): every element of Q, K and V, including rows with no visible key
    (Sq > Sk, bottom-right causal)."""
    rng = np.random.default_rng(Hq * 100 + Sq * 10 + Sk)
    d, scale, h = 3, 0.7, 1e-6
    q, k, v = _rand(1, Hq, Sq, d, rng=rng), _rand(1, Hkv, Sk, d, rng=rng), _rand(1, Hkv, Sk, d, rng=rng)
    w = _rand(1, Hq, Sq, d, rng=rng)
    _, grads = _loss_and_grads(q, k, v, w, causal, scale)
    for x, g in zip((q, k, v), grads):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            old = x[idx]
            x[idx] = old + h
            lp, _ = _loss_and_grads(q, k, v, w, causal, scale)
            x[idx] = old - h
            lm, _ = _loss_and_grads(q, k, v, w, causal, scale)
            x[idx] = old
            num[idx] = (lp - lm) / (2 * h)
        np.testing.assert_allclose(g, num, atol=1e-7, rtol=1e-6)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_torch_autograd(causal):
    """fp64 autograd of a forward written here with torch ops (a separate code
    path from the oracle's hand-derived gradient), with GQA by repeating K/V heads."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(77)
    B, Hq, Hkv, Sq, Sk, d, scale = 2, 4, 2, 9, 11, 5, 0.4
    q, k, v = _rand(B, Hq, Sq, d, rng=rng), _rand(B, Hkv, Sk, d, rng=rng), _rand(B, Hkv, Sk, d, rng=rng)
    w = _rand(B, Hq, Sq, d, rng=rng)
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    kk = tk.repeat_interleave(Hq // Hkv, dim=1)
    vv = tv.repeat_interleave(Hq // Hkv, dim=1)
    s = scale * torch.matmul(tq, kk.transpose(-1, -2))
    if causal:
        i = torch.arange(Sq)[:, None]
        j = torch.arange(Sk)[None, :]
        s = s.masked_fill(j > i + (Sk - Sq), float("-inf"))
    o = torch.matmul(torch.softmax(s, dim=-1), vv)
    (o * torch.tensor(w)).sum().backward()
    dq, dk, dv = oracle.sdpa_backward(q, k, v, w, causal, scale)
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-12)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_key_shift_and_value_sum(causal):
    """Adding a common vector to every key moves no probability, so the
    gradients of the keys sum to zero; the probabilities of a row sum to 1, so
    the value gradients sum to the sum of dO over the rows that see a key."""
    rng = np.random.default_rng(5)
    B, Hq, Hkv, Sq, Sk, d = 1, 4, 2, 8, 6, 4
    q, k, v = _rand(B, Hq, Sq, d, rng=rng), _rand(B, Hkv, Sk, d, rng=rng), _rand(B, Hkv, Sk, d, rng=rng)
    do = _rand(B, Hq, Sq, d, rng=rng)
    dq, dk, dv = oracle.sdpa_backward(q, k, v, do, causal, 0.6)
    np.testing.assert_allclose(dk.sum(axis=2), 0.0, atol=1e-12)
    rows = (np.arange(Sq) + (Sk - Sq) >= 0) if causal else np.ones(Sq, bool)
    g = Hq // Hkv
    want = do[:, :, rows].sum(axis=2).reshape(B, Hkv, g, d).sum(axis=2)
    np.testing.assert_allclose(dv.sum(axis=2), want, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_constant_values_give_no_score_gradient(causal):
    """With every value row equal, O does not depend on the scores at all, so
    dQ = dK = 0 exactly (up to rounding); dV still carries dO."""
    rng = np.random.default_rng(6)
    q, k = _rand(1, 2, 7, 4, rng=rng), _rand(1, 2, 7, 4, rng=rng)
    v = np.broadcast_to(_rand(1, 2, 1, 4, rng=rng), (1, 2, 7, 4)).copy()
    do = _rand(1, 2, 7, 4, rng=rng)
    dq, dk, dv = oracle.sdpa_backward(q, k, v, do, causal, 0.5)
    assert np.abs(dq).max() < 1e-12 and np.abs(dk).max() < 1e-12
    assert np.abs(dv).max() > 0.1


def _run_bwd_pins():
    failed = []
    checks = {
        "fd": lambda: test_backward_matches_finite_differences(2, 1, 5, 7, True),
        "shift": lambda: test_backward_key_shift_and_value_sum(True),
        "const_v": lambda: test_backward_constant_values_give_no_score_gradient(False),
    }
    for name, fn in checks.items():
        try:
            fn()
        except (AssertionError, ValueError, IndexError):
            failed.append(name)
    return failed


def test_backward_pins_pass_on_the_oracle():
    assert _run_bwd_pins() == []


_orig_attend_grad = oa._attend_grad


def _grad_no_delta(q, k, v, do, vis, scale):
    _, _, P = oa._attend(q, k, v, vis, scale)
    dS = P * (do @ v.T)
    return scale * (dS @ k), scale * (dS.T @ q), P.T @ do


def _grad_no_scale(q, k, v, do, vis, scale):
    dq, dk, dv = _orig_attend_grad(q, k, v, do, vis, scale)
    return dq / scale, dk / scale, dv


def _grad_dk_from_do(q, k, v, do, vis, scale):
    _, _, P = oa._attend(q, k, v, vis, scale)
    dP = do @ v.T
    dS = P * (dP - (P * dP).sum(axis=1)[:, None])
    return scale * (dS @ k), scale * (dS.T @ do), P.T @ do


def _grad_dv_from_q(q, k, v, do, vis, scale):
    dq, dk, _ = _orig_attend_grad(q, k, v, do, vis, scale)
    _, _, P = oa._attend(q, k, v, vis, scale)
    return dq, dk, P.T @ q


def _sdpa_backward_gqa_overwrite(q, k, v, do, causal, scale):
    q, k, v, do = (np.asarray(x, np.float64) for x in (q, k, v, do))
    B, Hq, Sq, d = q.shape
    Hkv, Sk = k.shape[1], k.shape[2]
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    vis = oa._visible(np.arange(Sq), Sq, Sk, causal)
    for b in range(B):
        for hq in range(Hq):
            kvh = oa.kv_head_of(hq, Hq, Hkv)
            dq[b, hq], dk[b, kvh], dv[b, kvh] = oa._attend_grad(q[b, hq], k[b, kvh], v[b, kvh], do[b, hq], vis, scale)
    return dq, dk, dv


@pytest.mark.parametrize("mutant,attr", [
    (_grad_no_delta, "_attend_grad"),
    (_grad_no_scale, "_attend_grad"),
    (_grad_dk_from_do, "_attend_grad"),
    (_grad_dv_from_q, "_attend_grad"),
    (_sdpa_backward_gqa_overwrite, "sdpa_backward"),
])
def test_backward_planted_mistakes_are_caught(monkeypatch, mutant, attr):
    monkeypatch.setattr(oa, attr, mutant)
    if attr == "sdpa_backward":
        monkeypatch.setattr(oracle, "sdpa_backward", mutant)
    assert _run_bwd_pins(), f"no backward pin caught the planted mistake in {attr}"
