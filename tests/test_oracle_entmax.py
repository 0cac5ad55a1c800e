"""Pins of the oracle's 1.5-entmax (tau by bisection, and the attention built
on it).

p_t = [z_t / 2 - tau]_+^2 with sum p = 1.  Pinned against the exact
sort-based solution (for support size k the quadratic
k tau^2 - 2 tau S1 + S2 - 1 = 0 over the k largest u = z / 2, support the
largest k with u_k > tau_k), the two-logit closed form, equal logits (uniform),
translation (tau shifts by c / 2), and attention over every page against a
dense entmax written here.
"""
import numpy as np

import oracle
from sparse_kv_cache_amd import workloads as W


def tau_by_sort(z):
    u = np.sort(np.asarray(z, dtype=np.float64) / 2.0)[::-1]
    best = None
    s1 = s2 = 0.0
    for k in range(1, len(u) + 1):
        s1 += u[k - 1]
        s2 += u[k - 1] ** 2
        disc = s1 * s1 - k * (s2 - 1.0)
        tau = (s1 - np.sqrt(max(disc, 0.0))) / k
        if u[k - 1] > tau:
            best = tau
    return best


def probs(z, tau):
    d = np.asarray(z, dtype=np.float64) / 2.0 - tau
    return np.where(d > 0, d * d, 0.0)


def test_tau_matches_the_sort_based_solution():
    rng = np.random.default_rng(0)
    for n in (1, 2, 3, 7, 64, 1000):
        for scale in (0.1, 1.0, 5.0, 40.0):
            z = rng.standard_normal(n) * scale
            t = oracle.entmax15_tau(z)
            assert abs(t - tau_by_sort(z)) <= 1e-12 * max(1.0, abs(t))
            p = probs(z, t)
            assert abs(p.sum() - 1.0) < 1e-12
            assert np.all(p >= 0)


def test_two_logits_closed_form():
    for u1, u2 in [(0.3, 0.1), (2.0, 1.5), (0.0, -0.9), (1.0, -0.2), (5.0, 1.0)]:
        z = np.array([2 * u1, 2 * u2])
        t = oracle.entmax15_tau(z)
        if u1 - u2 >= 1.0:
            want = u1 - 1.0
        else:
            m, dl = (u1 + u2) / 2, (u1 - u2) / 2
            want = m - np.sqrt(0.5 - dl * dl)
        assert abs(t - want) < 1e-12
    # a gap of at least 1 in u leaves one token with all the mass
    p = probs([4.0, 1.9], oracle.entmax15_tau([4.0, 1.9]))
    np.testing.assert_allclose(p, [1.0, 0.0], atol=1e-12)


def test_equal_logits_are_uniform_and_translation_shifts_tau():
    for n in (1, 4, 33):
        z = np.full(n, 0.7)
        t = oracle.entmax15_tau(z)
        assert abs(t - (0.35 - 1.0 / np.sqrt(n))) < 1e-12
        np.testing.assert_allclose(probs(z, t), np.full(n, 1.0 / n), atol=1e-12)
    z = np.random.default_rng(1).standard_normal(50) * 3
    assert abs(oracle.entmax15_tau(z + 4.2) - oracle.entmax15_tau(z) - 2.1) < 1e-12


def _dense(qrow, cache, h, bt_row, S, P, scale):
    pages = (S + P - 1) // P
    ks, vs = [], []
    for p in range(pages):
        n = min(P, S - p * P)
        blk = int(bt_row[p])
        ks.append(oracle.bf16_decode(cache[0, blk, :n, h]))
        vs.append(oracle.bf16_decode(cache[1, blk, :n, h]))
    K, V = np.concatenate(ks), np.concatenate(vs)
    z = scale * (K @ qrow)
    t = tau_by_sort(z)
    return probs(z, t) @ V, t


def test_attention_over_all_pages_is_dense_entmax():
    wl = W.small_case(seed=90, H_q=4, H_kv=2, min_len=5)
    cache = W.bf16_bits(W.make_cache(wl))
    q = W.make_queries(wl).double().numpy()
    for b in range(wl.B):
        S = int(wl.seq_lens[b])
        pages = np.arange(int(wl.pages()[b]), dtype=np.int32)
        for i in range(wl.H_q):
            for sc in (wl.softmax_scale, 1.0):      # a sparse and a sparser case
                o, t = oracle.attend_entmax15(q[b, i], cache, i // wl.G, wl.block_table[b],
                                              S, pages, sc)
                ro, rt = _dense(q[b, i], cache, i // wl.G, wl.block_table[b], S, wl.P, sc)
                np.testing.assert_allclose(o, ro, rtol=1e-11, atol=1e-11)
                assert abs(t - rt) < 1e-11


def test_single_token_returns_its_value_and_empty_is_zero():
    wl = W.small_case(seed=91, B=1, H_q=1, H_kv=1, min_len=40)
    cache = W.bf16_bits(W.make_cache(wl))
    q = W.make_queries(wl).double().numpy()
    S = int(wl.seq_lens[0])
    last = (S - 1) // wl.P
    # the tail page holds a single row when S % P == 1; emulate with S' = last*P + 1
    S1 = last * wl.P + 1
    o, t = oracle.attend_entmax15(q[0, 0], cache, 0, wl.block_table[0], S1,
                                  np.array([last], dtype=np.int32), wl.softmax_scale)
    v = oracle.bf16_decode(cache[1, int(wl.block_table[0, last]), 0, 0])
    np.testing.assert_allclose(o, v, atol=1e-12)
    o, t = oracle.attend_entmax15(q[0, 0], cache, 0, wl.block_table[0], S,
                                  np.array([], dtype=np.int32), wl.softmax_scale)
    assert np.all(o == 0) and t == -np.inf


def test_alibi_attention_over_all_pages_is_dense_entmax_with_the_bias():
    wl = W.small_case(seed=92, H_q=2, H_kv=1, min_len=5)
    cache = W.bf16_bits(W.make_cache(wl))
    q = W.make_queries(wl).double().numpy()
    for b in range(wl.B):
        S = int(wl.seq_lens[b])
        N = int(wl.pages()[b])
        pages = np.arange(N, dtype=np.int32)
        ks, vs = [], []
        for p in range(N):
            n = min(wl.P, S - p * wl.P)
            blk = int(wl.block_table[b, p])
            ks.append(oracle.bf16_decode(cache[0, blk, :n, 0]))
            vs.append(oracle.bf16_decode(cache[1, blk, :n, 0]))
        K, V = np.concatenate(ks), np.concatenate(vs)
        for slope in (0.0, 0.0625, 0.5):
            z = wl.softmax_scale * (K @ q[b, 0]) + slope * (np.arange(S) - (S - 1))
            rt = tau_by_sort(z)
            o, t = oracle.attend_entmax15(q[b, 0], cache, 0, wl.block_table[b], S, pages,
                                          wl.softmax_scale, slope=slope)
            np.testing.assert_allclose(o, probs(z, rt) @ V, rtol=1e-11, atol=1e-11)
            assert abs(t - rt) < 1e-11
