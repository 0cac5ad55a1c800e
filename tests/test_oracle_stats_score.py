"""Pins of the oracle's page statistics and page score.

Statistics: brute force over explicitly gathered rows, the ordering
invariant min <= mean <= max, a constant page, and invariance under a change
of block table.  Score: the Quest bound is at least the true max of q.k on
every page, the mean term equals the page mean of q.k, q >= 0 reduces the
bound to q.kmax, a constant page makes both terms the single q.k, and the
bound built from kmax alone fails when q has a negative coordinate.
"""
import numpy as np
import torch

import oracle
from sparse_kv_cache_amd import workloads as W


def _case(seed, **kw):
    wl = W.small_case(seed=seed, **kw)
    cache = W.bf16_bits(W.make_cache(wl))
    q = W.make_queries(wl).double().numpy()
    return wl, cache, q


def _page_rows(wl, cache, b, p, kv=0):
    """[n, H_kv, D] float64 rows of logical page p of request b."""
    S = int(wl.seq_lens[b])
    n = min(wl.P, S - p * wl.P)
    blk = int(wl.block_table[b, p])
    return oracle.bf16_decode(cache[kv, blk, :n])


def test_stats_brute_force_and_order():
    for seed in range(4):
        wl, cache, _ = _case(seed, min_len=1)
        mn, mx, me = oracle.page_stats(cache, wl.block_table, wl.seq_lens, wl.P)
        for b in range(wl.B):
            for p in range(int(wl.pages()[b])):
                rows = _page_rows(wl, cache, b, p)
                blk = int(wl.block_table[b, p])
                assert np.array_equal(mn[blk], rows.min(0))
                assert np.array_equal(mx[blk], rows.max(0))
                np.testing.assert_allclose(me[blk], rows.sum(0) / rows.shape[0],
                                           rtol=1e-14, atol=1e-15)
                assert np.all(mn[blk] <= me[blk] + 1e-15)
                assert np.all(me[blk] <= mx[blk] + 1e-15)


def test_stats_constant_page_and_partial_tail():
    wl = W.small_case(seed=7, B=1, H_q=2, H_kv=1, D=8, P=16, max_pages=3)
    wl.seq_lens[:] = 16 + 5          # a full page and a 5-row tail
    cache = np.zeros((2, wl.num_blocks, 16, 1, 8), dtype=np.uint16)
    row = oracle.double_to_bf16(np.linspace(-2, 3, 8))
    b0, b1 = int(wl.block_table[0, 0]), int(wl.block_table[0, 1])
    cache[0, b0, :, 0] = row
    cache[0, b1, :5, 0] = row
    cache[0, b1, 5:, 0] = oracle.double_to_bf16(np.full(8, 99.0))  # stale rows
    mn, mx, me = oracle.page_stats(cache, wl.block_table, wl.seq_lens, 16)
    r = oracle.bf16_decode(row)
    for blk in (b0, b1):
        assert np.array_equal(mn[blk, 0], r)
        assert np.array_equal(mx[blk, 0], r)
        np.testing.assert_allclose(me[blk, 0], r, rtol=1e-15)


def test_stats_invariant_under_block_table():
    wl, cache, _ = _case(11, min_len=30)
    mn, mx, me = oracle.page_stats(cache, wl.block_table, wl.seq_lens, wl.P)
    # move every page to a different physical block (reverse order)
    perm = np.arange(wl.num_blocks)[::-1].copy()
    cache2 = np.empty_like(cache)
    cache2[:, perm] = cache
    bt2 = perm[wl.block_table].astype(np.int32)
    mn2, mx2, me2 = oracle.page_stats(cache2, bt2, wl.seq_lens, wl.P)
    for b in range(wl.B):
        for p in range(int(wl.pages()[b])):
            x, y = int(wl.block_table[b, p]), int(bt2[b, p])
            assert np.array_equal(mn[x], mn2[y])
            assert np.array_equal(mx[x], mx2[y])
            assert np.array_equal(me[x], me2[y])


def _scores(wl, cache, q, w_avg, w_peak):
    st = oracle.page_stats(cache, wl.block_table, wl.seq_lens, wl.P)
    return oracle.page_score(q, *st, wl.block_table, wl.seq_lens, wl.P,
                             w_avg, w_peak)


def test_peak_bound_dominates_true_max_and_mean_identity():
    for seed in range(3):
        wl, cache, q = _case(20 + seed, min_len=20)
        peak = _scores(wl, cache, q, 0.0, 1.0)
        avg = _scores(wl, cache, q, 1.0, 0.0)
        G = wl.G
        for b in range(wl.B):
            for i in range(wl.H_q):
                for p in range(int(wl.pages()[b])):
                    rows = _page_rows(wl, cache, b, p)[:, i // G, :]
                    dots = rows @ q[b, i]
                    u = peak[b, i, p]
                    assert u >= dots.max() - 1e-12 * max(1.0, abs(u))
                    np.testing.assert_allclose(avg[b, i, p], dots.mean(),
                                               rtol=1e-12, atol=1e-12)


def test_combined_score_is_weighted_sum():
    wl, cache, q = _case(30)
    a = _scores(wl, cache, q, 1.0, 0.0)
    u = _scores(wl, cache, q, 0.0, 1.0)
    s = _scores(wl, cache, q, 0.75, -1.5)
    m = ~np.isnan(s)
    np.testing.assert_allclose(s[m], 0.75 * a[m] - 1.5 * u[m], rtol=1e-12, atol=1e-12)


def test_nonnegative_query_reduces_to_kmax():
    wl, cache, q = _case(31)
    q = np.abs(q)
    u = _scores(wl, cache, q, 0.0, 1.0)
    mn, mx, me = oracle.page_stats(cache, wl.block_table, wl.seq_lens, wl.P)
    for b in range(wl.B):
        for i in range(wl.H_q):
            for p in range(int(wl.pages()[b])):
                blk = int(wl.block_table[b, p])
                np.testing.assert_allclose(u[b, i, p], q[b, i] @ mx[blk, i // wl.G],
                                           rtol=1e-12)


def test_constant_page_makes_both_terms_equal():
    wl = W.small_case(seed=32, B=1, H_q=2, H_kv=1, D=16, P=16, max_pages=2)
    wl.seq_lens[:] = 32
    rng = np.random.default_rng(0)
    cache = np.zeros((2, wl.num_blocks, 16, 1, 16), dtype=np.uint16)
    for p in range(2):
        row = oracle.double_to_bf16(rng.standard_normal(16))
        cache[0, int(wl.block_table[0, p]), :, 0] = row
    q = rng.standard_normal((1, 2, 16))
    a = _scores(wl, cache, q, 1.0, 0.0)
    u = _scores(wl, cache, q, 0.0, 1.0)
    for p in range(2):
        k = oracle.bf16_decode(cache[0, int(wl.block_table[0, p]), 0, 0])
        for i in range(2):
            np.testing.assert_allclose(a[0, i, p], q[0, i] @ k, rtol=1e-12)
            np.testing.assert_allclose(u[0, i, p], q[0, i] @ k, rtol=1e-12)


def test_kmax_only_bound_fails_for_signed_query():
    # Why both envelopes are needed: with a negative coordinate, q.kmax can
    # fall below the true max of q.k, while the two-envelope bound cannot.
    rows = np.array([[1.0, -3.0], [2.0, 1.0]])
    q = np.array([1.0, -1.0])
    true_max = (rows @ q).max()                       # 4.0
    kmax_only = q @ rows.max(0)                       # 2 - 1 = 1
    assert kmax_only < true_max
    wl = W.small_case(seed=33, B=1, H_q=1, H_kv=1, D=2, P=16, max_pages=1)
    wl.seq_lens[:] = 2
    cache = np.zeros((2, wl.num_blocks, 16, 1, 2), dtype=np.uint16)
    cache[0, int(wl.block_table[0, 0]), :2, 0] = oracle.double_to_bf16(rows)
    u = _scores(wl, cache, q[None, None, :], 0.0, 1.0)[0, 0, 0]
    assert u >= true_max
    assert u == 1.0 * 2.0 + (-1.0) * (-3.0)           # max(q.max, q.min) per dim


def test_scores_independent_of_physical_placement():
    wl, cache, q = _case(34)
    s1 = _scores(wl, cache, q, 1.0, 0.5)
    perm = np.random.default_rng(5).permutation(wl.num_blocks)
    cache2 = np.empty_like(cache)
    cache2[:, perm] = cache
    wl2 = W.small_case(seed=34)
    wl2.block_table = perm[wl.block_table].astype(np.int32)
    s2 = _scores(wl2, cache2, q, 1.0, 0.5)
    assert np.array_equal(np.isnan(s1), np.isnan(s2))
    m = ~np.isnan(s1)
    assert np.array_equal(s1[m], s2[m])
    assert torch.__version__  # torch present for the generators


# ----------------------------------------------------- group-shared scores

def _gscores(wl, cache, q, w_avg, w_peak):
    st = oracle.page_stats(cache, wl.block_table, wl.seq_lens, wl.P)
    return oracle.page_score_group(q, *st, wl.block_table, wl.seq_lens, wl.P,
                                   w_avg, w_peak)


def test_group_mean_term_is_page_mean_of_the_group_mean_query():
    # The mean term is linear in q: the group's mean score equals the page
    # mean of q_bar . k with q_bar the group's mean query, from raw rows.
    for seed in range(3):
        wl, cache, q = _case(40 + seed, H_q=8, H_kv=2, min_len=20)
        avg = _gscores(wl, cache, q, 1.0, 0.0)
        G = wl.G
        for b in range(wl.B):
            for h in range(wl.H_kv):
                qbar = q[b, h * G:(h + 1) * G].mean(0)
                for p in range(int(wl.pages()[b])):
                    rows = _page_rows(wl, cache, b, p)[:, h, :]
                    np.testing.assert_allclose(avg[b, h, p], (rows @ qbar).mean(),
                                               rtol=1e-12, atol=1e-12)


def test_group_peak_bounds_every_head_average_logit():
    # mean over g of max_t q_g.k_t >= max_t of the mean logit: the group peak
    # term bounds the best mean logit of the page (brute force over rows).
    for seed in range(3):
        wl, cache, q = _case(50 + seed, H_q=6, H_kv=2, min_len=20)
        u = _gscores(wl, cache, q, 0.0, 1.0)
        G = wl.G
        for b in range(wl.B):
            for h in range(wl.H_kv):
                for p in range(int(wl.pages()[b])):
                    rows = _page_rows(wl, cache, b, p)[:, h, :]
                    per_head_max = (rows @ q[b, h * G:(h + 1) * G].T).max(0)
                    assert u[b, h, p] >= per_head_max.mean() - 1e-12 * max(1.0, abs(u[b, h, p]))


def test_group_of_one_is_the_per_head_score():
    wl, cache, q = _case(60, H_q=3, H_kv=3)
    a = _gscores(wl, cache, q, 0.8, -0.3)
    b = _scores(wl, cache, q, 0.8, -0.3)
    m = ~np.isnan(b)
    assert np.array_equal(np.isnan(a), np.isnan(b))
    np.testing.assert_allclose(a[m], b[m], rtol=1e-13, atol=1e-13)


def test_group_score_ignores_head_order_within_a_group():
    wl, cache, q = _case(61, H_q=8, H_kv=2)
    a = _gscores(wl, cache, q, 1.0, 0.5)
    q2 = q.copy()
    rng = np.random.default_rng(1)
    for h in range(2):
        q2[:, h * 4:(h + 1) * 4] = q[:, h * 4 + rng.permutation(4)]
    b = _gscores(wl, cache, q2, 1.0, 0.5)
    m = ~np.isnan(a)
    np.testing.assert_allclose(a[m], b[m], rtol=1e-13, atol=1e-13)
    # and heads of the other group do not leak in
    q3 = q.copy()
    q3[:, 4:] = rng.standard_normal(q3[:, 4:].shape)
    c = _gscores(wl, cache, q3, 1.0, 0.5)
    np.testing.assert_allclose(a[:, 0][m[:, 0]], c[:, 0][m[:, 0]], rtol=1e-13, atol=1e-13)
