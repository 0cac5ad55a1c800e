"""Pins of the oracle's ALiBi-aware page score and ALiBi attention.

The bias of a key at logical position t is slope * (t - (S - 1)).  Pinned
against brute force over raw rows: the mean term is the page mean of the
biased q.k (in q.k units, slope / scale), the peak term bounds the page's best
biased q.k and is tight on a constant page; a zero slope gives back the plain
score and attention; attention over every page equals a dense softmax written
here in numpy; a steep slope concentrates attention on the newest token.
"""
import numpy as np

import oracle
from sparse_kv_cache_amd import workloads as W


def _case(seed, **kw):
    wl = W.small_case(seed=seed, **kw)
    cache = W.bf16_bits(W.make_cache(wl))
    q = W.make_queries(wl).double().numpy()
    return wl, cache, q


def _rows(wl, cache, b, p, kv=0):
    S = int(wl.seq_lens[b])
    n = min(wl.P, S - p * wl.P)
    return oracle.bf16_decode(cache[kv, int(wl.block_table[b, p]), :n])


def _alibi_scores(wl, cache, q, w_avg, w_peak, alibi, aggregate=False):
    st = oracle.page_stats(cache, wl.block_table, wl.seq_lens, wl.P)
    return oracle.page_score_alibi(q, *st, wl.block_table, wl.seq_lens, wl.P, w_avg,
                                   w_peak, alibi, aggregate)


def test_zero_slope_is_the_plain_score():
    wl, cache, q = _case(70, H_q=8, H_kv=2)
    st = oracle.page_stats(cache, wl.block_table, wl.seq_lens, wl.P)
    z = np.zeros(wl.H_q)
    a = oracle.page_score_alibi(q, *st, wl.block_table, wl.seq_lens, wl.P, 0.7, 0.4, z)
    b = oracle.page_score(q, *st, wl.block_table, wl.seq_lens, wl.P, 0.7, 0.4)
    m = ~np.isnan(b)
    np.testing.assert_array_equal(np.isnan(a), np.isnan(b))
    np.testing.assert_allclose(a[m], b[m], rtol=1e-14, atol=1e-14)
    a = oracle.page_score_alibi(q, *st, wl.block_table, wl.seq_lens, wl.P, 0.7, 0.4, z, True)
    b = oracle.page_score_group(q, *st, wl.block_table, wl.seq_lens, wl.P, 0.7, 0.4)
    np.testing.assert_allclose(a[~np.isnan(b)], b[~np.isnan(b)], rtol=1e-14, atol=1e-14)


def test_mean_term_and_peak_bound_with_bias_by_brute_force():
    for seed in range(3):
        wl, cache, q = _case(71 + seed, H_q=4, H_kv=2, min_len=20, P=4 + 12 * (seed % 2))
        alibi = np.array([0.0, 0.05, 0.5, 2.0])
        avg = _alibi_scores(wl, cache, q, 1.0, 0.0, alibi)
        peak = _alibi_scores(wl, cache, q, 0.0, 1.0, alibi)
        for b in range(wl.B):
            S = int(wl.seq_lens[b])
            for i in range(wl.H_q):
                for p in range(int(wl.pages()[b])):
                    rows = _rows(wl, cache, b, p)[:, i // wl.G, :]
                    pos = p * wl.P + np.arange(rows.shape[0])
                    biased = rows @ q[b, i] + alibi[i] * (pos - (S - 1))
                    np.testing.assert_allclose(avg[b, i, p], biased.mean(),
                                               rtol=1e-12, atol=1e-12)
                    u = peak[b, i, p]
                    assert u >= biased.max() - 1e-12 * max(1.0, abs(u))


def test_peak_bound_is_tight_on_a_constant_page():
    wl = W.small_case(seed=74, B=1, H_q=1, H_kv=1, D=8, P=16, max_pages=3)
    wl.seq_lens[:] = 40
    rng = np.random.default_rng(0)
    cache = np.zeros((2, wl.num_blocks, 16, 1, 8), dtype=np.uint16)
    for p in range(3):
        cache[0, int(wl.block_table[0, p]), :, 0] = oracle.double_to_bf16(rng.standard_normal(8))
    q = rng.standard_normal((1, 1, 8))
    a = np.array([0.3])
    u = _alibi_scores(wl, cache, q, 0.0, 1.0, a)
    for p in range(3):
        k = oracle.bf16_decode(cache[0, int(wl.block_table[0, p]), 0, 0])
        n = min(16, 40 - 16 * p)
        best = q[0, 0] @ k + 0.3 * (16 * p + n - 1 - 39)
        np.testing.assert_allclose(u[0, 0, p], best, rtol=1e-13, atol=1e-13)


def test_group_aggregate_is_the_group_mean():
    wl, cache, q = _case(75, H_q=6, H_kv=2)
    alibi = np.linspace(0.01, 0.6, 6)
    per = _alibi_scores(wl, cache, q, 1.0, 0.5, alibi)
    agg = _alibi_scores(wl, cache, q, 1.0, 0.5, alibi, aggregate=True)
    want = per.reshape(wl.B, 2, 3, -1).mean(axis=2)
    m = ~np.isnan(want)
    np.testing.assert_allclose(agg[m], want[m], rtol=1e-13, atol=1e-13)


def _dense_alibi(qrow, cache, h, bt_row, S, P, scale, slope):
    """Softmax over every token of the request, written directly."""
    pages = (S + P - 1) // P
    ks, vs, pos = [], [], []
    for p in range(pages):
        n = min(P, S - p * P)
        blk = int(bt_row[p])
        ks.append(oracle.bf16_decode(cache[0, blk, :n, h]))
        vs.append(oracle.bf16_decode(cache[1, blk, :n, h]))
        pos.append(p * P + np.arange(n))
    K, V, t = np.concatenate(ks), np.concatenate(vs), np.concatenate(pos)
    z = scale * (K @ qrow) + slope * (t - (S - 1))
    w = np.exp(z - z.max())
    return (w[:, None] * V).sum(0) / w.sum(), z.max() + np.log(w.sum())


def test_attention_over_all_pages_is_dense_alibi_softmax():
    wl, cache, q = _case(76, H_q=4, H_kv=2, min_len=5)
    for b in range(wl.B):
        S = int(wl.seq_lens[b])
        pages = np.arange(int(wl.pages()[b]), dtype=np.int32)
        for i, slope in enumerate([0.0, 0.02, 0.3, 1.5]):
            o, lse = oracle.attend_alibi(q[b, i], cache, i // wl.G, wl.block_table[b], S,
                                         pages, wl.softmax_scale, slope)
            ro, rl = _dense_alibi(q[b, i], cache, i // wl.G, wl.block_table[b], S, wl.P,
                                  wl.softmax_scale, slope)
            np.testing.assert_allclose(o, ro, rtol=1e-12, atol=1e-12)
            assert abs(lse - rl) < 1e-12
            if slope == 0.0:
                o0, l0 = oracle.attend(q[b, i], cache, i // wl.G, wl.block_table[b], S,
                                       pages, wl.softmax_scale)
                np.testing.assert_allclose(o, o0, rtol=1e-13, atol=1e-13)


def test_steep_slope_attends_to_the_newest_token():
    wl, cache, q = _case(77, B=1, H_q=2, H_kv=1, min_len=30)
    S = int(wl.seq_lens[0])
    pages = np.arange(int(wl.pages()[0]), dtype=np.int32)
    o, _ = oracle.attend_alibi(q[0, 0], cache, 0, wl.block_table[0], S, pages,
                               wl.softmax_scale, 200.0)
    last = (S - 1) // wl.P
    v = oracle.bf16_decode(cache[1, int(wl.block_table[0, last]), (S - 1) % wl.P, 0])
    np.testing.assert_allclose(o, v, rtol=0, atol=1e-12)
