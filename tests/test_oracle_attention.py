"""Pins of the oracle's attention over selected pages and its LSE merge.

Attention: with every page selected it equals dense softmax attention written
independently over all tokens in logical order (numpy, no paging); a single
token gives o = v and lse = its logit; two identical keys give the mean of
their values.  Merge: any partition of the token set, attended part by part
and merged, equals single-shot attention; the +inf / -inf rules of the
MergeAttnStates test on the vllm.cpp page.
"""
import numpy as np

import oracle
from sparse_kv_cache_amd import workloads as W


def _dense(q, keys, vals, scale):
    l = scale * keys @ q
    w = np.exp(l - l.max())
    return (w[:, None] * vals).sum(0) / w.sum(), l.max() + np.log(w.sum())


def _logical_tokens(wl, cache, b, h):
    S = int(wl.seq_lens[b])
    ks, vs = [], []
    for t in range(S):
        blk = int(wl.block_table[b, t // wl.P])
        ks.append(oracle.bf16_decode(cache[0, blk, t % wl.P, h]))
        vs.append(oracle.bf16_decode(cache[1, blk, t % wl.P, h]))
    return np.array(ks), np.array(vs)


def test_all_pages_equals_dense_attention():
    for seed in range(3):
        wl = W.small_case(seed=40 + seed, min_len=1)
        cache = W.bf16_bits(W.make_cache(wl))
        q = W.make_queries(wl).double().numpy()
        for b in range(wl.B):
            N = int(wl.pages()[b])
            for i in range(wl.H_q):
                h = i // wl.G
                o, lse = oracle.attend(q[b, i], cache, h, wl.block_table[b],
                                       wl.seq_lens[b], np.arange(N), 0.125)
                k, v = _logical_tokens(wl, cache, b, h)
                o2, lse2 = _dense(q[b, i], k, v, 0.125)
                np.testing.assert_allclose(o, o2, rtol=1e-12, atol=1e-13)
                np.testing.assert_allclose(lse, lse2, rtol=1e-13, atol=1e-13)


def test_single_token_and_identical_keys():
    wl = W.small_case(seed=50, B=1, H_q=1, H_kv=1, D=8, P=16, max_pages=2)
    wl.seq_lens[:] = 17                      # page 1 holds one token
    rng = np.random.default_rng(0)
    cache = np.zeros((2, wl.num_blocks, 16, 1, 8), dtype=np.uint16)
    b1 = int(wl.block_table[0, 1])
    k = oracle.double_to_bf16(rng.standard_normal(8))
    v = oracle.double_to_bf16(rng.standard_normal(8))
    cache[0, b1, 0, 0], cache[1, b1, 0, 0] = k, v
    q = rng.standard_normal(8)
    o, lse = oracle.attend(q, cache, 0, wl.block_table[0], 17, [1], 0.5)
    np.testing.assert_array_equal(o, oracle.bf16_decode(v))
    np.testing.assert_allclose(lse, 0.5 * q @ oracle.bf16_decode(k), rtol=1e-15)
    # two identical keys in page 0 rows 0 and 1 with different values
    b0 = int(wl.block_table[0, 0])
    cache2 = np.zeros_like(cache)
    cache2[0, b0, :2, 0] = k
    v2 = oracle.double_to_bf16(rng.standard_normal((2, 8)))
    cache2[1, b0, :2, 0] = v2
    o, lse = oracle.attend(q, cache2, 0, wl.block_table[0], 2, [0], 0.5)
    np.testing.assert_allclose(o, oracle.bf16_decode(v2).mean(0), rtol=1e-14)
    np.testing.assert_allclose(lse, 0.5 * q @ oracle.bf16_decode(k) + np.log(2),
                               rtol=1e-14)


def test_empty_selection_is_minus_inf():
    wl = W.small_case(seed=51)
    cache = W.bf16_bits(W.make_cache(wl))
    o, lse = oracle.attend(np.ones(wl.D), cache, 0, wl.block_table[0],
                           wl.seq_lens[0], [], 0.1)
    assert lse == -np.inf and np.all(o == 0)


def test_chunked_merge_equals_single_shot():
    rng = np.random.default_rng(3)
    for seed in range(4):
        wl = W.small_case(seed=60 + seed, min_len=40)
        cache = W.bf16_bits(W.make_cache(wl))
        q = W.make_queries(wl).double().numpy()
        for b in range(wl.B):
            N = int(wl.pages()[b])
            pages = np.sort(rng.choice(N, size=max(1, N // 2), replace=False))
            for i in range(wl.H_q):
                full, lfull = oracle.attend(q[b, i], cache, i // wl.G,
                                            wl.block_table[b], wl.seq_lens[b],
                                            pages, 0.2)
                # random partition into contiguous groups, some empty
                cuts = np.sort(rng.integers(0, len(pages) + 1, size=3))
                groups = np.split(pages, cuts)
                parts = [oracle.attend(q[b, i], cache, i // wl.G,
                                       wl.block_table[b], wl.seq_lens[b], g, 0.2)
                         for g in groups]
                o, l = oracle.lse_merge(np.array([p[0] for p in parts]),
                                        np.array([p[1] for p in parts]))
                np.testing.assert_allclose(o, full, rtol=1e-12, atol=1e-12)
                np.testing.assert_allclose(l, lfull, rtol=1e-12, atol=1e-12)


def test_merge_edge_cases():
    rng = np.random.default_rng(4)
    a, c = rng.standard_normal(5), rng.standard_normal(5)
    # prefix has no keys: the other partial passes through
    o, l = oracle.lse_merge(np.array([a, c]), np.array([-np.inf, 0.7]))
    np.testing.assert_allclose(o, c, rtol=1e-15)
    assert l == 0.7
    # both -inf: emit the first partial, lse -inf
    o, l = oracle.lse_merge(np.array([a, c]), np.array([-np.inf, -np.inf]))
    np.testing.assert_array_equal(o, a)
    assert l == -np.inf
    # +inf is read as -inf
    o, l = oracle.lse_merge(np.array([a, c]), np.array([np.inf, 0.25]))
    np.testing.assert_allclose(o, c, rtol=1e-15)
    assert l == 0.25
    o, l = oracle.lse_merge(np.array([a, c]), np.array([np.inf, -np.inf]))
    np.testing.assert_array_equal(o, a)
    assert l == -np.inf
    # two equal lse values average the partials and add ln 2
    o, l = oracle.lse_merge(np.array([a, c]), np.array([1.5, 1.5]))
    np.testing.assert_allclose(o, (a + c) / 2, rtol=1e-14)
    np.testing.assert_allclose(l, 1.5 + np.log(2), rtol=1e-15)
