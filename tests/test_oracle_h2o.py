"""Pins of the oracle's append / reset and the token-level H2O accumulator.

* The accumulator reproduces the digits the vortex_torch pull request prints
  for its execute-mode recurrence (128 tokens x 800 steps, inputs regenerated
  from the seeds the page's script uses): rel.err, top-32 overlap, max, and the
  response to a changed final step, for decay 0.984375 and 1.0.
* Closed forms: each step adds exactly one unit of probability mass, so the
  exact mass after n steps is (1 - d^n) / (1 - d); with bf16 storage the
  oracle stays within the page's 10 % bound.  decay = 1 is the plain running
  sum.  A constant input settles at a bf16 fixed point of the recurrence.
* The flow-level harness of the page's hardware follow-up (seq 128, group 4,
  bos 4, eos 8, 600 steps, keys with a per-token affinity along a direction
  the queries lean towards), re-run on CPU-drawn inputs against its
  thresholds and an unrounded float64 recurrence written here.
* Append writes exactly the new bytes and zeroes the written hh slots only.
* The per-head reading of the GQA token flow (each query head's softmax,
  averaged over the group): a three-token closed form where it differs from
  the group-mean query, exact rational weights on tiny inputs, G = 1 and
  identical group queries reduce it to the group-mean step, one unit of mass
  per step inside the window only, head order within a group is irrelevant and
  a group reaches only its own kv head.
"""
import json
import os

import numpy as np
import torch

import oracle
from sparse_kv_cache_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _page_probs():
    """The execute-mode input recipe printed on the page (CPU generators)."""
    torch.manual_seed(0)
    affinity = torch.randn(128) * 1.5
    g = torch.Generator().manual_seed(1)
    rows = [torch.softmax(affinity + torch.randn(128, generator=g) * 0.5, 0)
            for _ in range(800)]
    return torch.stack(rows).double().numpy()   # exact widening of float32


def _run(probs, decay):
    hh = np.zeros(probs.shape[1], dtype=np.uint16)
    for row in probs:
        oracle.h2o_recurrence(row, hh, decay)
    return oracle.bf16_decode(hh)


def _exact(probs, decay):
    d = oracle.bf16_decode(oracle.double_to_bf16(decay))
    acc = np.zeros(probs.shape[1])
    for row in probs:
        acc = row + d * acc
    return acc


def _topk_set(x, k):
    # torch.topk on the values, as the page's script does
    return set(torch.from_numpy(np.asarray(x)).topk(k).indices.tolist())


def test_recurrence_reproduces_printed_digits():
    gold = json.load(open(os.path.join(GOLDEN, "h2o_recurrence_printed.json")))
    probs = _page_probs()
    for key, want in gold["printed"].items():
        decay = float(key)
        got = _run(probs, decay)
        ref = _exact(probs, decay)
        rel = np.abs(got - ref).max() / np.abs(ref).max()
        assert f"{rel:.2e}" == want["rel_err"]
        ov = len(_topk_set(got, 32) & _topk_set(ref, 32)) / 32
        assert f"{ov:.0%}" == want["topk_overlap"]
        if "max" in want:
            assert f"{got.max():.1f}" == want["max"]
        changed = probs.copy()
        changed[-1] = probs[-1] * 0 + np.float32(1.0) / np.float32(128)
        moved = np.abs(_run(changed, decay) - got).max()
        assert f"{moved:.3e}" == want["changed_step_delta"]
    th = gold["thresholds"]
    got = _run(probs, 0.984375)
    ref = _exact(probs, 0.984375)
    assert np.abs(got - ref).max() / np.abs(ref).max() < th["rel_err_below"]
    assert got.max() < th["max_below"]


def test_mass_closed_form_and_plain_sum():
    rng = np.random.default_rng(0)
    n_tok, d = 200, 0.984375
    hh = np.zeros(n_tok, dtype=np.uint16)
    for n in range(1, 257):
        p = rng.dirichlet(np.full(n_tok, 0.3))
        oracle.h2o_recurrence(p, hh, d)
        if n in (1, 64, 256):
            exact = (1 - d ** n) / (1 - d)
            mass = oracle.bf16_decode(hh).sum()
            assert abs(mass / exact - 1) <= 0.10, (n, mass, exact)
    # decay = 1: the plain running sum, rounded to bf16 after every add; with
    # power-of-two increments the sum is exact
    hh = np.zeros(4, dtype=np.uint16)
    for _ in range(16):
        oracle.h2o_recurrence(np.full(4, 2.0 ** -4), hh, 1.0)
    np.testing.assert_array_equal(oracle.bf16_decode(hh), np.ones(4))
    # and matches a library bf16 round of float32 sums for general inputs
    hh = np.zeros(64, dtype=np.uint16)
    lib = torch.zeros(64, dtype=torch.bfloat16)
    for _ in range(50):
        p = rng.random(64) * 0.1
        pb = torch.from_numpy(p).float().to(torch.bfloat16)
        lib = (pb.float() + lib.float()).to(torch.bfloat16)
        oracle.h2o_recurrence(p, hh, 1.0)
    np.testing.assert_array_equal(oracle.bf16_decode(hh), lib.double().numpy())


def test_constant_input_settles_at_a_fixed_point():
    d = 0.984375
    for p in (2.0 ** -7, 0.013, 0.2):
        hh = np.zeros(1, dtype=np.uint16)
        for _ in range(3000):
            oracle.h2o_recurrence(np.array([p]), hh, d)
        v = oracle.bf16_decode(hh)[0]
        before = hh.copy()
        oracle.h2o_recurrence(np.array([p]), hh, d)
        assert hh[0] == before[0]                     # a fixed point
        pb = oracle.bf16_decode(oracle.double_to_bf16(p))
        ulp = 2.0 ** (np.floor(np.log2(v)) - 7)
        # the rounding can only hold v where the pull towards p/(1-d) is
        # under half an ulp
        assert abs(pb - (1 - d) * v) <= ulp / 2 + 1e-18
        assert v <= pb / (1 - d) + ulp


def test_flow_harness_thresholds_on_cpu_inputs():
    gold = json.load(open(os.path.join(GOLDEN, "h2o_flow_thresholds.json")))
    S, steps, G, D = gold["seq_len"], gold["steps"], gold["group_size"], gold["head_dim"]
    bos, eos, topk = gold["bos"], gold["eos"], gold["topk"]
    g = torch.Generator().manual_seed(0)
    u = torch.randn(D, generator=g, dtype=torch.float64)
    u = u / u.norm()
    affinity = torch.randn(S, generator=g, dtype=torch.float64) * 2.0
    k = (torch.randn(S, D, generator=g, dtype=torch.float64)
         + affinity[:, None] * u[None, :]).float().to(torch.bfloat16)
    cache = np.zeros((2, S, 1, 1, D), dtype=np.uint16)
    cache[0, :, 0, 0] = W.bf16_bits(k)
    bt = np.arange(S, dtype=np.int32)[None, :]
    sl = np.array([S], dtype=np.int32)
    hh = np.zeros((S, 1), dtype=np.uint16)
    decay, scale = 0.984375, D ** -0.5
    kd = k.double().numpy()
    ref = np.zeros(S)
    for step in range(steps):
        q = (torch.randn(1, G, D, generator=g, dtype=torch.float64) * 0.3
             + u[None, None, :]).float().to(torch.bfloat16).double().numpy()
        sc = oracle.h2o_step(q, cache, bt, sl, hh, bos, eos, scale, decay)
        # unrounded float64 recurrence over the window [bos, S - eos)
        l = scale * kd @ q[0].mean(0)
        p = np.zeros(S)
        w = np.exp(l[bos:S - eos] - l[bos:S - eos].max())
        p[bos:S - eos] = w / w.sum()
        ref = p + decay * ref
    got = oracle.bf16_decode(hh[:, 0])
    np.testing.assert_array_equal(sc[0, 0], got)
    rel = np.abs(got - ref).max() / np.abs(ref).max()
    assert rel < gold["final_rel_err_below"]
    predicted = (1 - decay ** steps) / (1 - decay)
    assert 1 - got.sum() / predicted <= gold["mass_loss_at_most"]
    # entries outside the window are never touched
    assert np.all(got[:bos] == 0) and np.all(got[S - eos:] == 0)
    # overlap must be complete whenever the boundary is wider than one ulp
    srt = np.sort(ref[ref > 0])[::-1]
    gap = srt[topk - 1] - srt[topk]
    ulp = srt[topk - 1] * 2.0 ** -8
    ov = len(_topk_set(got, topk) & _topk_set(ref, topk)) / topk
    assert gap <= ulp or ov == 1.0


def test_append_writes_bytes_and_resets_only_written_slots():
    wl = W.small_case(seed=70, B=3, H_q=4, H_kv=2, D=16, P=1, max_pages=40,
                      min_len=2)
    cache = W.bf16_bits(W.make_cache(wl)).copy()
    before = cache.copy()
    kn, vn = (W.bf16_bits(t) for t in W.make_new_kv(wl))
    hh = np.full((wl.num_blocks, wl.H_kv), 0x40F0, dtype=np.uint16)   # 7.5
    oracle.append(cache, wl.block_table, wl.seq_lens, kn, vn, hh)
    touched = set()
    for b in range(wl.B):
        pos = int(wl.seq_lens[b]) - 1
        blk = int(wl.block_table[b, pos])
        np.testing.assert_array_equal(cache[0, blk, 0], kn[b])
        np.testing.assert_array_equal(cache[1, blk, 0], vn[b])
        assert np.all(hh[blk] == 0)
        touched.add(blk)
    rest = np.array(sorted(set(range(wl.num_blocks)) - touched))
    assert np.all(hh[rest] == 0x40F0)
    np.testing.assert_array_equal(cache[:, rest], before[:, rest])
    # paged append (P = 16): row (S-1) % 16 of the tail block
    wl = W.small_case(seed=71, B=2, H_q=2, H_kv=1, D=8, P=16, max_pages=4)
    cache = W.bf16_bits(W.make_cache(wl)).copy()
    before = cache.copy()
    kn, vn = (W.bf16_bits(t) for t in W.make_new_kv(wl))
    oracle.append(cache, wl.block_table, wl.seq_lens, kn, vn, None)
    for b in range(wl.B):
        pos = int(wl.seq_lens[b]) - 1
        blk = int(wl.block_table[b, pos // 16])
        np.testing.assert_array_equal(cache[0, blk, pos % 16], kn[b])
        before[0, blk, pos % 16] = kn[b]
        before[1, blk, pos % 16] = vn[b]
    np.testing.assert_array_equal(cache, before)


# --------------------------------------------------------------------------
# per-head reading of the GQA token flow: each query head's own softmax over
# the window, averaged over the group


def _token_case(keys, H_kv=1):
    """Cache [2, S, 1, H_kv, D] holding `keys` ([S, H_kv, D] bf16-exact floats)
    under a contiguous block table, one request."""
    keys = np.asarray(keys, dtype=np.float64)
    S, _, D = keys.shape
    cache = np.zeros((2, S, 1, H_kv, D), dtype=np.uint16)
    cache[0, :, 0] = oracle.double_to_bf16(keys)
    assert np.array_equal(oracle.bf16_decode(cache[0, :, 0]), keys)
    bt = np.arange(S, dtype=np.int32)[None, :]
    sl = np.array([S], dtype=np.int32)
    return cache, bt, sl


def test_per_head_closed_form_three_tokens():
    # keys e1, e2, 0; head 0 asks along e1, head 1 along e2 (q = c e_i, scale 1)
    D, c = 8, 2.0
    keys = np.zeros((3, 1, D))
    keys[0, 0, 0] = 1.0
    keys[1, 0, 1] = 1.0
    cache, bt, sl = _token_case(keys)
    q = np.zeros((1, 2, D))
    q[0, 0, 0] = c
    q[0, 1, 1] = c
    e = np.exp(c)
    # each head: (e, 1, 1) / (e + 2) and (1, e, 1) / (e + 2); their mean
    heads = np.array([(e + 1) / 2, (e + 1) / 2, 1.0]) / (e + 2)
    # the group-mean query c/2 (e1 + e2) gives softmax(c/2, c/2, 0)
    mean_q = np.array([np.exp(c / 2), np.exp(c / 2), 1.0]) / (2 * np.exp(c / 2) + 1)
    assert np.abs(heads - mean_q).max() > 0.02          # the readings differ here
    d = 0.984375
    for per_head, want in ((True, heads), (False, mean_q)):
        hh = np.zeros((3, 1), dtype=np.uint16)
        sc = oracle.h2o_step(q, cache, bt, sl, hh, 0, 0, 1.0, d, per_head=per_head)
        np.testing.assert_array_equal(hh[:, 0], oracle.double_to_bf16(want))
        np.testing.assert_array_equal(sc[0, 0, :3], oracle.bf16_decode(hh[:, 0]))
        # second step: bf16(bf16(p) + bf16(d) * hh)
        first = oracle.bf16_decode(hh[:, 0]).copy()
        oracle.h2o_step(q, cache, bt, sl, hh, 0, 0, 1.0, d, per_head=per_head)
        pb = oracle.bf16_decode(oracle.double_to_bf16(want))
        np.testing.assert_array_equal(hh[:, 0], oracle.double_to_bf16(pb + d * first))


def _random_token_case(seed, B=2, H_q=8, H_kv=2, D=16, S=40):
    rng = np.random.default_rng(seed)
    cache = oracle.double_to_bf16(rng.standard_normal((2, B * S, 1, H_kv, D)))
    bt = rng.permutation(B * S).astype(np.int32).reshape(B, S)
    sl = np.array([S, S - 13][:B], dtype=np.int32)
    q = rng.standard_normal((B, H_q, D))
    hh = oracle.double_to_bf16(rng.random((B * S, H_kv)) * 4)
    return cache, bt, sl, q, hh


def test_per_head_reduces_to_group_mean_cases():
    # G = 1: both readings are the same step, bit for bit
    cache, bt, sl, q, hh0 = _random_token_case(80, H_q=2, H_kv=2)
    a, b = hh0.copy(), hh0.copy()
    sa = oracle.h2o_step(q, cache, bt, sl, a, 2, 3, 0.25, 0.984375, per_head=True)
    sb = oracle.h2o_step(q, cache, bt, sl, b, 2, 3, 0.25, 0.984375)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(sa, sb)
    # identical queries within each group: the same probabilities (up to the
    # float64 rounding of the two averages, so at most one bf16 step apart)
    cache, bt, sl, q, hh0 = _random_token_case(81, H_q=8, H_kv=2)
    q[:, 1:4] = q[:, 0:1]
    q[:, 5:8] = q[:, 4:5]
    a, b = hh0.copy(), hh0.copy()
    oracle.h2o_step(q, cache, bt, sl, a, 2, 3, 0.25, 0.984375, per_head=True)
    oracle.h2o_step(q, cache, bt, sl, b, 2, 3, 0.25, 0.984375)
    apart = np.abs(a.astype(np.int64) - b.astype(np.int64))
    assert apart.max() <= 1 and (apart == 0).mean() > 0.95


def test_per_head_window_mass_order_and_groups():
    B, H_q, H_kv, S, bos, eos = 2, 8, 2, 40, 2, 3
    cache, bt, sl, q, hh0 = _random_token_case(82, B, H_q, H_kv, S=S)
    # one unit of mass per (request, kv head), only inside [bos, S - eos)
    hh = np.zeros_like(hh0)
    oracle.h2o_step(q, cache, bt, sl, hh, bos, eos, 0.25, 0.984375, per_head=True)
    for b in range(B):
        n = int(sl[b])
        v = oracle.bf16_decode(hh[bt[b, :n]])
        assert np.all(v[:bos] == 0) and np.all(v[n - eos:] == 0)
        assert np.all(v[bos:n - eos] > 0)
        assert np.all(np.abs(v.sum(0) - 1) <= (n - bos - eos) * 2.0 ** -9)
    # mass after n steps from zero: (1 - d^n) / (1 - d) within the 10 % bound
    d, steps = 0.984375, 200
    hh = np.zeros_like(hh0)
    rng = np.random.default_rng(3)
    for _ in range(steps):
        qq = rng.standard_normal(q.shape)
        oracle.h2o_step(qq, cache, bt, sl, hh, bos, eos, 0.25, d, per_head=True)
    exact = (1 - d ** steps) / (1 - d)
    for b in range(B):
        mass = oracle.bf16_decode(hh[bt[b, :int(sl[b])]]).sum(0)
        assert np.all(np.abs(mass / exact - 1) <= 0.10), mass
    # the head order within a group does not matter
    perm = np.array([2, 0, 3, 1, 5, 7, 4, 6])
    a, b = hh0.copy(), hh0.copy()
    oracle.h2o_step(q, cache, bt, sl, a, bos, eos, 0.25, d, per_head=True)
    oracle.h2o_step(q[:, perm], cache, bt, sl, b, bos, eos, 0.25, d, per_head=True)
    assert np.abs(a.astype(np.int64) - b.astype(np.int64)).max() <= 1
    # a group's queries reach only its own kv head
    q2 = q.copy()
    q2[:, 4:] = rng.standard_normal((B, 4, q.shape[2])) * 3
    c = hh0.copy()
    oracle.h2o_step(q2, cache, bt, sl, c, bos, eos, 0.25, d, per_head=True)
    np.testing.assert_array_equal(c[:, 0], a[:, 0])
    assert not np.array_equal(c[:, 1], a[:, 1])


def test_per_head_matches_brute_force_on_tiny_inputs():
    # the definition written out with exact rational weights: logits chosen so
    # every head's softmax is a ratio of small integers (exp of log-integers)
    D = 4
    keys = np.zeros((4, 1, D))
    keys[:, 0, 0] = [1.0, 0.0, 0.0, 0.0]
    keys[:, 0, 1] = [0.0, 1.0, 0.0, 0.0]
    keys[:, 0, 2] = [0.0, 0.0, 1.0, 0.0]
    cache, bt, sl = _token_case(keys)
    q = np.zeros((1, 4, D))
    q[0, 0, :3] = np.log([3.0, 1.0, 1.0])      # exp logits 3, 1, 1, 1 -> /6
    q[0, 1, :3] = np.log([1.0, 5.0, 1.0])      # 1, 5, 1, 1 -> /8
    q[0, 2, :3] = np.log([1.0, 1.0, 7.0])      # 1, 1, 7, 1 -> /10
    q[0, 3, :3] = np.log([2.0, 2.0, 2.0])      # 2, 2, 2, 1 -> /7
    probs = np.array([[3, 1, 1, 1], [1, 5, 1, 1], [1, 1, 7, 1], [2, 2, 2, 1]], float)
    probs /= probs.sum(1, keepdims=True)
    want = probs.mean(0)
    hh = np.zeros((4, 1), dtype=np.uint16)
    oracle.h2o_step(q, cache, bt, sl, hh, 0, 0, 1.0, 0.984375, per_head=True)
    np.testing.assert_array_equal(hh[:, 0], oracle.double_to_bf16(want))
