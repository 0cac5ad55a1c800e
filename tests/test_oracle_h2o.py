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
