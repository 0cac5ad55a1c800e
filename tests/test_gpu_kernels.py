"""GPU parity of each entry point against the float64 oracle, on small seeded
cases that span several tiles, ragged tails and the degenerate cases (one
token, budget >= N, budget 1, empty splits, exact ties, -0.0, +/-inf lse).
All calls go through the C ABI (sparse_kv_cache_amd binding)."""
import numpy as np
import pytest
import torch

import oracle
import sparse_kv_cache_amd as skv
from sparse_kv_cache_amd import workloads as W
from sparse_kv_cache_amd.decode import SparseDecoder

from parity import (OUT_ATOL, bits, check_attention, check_gauss_row, check_partials,
                    check_group_select_decode_matches, check_scores,
                    check_split_select_decode_matches, check_decoder_partials,
                    check_token_fused_matches, check_scores_alibi, check_scores_group, page_rows,
                    check_selection_exact, check_selection_vs_oracle,
                    check_stats, dev, per_head_rows, poison, say,
                    selection_rows, bf16_bits_apart, check_sel_blk)

pytestmark = pytest.mark.gpu

# seed, B, H_q, H_kv, D, P, max_pages, topk, frac, bos, eos, splits, w_avg, w_peak
PAGE_CASES = [
    (0, 2, 4, 2, 64, 16, 9, 3, 0.0, 0, 1, 2, 1.0, 1.0),
    (1, 3, 8, 2, 128, 16, 20, 5, 0.0, 0, 1, 3, 1.0, 0.5),
    (2, 2, 7, 1, 128, 16, 12, 4, 0.0, 1, 2, 4, 0.5, -1.0),
    (3, 2, 3, 3, 64, 4, 30, 6, 0.2, 0, 1, 5, 1.0, 1.0),
    (4, 2, 16, 2, 128, 16, 40, 9, 0.0, 0, 1, 8, 1.0, 1.0),
    (5, 1, 16, 1, 64, 1, 200, 17, 0.0, 2, 3, 3, 1.0, 1.0),
    (6, 2, 8, 2, 128, 16, 6, 50, 0.0, 0, 1, 4, 1.0, 1.0),
    (7, 4, 4, 4, 128, 16, 3, 1, 0.0, 0, 1, 1, 1.0, 1.0),
    (8, 2, 32, 8, 128, 16, 64, 16, 0.0, 0, 1, 8, 1.0, 0.5),
    (9, 2, 12, 4, 64, 8, 25, 7, 0.3, 1, 1, 2, 1.0, 2.0),
    (10, 1, 6, 2, 128, 2, 80, 9, 0.0, 0, 1, 16, 1.0, 1.0),
    # more splits than selection capacity: most chunks start past the row
    (11, 2, 8, 2, 128, 16, 24, 4, 0.0, 0, 1, 32, 1.0, 1.0),
    # split counts the in-decode selection's 16-wave blocks do not divide
    # (waves past the last split stay for the selection only)
    (12, 2, 8, 2, 128, 16, 30, 6, 0.0, 0, 1, 20, 1.0, 1.0),
    (13, 1, 16, 2, 64, 16, 300, 24, 0.0, 1, 1, 12, 1.0, 0.5),
]


def _decoder(wl):
    return SparseDecoder(wl.B, wl.H_q, wl.H_kv, wl.D, wl.num_blocks, wl.P,
                         wl.bt_ld, topk_pages=wl.topk_pages, topk_frac=wl.topk_frac,
                         bos=wl.bos, eos=wl.eos, w_avg=wl.w_avg, w_peak=wl.w_peak,
                         scale=wl.softmax_scale, num_splits=wl.num_splits)


def check_one_launch_step(d, q, cache, bt, sl):
    """sparse_page_decode (score + select + decode + merge in one launch)
    against the separate launches already in d's buffers."""
    ref_s, ref_idx = d.scores.clone(), d.sel_idx.clone()
    ref_cnt, ref_blk = d.sel_cnt.clone(), d.sel_blk.clone()
    o_ref, l_ref = d.out.clone(), d.lse.clone()
    d.keep_scores = d.keep_selection = True
    d.scores.fill_(float("nan"))
    d.sel_idx.fill_(-7); d.sel_cnt.fill_(-7); d.sel_blk.fill_(-7)
    d.out.fill_(float("nan")); d.lse.fill_(float("nan"))
    d.score_select_attend(q, cache, bt, sl)
    torch.cuda.synchronize()
    valid = ~torch.isnan(ref_s)
    assert torch.equal(torch.isnan(d.scores), ~valid), "one-launch scores: written set differs"
    # same arithmetic; with ALiBi the slope / scale is rounded on a different
    # side, so the bound is relative to the row's largest magnitude (the bias
    # and the q.k terms can cancel)
    rowmax = torch.nan_to_num(ref_s.abs(), nan=0.0).amax(dim=2, keepdim=True)
    err = torch.nan_to_num((d.scores - ref_s).abs(), nan=0.0)
    assert torch.all(err <= 4e-6 * rowmax + 1e-6), \
        f"one-launch scores differ by {float(err.max())}"
    if not torch.equal(d.scores[valid], ref_s[valid]):
        # its selection must be exact on its own scores
        gs = d.scores.cpu().numpy()
        N = np.repeat((sl.cpu().numpy().astype(np.int64) + d.P - 1) // d.P, d.H_q)
        check_selection_exact(d.sel_idx.cpu().numpy().reshape(-1, d.k_cap),
                              d.sel_cnt.cpu().numpy().reshape(-1),
                              gs.reshape(-1, gs.shape[2]), N, d.topk_pages, d.topk_frac,
                              d.bos, d.eos)
    if torch.equal(d.sel_idx, ref_idx) and torch.equal(d.sel_cnt, ref_cnt):
        assert torch.equal(d.sel_blk, ref_blk)
        assert torch.allclose(o_ref, d.out, rtol=0, atol=1e-5), "one-launch output differs"
        assert torch.allclose(l_ref, d.lse, rtol=0, atol=1e-5), "one-launch lse differs"
    else:
        assert torch.equal(torch.isnan(d.scores), ~valid)   # (selection differs at a tie)
    d.keep_scores = d.keep_selection = False


def run_page_case(wl, cache_cpu, q_cpu, exact_ties=False):
    cache = dev(cache_cpu)
    q = dev(q_cpu)
    bt = dev(wl.block_table)
    sl = dev(wl.seq_lens)
    d = _decoder(wl)
    d.keep_partials = True
    poison(d)
    d.k_min.fill_(float("nan")); d.k_max.fill_(float("nan")); d.k_mean.fill_(float("nan"))
    d.rebuild_stats(cache, bt, sl)
    d.score(q, bt, sl)
    d.select(sl, bt)
    d.attend(q, cache, bt, sl)
    d.merge()
    torch.cuda.synchronize()
    # the same decode through the block table instead of the selection's ids
    o_with = d.out.clone()
    d.use_sel_blk = False
    d.out.fill_(float("nan"))
    d.attend(q, cache, bt, sl)
    d.merge()
    torch.cuda.synchronize()
    # (the two paths may use different kernels and summation orders)
    assert torch.allclose(o_with, d.out, rtol=0, atol=1e-5), \
        "decode differs with / without sel_blk"
    d.use_sel_blk = True
    if d.fused:
        # the in-block merge against the separate merge launch
        lse_f = d.lse.clone()
        d.fused = False
        d.out.fill_(float("nan"))
        d.lse.fill_(float("nan"))
        d.attend(q, cache, bt, sl)
        d.merge()
        torch.cuda.synchronize()
        assert torch.allclose(o_with, d.out, rtol=0, atol=1e-5), "merged decode differs"
        assert torch.allclose(lse_f, d.lse, rtol=0, atol=1e-5, equal_nan=False), \
            "merged decode lse differs"
        d.fused = True
    if d.select_in_decode:
        # selection inside the decode launch: the same selection as page_topk
        # and the same output
        ref_idx, ref_cnt, ref_blk = d.sel_idx.clone(), d.sel_cnt.clone(), d.sel_blk.clone()
        o_ref, l_ref = d.out.clone(), d.lse.clone()
        d.keep_selection = True
        d.sel_idx.fill_(-7); d.sel_cnt.fill_(-7); d.sel_blk.fill_(-7)
        d.out.fill_(float("nan")); d.lse.fill_(float("nan"))
        d.select_attend(q, cache, bt, sl)
        torch.cuda.synchronize()
        assert torch.equal(d.sel_idx, ref_idx) and torch.equal(d.sel_cnt, ref_cnt)
        assert torch.equal(d.sel_blk, ref_blk)
        assert torch.allclose(o_ref, d.out, rtol=0, atol=1e-5), "select+decode differs"
        assert torch.allclose(l_ref, d.lse, rtol=0, atol=1e-5), "select+decode lse differs"
    if d.score_in_decode:
        check_one_launch_step(d, q, cache, bt, sl)
    if d.select_in_split_decode:
        check_split_select_decode_matches(d, q, cache, bt, sl)

    cb = bits(cache)
    qd = q_cpu.double().numpy()
    used = W.referenced_blocks(wl)
    gmin, gmax = bits(d.k_min), bits(d.k_max)
    gmean = d.k_mean.cpu().numpy()
    st = check_stats(gmin, gmax, gmean, cb, wl.block_table, wl.seq_lens, wl.P, used)
    # the score kernel in isolation: oracle fed the GPU statistics
    gst = (oracle.bf16_decode(gmin), oracle.bf16_decode(gmax), gmean.astype(np.float64))
    gs = d.scores.cpu().numpy()
    check_scores(gs, qd, gst, wl.block_table, wl.seq_lens, wl.P, wl.w_avg, wl.w_peak)
    # the top-k kernel in isolation: oracle fed the GPU scores
    N = wl.pages()
    sel_idx = d.sel_idx.cpu().numpy().reshape(-1, d.k_cap)
    sel_cnt = d.sel_cnt.cpu().numpy().reshape(-1)
    rowsN = np.repeat(N, wl.H_q)
    check_selection_exact(sel_idx, sel_cnt, gs.reshape(-1, wl.bt_ld), rowsN,
                          wl.topk_pages, wl.topk_frac, wl.bos, wl.eos)
    check_sel_blk(d.sel_blk.cpu().numpy(), d.sel_idx.cpu().numpy(), wl.block_table)
    # end to end: oracle statistics and scores in float64
    ref_scores = oracle.page_score(qd, *st, wl.block_table, wl.seq_lens, wl.P,
                                   wl.w_avg, wl.w_peak)
    rows = selection_rows(sel_idx, sel_cnt)
    ex = check_selection_vs_oracle(rows, ref_scores.reshape(-1, wl.bt_ld), rowsN,
                                   wl.topk_pages, wl.topk_frac, wl.bos, wl.eos)
    if exact_ties:
        assert ex == 0
    # attention over the GPU's own selection
    per = per_head_rows(rows, wl.B, wl.H_q, wl.H_q)
    check_partials(d.o_part.cpu().numpy(), d.lse_part.cpu().numpy(), qd, cb,
                   wl.block_table, wl.seq_lens, per, wl.G, wl.softmax_scale, d.k_cap)
    if d.select_in_split_decode:
        check_decoder_partials(d, qd, cb, wl.block_table, wl.seq_lens, per, wl.G,
                               wl.softmax_scale)
    worst = check_attention(d.out.cpu().numpy(), d.lse.cpu().numpy(), qd, cb,
                            wl.block_table, wl.seq_lens, per, wl.G,
                            wl.softmax_scale)
    return worst, ex


@pytest.mark.parametrize("case", PAGE_CASES, ids=[f"page{c[0]}" for c in PAGE_CASES])
def test_page_level_step(case):
    (seed, B, H_q, H_kv, D, P, maxp, topk, frac, bos, eos, ns, wa, wp) = case
    say(f"[gpu] page-level case {case}")
    wl = W.small_case(seed=seed, B=B, H_q=H_q, H_kv=H_kv, D=D, P=P, max_pages=maxp,
                      topk_pages=topk, topk_frac=frac, bos=bos, eos=eos,
                      w_avg=wa, w_peak=wp, num_splits=ns)
    worst, ex = run_page_case(wl, W.make_cache(wl), W.make_queries(wl))
    say(f"  max |out - oracle| = {worst:.2e}, exempt rows {ex}")


def test_page_level_step_with_empty_and_one_token_requests():
    """A batch holding an empty request (S = 0: no page, nothing selected,
    output 0 with lse -inf), a one-token request and a full one, through
    every launch form of the page-level step."""
    say("[gpu] page-level step with S = 0 and S = 1 requests")
    wl = W.small_case(seed=90, B=4, H_q=8, H_kv=2, D=128, P=16, max_pages=12,
                      topk_pages=5, num_splits=4)
    wl.seq_lens = np.array([0, 1, 17, 12 * 16], dtype=np.int32)
    wl.block_table[3] = np.arange(12, dtype=np.int32) + 30
    worst, ex = run_page_case(wl, W.make_cache(wl), W.make_queries(wl))
    say(f"  max |out - oracle| = {worst:.2e}, exempt rows {ex}")


# The in-block selection (select + decode, and the one launch) holds 1, 4 or 8
# entries per thread for rows of up to 512, 2048 and 4096 pages (the longest
# row the one launch takes); its decode has a page-size-16 form and a generic
# one, with and without ALiBi, at D = 64 and 128.  One case per combination.
# seed, B, H_q, H_kv, D, P, max_pages, min_pages, topk, splits, alibi
LONG_ROW_CASES = [
    (70, 2, 8, 2, 128, 16, 1500, 600, 300, 8, False),
    (71, 1, 4, 1, 64, 16, 4096, 2500, 2000, 8, False),
    (72, 2, 8, 2, 128, 16, 4096, 2300, 700, 6, False),
    (73, 2, 4, 2, 64, 16, 1200, 600, 200, 4, False),
    (74, 2, 8, 2, 128, 8, 300, 100, 40, 8, False),
    (75, 2, 8, 2, 128, 4, 1800, 700, 250, 8, False),
    (76, 1, 8, 2, 128, 2, 4096, 2200, 900, 5, False),
    (77, 2, 4, 1, 64, 4, 1500, 600, 300, 8, False),
    (78, 1, 4, 2, 64, 8, 4000, 2100, 1000, 3, False),
    (79, 2, 6, 3, 64, 8, 400, 100, 30, 7, False),
    (84, 2, 8, 2, 128, 16, 1500, 600, 300, 8, True),
    (85, 1, 8, 2, 128, 16, 4096, 2300, 700, 6, True),
    (86, 2, 4, 2, 64, 16, 300, 100, 40, 4, True),
    (87, 2, 4, 2, 64, 16, 1200, 600, 200, 8, True),
    (88, 1, 4, 1, 64, 16, 4096, 2500, 2000, 8, True),
    (89, 2, 8, 2, 128, 8, 300, 100, 40, 8, True),
    (90, 2, 8, 2, 128, 4, 1800, 700, 250, 8, True),
    (91, 1, 8, 2, 128, 2, 4096, 2200, 900, 5, True),
    (92, 2, 6, 3, 64, 8, 400, 100, 30, 7, True),
    (93, 2, 4, 1, 64, 4, 1500, 600, 300, 8, True),
    (94, 1, 4, 2, 64, 8, 4000, 2100, 1000, 3, True),
]


@pytest.mark.parametrize("case", LONG_ROW_CASES, ids=[f"rows{c[0]}" for c in LONG_ROW_CASES])
def test_page_level_step_long_rows(case):
    (seed, B, H_q, H_kv, D, P, maxp, minp, topk, ns, al) = case
    say(f"[gpu] page-level rows {case}")
    wl = W.small_case(seed=seed, B=B, H_q=H_q, H_kv=H_kv, D=D, P=P, max_pages=maxp,
                      topk_pages=topk, num_splits=ns, min_len=minp * P)
    d = _decoder(wl)
    assert d.fused and d.select_in_decode and d.score_in_decode
    del d
    cache, q = W.make_cache(wl), W.make_queries(wl)
    if al:
        from sparse_kv_cache_amd.decode import alibi_slopes
        slopes = alibi_slopes(H_q, device="cpu").numpy()
        worst, ex = run_alibi_case(wl, cache, q, False, slopes)
    else:
        worst, ex = run_page_case(wl, cache, q)
    say(f"  max |out - oracle| = {worst:.2e}, exempt rows {ex}")


# seed, B, H_q, H_kv, D, P, max_pages, min_pages, topk, splits, alibi: the
# selection inside the split decode at its limits (rows of 8192, k_cap 4096;
# the generic page size's 8-wave blocks with 16 entries a thread; a few
# hundred splits; 4096 splits, most of them past the selection)
SPLIT_ROW_CASES = [
    (100, 1, 4, 2, 64, 16, 8192, 7000, 4096, 64, False),
    (101, 1, 2, 1, 64, 4, 8192, 6000, 1500, 40, False),
    (102, 2, 4, 2, 64, 16, 3000, 1000, 800, 300, False),
    (103, 1, 4, 2, 128, 16, 8192, 8000, 256, 4096, False),
    (104, 1, 4, 2, 64, 16, 8192, 7000, 3000, 48, True),
]


@pytest.mark.parametrize("case", SPLIT_ROW_CASES, ids=[f"split{c[0]}" for c in SPLIT_ROW_CASES])
def test_split_select_decode_at_its_limits(case):
    (seed, B, H_q, H_kv, D, P, maxp, minp, topk, ns, al) = case
    say(f"[gpu] split select-decode {case}")
    wl = W.small_case(seed=seed, B=B, H_q=H_q, H_kv=H_kv, D=D, P=P, max_pages=maxp,
                      topk_pages=topk, num_splits=ns, min_len=minp * P)
    d = _decoder(wl)
    assert d.select_in_split_decode and not d.fused
    del d
    cache, q = W.make_cache(wl), W.make_queries(wl)
    if al:
        from sparse_kv_cache_amd.decode import alibi_slopes
        slopes = alibi_slopes(H_q, device="cpu").numpy()
        worst, ex = run_alibi_case(wl, cache, q, False, slopes)
    else:
        worst, ex = run_page_case(wl, cache, q)
    say(f"  max |out - oracle| = {worst:.2e}, exempt rows {ex}")


# seed, D, P, max_pages, min_pages, topk, frac, bos, eos, splits, alibi: the
# split select-decode's ranked window between reserved leading and trailing
# pages, with a budget that grows with the row (topk_frac)
SPLIT_WINDOW_CASES = [
    (106, 128, 16, 6000, 3000, 100, 0.05, 3, 5, 24, False),
    (107, 64, 4, 5000, 1000, 20, 0.1, 7, 2, 40, True),
]


@pytest.mark.parametrize("case", SPLIT_WINDOW_CASES,
                         ids=[f"window{c[0]}" for c in SPLIT_WINDOW_CASES])
def test_split_select_decode_reserved_window_and_fraction(case):
    (seed, D, P, maxp, minp, topk, frac, bos, eos, ns, al) = case
    say(f"[gpu] split select-decode with a reserved window {case}")
    wl = W.small_case(seed=seed, B=2, H_q=4, H_kv=2, D=D, P=P, max_pages=maxp,
                      topk_pages=topk, topk_frac=frac, bos=bos, eos=eos, num_splits=ns,
                      min_len=minp * P)
    d = _decoder(wl)
    assert d.select_in_split_decode
    del d
    cache, q = W.make_cache(wl), W.make_queries(wl)
    if al:
        from sparse_kv_cache_amd.decode import alibi_slopes
        worst, ex = run_alibi_case(wl, cache, q, False, alibi_slopes(4, device="cpu").numpy())
    else:
        worst, ex = run_page_case(wl, cache, q)
    say(f"  max |out - oracle| = {worst:.2e}, exempt rows {ex}")


def _short_rows(wl, pages):
    """Cap every request at `pages` pages (a ragged tail kept): the block-table
    row keeps its width, which sets how many selection entries a thread of the
    in-decode top-k holds, while the data and the oracle's work stay small."""
    cap = pages * wl.P - (np.arange(wl.B) % wl.P)
    wl.seq_lens = np.minimum(wl.seq_lens, cap).astype(np.int32)
    return wl


# (page size, row width): every entries-per-thread count of the split
# select-decode (1-8 with 16-wave blocks at page size 16, 1-16 with 8-wave
# blocks below it)
SPLIT_FORMS = [(16, 600), (16, 1500), (16, 3000), (16, 6000),
               (4, 400), (4, 900), (4, 1800), (4, 3500), (4, 7000)]


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("alibi", [False, True], ids=["plain", "alibi"])
@pytest.mark.parametrize("P,ld", SPLIT_FORMS, ids=[f"P{p}-ld{l}" for p, l in SPLIT_FORMS])
def test_split_select_decode_every_form(P, ld, alibi, D):
    say(f"[gpu] split select-decode form P={P} ld={ld} alibi={alibi} D={D}")
    wl = _short_rows(W.small_case(seed=110 + ld % 89, B=2, H_q=4, H_kv=2, D=D, P=P,
                                  max_pages=ld, topk_pages=10, num_splits=12), 40)
    d = _decoder(wl)
    assert d.select_in_split_decode and not d.fused
    del d
    cache, q = W.make_cache(wl), W.make_queries(wl)
    if alibi:
        from sparse_kv_cache_amd.decode import alibi_slopes
        worst, ex = run_alibi_case(wl, cache, q, False, alibi_slopes(4, device="cpu").numpy())
    else:
        worst, ex = run_page_case(wl, cache, q)
    say(f"  max |out - oracle| = {worst:.2e}, exempt rows {ex}")


# row widths for every entries-per-thread count (4, 8, 12, 16) of the group
# decode's in-block selection
GROUP_FORMS = [100, 3000, 5000, 7000]


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("alibi", [False, True], ids=["plain", "alibi"])
@pytest.mark.parametrize("ld", GROUP_FORMS)
def test_group_select_decode_every_form(ld, alibi, D):
    say(f"[gpu] group select-decode form ld={ld} alibi={alibi} D={D}")
    wl = _short_rows(W.small_case(seed=120 + ld % 83, B=2, H_q=8, H_kv=2, D=D, P=16,
                                  max_pages=ld, topk_pages=10, num_splits=4), 40)
    cache, q = W.make_cache(wl), W.make_queries(wl)
    if alibi:
        from sparse_kv_cache_amd.decode import alibi_slopes
        worst, ex = run_alibi_case(wl, cache, q, True, alibi_slopes(8, device="cpu").numpy())
    else:
        worst, ex = run_group_case(wl, cache, q)
    say(f"  max |out - oracle| = {worst:.2e}, exempt rows {ex}")


@pytest.mark.parametrize("alibi", [False, True], ids=["plain", "alibi"])
def test_group_select_decode_sixteen_heads(alibi):
    """A query group of 16 (every column of the matrix-core tile) sharing one
    selection over rows of up to 3,000 pages."""
    say(f"[gpu] group select-decode, G = 16, alibi={alibi}")
    wl = _short_rows(W.small_case(seed=131, B=2, H_q=32, H_kv=2, D=128, P=16,
                                  max_pages=3000, topk_pages=24, num_splits=6), 300)
    cache, q = W.make_cache(wl), W.make_queries(wl)
    if alibi:
        from sparse_kv_cache_amd.decode import alibi_slopes
        worst, ex = run_alibi_case(wl, cache, q, True, alibi_slopes(32, device="cpu").numpy())
    else:
        worst, ex = run_group_case(wl, cache, q)
    say(f"  max |out - oracle| = {worst:.2e}, exempt rows {ex}")


def test_bandwidth_references_run():
    """The two read-only references (measurement tools, no arithmetic of the
    method) run over valid inputs, at both head sizes; their sink is written
    only when a read word equals a sentinel, which zeros never do."""
    say("[gpu] bandwidth references")
    sink = torch.zeros(1024, dtype=torch.int32, device="cuda")
    skv.skv_ref_stream_read(torch.zeros(1 << 22, dtype=torch.uint8, device="cuda"), sink)
    for D in (64, 128):
        kv = torch.zeros((2, 8, 16, 2, D), dtype=torch.bfloat16, device="cuda")
        items = torch.tensor([[blk, h, n] for blk in range(8) for h in range(2) for n in (16, 5)],
                             dtype=torch.int32, device="cuda")
        skv.skv_ref_gather_read(kv, items, sink)
    torch.cuda.synchronize()
    assert int(sink.abs().sum().item()) == 0


def test_page_level_step_with_128_query_heads():
    """128 query heads over 8 kv heads (G = 16) at D = 64."""
    say("[gpu] page-level step, 128 query heads")
    wl = W.small_case(seed=91, B=2, H_q=128, H_kv=8, D=64, P=16, max_pages=10,
                      topk_pages=4, num_splits=2)
    worst, ex = run_page_case(wl, W.make_cache(wl), W.make_queries(wl))
    say(f"  max |out - oracle| = {worst:.2e}, exempt rows {ex}")


# (D, H_q, H_kv): group slices of 1, 2, 4 and 8 query heads (and two of 8)
SCORE_SHAPES = [(64, 2, 2), (64, 4, 2), (64, 8, 2), (64, 16, 2), (64, 32, 2),
                (128, 2, 2), (128, 4, 2), (128, 8, 2), (128, 16, 2), (128, 32, 2)]


@pytest.mark.parametrize("D,H_q,H_kv", SCORE_SHAPES,
                         ids=[f"D{d}-G{h // k}" for d, h, k in SCORE_SHAPES])
def test_page_score_both_block_shapes(D, H_q, H_kv):
    """page_score runs 8-wave blocks while its 4-wave grid fits on the
    device at once (at most 2048 blocks) and 4-wave blocks past that. The grid
    follows the block-table row length (blocks past a request's pages return
    at once), so the same batch scored through a short and a long row takes
    both shapes; each must match the oracle fed the same statistics, for
    every group-slice width."""
    say(f"[gpu] page_score block shapes, D={D} G={H_q // H_kv}")
    B, P = 32, 16
    wl = W.small_case(seed=97, B=B, H_q=H_q, H_kv=H_kv, D=D, P=P, max_pages=40)
    cache = dev(W.make_cache(wl))
    q_cpu = W.make_queries(wl)
    q, sl = dev(q_cpu), dev(wl.seq_lens)
    k_min = torch.empty((wl.num_blocks, H_kv, D), dtype=torch.bfloat16, device="cuda")
    k_max = torch.empty_like(k_min)
    k_mean = torch.empty((wl.num_blocks, H_kv, D), dtype=torch.float32, device="cuda")
    ppw, slices = 64 // (D // 8), -(-(H_q // H_kv) // 8)
    for ld in (48, 2100):
        tiles4 = -(-ld // (2 * 4 * ppw))
        assert (H_kv * slices * tiles4 * B <= 2048) == (ld == 48)
        bt_np = np.zeros((B, ld), dtype=np.int32)
        bt_np[:, :wl.block_table.shape[1]] = wl.block_table
        bt = dev(bt_np)
        skv.pagestats_update(cache, k_min, k_max, k_mean, bt, sl)
        scores = torch.full((B, H_q, ld), float("nan"), device="cuda")
        skv.page_score(q, k_min, k_max, k_mean, bt, sl, P, wl.w_avg, wl.w_peak, scores)
        torch.cuda.synchronize()
        gst = (oracle.bf16_decode(bits(k_min)), oracle.bf16_decode(bits(k_max)),
               k_mean.cpu().numpy().astype(np.float64))
        check_scores(scores.cpu().numpy(), q_cpu.double().numpy(), gst, bt_np, wl.seq_lens,
                     P, wl.w_avg, wl.w_peak)


# seed, B, H_q, H_kv, D, P, max_pages, topk, frac, bos, eos, splits, w_avg, w_peak
GROUP_CASES = [
    (40, 2, 8, 2, 128, 16, 20, 5, 0.0, 0, 1, 3, 1.0, 1.0),
    (41, 3, 16, 1, 64, 16, 33, 9, 0.0, 1, 1, 4, 1.0, 0.5),
    (42, 2, 12, 4, 128, 4, 30, 7, 0.2, 0, 1, 2, 0.5, 1.0),
    (43, 1, 64, 8, 128, 16, 70, 16, 0.0, 0, 1, 8, 1.0, 1.0),
    (44, 2, 4, 2, 64, 1, 150, 20, 0.0, 2, 3, 5, 1.0, 1.0),
    (45, 2, 6, 3, 128, 16, 5, 50, 0.0, 0, 1, 2, 1.0, 1.0),
    # rows up to 8192 with k_cap 4096 (the in-decode selection's 16 entries a
    # thread), and a generic page size with a reserved window
    (46, 1, 8, 2, 64, 16, 8192, 4096, 0.0, 0, 1, 8, 1.0, 1.0),
    (47, 2, 8, 4, 128, 4, 6000, 1000, 0.0, 1, 2, 16, 1.0, 0.5),
]


def run_group_case(wl, cache_cpu, q_cpu):
    """Page level with one selection per kv head, shared by its query group."""
    cache = dev(cache_cpu)
    q = dev(q_cpu)
    bt = dev(wl.block_table)
    sl = dev(wl.seq_lens)
    d = SparseDecoder(wl.B, wl.H_q, wl.H_kv, wl.D, wl.num_blocks, wl.P, wl.bt_ld,
                      topk_pages=wl.topk_pages, topk_frac=wl.topk_frac, bos=wl.bos,
                      eos=wl.eos, w_avg=wl.w_avg, w_peak=wl.w_peak,
                      scale=wl.softmax_scale, num_splits=wl.num_splits,
                      group_select=True)
    assert d.H_sel == wl.H_kv
    poison(d)
    d.rebuild_stats(cache, bt, sl)
    d.score(q, bt, sl)
    d.select(sl, bt)
    d.attend(q, cache, bt, sl)
    d.merge()
    torch.cuda.synchronize()

    cb = bits(cache)
    qd = q_cpu.double().numpy()
    used = W.referenced_blocks(wl)
    st = check_stats(bits(d.k_min), bits(d.k_max), d.k_mean.cpu().numpy(), cb,
                     wl.block_table, wl.seq_lens, wl.P, used)
    gst = (oracle.bf16_decode(bits(d.k_min)), oracle.bf16_decode(bits(d.k_max)),
           d.k_mean.cpu().numpy().astype(np.float64))
    gs = d.scores.cpu().numpy()
    check_scores_group(gs, qd, gst, wl.block_table, wl.seq_lens, wl.P, wl.w_avg,
                       wl.w_peak)
    N = wl.pages()
    sel_idx = d.sel_idx.cpu().numpy().reshape(-1, d.k_cap)
    sel_cnt = d.sel_cnt.cpu().numpy().reshape(-1)
    rowsN = np.repeat(N, wl.H_kv)
    check_selection_exact(sel_idx, sel_cnt, gs.reshape(-1, wl.bt_ld), rowsN,
                          wl.topk_pages, wl.topk_frac, wl.bos, wl.eos)
    check_sel_blk(d.sel_blk.cpu().numpy(), d.sel_idx.cpu().numpy(), wl.block_table)
    ref_scores = oracle.page_score_group(qd, *st, wl.block_table, wl.seq_lens, wl.P,
                                         wl.w_avg, wl.w_peak)
    rows = selection_rows(sel_idx, sel_cnt)
    ex = check_selection_vs_oracle(rows, ref_scores.reshape(-1, wl.bt_ld), rowsN,
                                   wl.topk_pages, wl.topk_frac, wl.bos, wl.eos)
    per = per_head_rows(rows, wl.B, wl.H_q, wl.H_kv)
    check_partials(d.o_part.cpu().numpy(), d.lse_part.cpu().numpy(), qd, cb,
                   wl.block_table, wl.seq_lens, per, wl.G, wl.softmax_scale, d.k_cap)
    worst = check_attention(d.out.cpu().numpy(), d.lse.cpu().numpy(), qd, cb,
                            wl.block_table, wl.seq_lens, per, wl.G, wl.softmax_scale)
    if d.select_in_group_decode:
        check_group_select_decode_matches(d, q, cache, bt, sl)
    return worst, ex


@pytest.mark.parametrize("case", GROUP_CASES, ids=[f"group{c[0]}" for c in GROUP_CASES])
def test_group_selection_step(case):
    (seed, B, H_q, H_kv, D, P, maxp, topk, frac, bos, eos, ns, wa, wp) = case
    say(f"[gpu] group-selection case {case}")
    wl = W.small_case(seed=seed, B=B, H_q=H_q, H_kv=H_kv, D=D, P=P, max_pages=maxp,
                      topk_pages=topk, topk_frac=frac, bos=bos, eos=eos,
                      w_avg=wa, w_peak=wp, num_splits=ns)
    worst, ex = run_group_case(wl, W.make_cache(wl), W.make_queries(wl))
    say(f"  max |out - oracle| = {worst:.2e}, exempt rows {ex}")


# seed, B, H_q, H_kv, D, P, max_pages, topk, splits, group_select
ALIBI_CASES = [
    (80, 2, 8, 2, 128, 16, 30, 6, 3, False),
    (81, 2, 4, 4, 64, 4, 40, 7, 4, False),
    (82, 1, 16, 2, 128, 16, 50, 9, 5, True),
    (83, 2, 6, 3, 64, 1, 120, 20, 2, True),
    # more splits than a block merges: the selection inside the split decode
    # (8-wave blocks at page size 4, 16-wave blocks at 16)
    (84, 2, 8, 2, 128, 4, 60, 9, 12, False),
    (85, 1, 16, 2, 128, 16, 200, 12, 20, False),
]


def run_alibi_case(wl, cache_cpu, q_cpu, group, slopes_np):
    """Page level with ALiBi slopes, per-head or group-shared selection."""
    from sparse_kv_cache_amd.decode import alibi_slopes  # noqa: F401 (API presence)
    cache = dev(cache_cpu)
    q = dev(q_cpu)
    bt = dev(wl.block_table)
    sl = dev(wl.seq_lens)
    slopes = torch.from_numpy(slopes_np.astype(np.float32)).cuda()
    d = SparseDecoder(wl.B, wl.H_q, wl.H_kv, wl.D, wl.num_blocks, wl.P, wl.bt_ld,
                      topk_pages=wl.topk_pages, topk_frac=wl.topk_frac, bos=wl.bos,
                      eos=wl.eos, w_avg=wl.w_avg, w_peak=wl.w_peak,
                      scale=wl.softmax_scale, num_splits=wl.num_splits,
                      group_select=group, alibi_slopes=slopes)
    d.keep_partials = True
    poison(d)
    d.rebuild_stats(cache, bt, sl)
    d.score(q, bt, sl)
    d.select(sl, bt)
    d.attend(q, cache, bt, sl)
    d.merge()
    torch.cuda.synchronize()
    cb = bits(cache)
    qd = q_cpu.double().numpy()
    st = check_stats(bits(d.k_min), bits(d.k_max), d.k_mean.cpu().numpy(), cb,
                     wl.block_table, wl.seq_lens, wl.P, W.referenced_blocks(wl))
    gst = (oracle.bf16_decode(bits(d.k_min)), oracle.bf16_decode(bits(d.k_max)),
           d.k_mean.cpu().numpy().astype(np.float64))
    # the score in q.k units takes slope / scale, as the decoder passes it
    a_score = d.alibi_score.cpu().numpy().astype(np.float64)
    gs = d.scores.cpu().numpy()
    check_scores_alibi(gs, qd, gst, wl.block_table, wl.seq_lens, wl.P, wl.w_avg,
                       wl.w_peak, a_score, group)
    H_sel = d.H_sel
    N = wl.pages()
    sel_idx = d.sel_idx.cpu().numpy().reshape(-1, d.k_cap)
    sel_cnt = d.sel_cnt.cpu().numpy().reshape(-1)
    rowsN = np.repeat(N, H_sel)
    check_selection_exact(sel_idx, sel_cnt, gs.reshape(-1, wl.bt_ld), rowsN,
                          wl.topk_pages, wl.topk_frac, wl.bos, wl.eos)
    ref_scores = oracle.page_score_alibi(qd, *st, wl.block_table, wl.seq_lens, wl.P,
                                         wl.w_avg, wl.w_peak, a_score, group)
    rows = selection_rows(sel_idx, sel_cnt)
    ex = check_selection_vs_oracle(rows, ref_scores.reshape(-1, wl.bt_ld), rowsN,
                                   wl.topk_pages, wl.topk_frac, wl.bos, wl.eos)
    per = per_head_rows(rows, wl.B, wl.H_q, H_sel)
    sl64 = slopes.cpu().numpy().astype(np.float64)
    if d.select_in_decode:
        # selection inside the decode launch: page_topk's selection and the
        # same output as the separate launches
        ref_idx, ref_cnt, ref_blk = d.sel_idx.clone(), d.sel_cnt.clone(), d.sel_blk.clone()
        o_ref, l_ref = d.out.clone(), d.lse.clone()
        d.keep_selection = True
        d.sel_idx.fill_(-7); d.sel_cnt.fill_(-7); d.sel_blk.fill_(-7)
        d.out.fill_(float("nan")); d.lse.fill_(float("nan"))
        d.select_attend(q, cache, bt, sl)
        torch.cuda.synchronize()
        assert torch.equal(d.sel_idx, ref_idx) and torch.equal(d.sel_cnt, ref_cnt)
        assert torch.equal(d.sel_blk, ref_blk)
        assert torch.allclose(o_ref, d.out, rtol=0, atol=1e-5), "select+decode differs"
        assert torch.allclose(l_ref, d.lse, rtol=0, atol=1e-5), "select+decode lse differs"
        d.keep_selection = False
    if d.score_in_decode:
        d.fused = False            # the reference buffers from separate launches
        d.attend(q, cache, bt, sl)
        d.merge()
        d.fused = True
        torch.cuda.synchronize()
        check_one_launch_step(d, q, cache, bt, sl)
    if d.select_in_split_decode:
        check_split_select_decode_matches(d, q, cache, bt, sl)
    check_partials(d.o_part.cpu().numpy(), d.lse_part.cpu().numpy(), qd, cb,
                   wl.block_table, wl.seq_lens, per, wl.G, wl.softmax_scale, d.k_cap,
                   slopes=sl64)
    if d.select_in_split_decode:
        check_decoder_partials(d, qd, cb, wl.block_table, wl.seq_lens, per, wl.G,
                               wl.softmax_scale, slopes=sl64)
    worst = check_attention(d.out.cpu().numpy(), d.lse.cpu().numpy(), qd, cb,
                            wl.block_table, wl.seq_lens, per, wl.G, wl.softmax_scale,
                            slopes=sl64)
    if d.select_in_group_decode:
        check_group_select_decode_matches(d, q, cache, bt, sl)
    return worst, ex


@pytest.mark.parametrize("case", ALIBI_CASES, ids=[f"alibi{c[0]}" for c in ALIBI_CASES])
def test_alibi_step(case):
    (seed, B, H_q, H_kv, D, P, maxp, topk, ns, group) = case
    say(f"[gpu] ALiBi case {case}")
    wl = W.small_case(seed=seed, B=B, H_q=H_q, H_kv=H_kv, D=D, P=P, max_pages=maxp,
                      topk_pages=topk, num_splits=ns)
    from sparse_kv_cache_amd.decode import alibi_slopes
    slopes = alibi_slopes(H_q, device="cpu").numpy()
    worst, ex = run_alibi_case(wl, W.make_cache(wl), W.make_queries(wl), group, slopes)
    say(f"  max |out - oracle| = {worst:.2e}, exempt rows {ex}")


# seed, B, H_q, H_kv, D, P, max_pages, topk, splits, group_select, scale
ENTMAX_CASES = [
    (95, 2, 8, 2, 128, 16, 30, 6, 3, False, None),
    (96, 2, 4, 4, 64, 4, 40, 7, 4, False, 1.0),
    (97, 1, 16, 2, 128, 16, 50, 9, 5, True, None),
    (98, 2, 6, 3, 64, 1, 120, 20, 2, True, 0.5),
    # 256 query rows: the merged launch's 8-wave blocks and the three-launch
    # tau pass's 256-thread blocks with the row in registers
    (99, 16, 16, 4, 64, 16, 12, 5, 3, False, None),
]


def run_entmax_case(wl, cache_cpu, q_cpu, group):
    """Page level with 1.5-entmax attention over the GPU's own selection."""
    cache = dev(cache_cpu)
    q = dev(q_cpu)
    bt = dev(wl.block_table)
    sl = dev(wl.seq_lens)
    d = SparseDecoder(wl.B, wl.H_q, wl.H_kv, wl.D, wl.num_blocks, wl.P, wl.bt_ld,
                      topk_pages=wl.topk_pages, topk_frac=wl.topk_frac, bos=wl.bos,
                      eos=wl.eos, w_avg=wl.w_avg, w_peak=wl.w_peak,
                      scale=wl.softmax_scale, num_splits=wl.num_splits,
                      group_select=group, attention="entmax15")
    poison(d)
    d.entmax_scratch.fill_(float("nan"))
    d.rebuild_stats(cache, bt, sl)
    d.score(q, bt, sl)
    d.select(sl, bt)
    torch.cuda.synchronize()
    cb = bits(cache)
    qd = q_cpu.double().numpy()
    sel_idx = d.sel_idx.cpu().numpy().reshape(-1, d.k_cap)
    sel_cnt = d.sel_cnt.cpu().numpy().reshape(-1)
    per = per_head_rows(selection_rows(sel_idx, sel_cnt), wl.B, wl.H_q, d.H_sel)
    ref = {}
    for b in range(wl.B):
        for i in range(wl.H_q):
            ref[b, i] = oracle.attend_entmax15(qd[b, i], cb, i // wl.G, wl.block_table[b],
                                               int(wl.seq_lens[b]), per[b][i],
                                               wl.softmax_scale)
    worst = 0.0
    # one merged launch, then the three launches + lse_merge
    for fused in (True, False):
        d.entmax_fused = fused
        d.out.fill_(float("nan"))
        d.entmax_tau().fill_(float("nan"))
        d.attend(q, cache, bt, sl)
        d.merge()
        torch.cuda.synchronize()
        out = d.out.cpu().numpy()
        gtau = d.entmax_tau().cpu().numpy()
        for (b, i), (o, tau) in ref.items():
            assert not np.any(np.isnan(out[b, i])), f"NaN output ({b},{i}) fused={fused}"
            e = np.abs(out[b, i].astype(np.float64) - o).max()
            worst = max(worst, e)
            assert e <= 2e-3, f"entmax out ({b},{i}) err {e} fused={fused}"
            if np.isinf(tau):
                assert np.isinf(gtau[b, i])
            else:
                assert abs(float(gtau[b, i]) - tau) <= 1e-4 * max(1.0, abs(tau)), \
                    f"tau ({b},{i}) {gtau[b, i]} vs {tau} fused={fused}"
    return worst


@pytest.mark.parametrize("case", ENTMAX_CASES, ids=[f"entmax{c[0]}" for c in ENTMAX_CASES])
def test_entmax_step(case):
    (seed, B, H_q, H_kv, D, P, maxp, topk, ns, group, scale) = case
    say(f"[gpu] 1.5-entmax case {case}")
    wl = W.small_case(seed=seed, B=B, H_q=H_q, H_kv=H_kv, D=D, P=P, max_pages=maxp,
                      topk_pages=topk, num_splits=ns)
    if scale is not None:
        wl.scale = scale
    worst = run_entmax_case(wl, W.make_cache(wl), W.make_queries(wl), group)
    say(f"  max |out - oracle| = {worst:.2e}")


# seed, B, H_q, H_kv, D, P, max_pages, bos, eos, splits, alibi, mixture, cap, scale
GAUSS_CASES = [
    (130, 2, 4, 2, 64, 16, 9, 0, 1, 2, False, None, None, None),
    (131, 3, 8, 2, 128, 16, 40, 0, 1, 4, True, None, None, None),
    (132, 2, 8, 2, 128, 16, 40, 0, 1, 4, False, True, None, None),
    (133, 2, 8, 2, 128, 16, 40, 0, 1, 4, True, False, None, None),
    (134, 2, 6, 2, 128, 8, 60, 1, 2, 3, False, None, 5, 1.0),
    (135, 1, 4, 1, 64, 16, 3, 0, 1, 1, True, None, None, None),
    (136, 2, 16, 2, 128, 16, 300, 0, 1, 8, True, None, None, None),
    (137, 1, 8, 8, 128, 16, 1100, 0, 1, 8, False, None, None, 0.25),
    (138, 2, 8, 4, 64, 4, 90, 2, 1, 5, True, None, 12, None),
    # page size 1 (every variance 0), D 64, no reserved tail page
    (140, 2, 4, 4, 64, 1, 120, 0, 0, 2, False, None, None, None),
    # D 64 with ALiBi, a binding cap, no reserved page, a sharper scale
    (141, 2, 8, 2, 64, 16, 50, 0, 0, 3, True, None, 4, 2.0),
    # D 64 with a group of 8 (the moments pass's widest head slice)
    (142, 2, 16, 2, 64, 16, 40, 0, 1, 4, False, None, None, None),
]


def run_gauss_case(wl, cache_in, q_cpu, slopes_np=None, mixture=None, cap=None, rows=None):
    """Gaussian-aware step: variance statistics, moments, tau-hat, selection
    and the 1.5-entmax decode over it, each against the oracle.  rows limits
    the checked (request, query head) rows (default all)."""
    cache = cache_in if cache_in.is_cuda else dev(cache_in)
    q = dev(q_cpu)
    bt = dev(wl.block_table)
    sl = dev(wl.seq_lens)
    slopes = None if slopes_np is None else dev(np.asarray(slopes_np, dtype=np.float32))
    d = SparseDecoder(wl.B, wl.H_q, wl.H_kv, wl.D, wl.num_blocks, wl.P, wl.bt_ld,
                      topk_pages=wl.topk_pages, bos=wl.bos, eos=wl.eos,
                      scale=wl.softmax_scale, num_splits=wl.num_splits,
                      selection="gauss", alibi_slopes=slopes, gauss_cap=cap,
                      gauss_mixture=mixture)
    poison(d)
    for t in (d.k_var, d.mu, d.var, d.tau_hat, d.entmax_scratch):
        t.fill_(float("nan"))
    d.rebuild_stats(cache, bt, sl)
    d.gauss_select(q, bt, sl)
    # the three-launch decode first, kept for comparison with the merged one
    d.entmax_fused = False
    d.attend(q, cache, bt, sl)
    d.merge()
    torch.cuda.synchronize()
    out3 = d.out.cpu().numpy()
    d.entmax_fused = True
    d.out.fill_(float("nan"))
    d.attend(q, cache, bt, sl)
    d.merge()
    torch.cuda.synchronize()
    cb = bits(cache)
    qd = q_cpu.double().numpy()
    scale = wl.softmax_scale
    _, _, kmean = oracle.page_stats(cb, wl.block_table, wl.seq_lens, wl.P)
    kvar = oracle.page_var(cb, wl.block_table, wl.seq_lens, wl.P)
    used = W.referenced_blocks(wl)
    gv = d.k_var.cpu().numpy()[used].astype(np.float64)
    ov = kvar[used]
    assert np.all(np.abs(gv - ov) <= 1e-5 * ov + 1e-6), \
        f"page variance err {np.abs(gv - ov).max()}"
    sl64 = None if slopes_np is None else np.asarray(slopes_np, np.float32).astype(np.float64)
    mu_o, var_o = oracle.gauss_moments(qd, kmean, kvar, wl.block_table, wl.seq_lens, wl.P,
                                       scale, alibi=sl64, ld=wl.bt_ld)
    g_mu, g_var = d.mu.cpu().numpy(), d.var.cpu().numpy()
    g_est, g_tau = d.est.cpu().numpy(), d.tau_hat.cpu().numpy()
    sel_idx, sel_cnt = d.sel_idx.cpu().numpy(), d.sel_cnt.cpu().numpy()
    check_sel_blk(d.sel_blk.cpu().numpy(), sel_idx, wl.block_table)
    out, etau = d.out.cpu().numpy(), d.entmax_tau().cpu().numpy()
    N_all = wl.pages()
    if rows is None:
        rows = [(b, i) for b in range(wl.B) for i in range(wl.H_q)]
    exempt, worst, counts = 0, 0.0, []
    for b, i in rows:
        S, N = int(wl.seq_lens[b]), int(N_all[b])
        h = i // wl.G
        cnt = int(sel_cnt[b, i])
        assert 0 < cnt <= d.k_cap and np.all(sel_idx[b, i, cnt:] == -1), f"({b},{i}) count"
        counts.append(cnt)
        n = page_rows(S, wl.P, N)
        blk = wl.block_table[b, :N]
        sd = np.sqrt(kvar[blk, h])
        k1 = scale * ((np.abs(kmean[blk, h]) + sd) @ np.abs(qd[b, i]))
        q2 = scale * scale * float(qd[b, i] @ qd[b, i])
        bias = np.zeros(N)
        if sl64 is not None:
            bias = sl64[i] * (np.arange(N) * wl.P + 0.5 * (n - 1) - (S - 1))
        exempt += check_gauss_row(g_mu[b, i, :N], g_var[b, i, :N], g_est[b, i, :N],
                                  g_tau[b, i], sel_idx[b, i, :cnt], n, d.mixture, wl.bos,
                                  wl.eos, d.k_cap, mu_o[b, i, :N], var_o[b, i, :N], k1, q2,
                                  bias, (b, i))
        o, t = oracle.attend_entmax15(qd[b, i], cb, h, wl.block_table[b], S,
                                      sel_idx[b, i, :cnt], scale,
                                      slope=None if sl64 is None else sl64[i])
        assert not np.any(np.isnan(out[b, i])), f"NaN output ({b},{i})"
        e = max(np.abs(out[b, i].astype(np.float64) - o).max(),
                np.abs(out3[b, i].astype(np.float64) - o).max())
        worst = max(worst, e)
        assert e <= OUT_ATOL, f"gauss out ({b},{i}) err {e}"
        assert abs(float(etau[b, i]) - t) <= 1e-4 * max(1.0, abs(t)), \
            f"entmax tau ({b},{i}) {etau[b, i]} vs {t}"
    return worst, exempt, counts


@pytest.mark.parametrize("case", GAUSS_CASES, ids=[f"gauss{c[0]}" for c in GAUSS_CASES])
def test_gauss_step(case):
    (seed, B, H_q, H_kv, D, P, maxp, bos, eos, ns, alibi, mixture, cap, scale) = case
    say(f"[gpu] Gaussian-aware case {case}")
    wl = W.small_case(seed=seed, B=B, H_q=H_q, H_kv=H_kv, D=D, P=P, max_pages=maxp,
                      bos=bos, eos=eos, num_splits=ns)
    if scale is not None:
        wl.scale = scale
    from sparse_kv_cache_amd.decode import alibi_slopes
    slopes = alibi_slopes(H_q, device="cpu").numpy() if alibi else None
    worst, ex, counts = run_gauss_case(wl, W.make_cache(wl), W.make_queries(wl), slopes,
                                       mixture, cap)
    say(f"  max |out - oracle| = {worst:.2e}, exempt rows {ex}, pages selected "
        f"{min(counts)}..{max(counts)} of up to {int(wl.pages().max())}")


@pytest.mark.parametrize("alibi", [False, True])
def test_gauss_degenerate_pages(alibi):
    """A zero cache (every variance 0, every mean 0: equal estimates without
    ALiBi), one-token and exactly-full requests."""
    say(f"[gpu] Gaussian-aware degenerate pages, alibi={alibi}")
    wl = W.small_case(seed=139, B=3, H_q=4, H_kv=2, D=128, P=16, max_pages=6,
                      num_splits=2, min_len=20)
    wl.seq_lens = np.array([1, 16, 81], dtype=np.int32)
    perm = np.random.default_rng(139).permutation(wl.num_blocks).astype(np.int32)
    wl.block_table = perm[:wl.B * 6].reshape(wl.B, 6).copy()
    from sparse_kv_cache_amd.decode import alibi_slopes
    slopes = alibi_slopes(wl.H_q, device="cpu").numpy() if alibi else None
    cache = torch.zeros((2, wl.num_blocks, 16, 2, 128), dtype=torch.bfloat16)
    cache[1].normal_(generator=torch.Generator().manual_seed(5))
    run_gauss_case(wl, cache, W.make_queries(wl), slopes)
    run_gauss_case(wl, W.make_cache(wl), W.make_queries(wl), slopes)


def test_all_equal_scores_tie_break_to_lower_index():
    say("[gpu] zero cache: every score ties")
    wl = W.small_case(seed=20, B=2, H_q=4, H_kv=2, D=128, P=16, max_pages=30,
                      topk_pages=5, num_splits=3, min_len=100)
    cache = torch.zeros((2, wl.num_blocks, 16, 2, 128), dtype=torch.bfloat16)
    worst, ex = run_page_case(wl, cache, W.make_queries(wl), exact_ties=True)


def test_topk_rows_against_oracle_all_sizes():
    rng = np.random.default_rng(0)
    for ld in (1, 5, 64, 1000, 1024, 2048, 2049, 4096, 5000, 8192, 12000, 16384,
               20000, 32768):
        B, H = 3, 2
        say(f"[gpu] page_topk score_ld={ld}")
        sl = rng.integers(1, ld, size=B, endpoint=True).astype(np.int32)
        sc = rng.integers(-6, 7, size=(B, H, ld)).astype(np.float32)      # ties
        sc[0] = rng.standard_normal((H, ld)).astype(np.float32)
        sc[..., ::7] = -0.0
        sc[..., 3::11] = 0.0
        for topk, frac, bos, eos in ((1, 0.0, 0, 1), (7, 0.0, 2, 3), (3, 0.1, 0, 1),
                                     (ld + 5, 0.0, 0, 1), (max(1, ld // 3), 0.0, 0, 0)):
            k_cap = min(max(topk, int(np.floor(np.float64(np.float32(frac)) * ld)),
                            bos + eos), ld)
            k_cap = max(k_cap, 1)
            scores = dev(sc)
            idx = torch.full((B, H, k_cap), -7, dtype=torch.int32, device="cuda")
            cnt = torch.full((B, H), -7, dtype=torch.int32, device="cuda")
            skv.page_topk(scores, dev(sl), 1, topk, idx, cnt, frac, bos, eos)
            torch.cuda.synchronize()
            check_selection_exact(idx.cpu().numpy().reshape(-1, k_cap),
                                  cnt.cpu().numpy().reshape(-1),
                                  sc.reshape(-1, ld).astype(np.float64),
                                  np.repeat(sl, H), topk, frac, bos, eos)


def test_topk_many_rows_all_sizes():
    """Launches of more than 1024 rows (256-thread blocks and wider, reading
    only a row's valid entries) at every row-length class, and a launch of
    exactly 1024 rows (the last that reads whole rows eagerly)."""
    rng = np.random.default_rng(1)
    for B, H, ld in ((33, 32, 1000), (33, 32, 2000), (33, 32, 4000), (33, 32, 8000),
                     (33, 32, 16000), (33, 32, 32768), (32, 32, 3000)):
        say(f"[gpu] page_topk {B * H} rows, score_ld={ld}")
        sl = rng.integers(1, ld, size=B, endpoint=True).astype(np.int32)
        sc = rng.standard_normal((B, H, ld)).astype(np.float32)
        sc[::2, :, ::5] = np.round(sc[::2, :, ::5])          # ties in half the requests
        sc[1::4] = rng.integers(-3, 4, size=sc[1::4].shape)   # and whole rows of them
        topk, frac, bos, eos = max(1, ld // 10), 0.0, 1, 2
        k_cap = min(max(topk, bos + eos), ld)
        scores = dev(sc)
        idx = torch.full((B, H, k_cap), -7, dtype=torch.int32, device="cuda")
        cnt = torch.full((B, H), -7, dtype=torch.int32, device="cuda")
        skv.page_topk(scores, dev(sl), 1, topk, idx, cnt, frac, bos, eos)
        torch.cuda.synchronize()
        check_selection_exact(idx.cpu().numpy().reshape(-1, k_cap),
                              cnt.cpu().numpy().reshape(-1), sc.reshape(-1, ld),
                              np.repeat(sl, H), topk, frac, bos, eos)


def test_gauss_select_rows_all_sizes():
    """gauss_select on synthetic moment rows at every launch shape: under 1024
    rows at the row lengths of the 1024-thread blocks (4, 16 and 32 pages a
    thread), 1024 and more rows at the lengths of the 256- and 512-thread
    blocks; single Gaussian and mixture, with and without a binding cap."""
    from parity import check_gauss_select_row
    rng = np.random.default_rng(3)
    P = 16
    for B, H, ld, mixture, cap in ((2, 3, 3000, False, None), (2, 3, 12000, True, None),
                                   (1, 2, 20000, False, 64), (33, 32, 1500, True, None),
                                   (33, 32, 3000, False, 40), (33, 32, 6000, True, None)):
        say(f"[gpu] gauss_select {B * H} rows, ld={ld}, mixture={mixture}, cap={cap}")
        sl = rng.integers(1, ld * P, size=B, endpoint=True).astype(np.int32)
        mu = rng.normal(0.0, 0.5, size=(B, H, ld)).astype(np.float32)
        mu += (rng.random((B, H, ld)) < 0.01) * np.float32(3.0)      # a few strong pages
        var = rng.gamma(2.0, 0.05, size=(B, H, ld)).astype(np.float32)
        var[..., ::13] = 0.0
        k_cap = ld if cap is None else cap
        bt = np.tile(np.arange(ld, dtype=np.int32), (B, 1))
        est = torch.full((B, H, ld), float("nan"), device="cuda")
        tau = torch.full((B, H), float("nan"), device="cuda")
        idx = torch.full((B, H, k_cap), -7, dtype=torch.int32, device="cuda")
        cnt = torch.full((B, H), -7, dtype=torch.int32, device="cuda")
        skv.gauss_select(dev(mu), dev(var), dev(sl), P, dev(bt), mixture, k_cap, est, idx,
                         cnt, tau=tau, reserved_bos=0, reserved_eos=1)
        torch.cuda.synchronize()
        g_est, g_tau = est.cpu().numpy(), tau.cpu().numpy()
        g_idx, g_cnt = idx.cpu().numpy(), cnt.cpu().numpy()
        for b in range(B):
            N = (int(sl[b]) + P - 1) // P
            n = np.minimum(P, int(sl[b]) - np.arange(N) * P).astype(np.int32)
            for h in range(H):
                check_gauss_select_row(mu[b, h, :N], var[b, h, :N], g_est[b, h, :N],
                                       g_tau[b, h], g_idx[b, h, :g_cnt[b, h]], n, mixture,
                                       0, 1, k_cap, (b, h))


@pytest.mark.parametrize("ns", [1, 9, 16, 17, 32, 33, 64, 300])
def test_lse_merge_edge_cases_and_random(ns):
    """Up to 8 splits per thread (16 at D = 128, 32 at D = 64) take the
    register-resident kernel, in both of its widths; more take the LDS-staged
    passes."""
    say(f"[gpu] lse_merge, {ns} splits")
    rng = np.random.default_rng(1 + ns)
    for D in (64, 128):
        rows = 37
        o = rng.standard_normal((rows, ns, D)).astype(np.float32)
        l = (rng.standard_normal((rows, ns)) * 3).astype(np.float32)
        l[0, :] = -np.inf                     # every split empty
        l[1, :min(4, ns - 1)] = -np.inf
        l[2, min(2, ns - 1)] = np.inf         # +inf is read as -inf
        l[3, :] = -np.inf
        l[3, min(5, ns - 1)] = np.inf
        l[4, 0] = 80.0                        # large spread
        out = torch.full((rows, D), float("nan"), device="cuda")
        lse = torch.full((rows,), float("nan"), device="cuda")
        skv.lse_merge(dev(o), dev(l), out, lse)
        torch.cuda.synchronize()
        go, gl = out.cpu().numpy(), lse.cpu().numpy()
        for r in range(rows):
            want, wl_ = oracle.lse_merge(o[r].astype(np.float64), l[r].astype(np.float64))
            np.testing.assert_allclose(go[r], want, rtol=1e-5, atol=1e-5)
            if np.isinf(wl_):
                assert np.isinf(gl[r]) and gl[r] < 0
            else:
                assert abs(gl[r] - wl_) <= 1e-5
        np.testing.assert_array_equal(go[0], o[0, 0])
        np.testing.assert_array_equal(go[3], o[3, 0])


@pytest.mark.parametrize("P", [16, 4, 1])
def test_append_refresh_and_reset(P):
    say(f"[gpu] pagestats append P={P}")
    wl = W.small_case(seed=30 + P, B=5, H_q=8, H_kv=2, D=128, P=P,
                      max_pages=max(3, 48 // P), min_len=1)
    cache_cpu = W.make_cache(wl)
    cache = dev(cache_cpu)
    bt, sl = dev(wl.block_table), dev(wl.seq_lens)
    kn, vn = W.make_new_kv(wl, step=3)
    hh = torch.full((wl.num_blocks * P, wl.H_kv), 7.5, dtype=torch.bfloat16,
                    device="cuda")
    kmin = torch.full((wl.num_blocks, 2, 128), float("nan"), dtype=torch.bfloat16,
                      device="cuda")
    kmax = kmin.clone()
    kmean = torch.full((wl.num_blocks, 2, 128), float("nan"), device="cuda")
    skv.pagestats_update(cache, kmin, kmax, kmean, bt, sl)          # rebuild
    skv.pagestats_update(cache, kmin, kmax, kmean, bt, sl, dev(kn), dev(vn), hh)
    torch.cuda.synchronize()
    cb = bits(cache_cpu).copy()
    hh_ref = bits(torch.full((wl.num_blocks * P, wl.H_kv), 7.5,
                             dtype=torch.bfloat16)).copy()
    oracle.append(cb, wl.block_table, wl.seq_lens, bits(kn), bits(vn), hh_ref)
    assert np.array_equal(bits(cache), cb), "cache bytes differ after append"
    assert np.array_equal(bits(hh), hh_ref), "hh reset differs"
    used = W.referenced_blocks(wl)
    check_stats(bits(kmin), bits(kmax), kmean.cpu().numpy(), cb, wl.block_table,
                wl.seq_lens, P, used)


@pytest.mark.parametrize("reading,H_q,H_kv,D,eos", [
    ("group_mean", 8, 2, 128, 8), ("per_head", 8, 2, 128, 8), ("per_head", 80, 16, 128, 8),
    # no reserved tail: the newest token's logit is taken (from k_new in the
    # fused step's append)
    ("group_mean", 8, 2, 128, 0), ("per_head", 12, 4, 64, 0),
    ("per_head", 12, 4, 64, 8), ("group_mean", 12, 4, 64, 8),
    # G = 16 (every column of the matrix-core tile), one kv head, and three kv
    # heads (rows dealt token-major in the group-mean pass)
    ("per_head", 16, 1, 64, 8), ("per_head", 48, 3, 128, 8), ("group_mean", 48, 3, 128, 8),
    # every key-row load depth of the group-mean pass (rows of 4 * H_kv tokens
    # per wave, head-major where H_kv divides 16, else token-major) and every
    # tile count per wave of the per-head pass, at both head sizes
    ("group_mean", 8, 4, 128, 8), ("group_mean", 12, 6, 128, 8), ("group_mean", 24, 12, 128, 8),
    ("group_mean", 32, 16, 128, 8), ("group_mean", 6, 3, 64, 8), ("group_mean", 16, 8, 64, 8),
    ("group_mean", 12, 6, 64, 8), ("group_mean", 20, 10, 64, 8), ("group_mean", 32, 16, 64, 8),
    ("per_head", 40, 10, 128, 8), ("per_head", 16, 8, 64, 8), ("per_head", 24, 12, 64, 8),
    ("per_head", 32, 16, 64, 8)])
def test_token_level_step_teacher_forced(reading, H_q, H_kv, D, eos):
    _token_teacher_forced(reading, H_q, H_kv, D, eos)


@pytest.mark.parametrize("reading", ["group_mean", "per_head"])
def test_token_level_step_long_splits(reading):
    """More than 64 tokens a split (200 selected over 2 splits): the
    two-launch step's group decode folds a split's row groups over 8 waves,
    the standalone one over 4, so their partials agree to within rounding
    rather than bit for bit; both must match the oracle."""
    _token_teacher_forced(reading, 8, 2, 128, 1, topk=200, splits=2)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("S0", [3000, 5000, 7000])
@pytest.mark.parametrize("reading", ["group_mean", "per_head"])
def test_token_level_step_long_rows(reading, S0, D):
    """Rows of 3,000, 5,000 and 7,000 tokens: the two-launch step's in-block
    selection at 8, 12 and 16 entries a thread."""
    _token_teacher_forced(reading, 8, 2, D, 1, topk=40, splits=5, S0=S0, steps=2)


def _token_teacher_forced(reading, H_q, H_kv, D, eos, topk=40, splits=5, S0=300, steps=6):
    say(f"[gpu] h2o small, teacher forced, {reading} H_q {H_q} H_kv {H_kv} D {D} eos {eos} "
        f"top-{topk} over {splits} splits, {S0} tokens")
    B = 3
    wl = W.h2o_token(seed=40, steps=steps, prompt=S0, B=B)
    wl.H_q, wl.H_kv, wl.D = H_q, H_kv, D
    wl.bos, wl.eos, wl.topk_pages, wl.num_splits = 4, eos, topk, splits
    wl.seq_lens = np.array([S0, S0 - 37, 11], dtype=np.int32)
    cache = dev(W.make_cache(wl))
    bt = dev(wl.block_table)
    d = SparseDecoder(B, H_q, H_kv, D, wl.num_blocks, 1, wl.bt_ld,
                      topk_pages=wl.topk_pages, bos=wl.bos, eos=wl.eos,
                      scale=wl.softmax_scale, num_splits=wl.num_splits,
                      token_level=True, h2o_softmax=reading)
    d.hh.copy_(W.make_hh(wl).cuda())
    for step in range(wl.steps):
        sl_np = wl.seq_lens_at(step)
        sl = dev(sl_np)
        q_cpu = W.make_queries(wl, step)
        q = dev(q_cpu)
        kn, vn = W.make_new_kv(wl, step)
        pre_cache, pre_hh = bits(cache).copy(), bits(d.hh).copy()
        pre_cache_dev, pre_append_hh_dev = cache.clone(), d.hh.clone()
        poison(d)
        d.append(cache, bt, sl, dev(kn), dev(vn))
        torch.cuda.synchronize()
        oracle.append(pre_cache, wl.block_table, sl_np, bits(kn), bits(vn), pre_hh)
        assert np.array_equal(bits(cache), pre_cache)
        assert np.array_equal(bits(d.hh), pre_hh)
        pre_hh_dev = d.hh.clone()
        d.accumulate(q, cache, bt, sl)
        d.select(sl, bt)
        d.attend(q, cache, bt, sl)
        d.merge()
        torch.cuda.synchronize()
        hh_ref = pre_hh.copy()
        qd = q_cpu.double().numpy()
        ref_scores = oracle.h2o_step(qd, pre_cache, wl.block_table, sl_np, hh_ref,
                                     wl.bos, wl.eos, wl.softmax_scale, wl.decay,
                                     per_head=(reading == "per_head"))
        gh = bits(d.hh)
        apart = bf16_bits_apart(gh, hh_ref)
        assert apart.max() <= 1, f"step {step}: hh more than one ulp off"
        gs = d.scores.cpu().numpy()
        for b in range(B):
            n = int(sl_np[b])
            slots = wl.block_table[b, :n]
            np.testing.assert_array_equal(gs[b, :, :n].T, oracle.bf16_decode(gh[slots]))
        sel_idx = d.sel_idx.cpu().numpy().reshape(-1, d.k_cap)
        sel_cnt = d.sel_cnt.cpu().numpy().reshape(-1)
        Nrows = np.repeat(sl_np, H_kv)
        check_selection_exact(sel_idx, sel_cnt, gs.reshape(-1, wl.bt_ld), Nrows,
                              wl.topk_pages, 0.0, wl.bos, wl.eos)
        rows = selection_rows(sel_idx, sel_cnt)
        check_selection_vs_oracle(rows, ref_scores.reshape(-1, wl.bt_ld), Nrows,
                                  wl.topk_pages, 0.0, wl.bos, wl.eos, token_level=True)
        per = per_head_rows(rows, B, H_q, H_kv)
        check_partials(d.o_part.cpu().numpy(), d.lse_part.cpu().numpy(), qd,
                       bits(cache), wl.block_table, sl_np, per, H_q // H_kv,
                       wl.softmax_scale, d.k_cap)
        check_attention(d.out.cpu().numpy(), d.lse.cpu().numpy(), qd, bits(cache),
                        wl.block_table, sl_np, per, H_q // H_kv, wl.softmax_scale)
        if d.token_fused:
            check_token_fused_matches(d, q, cache, bt, sl, pre_hh_dev)
            # and with the append inside the first launch
            check_token_fused_matches(d, q, cache, bt, sl, pre_append_hh_dev, dev(kn),
                                      dev(vn), pre_cache_dev)
        say(f"  step {step}: hh ulps off max {apart.max()}, "
            f"{int((apart > 0).sum())} of {apart.size}")


def test_invalid_arguments_raise_before_launch():
    say("[gpu] argument errors")
    q = torch.zeros((1, 4, 96), device="cuda")
    with pytest.raises(skv.SparseKVError) as e:
        skv.lse_merge(torch.zeros((1, 2, 96), device="cuda"),
                      torch.zeros((1, 2), device="cuda"), torch.zeros((1, 96), device="cuda"))
    assert e.value.code == -22
    with pytest.raises(TypeError):
        skv.page_score(q.double(), None, None, None, None, None, 16, 1, 1, None)


@pytest.mark.parametrize("mode", ["one_launch", "select_decode", "separate", "group", "gauss",
                                  "entmax", "gauss_merged", "entmax_merged"])
def test_graph_replays_match_eager(mode):
    """bench.py times HIP-graph replays of the step: each replay, with eager
    work and new queries in between, must give the eager step's bits."""
    say(f"[gpu] graph replay vs eager, {mode}")
    wl = W.small_case(seed=150, B=3, H_q=8, H_kv=2, D=128, P=16, max_pages=40,
                      topk_pages=6, num_splits=4, min_len=40)
    kw = {}
    if mode == "separate":
        kw["fuse_merge"] = False
    elif mode == "group":
        kw["group_select"] = True
    elif mode.startswith("gauss"):
        kw["selection"] = "gauss"
    elif mode.startswith("entmax"):
        kw["attention"] = "entmax15"
    d = SparseDecoder.for_workload(wl, device="cuda", **kw)
    # the one-launch 1.5-entmax decode, also for this small batch
    d.entmax_fused = mode.endswith("_merged")
    if mode == "select_decode":
        # the form batches past the one-launch row limit take: page_score,
        # then selection, decode and merge in one launch
        assert d.score_in_decode and d.select_in_decode
        d.score_in_decode = False
    cache = dev(W.make_cache(wl))
    bt, sl = dev(wl.block_table), dev(wl.seq_lens)
    q = dev(W.make_queries(wl, 0))
    d.rebuild_stats(cache, bt, sl)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        d.step(q, cache, bt, sl)
    torch.cuda.synchronize()
    for step in range(3):
        q.copy_(dev(W.make_queries(wl, step + 1)))
        scratch = torch.randn(1 << 20, device="cuda").sum()     # eager work between
        g.replay()
        torch.cuda.synchronize()
        got = (d.out.clone(), d.lse.clone())
        d.out.fill_(float("nan"))
        d.step(q, cache, bt, sl)
        torch.cuda.synchronize()
        assert torch.isfinite(scratch)
        assert torch.equal(got[0], d.out), f"replay {step}: out differs from eager"
        assert torch.equal(got[1], d.lse), f"replay {step}: lse differs from eager"


@pytest.mark.parametrize("reading", ["group_mean", "per_head"])
def test_token_fused_append_past_the_table_writes_nothing(reading):
    """h2o_select_decode given k_new / v_new: a request whose new token lies
    past its block-table row (S - 1 >= bt_ld) appends nothing, as
    pagestats_update does; the others append. The step equals
    pagestats_update followed by the call without k_new, bit for bit."""
    say(f"[gpu] token-level append inside the first launch, row past the table, {reading}")
    S0, B = 300, 3
    wl = W.h2o_token(seed=43, steps=2, prompt=S0, B=B)
    wl.H_q, wl.H_kv, wl.D = 8, 2, 128
    wl.bos, wl.eos, wl.topk_pages, wl.num_splits = 2, 0, 40, 4
    wl.seq_lens = np.array([S0, wl.bt_ld + 1, 11], dtype=np.int32)
    d = SparseDecoder(B, wl.H_q, wl.H_kv, wl.D, wl.num_blocks, 1, wl.bt_ld,
                      topk_pages=wl.topk_pages, bos=wl.bos, eos=wl.eos,
                      scale=wl.softmax_scale, num_splits=wl.num_splits,
                      token_level=True, h2o_softmax=reading)
    assert d.token_fused
    hh0 = W.make_hh(wl).cuda()
    cache0 = dev(W.make_cache(wl))
    bt, sl = dev(wl.block_table), dev(wl.seq_lens)
    q = dev(W.make_queries(wl, 0))
    kn, vn = (dev(t) for t in W.make_new_kv(wl, 0))
    cache_a = cache0.clone()
    d.hh.copy_(hh0)
    d.append(cache_a, bt, sl, kn, vn)
    d.accumulate_select_attend(q, cache_a, bt, sl)
    d.merge()
    torch.cuda.synchronize()
    ref = (d.hh.clone(), d.out.clone(), d.lse.clone())
    cache_b = cache0.clone()
    d.hh.copy_(hh0)
    d.out.fill_(float("nan"))
    d.accumulate_select_attend(q, cache_b, bt, sl, kn, vn)
    d.merge()
    torch.cuda.synchronize()
    assert torch.equal(cache_a, cache_b), "appended cache differs"
    for name, a, b in zip(("hh", "out", "lse"), ref, (d.hh, d.out, d.lse)):
        assert torch.equal(a, b), f"{name} differs from append + separate call"
    # only requests 0 and 2 wrote a row
    written = [int(wl.block_table[b, int(wl.seq_lens[b]) - 1]) for b in (0, 2)]
    keep = torch.ones(cache0.shape[1], dtype=torch.bool, device="cuda")
    keep[written] = False
    assert torch.equal(cache_b[:, keep], cache0[:, keep]), "a row was written past the table"
    assert not torch.equal(cache_b[:, written], cache0[:, written])


@pytest.mark.parametrize("reading", ["group_mean", "per_head"])
def test_token_level_graph_replays_match_eager(reading):
    """The token-level step (accumulate, select, attend, merge) captured in a
    graph: from the same hh, every replay must give the eager step's output,
    lse and updated hh, bit for bit."""
    say(f"[gpu] token-level graph replay vs eager, {reading}")
    S0, B = 300, 3
    wl = W.h2o_token(seed=41, steps=4, prompt=S0, B=B)
    wl.H_q, wl.H_kv, wl.D = 8, 2, 128
    wl.topk_pages, wl.num_splits = 40, 4
    wl.seq_lens = np.array([S0, S0 - 37, 11], dtype=np.int32)
    d = SparseDecoder(B, wl.H_q, wl.H_kv, wl.D, wl.num_blocks, 1, wl.bt_ld,
                      topk_pages=wl.topk_pages, bos=wl.bos, eos=wl.eos,
                      scale=wl.softmax_scale, num_splits=wl.num_splits,
                      token_level=True, h2o_softmax=reading)
    d.hh.copy_(W.make_hh(wl).cuda())
    cache = dev(W.make_cache(wl))
    bt, sl = dev(wl.block_table), dev(wl.seq_lens)
    q = dev(W.make_queries(wl, 0))
    torch.cuda.synchronize()
    hh0 = d.hh.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        d.step(q, cache, bt, sl)
    torch.cuda.synchronize()
    for step in range(3):
        q.copy_(dev(W.make_queries(wl, step + 1)))
        d.hh.copy_(hh0)
        scratch = torch.randn(1 << 20, device="cuda").sum()     # eager work between
        g.replay()
        torch.cuda.synchronize()
        got = (d.out.clone(), d.lse.clone(), d.hh.clone())
        d.hh.copy_(hh0)
        d.out.fill_(float("nan"))
        d.step(q, cache, bt, sl)
        torch.cuda.synchronize()
        assert torch.isfinite(scratch)
        assert torch.equal(got[0], d.out), f"replay {step}: out differs from eager"
        assert torch.equal(got[1], d.lse), f"replay {step}: lse differs from eager"
        assert torch.equal(got[2], d.hh), f"replay {step}: hh differs from eager"
        hh0 = d.hh.clone()


def test_gauss_append_refreshes_tail_variance():
    """Gaussian-aware decoder over appends: pagestats_update's tail refresh
    and page_var_update(tail_only) keep every page's mean and variance equal
    to the oracle's statistics of the grown cache (pages crossing a boundary
    included)."""
    say("[gpu] Gaussian-aware statistics over 20 appends")
    wl = W.high_batch(seed=160, steps=20, B=3, num_blocks=120, smin=17, smax=150)
    d = SparseDecoder.for_workload(wl, device="cuda", selection="gauss")
    cache = dev(W.make_cache(wl))
    bt = dev(wl.block_table)
    d.k_var.fill_(float("nan"))
    d.rebuild_stats(cache, bt, dev(wl.seq_lens))
    for step in range(wl.steps):
        kn, vn = W.make_new_kv(wl, step)
        d.append(cache, bt, dev(wl.seq_lens_at(step)), dev(kn), dev(vn))
    torch.cuda.synchronize()
    sl = wl.seq_lens_at(wl.steps - 1)
    cb = bits(cache)
    used = np.unique(np.concatenate(
        [wl.block_table[b, :(int(sl[b]) + wl.P - 1) // wl.P] for b in range(wl.B)]))
    check_stats(bits(d.k_min), bits(d.k_max), d.k_mean.cpu().numpy(), cb, wl.block_table,
                sl, wl.P, used)
    ov = oracle.page_var(cb, wl.block_table, sl, wl.P)[used]
    gv = d.k_var.cpu().numpy()[used].astype(np.float64)
    assert np.all(np.abs(gv - ov) <= 1e-5 * ov + 1e-6), \
        f"variance after appends off by {np.abs(gv - ov).max()}"


@pytest.mark.parametrize("mode", ["one_launch", "separate", "group", "entmax", "gauss",
                                  "token_group_mean", "token_per_head"])
def test_empty_batch_is_a_no_op(mode):
    """B = 0 through every entry point of a step: each call returns OK without
    touching memory (empty tensors carry NULL data pointers), and the cache
    is left as it was."""
    say(f"[gpu] empty batch, {mode}")
    token = mode.startswith("token")
    P, H_q, H_kv, D, NB, ld = (1 if token else 16), 8, 2, 128, 64, 32
    kw = dict(topk_pages=4, num_splits=2, token_level=token)
    if mode == "separate":
        kw["fuse_merge"] = False
    if mode == "group":
        kw["group_select"] = True
    if mode == "entmax":
        kw["attention"] = "entmax15"
    if mode == "gauss":
        kw["selection"] = "gauss"
    if token:
        kw["h2o_softmax"] = "per_head" if mode == "token_per_head" else "group_mean"
    d = SparseDecoder(0, H_q, H_kv, D, NB, P, ld, **kw)
    g = torch.Generator(device="cuda").manual_seed(5)
    cache = torch.randn((2, NB, P, H_kv, D), generator=g, device="cuda").to(torch.bfloat16)
    before = cache.clone()
    q = torch.empty((0, H_q, D), device="cuda")
    bt = torch.empty((0, ld), dtype=torch.int32, device="cuda")
    sl = torch.empty((0,), dtype=torch.int32, device="cuda")
    kn = torch.empty((0, H_kv, D), dtype=torch.bfloat16, device="cuda")
    if not token:
        d.rebuild_stats(cache, bt, sl)
    if token:
        d.append(cache, bt, sl, kn, kn.clone())
        d.accumulate(q, cache, bt, sl)
        d.select(sl, bt)
        d.attend(q, cache, bt, sl)
        d.merge()
        out = d.out
    else:
        out, _ = d.step(q, cache, bt, sl, kn, kn.clone())
    torch.cuda.synchronize()
    assert out.shape[0] == 0
    assert torch.equal(cache, before)
