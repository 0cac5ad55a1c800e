"""Helpers of the GPU-vs-oracle parity tests.

Parity rules (stated once here, used by every GPU test):
  * k_min / k_max: bit-exact.  k_mean: within the recursive-summation bound
    n * 2^-24 * sum_t |k_t| / n of an fp32 sum of n bf16 values, plus 1e-7.
  * page scores, kernel in isolation (oracle fed the GPU's own statistics):
    within 2 * D * 2^-24 * sum_d |term_d| (fp32 dot-product bound).
  * selection, kernel in isolation (oracle fed the GPU's fp32 scores):
    identical index lists.  End to end (oracle from the cache in float64):
    identical, except rows whose k-th and (k+1)-th oracle scores differ by
    less than 1e-5 relative (page level) or by at most one bf16 ulp of the
    k-th value (token level); such rows must still hold every candidate
    ranked clearly above the boundary and none ranked clearly below it.
  * attention (oracle over the GPU's own selection): out within 2e-3
    absolute, lse within 1e-4 absolute; split partials likewise.
  * hh (token level, oracle fed the GPU's pre-step hh): at most one bf16 ulp
    apart (bit patterns of non-negative values differ by <= 1).
Outputs are poisoned (NaN / -7) before each GPU call so unwritten elements
fail.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from sparse_kv_cache_amd import workloads as W

OUT_ATOL = 2e-3
LSE_ATOL = 1e-4
PAGE_GAP_REL = 1e-5


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a)) if isinstance(a, np.ndarray) else a
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda().contiguous()


def poison(dec):
    for t in (dec.scores, dec.o_part, dec.lse_part, dec.o_blk, dec.lse_blk, dec.out,
              dec.lse):
        if t is not None:
            t.fill_(float("nan"))
    dec.sel_idx.fill_(-7)
    dec.sel_cnt.fill_(-7)
    dec.sel_blk.fill_(-7)


def group_forms_fold_alike(dec):
    """Whether the group decode's two forms fold a split's rows in the same
    order: the standalone kernel deals a split's 16-row groups to 4 waves, the
    in-block-selection form (and the token-level step's) to 8, each wave
    folding groups w, w + waves, ... before the waves merge; with at most 4
    groups per split both forms fold the same groups in the same order."""
    epg = max(1, 16 // dec.P)                       # entries per 16-row group
    per_split = -(-dec.k_cap // dec.decode_splits)
    return -(-per_split // epg) <= 4


def check_close_partials(o_ref, l_ref, o, l, what):
    """The same attention states folded in another order: the online softmax
    rescales by other running maxima and splits other probabilities into
    bf16 hi + lo halves (about 16 significant bits), so the values agree to
    about 1e-5 of the row's magnitude; empty entries match exactly."""
    a, b = o_ref.reshape(-1, o_ref.shape[-1]), o.reshape(-1, o.shape[-1])
    assert torch.isfinite(b).all(), f"{what}: not finite"
    scale = a.abs().amax(dim=1, keepdim=True).clamp_min(1.0)
    err = ((a - b).abs() / scale).max().item()
    assert err <= 1e-4, f"{what}: output differs by {err} of the row's magnitude"
    la, lb = l_ref.reshape(-1), l.reshape(-1)
    fin = torch.isfinite(la)
    assert torch.equal(torch.isfinite(lb), fin), f"{what}: lse finiteness differs"
    assert torch.equal(la[~fin], lb[~fin]), f"{what}: empty entries' lse differs"
    if fin.any():
        e = ((la[fin] - lb[fin]).abs() / la[fin].abs().clamp_min(1.0)).max().item()
        assert e <= 1e-5, f"{what}: lse differs by {e}"


def check_group_select_decode_matches(dec, q, cache, bt, sl):
    """With a selection shared by each kv head's group, the one-launch form
    (selection inside the group decode) must give exactly the selection and
    block ids the separate page_topk + sparse_paged_decode (+ lse_merge)
    launches just wrote into dec's buffers, and their partials and merged
    output: bit for bit where both forms fold a split's rows alike
    (group_forms_fold_alike), else to within that refolding's rounding."""
    assert dec.select_in_group_decode
    ref = [t.clone() for t in (dec.sel_idx, dec.sel_cnt, dec.sel_blk, dec.o_part,
                               dec.lse_part, dec.out, dec.lse)]
    for t in (dec.o_part, dec.lse_part, dec.out, dec.lse):
        t.fill_(float("nan"))
    for t in (dec.sel_idx, dec.sel_cnt, dec.sel_blk):
        t.fill_(-7)
    keep = dec.keep_selection
    dec.keep_selection = True
    dec.select_attend_group(q, cache, bt, sl)
    dec.merge()
    dec.keep_selection = keep
    torch.cuda.synchronize()
    exact = group_forms_fold_alike(dec)
    names = ("sel_idx", "sel_cnt", "sel_blk", "o_part", "lse_part", "out", "lse")
    got = (dec.sel_idx, dec.sel_cnt, dec.sel_blk, dec.o_part, dec.lse_part, dec.out, dec.lse)
    for name, a, b in zip(names, ref, got):
        if exact or name.startswith("sel"):
            assert torch.equal(a, b), f"select-in-decode {name} differs from separate launches"
    if not exact:
        check_close_partials(ref[3], ref[4], dec.o_part, dec.lse_part, "select-in-decode partials")
        check_close_partials(ref[5], ref[6], dec.out, dec.lse, "select-in-decode output")


def check_split_select_decode_matches(dec, q, cache, bt, sl):
    """With one selection per query head and more splits than a block merges,
    the one-launch form (selection inside the split decode) must give exactly
    the bits the separate page_topk + sparse_paged_decode + lse_merge launches
    just wrote into dec's buffers: selection, block ids, partials, merged
    output."""
    assert dec.select_in_split_decode
    ref = [t.clone() for t in (dec.sel_idx, dec.sel_cnt, dec.sel_blk, dec.o_part,
                               dec.lse_part, dec.out, dec.lse)]
    for t in (dec.o_part, dec.lse_part, dec.out, dec.lse):
        t.fill_(float("nan"))
    for t in (dec.sel_idx, dec.sel_cnt, dec.sel_blk):
        t.fill_(-7)
    keep = dec.keep_selection
    dec.keep_selection = True
    dec.select_attend_split(q, cache, bt, sl, blocks=False)
    dec.merge()
    dec.keep_selection = keep
    torch.cuda.synchronize()
    names = ("sel_idx", "sel_cnt", "sel_blk", "o_part", "lse_part", "out", "lse")
    for name, a, b in zip(names, ref, (dec.sel_idx, dec.sel_cnt, dec.sel_blk, dec.o_part,
                                       dec.lse_part, dec.out, dec.lse)):
        assert torch.equal(a, b), f"select-in-split-decode {name} differs from separate launches"
    # the block-merged form: the same selection; each block's partial the
    # merge of its splits' partials; the merged output the same up to the
    # order of the fold
    for t in (dec.o_blk, dec.lse_blk, dec.out, dec.lse):
        t.fill_(float("nan"))
    for t in (dec.sel_idx, dec.sel_cnt, dec.sel_blk):
        t.fill_(-7)
    dec.keep_selection = True
    dec.select_attend_split(q, cache, bt, sl, blocks=True)
    dec.merge()
    dec.keep_selection = keep
    torch.cuda.synchronize()
    for name, a, b in zip(names[:3], ref, (dec.sel_idx, dec.sel_cnt, dec.sel_blk)):
        assert torch.equal(a, b), f"block-merged split decode: {name} differs"
    check_block_partials(ref[3].cpu().numpy(), ref[4].cpu().numpy(),
                         dec.o_blk.cpu().numpy(), dec.lse_blk.cpu().numpy(),
                         split_block_waves(dec.P))
    check_close_partials(ref[5], ref[6], dec.out, dec.lse, "block-merged split decode output")


def split_block_waves(P):
    """Splits one block of the block-merged split decode holds at page size P."""
    import sparse_kv_cache_amd as skv
    return 4096 // skv.sparse_select_decode_split_blocks_count(4096, P)


def split_block_chunk(dec):
    """Selection entries one block partial of dec's block-merged split decode
    covers: its splits' chunks of ceil(k_cap / num_splits) entries each."""
    return split_block_waves(dec.P) * -(-dec.k_cap // dec.num_splits)


def check_decoder_partials(dec, q, cache_bits, bt, sl, rows_sel, G, scale, slopes=None,
                           rows=None, heads=None):
    """The partials dec's last decode wrote, against the oracle: one per
    split, and with the split select-decode also the block-merged ones when
    that form ran last.  rows / heads restrict the check (q, rows_sel, bt, sl
    are then already the restricted ones)."""
    def pick(t):
        a = t.cpu().numpy()
        if rows is not None:
            a = a[rows]
        return a if heads is None else a[:, heads]
    o, lse = dec.partials
    if o is not dec.o_part:
        check_partials(pick(o), pick(lse), q, cache_bits, bt, sl, rows_sel, G, scale,
                       dec.k_cap, slopes=slopes, chunk=split_block_chunk(dec))
    else:
        check_partials(pick(o), pick(lse), q, cache_bits, bt, sl, rows_sel, G, scale,
                       dec.k_cap, slopes=slopes)


def check_block_partials(o_part, lse_part, o_blk, lse_blk, wb):
    """Block j of a row holds the oracle's LSE merge of the row's split
    partials [j*wb, (j+1)*wb) (the kernel folds them in fp32 from the
    unnormalised states: about 1e-6 of the row's magnitude apart); a block of
    empty splits holds zeros and -inf."""
    B, H, ns, D = o_part.shape
    nb = o_blk.shape[2]
    assert nb == -(-ns // wb), f"{nb} block partials for {ns} splits of {wb}"
    for b in range(B):
        for i in range(H):
            for j in range(nb):
                lo, hi = j * wb, min(ns, (j + 1) * wb)
                o, lse = oracle.lse_merge(o_part[b, i, lo:hi], lse_part[b, i, lo:hi])
                if np.isinf(lse):
                    assert np.isinf(lse_blk[b, i, j]) and lse_blk[b, i, j] < 0, (b, i, j)
                    assert np.all(o_blk[b, i, j] == 0), (b, i, j)
                    continue
                g = o_blk[b, i, j].astype(np.float64)
                e = np.abs(g - o).max() / max(1.0, np.abs(o).max())
                assert e <= 1e-5, f"block partial ({b},{i},{j}) err {e}"
                assert abs(float(lse_blk[b, i, j]) - lse) <= lse_tol(lse), \
                    f"block lse ({b},{i},{j}) {lse_blk[b, i, j]} vs {lse}"


def check_token_fused_matches(dec, q, cache, bt, sl, pre_hh, k_new=None, v_new=None,
                              pre_cache=None):
    """Token level: after the separate launches (h2o_accumulate or its per-head
    form, page_topk_blk, sparse_paged_decode, lse_merge) have filled dec's
    buffers, rerun the step from the same accumulator (pre_hh, the device
    tensor's bytes before the step) through h2o_select_decode and require the
    same bits: accumulator, score rows, selection, partials, merged output.
    With k_new / v_new the rerun also does the append (pagestats_update's
    part of the step): pre_hh and pre_cache are then the tensors before the
    append, and the cache must come out equal as well."""
    assert dec.token_fused
    names = ("hh", "scores", "sel_idx", "sel_cnt", "sel_blk", "o_part", "lse_part", "out",
             "lse")
    ref = {n: getattr(dec, n).clone() for n in names}
    ref_cache = None
    if k_new is not None:
        ref_cache = cache.clone()
        cache.copy_(pre_cache)
    dec.hh.copy_(pre_hh)
    for n in ("scores", "o_part", "lse_part", "out", "lse"):
        getattr(dec, n).fill_(float("nan"))
    for n in ("sel_idx", "sel_cnt", "sel_blk"):
        getattr(dec, n).fill_(-7)
    keep = (dec.keep_selection, dec.keep_scores)
    dec.keep_selection = dec.keep_scores = True
    dec.accumulate_select_attend(q, cache, bt, sl, k_new, v_new)
    dec.merge()
    dec.keep_selection, dec.keep_scores = keep
    torch.cuda.synchronize()
    if ref_cache is not None:
        assert torch.equal(ref_cache, cache), "fused token step: the appended cache differs"
    N = sl.cpu().numpy()
    exact = group_forms_fold_alike(dec)
    for n in names:
        a, b = ref[n], getattr(dec, n)
        if n == "scores":   # entries past each request's length are not written
            for r in range(a.shape[0]):
                assert torch.equal(a[r, :, :int(N[r])], b[r, :, :int(N[r])]), \
                    f"fused token step: scores of request {r} differ"
            continue
        if exact or n not in ("o_part", "lse_part", "out", "lse"):
            assert torch.equal(a, b), f"fused token step: {n} differs from separate launches"
    if not exact:
        check_close_partials(ref["o_part"], ref["lse_part"], dec.o_part, dec.lse_part,
                             "fused token step partials")
        check_close_partials(ref["out"], ref["lse"], dec.out, dec.lse, "fused token step output")


def bits(t):
    return W.bf16_bits(t)


# ------------------------------------------------------------- sub-batch

def sub_batch(wl, cache_gpu, rows, seq_lens=None, extra=()):
    """Host copy of the blocks used by requests ``rows`` with a remapped
    block table.  ``extra`` are GPU tensors indexed by block on dim 0 (stats)
    gathered the same way.  Returns (cache_bits, bt, seq_lens, blocks, extras)."""
    sl = wl.seq_lens if seq_lens is None else np.asarray(seq_lens)
    rows = list(rows)
    N = (sl[rows].astype(np.int64) + wl.P - 1) // wl.P
    blocks = np.unique(np.concatenate([wl.block_table[b, :n] for b, n in zip(rows, N)]))
    idx = torch.from_numpy(blocks.astype(np.int64)).cuda()
    cache = bits(cache_gpu.index_select(1, idx))
    bt = np.zeros((len(rows), wl.bt_ld), dtype=np.int32)
    for r, (b, n) in enumerate(zip(rows, N)):
        bt[r, :n] = np.searchsorted(blocks, wl.block_table[b, :n])
    ex = [t.index_select(0, idx).cpu() for t in extra]
    return cache, bt, sl[rows].astype(np.int32), blocks, ex


# ----------------------------------------------------------------- checks

def check_stats(gpu_min, gpu_max, gpu_mean, cache_bits, bt, sl, P, blocks_used):
    """gpu_* indexed like the oracle's output (physical blocks of cache_bits)."""
    mn, mx, me = oracle.page_stats(cache_bits, bt, sl, P)
    gmin = oracle.bf16_decode(gpu_min[blocks_used])
    gmax = oracle.bf16_decode(gpu_max[blocks_used])
    assert np.array_equal(gmin, mn[blocks_used]), "k_min differs"
    assert np.array_equal(gmax, mx[blocks_used]), "k_max differs"
    # bound: n * u * sum|k| / n = u * sum|k|; sum|k| <= n * max(|min|, |max|)
    n = np.zeros(len(blocks_used))
    for b in range(bt.shape[0]):
        Nb = (int(sl[b]) + P - 1) // P
        for p in range(Nb):
            j = np.searchsorted(blocks_used, bt[b, p])
            n[j] = min(P, int(sl[b]) - p * P)
    amax = np.maximum(np.abs(mn[blocks_used]), np.abs(mx[blocks_used]))
    tol = (2.0 ** -24) * n[:, None, None] * amax + 1e-7
    err = np.abs(gpu_mean[blocks_used].astype(np.float64) - me[blocks_used])
    assert np.all(err <= tol), f"k_mean error {err.max()} over bound"
    return mn, mx, me


def score_abs_terms(q, mn, mx, me, bt, sl, P, w_avg, w_peak):
    M = np.maximum(np.abs(mn), np.abs(mx))
    return oracle.page_score(np.abs(q), -M, M, np.abs(me), bt, sl, P,
                             abs(w_avg), abs(w_peak))


def check_scores(gpu_scores, q, stats_d, bt, sl, P, w_avg, w_peak):
    """gpu_scores [B, H_q, ld] fp32 vs the oracle fed the same statistics."""
    mn, mx, me = stats_d
    ref = oracle.page_score(q, mn, mx, me, bt, sl, P, w_avg, w_peak,
                            ld=gpu_scores.shape[2])
    terms = score_abs_terms(q, mn, mx, me, bt, sl, P, w_avg, w_peak)
    D = q.shape[2]
    valid = ~np.isnan(ref)
    g = gpu_scores.astype(np.float64)
    assert not np.any(np.isnan(g[valid])), "unwritten score"
    err = np.abs(g[valid] - ref[valid])
    tol = 2 * D * 2.0 ** -24 * terms[valid] + 1e-6
    assert np.all(err <= tol), f"score error {err.max()} over bound"
    return ref


def check_scores_group(gpu_scores, q, stats_d, bt, sl, P, w_avg, w_peak):
    """gpu_scores [B, H_kv, ld] (group means) vs the oracle fed the same
    statistics; the bound is the per-head one averaged over the group plus
    the rounding of the group means of q and |q|."""
    mn, mx, me = stats_d
    ref = oracle.page_score_group(q, mn, mx, me, bt, sl, P, w_avg, w_peak,
                                  ld=gpu_scores.shape[2])
    B, H_q, D = q.shape
    H_kv = gpu_scores.shape[1]
    G = H_q // H_kv
    terms = score_abs_terms(q, mn, mx, me, bt, sl, P, w_avg, w_peak)
    terms = terms.reshape(B, H_kv, G, -1).mean(axis=2)
    valid = ~np.isnan(ref)
    g = gpu_scores.astype(np.float64)
    assert not np.any(np.isnan(g[valid])), "unwritten score"
    err = np.abs(g[valid] - ref[valid])
    tol = (2 * D + 2 * G) * 2.0 ** -24 * terms[valid] + 1e-6
    assert np.all(err <= tol), f"group score error {err.max()} over bound"
    return ref


def check_scores_alibi(gpu_scores, q, stats_d, bt, sl, P, w_avg, w_peak, alibi,
                       aggregate):
    """ALiBi-aware scores ([B, H_q, ld], or group means [B, H_kv, ld]) vs the
    oracle fed the same statistics; alibi [H_q] in score units.  The bound adds
    the fp32 rounding of the bias terms (|slope| * distance)."""
    mn, mx, me = stats_d
    ref = oracle.page_score_alibi(q, mn, mx, me, bt, sl, P, w_avg, w_peak, alibi,
                                  aggregate, ld=gpu_scores.shape[2])
    B, H_q, D = q.shape
    terms = score_abs_terms(q, mn, mx, me, bt, sl, P, w_avg, w_peak)
    bias = ((abs(w_avg) + abs(w_peak)) * np.abs(np.asarray(alibi))[None, :, None]
            * np.asarray(sl, dtype=np.float64)[:, None, None])
    tot = terms + bias
    if aggregate:
        H_kv = gpu_scores.shape[1]
        tot = tot.reshape(B, H_kv, H_q // H_kv, -1).mean(axis=2)
        G = H_q // H_kv
    else:
        G = 1
    valid = ~np.isnan(ref)
    g = gpu_scores.astype(np.float64)
    assert not np.any(np.isnan(g[valid])), "unwritten score"
    err = np.abs(g[valid] - ref[valid])
    tol = (2 * D + 2 * G + 8) * 2.0 ** -24 * tot[valid] + 1e-6
    assert np.all(err <= tol), f"ALiBi score error {err.max()} over bound"
    return ref


def selection_rows(sel_idx, sel_cnt):
    out = []
    for r in range(sel_cnt.shape[0]):
        c = int(sel_cnt[r])
        out.append(sel_idx[r, :c].tolist())
    return out


def check_padding(sel_idx, sel_cnt):
    for r in range(sel_cnt.shape[0]):
        c = int(sel_cnt[r])
        assert c >= 0
        assert np.all(sel_idx[r, c:] == -1), "padding not -1"


def check_selection_exact(gpu_idx, gpu_cnt, scores_rows, N_rows, topk, frac,
                          bos, eos):
    """GPU selection equals the oracle's on the same (GPU) scores."""
    check_padding(gpu_idx, gpu_cnt)
    for r, (s, n) in enumerate(zip(scores_rows, N_rows)):
        want = oracle.select(s[:n].astype(np.float64), topk, frac, bos, eos).tolist()
        got = gpu_idx[r, :int(gpu_cnt[r])].tolist()
        assert got == want, f"row {r}: selection differs from oracle on GPU scores"


def check_sel_blk(sel_blk, sel_idx, block_table):
    """sel_blk [B, H_sel, k_cap] holds block_table[b, p] of each selected p."""
    B = sel_idx.shape[0]
    for b in range(B):
        idx = sel_idx[b]
        want = np.where(idx >= 0, block_table[b][np.clip(idx, 0, None)], -1)
        assert np.array_equal(sel_blk[b], want), f"request {b}: sel_blk differs"


def _window(N, bos, eos):
    lo = min(bos, N)
    hi = max(N - eos, 0)
    return lo, max(hi, lo)


def check_selection_vs_oracle(gpu_rows, oracle_scores_rows, N_rows, topk, frac,
                              bos, eos, token_level=False):
    """End-to-end rule with the near-tie exemption.  Returns #exempt rows."""
    exempt = 0
    for r, (got, s, n) in enumerate(zip(gpu_rows, oracle_scores_rows, N_rows)):
        s = s[:n]
        want = oracle.select(s, topk, frac, bos, eos).tolist()
        if got == want:
            continue
        lo, hi = _window(n, bos, eos)
        k = oracle.budget(n, topk, frac)
        m = k - (n - (hi - lo))
        cand = sorted(range(lo, hi), key=lambda p: (-s[p], p))
        assert 0 < m < len(cand), f"row {r}: mismatch with no boundary"
        a, b = s[cand[m - 1]], s[cand[m]]
        if token_level:
            bound_ok = abs(a - b) <= 2.0 ** (np.floor(np.log2(max(abs(a), 2.0 ** -133))) - 7)
        else:
            den = max(abs(a), abs(b))
            bound_ok = den == 0 or abs(a - b) / den < PAGE_GAP_REL
        assert bound_ok, f"row {r}: selection differs away from a near tie"
        assert len(got) == len(want), f"row {r}: wrong count"
        gs = set(got)
        band = (2.0 ** (np.floor(np.log2(max(abs(a), 2.0 ** -133))) - 7) if token_level
                else PAGE_GAP_REL * max(abs(a), abs(b)))
        for p in range(n):
            if p < lo or p >= hi:
                assert p in gs, f"row {r}: reserved page {p} missing"
            elif s[p] > a + band:
                assert p in gs, f"row {r}: page {p} clearly above the boundary missing"
            elif s[p] < b - band:
                assert p not in gs, f"row {r}: page {p} clearly below the boundary taken"
        exempt += 1
    return exempt


def _attend(q_row, cache_bits, h, bt_row, S, pages, scale, slopes, i):
    if slopes is None:
        return oracle.attend(q_row, cache_bits, h, bt_row, S, pages, scale)
    return oracle.attend_alibi(q_row, cache_bits, h, bt_row, S, pages, scale,
                               float(slopes[i]))


def lse_tol(lse):
    """1e-4 absolute, plus 8 fp32 ulps of |lse|: an ALiBi bias far from the
    query puts |lse| near 1e5, where one fp32 ulp is about 0.01."""
    return LSE_ATOL + 8.0 * 2.0 ** -23 * abs(lse)


def check_attention(gpu_out, gpu_lse, q, cache_bits, bt, sl, rows_sel, G, scale,
                    slopes=None):
    """gpu_out [B, H_q, D], gpu_lse [B, H_q]; rows_sel[b][i] = pages;
    slopes [H_q] = ALiBi slopes (or None)."""
    B, H_q, D = q.shape
    worst = 0.0
    for b in range(B):
        for i in range(H_q):
            o, lse = _attend(q[b, i], cache_bits, i // G, bt[b], sl[b],
                             rows_sel[b][i], scale, slopes, i)
            go = gpu_out[b, i].astype(np.float64)
            assert not np.any(np.isnan(go)), f"NaN output at ({b},{i})"
            e = np.abs(go - o).max()
            worst = max(worst, e)
            assert e <= OUT_ATOL, f"out ({b},{i}) err {e}"
            if np.isinf(lse):
                assert np.isinf(gpu_lse[b, i]) and gpu_lse[b, i] < 0
            else:
                assert abs(float(gpu_lse[b, i]) - lse) <= lse_tol(lse), \
                    f"lse ({b},{i}) {gpu_lse[b, i]} vs {lse}"
    return worst


def check_partials(o_part, lse_part, q, cache_bits, bt, sl, rows_sel, G, scale,
                   k_cap, slopes=None, chunk=None):
    """Partial s of a row holds entries [s*c, (s+1)*c): c = chunk, by default
    ceil(k_cap/splits) (one partial per split)."""
    B, H_q, ns, D = o_part.shape
    c = -(-k_cap // ns) if chunk is None else chunk
    for b in range(B):
        for i in range(H_q):
            pages = list(rows_sel[b][i])
            for s in range(ns):
                chunk = pages[s * c:(s + 1) * c] if c else []
                o, lse = _attend(q[b, i], cache_bits, i // G, bt[b], sl[b], chunk,
                                 scale, slopes, i)
                if np.isinf(lse):
                    assert np.isinf(lse_part[b, i, s]) and lse_part[b, i, s] < 0
                    assert np.all(o_part[b, i, s] == 0)
                    continue
                e = np.abs(o_part[b, i, s].astype(np.float64) - o).max()
                assert e <= OUT_ATOL, f"partial ({b},{i},{s}) err {e}"
                assert abs(float(lse_part[b, i, s]) - lse) <= lse_tol(lse), \
                    f"partial lse ({b},{i},{s}) {lse_part[b, i, s]} vs {lse}"


def per_head_rows(sel_rows, B, H_q, H_sel):
    """Expand selection rows to [b][i] (shared rows serve the whole group)."""
    G = H_q // H_sel
    out = []
    for b in range(B):
        out.append([sel_rows[b * H_sel + i // G] for i in range(H_q)])
    return out


def bf16_bits_apart(a_bits, b_bits):
    return np.abs(a_bits.astype(np.int64) - b_bits.astype(np.int64))


# ------------------------------------------------- Gaussian-aware selection

def page_rows(S, P, N):
    """Valid rows of each of the N pages of a request of S tokens."""
    return np.array([min(P, S - p * P) for p in range(N)], dtype=np.int32)


def check_gauss_select_row(g_mu, g_var, g_est, g_tau, g_sel, n, mixture, bos, eos, k_cap,
                           row):
    """The selection step of one row given the moments it was fed (g_mu,
    g_var fp32): tau-hat against the oracle's solve on those moments, the
    estimates mu + sigma sqrt(2 ln n), and the selection exact on the GPU's
    own fp32 estimates and tau-hat."""
    N = n.shape[0]
    t_o = oracle.gauss_tau(g_mu.astype(np.float64), g_var.astype(np.float64), n, mixture)
    assert abs(float(g_tau) - t_o) <= 1e-6 * max(1.0, abs(t_o)), \
        f"row {row}: tau-hat {g_tau} vs oracle {t_o} on the same moments"
    c = np.where(n > 1, np.sqrt(2.0 * np.log(np.maximum(n, 1))), 0.0)
    e_o = g_mu.astype(np.float64) + np.sqrt(np.maximum(g_var.astype(np.float64), 0)) * c
    tol_e = 1e-6 * (np.abs(g_mu) + np.sqrt(np.maximum(g_var, 0)) * c) + 1e-7
    assert np.all(np.abs(g_est - e_o) <= tol_e), f"row {row}: estimate error"
    lo, hi = min(bos, N), max(N - eos, 0)
    hi = max(hi, lo)
    half = np.float32(0.5) * g_est.astype(np.float32)
    qual = int(np.count_nonzero(half[lo:hi] > np.float32(g_tau)))
    budget = max(1, min(k_cap, qual + N - (hi - lo)))
    want = oracle.select(g_est.astype(np.float64), budget, 0.0, bos, eos).tolist()[:k_cap]
    assert list(g_sel) == want, f"row {row}: selection differs on the GPU's own values"


def check_gauss_row(g_mu, g_var, g_est, g_tau, g_sel, n, mixture, bos, eos, k_cap,
                    mu_o, var_o, k1, q2, bias, row):
    """One (request, query head) row of the Gaussian-aware path.

    g_*   the GPU's moments, estimates, tau-hat (fp32) and selection;
    mu_o, var_o  the oracle's moments from the oracle's statistics;
    k1    scale * sum_d |q_d| (|mean_d| + sd_d): the magnitude the fp32 mean
          and dot product round against; q2 = scale^2 sum_d q_d^2;
    bias  the ALiBi part of mu_o (0 without ALiBi).
    Returns True when the end-to-end selection differs from the oracle's only
    at pages within the tolerance band of tau-hat (an exempt row)."""
    N = n.shape[0]
    # moments against the oracle
    e_mu = np.abs(g_mu - mu_o)
    tol_mu = 8e-6 * k1 + 2e-7 * np.abs(bias) + 1e-7
    assert np.all(e_mu <= tol_mu), f"row {row}: mu err {e_mu.max()} (tol {tol_mu.min()})"
    e_var = np.abs(g_var - var_o)
    tol_var = 1e-5 * var_o + 1e-8 * (1.0 + q2)
    assert np.all(e_var <= tol_var), f"row {row}: var err {e_var.max()}"
    check_gauss_select_row(g_mu, g_var, g_est, g_tau, g_sel, n, mixture, bos, eos, k_cap,
                           row)
    c = np.where(n > 1, np.sqrt(2.0 * np.log(np.maximum(n, 1))), 0.0)
    # end to end: the oracle's tau-hat and selection from its own moments
    t_full = oracle.gauss_tau(mu_o, var_o, n, mixture)
    assert abs(float(g_tau) - t_full) <= 1e-4 * max(1.0, abs(t_full)), \
        f"row {row}: tau-hat {g_tau} vs end-to-end oracle {t_full}"
    full = oracle.gauss_select(mu_o, var_o, n, t_full, bos, eos, k_cap).tolist()
    if full == list(g_sel):
        return False
    est_full = mu_o + np.sqrt(var_o) * c
    band = 1e-4 * max(1.0, abs(t_full)) + 1e-5 * np.abs(est_full)
    if len(full) >= k_cap or len(g_sel) >= k_cap:
        # the cap ranks by estimate: near-equal estimates may trade places
        assert len(full) == len(g_sel), f"row {row}: capped counts differ"
        return True
    for p in set(full) ^ set(g_sel):
        assert abs(est_full[p] / 2 - t_full) <= band[p], \
            f"row {row}: page {p} selected differently away from tau-hat"
    return True
