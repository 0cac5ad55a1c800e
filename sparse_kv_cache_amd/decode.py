"""Decode-step composites over the C ABI.

``SparseDecoder`` owns the per-step device buffers (page statistics, scores,
selections, split partials, outputs) for one cache shape and calls the
library's entry points in the order of a decode step:

  page level   [pagestats_update (append)] -> page_score -> page_topk
               -> sparse_paged_decode -> lse_merge
  group level  as page level with page_score_group: one selection per kv
               head, shared by its query group
  token level  pagestats_update (append + hh reset) -> h2o_accumulate (or
               h2o_accumulate_heads: per-head softmax averaged over the group)
               -> page_topk (per kv head) -> sparse_paged_decode -> lse_merge,
               as two launches when rows fit (h2o_select_decode: the append
               and the logits pass, then the update, the selection and the
               decode in one kernel), then lse_merge
  Gaussian     [pagestats_update + page_var_update (tail page)]
               -> gauss_moments -> gauss_select -> entmax15_paged_decode
               -> lse_merge

With one selection per query head and at most 8 splits the decoder fuses
launches: the merge runs inside the decode (sparse_paged_decode_merged), the
selection too when rows fit (sparse_select_decode, after page_score), and up
to ONE_LAUNCH_ROWS query rows the whole page-level step is one launch
(sparse_page_decode).  Past that row count scoring stays a launch of its own,
since it reads each kv head's statistics once for the whole query group.
With more splits (rows of up to 8192 pages) the selection runs inside the
split decode (sparse_select_decode_split) and lse_merge follows.

This mirrors the decode call of the EntmaxKV README ("Quick start": score,
select, attend and append in one call) cut at kernel granularity.  Nothing
here computes: it allocates once and marshals arguments.
"""
from __future__ import annotations

import math

import torch

from . import (entmax15_paged_decode, entmax15_paged_decode_merged, entmax_scratch_floats,
               gauss_moments, gauss_select,
               h2o_accumulate, h2o_accumulate_heads, h2o_heads_scratch_floats,
               h2o_scratch_floats, h2o_select_decode, h2o_select_decode_scratch_floats,
               lse_merge, page_score, page_score_ex,
               page_score_group, page_topk, page_topk_blk, page_var_update,
               pagestats_update, sparse_page_decode, sparse_paged_decode,
               sparse_paged_decode_ex, sparse_paged_decode_merged, sparse_select_decode,
               sparse_select_decode_group, sparse_select_decode_split,
               sparse_select_decode_split_blocks, sparse_select_decode_split_blocks_count)


def alibi_slopes(H, device="cuda"):
    """The standard geometric ALiBi slopes 2^(-8 (i + 1) / H) of H heads."""
    i = torch.arange(1, H + 1, dtype=torch.float64)
    return torch.pow(2.0, -8.0 * i / H).to(torch.float32).to(device)


# query rows up to which the page-level step runs as one launch
ONE_LAUNCH_ROWS = 512


def selection_capacity(score_ld, topk_pages, topk_frac=0.0, bos=0, eos=1):
    """Largest selection a row of at most score_ld entries can produce."""
    need = max(int(topk_pages), int(math.floor(float(topk_frac) * score_ld)),
               int(bos) + int(eos))
    return min(need, int(score_ld))


def validate_tables(block_table, seq_lens, num_blocks, page_size):
    """Debug check of the device-side contents the kernels trust: every
    request's length fits its block-table row (ceil(S / P) <= bt_ld) and every
    block id it uses lies in [0, num_blocks).  Copies both tensors to the host
    (a synchronising read); raises ValueError naming the first bad request.
    Not part of the step: call it, or pass validate=True to SparseDecoder,
    while debugging a caller."""
    bt = block_table.detach().cpu()
    sl = seq_lens.detach().cpu()
    if bt.dim() != 2 or sl.dim() != 1 or bt.shape[0] != sl.shape[0]:
        raise ValueError("block_table must be [B, bt_ld] and seq_lens [B]")
    ld = bt.shape[1]
    for b in range(sl.shape[0]):
        S = int(sl[b])
        if S < 0:
            raise ValueError(f"request {b}: seq_len {S} < 0")
        n = (S + page_size - 1) // page_size
        if n > ld:
            raise ValueError(f"request {b}: {S} tokens need {n} pages, the row holds {ld}")
        ids = bt[b, :n]
        if n and (int(ids.min()) < 0 or int(ids.max()) >= num_blocks):
            bad = int(ids[(ids < 0) | (ids >= num_blocks)][0])
            raise ValueError(f"request {b}: block id {bad} outside [0, {num_blocks})")


class SparseDecoder:
    """Buffers and call order of one decode step.

    kv_cache: bf16 [2, num_blocks, P, H_kv, D]; block_table int32 [B, bt_ld].
    token_level=True selects the H2O flow (page_size must be 1); its query
    group enters the accumulator through the group-mean query
    (h2o_softmax="group_mean") or through every head's own softmax, averaged
    over the group (h2o_softmax="per_head");
    group_select=True scores and selects once per kv head (page level);
    validate=True checks the block table and lengths on the host before each
    step (validate_tables; a debugging aid that synchronises);
    alibi_slopes (fp32 [H_q] on the device) adds ALiBi to scoring and decode.
    With one selection per query head and num_splits <= 8 the split merge runs
    inside the decode launch (fused); keep_partials also writes the partials.
    attention="entmax15" attends with 1.5-entmax instead of softmax (page
    level; three decode launches, then lse_merge).
    selection="gauss" selects per query head with the Gaussian-aware rule
    (adaptive page count, at most gauss_cap pages, default every page) and
    attends with 1.5-entmax; the page-mixture tau-hat is used for ALiBi heads
    and the single Gaussian otherwise, unless gauss_mixture says which."""

    def __init__(self, B, H_q, H_kv, D, num_blocks, page_size, bt_ld, *,
                 topk_pages, topk_frac=0.0, bos=0, eos=1, w_avg=1.0, w_peak=1.0,
                 scale=None, num_splits=1, decay=0.984375, token_level=False,
                 group_select=False, alibi_slopes=None, fuse_merge=True,
                 attention=None, selection="topk", gauss_cap=None, gauss_mixture=None,
                 h2o_softmax="group_mean", validate=False, device="cuda"):
        self.B, self.H_q, self.H_kv, self.D = B, H_q, H_kv, D
        self.num_blocks, self.P, self.bt_ld = num_blocks, page_size, bt_ld
        self.topk_pages, self.topk_frac = topk_pages, topk_frac
        self.bos, self.eos = bos, eos
        self.w_avg, self.w_peak = w_avg, w_peak
        self.scale = D ** -0.5 if scale is None else scale
        self.num_splits, self.decay = num_splits, decay
        self.token_level = token_level
        self.validate = bool(validate)
        self.group_select = bool(group_select) and not token_level
        dev = torch.device(device)
        if alibi_slopes is not None and token_level:
            raise ValueError("ALiBi is not part of the token-level flow")
        if h2o_softmax not in ("group_mean", "per_head"):
            raise ValueError("h2o_softmax must be 'group_mean' or 'per_head'")
        self.h2o_per_head = token_level and h2o_softmax == "per_head"
        if selection not in ("topk", "gauss"):
            raise ValueError("selection must be 'topk' or 'gauss'")
        if attention is None:
            attention = "entmax15" if selection == "gauss" else "softmax"
        if attention not in ("softmax", "entmax15"):
            raise ValueError("attention must be 'softmax' or 'entmax15'")
        if attention == "entmax15" and token_level:
            raise ValueError("1.5-entmax is built for the page-level flow")
        if selection == "gauss" and (token_level or group_select or attention != "entmax15"):
            raise ValueError("Gaussian-aware selection is per query head, page level, "
                             "with 1.5-entmax attention")
        self.attention = attention
        self.selection = selection
        self.gauss = selection == "gauss"
        self.mixture = (alibi_slopes is not None) if gauss_mixture is None else bool(gauss_mixture)
        self.alibi = alibi_slopes
        # the page score is in q.k units: slopes divided by the softmax scale
        self.alibi_score = None if alibi_slopes is None else alibi_slopes / self.scale
        self.H_sel = H_kv if (token_level or self.group_select) else H_q
        self.k_cap = selection_capacity(bt_ld, topk_pages, topk_frac, bos, eos)
        if self.gauss:
            cap = bt_ld if gauss_cap is None else int(gauss_cap)
            self.k_cap = max(1, min(bt_ld, max(cap, bos + eos)))
        f32, i32, bf = torch.float32, torch.int32, torch.bfloat16
        if token_level:
            if page_size != 1:
                raise ValueError("the token-level flow needs page_size 1")
            self.k_min = self.k_max = self.k_mean = None
            self.hh = torch.zeros((num_blocks, H_kv), dtype=bf, device=dev)
            n = (h2o_heads_scratch_floats(B, H_q, bt_ld) if self.h2o_per_head
                 else h2o_scratch_floats(B, H_kv, bt_ld))
            # (room for the fused step's accumulator copy as well)
            n = max(n, h2o_select_decode_scratch_floats(B, H_q, H_kv, bt_ld,
                                                        self.h2o_per_head))
            self.scratch = torch.empty(n, dtype=f32, device=dev)
        else:
            self.k_min = torch.empty((num_blocks, H_kv, D), dtype=bf, device=dev)
            self.k_max = torch.empty((num_blocks, H_kv, D), dtype=bf, device=dev)
            self.k_mean = torch.empty((num_blocks, H_kv, D), dtype=f32, device=dev)
            self.hh = None
            self.scratch = None
        self.scores = torch.empty((B, self.H_sel, bt_ld), dtype=f32, device=dev)
        self.sel_idx = torch.empty((B, self.H_sel, self.k_cap), dtype=i32, device=dev)
        self.sel_cnt = torch.empty((B, self.H_sel), dtype=i32, device=dev)
        self.sel_blk = torch.empty((B, self.H_sel, self.k_cap), dtype=i32, device=dev)
        self.use_sel_blk = True
        # A selection shared by a kv head's group is decoded by the matrix-core
        # group kernel, one block per (split, request, kv head): it runs best
        # with about one block per CU (256), so its split count follows the
        # grid, at most num_splits and at most one split per selected page.
        self.decode_splits = num_splits
        if self.H_sel == H_kv and H_q > H_kv:
            per = max(1, 256 // max(1, B * H_kv))
            self.decode_splits = max(1, min(num_splits, per, self.k_cap))
        self.o_part = torch.empty((B, H_q, self.decode_splits, D), dtype=f32, device=dev)
        self.lse_part = torch.empty((B, H_q, self.decode_splits), dtype=f32, device=dev)
        self.out = torch.empty((B, H_q, D), dtype=f32, device=dev)
        self.lse = torch.empty((B, H_q), dtype=f32, device=dev)
        self.fused = (bool(fuse_merge) and self.H_sel == H_q and num_splits <= 8
                      and attention == "softmax")
        self.keep_partials = False
        # selection inside the decode launch as well (score rows <= 4096)
        self.select_in_decode = self.fused and bt_ld <= 4096 and self.k_cap <= 4096
        # a selection shared by the group: selected inside the group decode
        # (rows of up to 8192), partials merged by lse_merge
        self.select_in_group_decode = (bool(fuse_merge) and self.H_sel == H_kv and H_q > H_kv
                                       and attention == "softmax" and bt_ld <= 8192
                                       and self.k_cap <= 4096)
        # token level: the accumulator update, the selection and the decode in
        # two launches (h2o_select_decode), then lse_merge
        self.token_fused = token_level and self.select_in_group_decode
        # one selection per query head with more splits than a block merges:
        # the selection inside the split decode (each block of a head derives
        # it), partials merged by lse_merge
        self.select_in_split_decode = (bool(fuse_merge) and self.H_sel == H_q
                                       and not self.fused and attention == "softmax"
                                       and selection == "topk" and bt_ld <= 8192
                                       and self.k_cap <= 4096)
        self.keep_selection = False
        # ... whose blocks also merge their splits, so lse_merge combines a
        # head's few block partials (split_blocks; False: one per split)
        self.split_blocks = True
        self.o_blk = self.lse_blk = None
        if self.select_in_split_decode:
            nb = sparse_select_decode_split_blocks_count(num_splits, page_size)
            self.o_blk = torch.empty((B, H_q, nb, D), dtype=f32, device=dev)
            self.lse_blk = torch.empty((B, H_q, nb), dtype=f32, device=dev)
        # the partials merge() combines: the last decode form's
        self.partials = (self.o_part, self.lse_part)
        # and scoring too: the whole page-level step in one launch, while the
        # device holds every block of it at once (two 8-wave blocks per CU,
        # 512 query rows); past that the separate page_score, which reads a
        # kv head's statistics once for its whole group instead of once per
        # query head, is faster (1024 rows: 97.7 against 106.2 us a step,
        # 4096: 750 against 879 us)
        sc_cap = (bt_ld + 3) // 4 * 4
        self.score_in_decode = (self.select_in_decode and not self.group_select
                                and B * H_q <= ONE_LAUNCH_ROWS
                                and (2 * sc_cap + 2 * self.k_cap) * 4 <= 48 * 1024)
        self.keep_scores = False
        self.k_var = self.mu = self.var = self.est = self.tau_hat = None
        if self.gauss:
            self.k_var = torch.empty((num_blocks, H_kv, D), dtype=f32, device=dev)
            self.mu = torch.empty((B, H_q, bt_ld), dtype=f32, device=dev)
            self.var = torch.empty((B, H_q, bt_ld), dtype=f32, device=dev)
            self.est = self.scores            # the estimates are the ranking scores
            self.tau_hat = torch.empty((B, H_q), dtype=f32, device=dev)
        self.entmax_scratch = None
        # 1.5-entmax in one merged launch (else three launches and lse_merge)
        # (a batch of fewer than 128 query rows with a fixed top-k budget
        # keeps the three launches and their num_splits chunks per row: one
        # block per row would leave the chip mostly idle; Gaussian-aware
        # selections are small, and the one launch wins there too)
        self.entmax_fused = (bool(fuse_merge) and attention == "entmax15"
                             and (B * H_q >= 128 or selection == "gauss"))
        if attention == "entmax15":
            n = entmax_scratch_floats(B, H_q, self.k_cap, page_size)
            self.entmax_scratch = torch.empty(n, dtype=f32, device=dev)
            self.entmax_tau_buf = torch.empty((B, H_q), dtype=f32, device=dev)

    @classmethod
    def for_workload(cls, wl, device="cuda", num_splits=None, group_select=False,
                     alibi_slopes=None, fuse_merge=True, attention=None,
                     selection="topk", gauss_cap=None, gauss_mixture=None,
                     h2o_softmax="group_mean"):
        return cls(wl.B, wl.H_q, wl.H_kv, wl.D, wl.num_blocks, wl.P, wl.bt_ld,
                   topk_pages=wl.topk_pages, topk_frac=wl.topk_frac, bos=wl.bos,
                   eos=wl.eos, w_avg=wl.w_avg, w_peak=wl.w_peak,
                   scale=wl.softmax_scale,
                   num_splits=wl.num_splits if num_splits is None else num_splits,
                   decay=wl.decay, token_level=(wl.name == "h2o_token"),
                   group_select=group_select, alibi_slopes=alibi_slopes,
                   fuse_merge=fuse_merge, attention=attention, selection=selection,
                   gauss_cap=gauss_cap, gauss_mixture=gauss_mixture,
                   h2o_softmax=h2o_softmax, device=device)

    # ------------------------------------------------------------ stages
    def rebuild_stats(self, kv_cache, block_table, seq_lens, stream=None):
        pagestats_update(kv_cache, self.k_min, self.k_max, self.k_mean,
                         block_table, seq_lens, stream=stream)
        if self.gauss:
            page_var_update(kv_cache, self.k_mean, self.k_var, block_table, seq_lens,
                            stream=stream)

    def append(self, kv_cache, block_table, seq_lens, k_new, v_new, stream=None):
        pagestats_update(kv_cache, self.k_min, self.k_max, self.k_mean,
                         block_table, seq_lens, k_new, v_new, self.hh,
                         stream=stream)
        if self.gauss:
            page_var_update(kv_cache, self.k_mean, self.k_var, block_table, seq_lens,
                            tail_only=True, stream=stream)

    def moments(self, q, block_table, seq_lens, stream=None):
        """Gaussian moments of every page's logits."""
        gauss_moments(q, self.k_mean, self.k_var, block_table, seq_lens, self.P,
                      self.scale, self.mu, self.var, alibi_slopes=self.alibi,
                      stream=stream)

    def select_gauss(self, seq_lens, block_table, stream=None):
        """tau-hat and the adaptive selection from the moments."""
        gauss_select(self.mu, self.var, seq_lens, self.P, block_table, self.mixture,
                     self.k_cap, self.est, self.sel_idx, self.sel_cnt, tau=self.tau_hat,
                     sel_blk=self.sel_blk if self.use_sel_blk else None,
                     reserved_bos=self.bos, reserved_eos=self.eos, stream=stream)

    def gauss_select(self, q, block_table, seq_lens, stream=None):
        """Moments, tau-hat and the adaptive selection (Gaussian-aware)."""
        self.moments(q, block_table, seq_lens, stream)
        self.select_gauss(seq_lens, block_table, stream)

    def score(self, q, block_table, seq_lens, stream=None):
        if self.token_level:
            raise RuntimeError("token-level scores come from h2o_accumulate")
        args = (q, self.k_min, self.k_max, self.k_mean, block_table, seq_lens, self.P,
                self.w_avg, self.w_peak, self.scores)
        if self.group_select:
            page_score_group(*args, alibi=self.alibi_score, stream=stream)
        elif self.alibi_score is not None:
            page_score_ex(*args, alibi=self.alibi_score, stream=stream)
        else:
            page_score(*args, stream=stream)

    def accumulate(self, q, kv_cache, block_table, seq_lens, stream=None):
        fn = h2o_accumulate_heads if self.h2o_per_head else h2o_accumulate
        fn(q, kv_cache, block_table, seq_lens, self.hh, self.scores,
                       self.scratch, self.scale, self.decay, self.bos, self.eos,
                       stream=stream)

    def select(self, seq_lens, block_table=None, stream=None):
        if self.use_sel_blk and block_table is not None:
            page_topk_blk(self.scores, seq_lens, self.P, self.topk_pages, self.sel_idx,
                          self.sel_cnt, block_table, self.sel_blk, self.topk_frac,
                          self.bos, self.eos, stream=stream)
        else:
            page_topk(self.scores, seq_lens, self.P, self.topk_pages, self.sel_idx,
                      self.sel_cnt, self.topk_frac, self.bos, self.eos, stream=stream)

    def attend(self, q, kv_cache, block_table, seq_lens, stream=None):
        self.partials = (self.o_part, self.lse_part)
        if self.attention == "entmax15" and self.entmax_fused:
            entmax15_paged_decode_merged(
                q, kv_cache, block_table, seq_lens, self.sel_idx, self.sel_cnt, self.scale,
                self.out, lse_out=self.lse, tau_out=self.entmax_tau_buf,
                scratch=self.entmax_scratch,
                sel_blk=self.sel_blk if self.use_sel_blk else None,
                alibi_slopes=self.alibi, stream=stream)
            return
        if self.attention == "entmax15":
            entmax15_paged_decode(q, kv_cache, block_table, seq_lens, self.sel_idx,
                                  self.sel_cnt, self.scale, self.o_part, self.lse_part,
                                  self.entmax_scratch,
                                  sel_blk=self.sel_blk if self.use_sel_blk else None,
                                  alibi_slopes=self.alibi, stream=stream)
            return
        if self.fused:
            parts = (self.o_part, self.lse_part) if self.keep_partials else (None, None)
            sparse_paged_decode_merged(
                q, kv_cache, block_table, seq_lens, self.sel_idx, self.sel_cnt,
                self.scale, self.num_splits, self.out, self.lse, o_part=parts[0],
                lse_part=parts[1], sel_blk=self.sel_blk if self.use_sel_blk else None,
                alibi_slopes=self.alibi, stream=stream)
            return
        if self.use_sel_blk or self.alibi is not None:
            sparse_paged_decode_ex(q, kv_cache, block_table, seq_lens, self.sel_idx,
                                   self.sel_cnt, self.scale, self.o_part, self.lse_part,
                                   sel_blk=self.sel_blk if self.use_sel_blk else None,
                                   alibi_slopes=self.alibi, stream=stream)
        else:
            sparse_paged_decode(q, kv_cache, block_table, seq_lens, self.sel_idx,
                                self.sel_cnt, self.scale, self.o_part, self.lse_part,
                                stream=stream)

    def select_attend(self, q, kv_cache, block_table, seq_lens, stream=None):
        """Selection, decode and merge in one launch (select_in_decode)."""
        keep = self.keep_selection
        sparse_select_decode(
            self.scores, q, kv_cache, block_table, seq_lens, self.topk_pages, self.k_cap,
            self.scale, self.num_splits, self.out, self.lse, topk_frac=self.topk_frac,
            reserved_bos=self.bos, reserved_eos=self.eos,
            sel_idx=self.sel_idx if keep else None, sel_cnt=self.sel_cnt if keep else None,
            sel_blk=self.sel_blk if keep else None, alibi_slopes=self.alibi, stream=stream)

    def select_attend_group(self, q, kv_cache, block_table, seq_lens, stream=None):
        """Selection (per kv head) and the group decode in one launch
        (select_in_group_decode); the partials still go through merge()."""
        keep = self.keep_selection
        self.partials = (self.o_part, self.lse_part)
        sparse_select_decode_group(
            self.scores, q, kv_cache, block_table, seq_lens, self.topk_pages, self.k_cap,
            self.scale, self.o_part, self.lse_part, topk_frac=self.topk_frac,
            reserved_bos=self.bos, reserved_eos=self.eos,
            sel_idx=self.sel_idx if keep else None, sel_cnt=self.sel_cnt if keep else None,
            sel_blk=self.sel_blk if keep else None, alibi_slopes=self.alibi, stream=stream)

    def select_attend_split(self, q, kv_cache, block_table, seq_lens, stream=None,
                            blocks=None):
        """Selection (per query head) and the split decode in one launch
        (select_in_split_decode); the partials go through merge(): one per
        block of splits (blocks, default split_blocks), else one per split."""
        keep = self.keep_selection
        sel = dict(sel_idx=self.sel_idx if keep else None,
                   sel_cnt=self.sel_cnt if keep else None,
                   sel_blk=self.sel_blk if keep else None)
        if self.split_blocks if blocks is None else blocks:
            sparse_select_decode_split_blocks(
                self.scores, q, kv_cache, block_table, seq_lens, self.topk_pages, self.k_cap,
                self.scale, self.num_splits, self.o_blk, self.lse_blk,
                topk_frac=self.topk_frac, reserved_bos=self.bos, reserved_eos=self.eos,
                alibi_slopes=self.alibi, stream=stream, **sel)
            self.partials = (self.o_blk, self.lse_blk)
            return
        sparse_select_decode_split(
            self.scores, q, kv_cache, block_table, seq_lens, self.topk_pages, self.k_cap,
            self.scale, self.o_part, self.lse_part, topk_frac=self.topk_frac,
            reserved_bos=self.bos, reserved_eos=self.eos, alibi_slopes=self.alibi,
            stream=stream, **sel)
        self.partials = (self.o_part, self.lse_part)

    def accumulate_select_attend(self, q, kv_cache, block_table, seq_lens, k_new=None,
                                 v_new=None, stream=None):
        """Token level (token_fused): the append (when k_new is given),
        accumulate, select and decode in two launches; hh updated, partials
        for merge()."""
        keep = self.keep_selection
        self.partials = (self.o_part, self.lse_part)
        h2o_select_decode(
            q, kv_cache, block_table, seq_lens, self.hh, self.scratch, self.scale,
            self.topk_pages, self.k_cap, self.o_part, self.lse_part, decay=self.decay,
            reserved_bos=self.bos, reserved_eos=self.eos, per_head=self.h2o_per_head,
            scores=self.scores if self.keep_scores else None, topk_frac=self.topk_frac,
            sel_idx=self.sel_idx if keep else None, sel_cnt=self.sel_cnt if keep else None,
            sel_blk=self.sel_blk if keep else None, k_new=k_new, v_new=v_new,
            stream=stream)

    def score_select_attend(self, q, kv_cache, block_table, seq_lens, stream=None):
        """Score, select, decode and merge in one launch (score_in_decode)."""
        keep = self.keep_selection
        sparse_page_decode(
            q, kv_cache, self.k_min, self.k_max, self.k_mean, block_table, seq_lens,
            self.w_avg, self.w_peak, self.topk_pages, self.k_cap, self.scale,
            self.num_splits, self.out, self.lse, topk_frac=self.topk_frac,
            reserved_bos=self.bos, reserved_eos=self.eos,
            scores=self.scores if self.keep_scores else None,
            sel_idx=self.sel_idx if keep else None, sel_cnt=self.sel_cnt if keep else None,
            sel_blk=self.sel_blk if keep else None, alibi_slopes=self.alibi, stream=stream)

    def merge(self, stream=None):
        if self.fused or (self.attention == "entmax15" and self.entmax_fused):
            return                      # merged inside attend()
        o, lse = self.partials
        lse_merge(o, lse, self.out, self.lse, stream=stream)

    # -------------------------------------------------------------- step
    def step(self, q, kv_cache, block_table, seq_lens, k_new=None, v_new=None,
             stream=None):
        """One decode step; returns (out, lse) views of the decoder's buffers."""
        if self.validate:
            validate_tables(block_table, seq_lens, self.num_blocks, self.P)
        if self.token_fused:
            # the append runs inside the first of the two launches
            self.accumulate_select_attend(q, kv_cache, block_table, seq_lens, k_new, v_new,
                                          stream)
            self.merge(stream)
            return self.out, self.lse
        if k_new is not None:
            self.append(kv_cache, block_table, seq_lens, k_new, v_new, stream)
        if self.gauss:
            self.gauss_select(q, block_table, seq_lens, stream)
            self.attend(q, kv_cache, block_table, seq_lens, stream)
            self.merge(stream)
            return self.out, self.lse
        if self.score_in_decode:
            self.score_select_attend(q, kv_cache, block_table, seq_lens, stream)
            return self.out, self.lse
        if self.token_level:
            self.accumulate(q, kv_cache, block_table, seq_lens, stream)
        else:
            self.score(q, block_table, seq_lens, stream)
        if self.select_in_decode:
            self.select_attend(q, kv_cache, block_table, seq_lens, stream)
            return self.out, self.lse
        if self.select_in_group_decode:
            self.select_attend_group(q, kv_cache, block_table, seq_lens, stream)
            self.merge(stream)
            return self.out, self.lse
        if self.select_in_split_decode:
            self.select_attend_split(q, kv_cache, block_table, seq_lens, stream)
            self.merge(stream)
            return self.out, self.lse
        self.select(seq_lens, block_table, stream)
        self.attend(q, kv_cache, block_table, seq_lens, stream)
        self.merge(stream)
        return self.out, self.lse

    def entmax_tau(self):
        """tau per query head [B, H_q] of the last 1.5-entmax decode."""
        if self.entmax_fused:
            return self.entmax_tau_buf
        n = self.B * self.H_q
        return self.entmax_scratch[-n:].view(self.B, self.H_q)
