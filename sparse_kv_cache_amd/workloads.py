"""Seeded synthetic inputs for the five decode workloads.

This module only draws random numbers and lays out tables.  It holds none of
the method's arithmetic (no statistics, scores, selection or attention), so
the HIP path and the float64 oracle can both be fed from it without sharing
any of the computation.

Shapes and distributions follow the workload descriptions:
  mha_tiny      B=1, H_q=H_kv=4, D=64, P=16, S=1024, contiguous table, topk 8
  gqa_ragged    B=8, 32/8 heads, D=128, P=16, S ~ U[2048, 8192], 4096-block
                pool, reverse-interleaved table, per-page mean offsets
                N(0, 0.5^2) on K and V, topk 64, w_avg 1.0, w_peak 0.5
  h2o_token     P=1, B=4, 32/8 heads, D=128, 4096-token prompt then 256 decode
                steps of one token, bf16 hh accumulator, decay 0.984375,
                top-512 tokens per kv head
  long_context  B=1, 64/8 heads, D=128, P=16, S=131072, identity table, 2% of
                pages get +2 along one random unit direction in K, topk 256,
                64 splits
  high_batch    B=128, 32/8 heads, D=128, P=16, S ~ U[1024, 32768], shuffled
                table over a 300k-block pool, topk 10% (min 4), 32 steps
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch


@dataclasses.dataclass
class Workload:
    name: str
    B: int
    H_q: int
    H_kv: int
    D: int
    P: int
    num_blocks: int
    seq_lens: np.ndarray          # int32 [B]: tokens present at step 0
    block_table: np.ndarray       # int32 [B, bt_ld]
    topk_pages: int
    topk_frac: float = 0.0
    bos: int = 0
    eos: int = 1
    w_avg: float = 1.0
    w_peak: float = 1.0
    scale: float = 0.0            # resolved to D**-0.5 when 0
    num_splits: int = 1
    decay: float = 0.984375
    steps: int = 1                # decode steps in the workload's sequence
    mean_offset_sigma: float = 0.0
    shifted_page_frac: float = 0.0
    q_bf16: bool = False          # queries drawn as bf16 values (h2o_token)
    seed: int = 0

    @property
    def G(self) -> int:
        return self.H_q // self.H_kv

    @property
    def bt_ld(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def softmax_scale(self) -> float:
        return self.scale if self.scale > 0 else self.D ** -0.5

    def pages(self, seq_lens=None) -> np.ndarray:
        s = self.seq_lens if seq_lens is None else seq_lens
        return (np.asarray(s, dtype=np.int64) + self.P - 1) // self.P

    def seq_lens_at(self, step: int) -> np.ndarray:
        """Token counts after the append of decode step ``step`` (0-based) for
        sequence workloads; the static workloads ignore ``step``."""
        if self.steps > 1:
            return (self.seq_lens + step + 1).astype(np.int32)
        return self.seq_lens.astype(np.int32)


# ------------------------------------------------------------ workloads

def mha_tiny(seed: int = 1) -> Workload:
    bt = np.arange(64, dtype=np.int32)[None, :]
    return Workload("mha_tiny", B=1, H_q=4, H_kv=4, D=64, P=16, num_blocks=64,
                    seq_lens=np.array([1024], dtype=np.int32), block_table=bt,
                    topk_pages=8, w_avg=1.0, w_peak=1.0, num_splits=2, seed=seed)


def gqa_ragged(seed: int = 2) -> Workload:
    rng = np.random.default_rng(seed)
    B, NB, ld = 8, 4096, 512
    seq = rng.integers(2048, 8192, size=B, endpoint=True).astype(np.int32)
    p = np.arange(ld)[None, :]
    b = np.arange(B)[:, None]
    bt = (NB - 1 - (p * B + b)).astype(np.int32)   # reverse-interleaved
    return Workload("gqa_ragged", B=B, H_q=32, H_kv=8, D=128, P=16,
                    num_blocks=NB, seq_lens=seq, block_table=bt, topk_pages=64,
                    w_avg=1.0, w_peak=0.5, num_splits=8, mean_offset_sigma=0.5,
                    seed=seed)


def h2o_token(seed: int = 3, steps: int = 256, prompt: int = 4096,
              B: int = 4) -> Workload:
    ld = prompt + steps
    bt = (np.arange(B)[:, None] * ld + np.arange(ld)[None, :]).astype(np.int32)
    return Workload("h2o_token", B=B, H_q=32, H_kv=8, D=128, P=1,
                    num_blocks=B * ld,
                    seq_lens=np.full(B, prompt, dtype=np.int32), block_table=bt,
                    topk_pages=512, bos=0, eos=1, num_splits=8, steps=steps,
                    q_bf16=True, seed=seed)


def long_context(seed: int = 4) -> Workload:
    N = 8192
    bt = np.arange(N, dtype=np.int32)[None, :]
    return Workload("long_context", B=1, H_q=64, H_kv=8, D=128, P=16,
                    num_blocks=N, seq_lens=np.array([N * 16], dtype=np.int32),
                    block_table=bt, topk_pages=256, w_avg=1.0, w_peak=1.0,
                    num_splits=64, shifted_page_frac=0.02, seed=seed)


def high_batch(seed: int = 5, steps: int = 32, B: int = 128,
               num_blocks: int = 300_000, smin: int = 1024,
               smax: int = 32768) -> Workload:
    rng = np.random.default_rng(seed)
    seq = rng.integers(smin, smax, size=B, endpoint=True).astype(np.int32)
    need = (seq.astype(np.int64) + steps + 15) // 16
    ld = int(need.max())
    perm = rng.permutation(num_blocks).astype(np.int32)
    bt = np.zeros((B, ld), dtype=np.int32)
    off = 0
    for b in range(B):
        bt[b, :need[b]] = perm[off:off + need[b]]
        off += int(need[b])
    assert off <= num_blocks
    return Workload("high_batch", B=B, H_q=32, H_kv=8, D=128, P=16,
                    num_blocks=num_blocks, seq_lens=seq, block_table=bt,
                    topk_pages=4, topk_frac=0.1, w_avg=1.0, w_peak=1.0,
                    num_splits=8, steps=steps, seed=seed)


WORKLOADS = {
    "mha_tiny": mha_tiny,
    "gqa_ragged": gqa_ragged,
    "h2o_token": h2o_token,
    "long_context": long_context,
    "high_batch": high_batch,
}


# ------------------------------------------------------- tensor draws

def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def referenced_blocks(wl: Workload, steps: int | None = None) -> np.ndarray:
    """Physical blocks any request uses over the workload's sequence."""
    n = wl.steps if steps is None else steps
    last = wl.seq_lens.astype(np.int64) + (n if wl.steps > 1 else 0)
    pages = (last + wl.P - 1) // wl.P
    return np.unique(np.concatenate(
        [wl.block_table[b, :pages[b]] for b in range(wl.B)]))


def make_cache(wl: Workload, device="cpu", chunk_blocks: int = 16384):
    """bf16 cache [2, num_blocks, P, H_kv, D].  Referenced blocks get N(0,1)
    (plus the workload's structure); the rest of the pool is zero."""
    g = _gen(device, 1000 + wl.seed)
    cache = torch.zeros((2, wl.num_blocks, wl.P, wl.H_kv, wl.D),
                        dtype=torch.bfloat16, device=device)
    blocks = torch.from_numpy(referenced_blocks(wl).astype(np.int64)).to(device)
    shape = (wl.P, wl.H_kv, wl.D)
    for kv in range(2):
        for s in range(0, blocks.numel(), chunk_blocks):
            idx = blocks[s:s + chunk_blocks]
            x = torch.randn((idx.numel(),) + shape, generator=g, device=device,
                            dtype=torch.float32)
            if wl.mean_offset_sigma > 0:
                off = torch.randn((idx.numel(), 1, wl.H_kv, wl.D), generator=g,
                                  device=device) * wl.mean_offset_sigma
                x += off
            cache[kv].index_copy_(0, idx, x.to(torch.bfloat16))
    if wl.shifted_page_frac > 0:
        rng = np.random.default_rng(2000 + wl.seed)
        N = int(wl.pages()[0])
        n_shift = int(round(wl.shifted_page_frac * N))
        pages = np.sort(rng.choice(N, size=n_shift, replace=False))
        u = rng.standard_normal(wl.D)
        u /= np.linalg.norm(u)
        blk = torch.from_numpy(wl.block_table[0, pages].astype(np.int64)).to(device)
        uu = torch.from_numpy(2.0 * u).to(device=device, dtype=torch.float32)
        k = cache[0].index_select(0, blk).float() + uu
        cache[0].index_copy_(0, blk, k.to(torch.bfloat16))
    return cache


def make_queries(wl: Workload, step: int = 0, device="cpu"):
    """Query rows [B, H_q, D] as float32 (bf16-valued for h2o_token)."""
    g = _gen(device, 3000 + 7919 * wl.seed + step)
    q = torch.randn((wl.B, wl.H_q, wl.D), generator=g, device=device,
                    dtype=torch.float32)
    if wl.q_bf16:
        q = q.to(torch.bfloat16).float()
    return q


def make_new_kv(wl: Workload, step: int = 0, device="cpu"):
    """The token appended at a decode step: k_new, v_new bf16 [B, H_kv, D]."""
    g = _gen(device, 5000 + 7919 * wl.seed + step)
    kn = torch.randn((wl.B, wl.H_kv, wl.D), generator=g, device=device)
    vn = torch.randn((wl.B, wl.H_kv, wl.D), generator=g, device=device)
    return kn.to(torch.bfloat16), vn.to(torch.bfloat16)


def make_hh(wl: Workload, device="cpu", stale: float = 7.5):
    """bf16 hh accumulator [num_blocks, H_kv]: zero on the prompt slots (as a
    prefill would leave it), a stale value on every other slot so that each
    decode append exercises the reset of a recycled slot."""
    hh = torch.full((wl.num_blocks * wl.P, wl.H_kv), stale,
                    dtype=torch.bfloat16, device=device)
    for b in range(wl.B):
        slots = torch.from_numpy(
            wl.block_table[b, :int(wl.seq_lens[b])].astype(np.int64)).to(device)
        hh.index_fill_(0, slots, 0.0)
    return hh


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Host copy of a bf16 tensor as its uint16 bit patterns."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def small_case(seed=0, B=2, H_q=4, H_kv=2, D=64, P=16, max_pages=9,
               num_blocks=None, topk_pages=3, topk_frac=0.0, bos=0, eos=1,
               w_avg=1.0, w_peak=1.0, num_splits=2, min_len=1):
    """A small ragged case with a shuffled block table, for unit tests."""
    rng = np.random.default_rng(seed)
    seq = rng.integers(min_len, max_pages * P, size=B, endpoint=True).astype(np.int32)
    need = (seq.astype(np.int64) + P - 1) // P
    ld = int(max_pages)
    NB = int(num_blocks or (B * max_pages + 3))
    perm = rng.permutation(NB).astype(np.int32)
    bt = np.full((B, ld), 0, dtype=np.int32)
    off = 0
    for b in range(B):
        bt[b, :need[b]] = perm[off:off + need[b]]
        off += int(need[b])
    return Workload(f"small{seed}", B=B, H_q=H_q, H_kv=H_kv, D=D, P=P,
                    num_blocks=NB, seq_lens=seq, block_table=bt,
                    topk_pages=topk_pages, topk_frac=topk_frac, bos=bos, eos=eos,
                    w_avg=w_avg, w_peak=w_peak, num_splits=num_splits, seed=seed)

