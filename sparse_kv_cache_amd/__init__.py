"""sparse_kv_cache_amd -- page-scored sparse decode attention for MI355X.

Thin Python binding of the C ABI in ``include/sparsekv.h`` (libsparsekv.so,
hand-written HIP for gfx950).  Every function here only checks tensor
dtypes / shapes / devices, marshals ``data_ptr()`` values and the current HIP
stream, and calls the entry point of the same name; all arithmetic runs in the
library's kernels.  PyTorch supplies device memory and streams only.

The library is loaded on first use.  If it has not been built, every call
raises ``RuntimeError``: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "pagestats_update", "page_score", "page_score_ex", "page_score_group", "page_topk",
    "page_topk_blk", "sparse_paged_decode", "sparse_paged_decode_ex",
    "sparse_paged_decode_merged", "lse_merge",
    "h2o_accumulate", "h2o_scratch_floats", "h2o_accumulate_heads",
    "h2o_heads_scratch_floats", "h2o_accumulate_noalloc", "h2o_select_decode", "h2o_select_decode_scratch_floats", "NOALLOC_SCRATCH_FLOATS",
    "entmax15_paged_decode",
    "entmax_scratch_floats", "sparse_select_decode", "sparse_select_decode_group",
    "sparse_select_decode_split", "sparse_select_decode_split_blocks",
    "sparse_select_decode_split_blocks_count", "sparse_page_decode",
    "page_var_update", "gauss_moments", "gauss_select", "entmax15_paged_decode_merged",
    "skv_ref_stream_read", "skv_ref_gather_read", "library_path",
    "load_library", "SparseKVError", "EXPORTED_SYMBOLS",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsparsekv.so")
_lib = None

EXPORTED_SYMBOLS = (
    "pagestats_update", "page_score", "page_score_ex", "page_score_group", "page_topk",
    "page_topk_blk", "sparse_paged_decode", "sparse_paged_decode_ex",
    "sparse_paged_decode_merged", "lse_merge",
    "h2o_accumulate", "h2o_scratch_floats", "h2o_accumulate_heads",
    "h2o_heads_scratch_floats", "h2o_accumulate_noalloc", "h2o_select_decode", "h2o_select_decode_scratch_floats", "entmax15_paged_decode",
    "entmax_scratch_floats", "sparse_select_decode", "sparse_select_decode_group",
    "sparse_select_decode_split", "sparse_select_decode_split_blocks",
    "sparse_select_decode_split_blocks_count", "sparse_page_decode",
    "page_var_update", "gauss_moments", "gauss_select", "entmax15_paged_decode_merged",
    "skv_ref_stream_read", "skv_ref_gather_read", "sparsekv_last_error",
    "sparsekv_build_id",
)
# size of the fixed scratch of h2o_accumulate_noalloc (SKV_NOALLOC_SCRATCH_FLOATS)
NOALLOC_SCRATCH_FLOATS = 2 * 1024 * 1024
_INT_RETURNING = ("pagestats_update", "page_score", "page_score_ex", "page_score_group",
                  "page_topk", "page_topk_blk", "sparse_paged_decode",
                  "sparse_paged_decode_ex", "sparse_paged_decode_merged", "lse_merge",
                  "h2o_accumulate", "h2o_accumulate_heads", "h2o_accumulate_noalloc",
                  "h2o_select_decode",
                  "entmax15_paged_decode",
                  "sparse_select_decode", "sparse_select_decode_group",
                  "sparse_select_decode_split", "sparse_select_decode_split_blocks",
                  "sparse_page_decode", "page_var_update", "gauss_moments", "gauss_select",
                  "entmax15_paged_decode_merged", "skv_ref_stream_read",
                  "skv_ref_gather_read")


class SparseKVError(RuntimeError):
    """A non-zero return code from the library."""

    def __init__(self, fn, code, msg):
        super().__init__(f"{fn} returned {code}: {msg}")
        self.code = code


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libsparsekv.so (once).  Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            f"{_LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; "
            "g.build()'` (or python sparse_kv_cache_amd/build.py) first")
    lib = ctypes.CDLL(_LIB_PATH)
    V, I, L, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float
    # a library built from other sources than the tree holds may take other
    # arguments than the ones passed below: refuse it rather than call it
    lib.sparsekv_build_id.restype = ctypes.c_char_p
    lib.sparsekv_build_id.argtypes = []
    from . import build as _build
    if os.path.isdir(_build.CSRC):
        built, now = lib.sparsekv_build_id().decode(), _build.source_digest()
        if built != now:
            raise RuntimeError(
                f"{_LIB_PATH} was built from other sources (build id {built[:12]}, "
                f"sources {now[:12]}); rebuild it: python -c 'import __graft_entry__ "
                "as g; g.build()'")
    lib.sparsekv_last_error.restype = ctypes.c_char_p
    lib.sparsekv_last_error.argtypes = []
    lib.pagestats_update.argtypes = [V, L, I, I, I, V, V, V, V, L, V, I, V, V, V, V]
    lib.page_score.argtypes = [V, I, I, I, I, V, V, V, V, L, V, I, F, F, V, L, V]
    lib.page_score_ex.argtypes = [V, I, I, I, I, V, V, V, V, L, V, I, F, F, V, L, V, V]
    lib.page_score_group.argtypes = lib.page_score_ex.argtypes
    lib.page_topk.argtypes = [V, L, I, I, V, I, I, F, I, I, V, V, I, V]
    lib.page_topk_blk.argtypes = [V, L, I, I, V, I, I, F, I, I, V, V, I, V, L, V, V]
    lib.sparse_paged_decode.argtypes = [V, I, I, I, I, V, L, I, V, L, V, V, V, I, I, F, I,
                                        V, V, V]
    lib.sparse_paged_decode_ex.argtypes = [V, I, I, I, I, V, L, I, V, L, V, V, V, V, I,
                                           I, F, I, V, V, V, V]
    lib.sparse_paged_decode_merged.argtypes = [V, I, I, I, I, V, L, I, V, L, V, V, V, V,
                                               I, F, I, V, V, V, V, V, V]
    lib.lse_merge.argtypes = [V, V, I, I, I, V, V, V]
    lib.h2o_accumulate.argtypes = [V, I, I, I, I, V, L, I, V, L, V, I, I, F, F, V, V,
                                   L, V, L, V]
    lib.h2o_scratch_floats.argtypes = [I, I, L]
    lib.h2o_scratch_floats.restype = ctypes.c_int64
    lib.h2o_accumulate_heads.argtypes = lib.h2o_accumulate.argtypes
    lib.h2o_select_decode.argtypes = [V, I, I, I, I, V, L, I, V, L, V, I, I, F, F, I, V, V, L,
                                      I, F, I, I, V, V, V, V, V, V, V, V, L, V]
    lib.h2o_select_decode_scratch_floats.argtypes = [I, I, I, L, I]
    lib.h2o_select_decode_scratch_floats.restype = ctypes.c_int64
    lib.h2o_accumulate_noalloc.argtypes = [V, I, I, I, I, V, L, I, V, L, V, I, I, F, F, V, V,
                                           L, V]
    lib.h2o_heads_scratch_floats.argtypes = [I, I, L]
    lib.h2o_heads_scratch_floats.restype = ctypes.c_int64
    lib.entmax15_paged_decode.argtypes = [V, I, I, I, I, V, L, I, V, L, V, V, V, V, I, I,
                                          F, I, V, V, V, V, L, V]
    lib.entmax15_paged_decode_merged.argtypes = [V, I, I, I, I, V, L, I, V, L, V, V, V, V,
                                                 I, I, F, V, V, V, V, V, L, V]
    lib.page_var_update.argtypes = [V, L, I, I, I, V, V, V, L, V, I, I, V]
    lib.gauss_moments.argtypes = [V, I, I, I, I, V, V, V, L, V, I, F, V, V, V, L, V]
    lib.gauss_select.argtypes = [V, V, L, I, I, V, I, V, L, I, I, I, I, V, V, V, V, V, V]
    lib.entmax_scratch_floats.argtypes = [I, I, I, I]
    lib.sparse_select_decode.argtypes = [V, L, I, F, I, I, V, I, I, I, I, V, L, I, V, L, V,
                                         I, F, I, V, V, V, V, V, V, V]
    lib.sparse_select_decode_group.argtypes = [V, L, I, F, I, I, V, I, I, I, I, V, L, I, V,
                                               L, V, I, F, I, V, V, V, V, V, V, V]
    lib.sparse_select_decode_split.argtypes = lib.sparse_select_decode_group.argtypes
    lib.sparse_select_decode_split_blocks.argtypes = lib.sparse_select_decode_group.argtypes
    lib.sparse_select_decode_split_blocks_count.argtypes = [I, I]
    lib.sparse_select_decode_split_blocks_count.restype = ctypes.c_int
    lib.sparse_page_decode.argtypes = [V, I, I, I, I, V, L, I, V, V, V, V, L, V, F, F, I, F,
                                       I, I, I, F, I, V, V, V, V, V, V, V, V]
    lib.entmax_scratch_floats.restype = ctypes.c_int64
    lib.skv_ref_stream_read.argtypes = [V, L, V, V]
    lib.skv_ref_gather_read.argtypes = [V, L, I, I, I, V, L, V, V]
    for name in _INT_RETURNING:
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


# ----------------------------------------------------------------- helpers

def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(name, t, dtype, ndim=None, device=None):
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _rc(name, code):
    if code != 0:
        msg = load_library().sparsekv_last_error().decode(errors="replace")
        raise SparseKVError(name, code, msg)


# ------------------------------------------------------------ entry points

def pagestats_update(kv_cache, k_min, k_max, k_mean, block_table, seq_lens,
                     k_new=None, v_new=None, hh_score=None, stream=None):
    """Rebuild (k_new is None) or append-and-refresh the page statistics."""
    lib = load_library()
    _check("kv_cache", kv_cache, torch.bfloat16, 5)
    dev = kv_cache.device
    _, NB, P, H_kv, D = kv_cache.shape
    for n, t, dt in (("k_min", k_min, torch.bfloat16), ("k_max", k_max, torch.bfloat16),
                     ("k_mean", k_mean, torch.float32)):
        _check(n, t, dt, 3, dev)
        if t is not None and tuple(t.shape) != (NB, H_kv, D):
            raise ValueError(f"{n} must be [num_blocks, H_kv, D]")
    _check("block_table", block_table, torch.int32, 2, dev)
    _check("seq_lens", seq_lens, torch.int32, 1, dev)
    _check("k_new", k_new, torch.bfloat16, 3, dev)
    _check("v_new", v_new, torch.bfloat16, 3, dev)
    _check("hh_score", hh_score, torch.bfloat16, 2, dev)
    B = seq_lens.shape[0]
    if block_table.shape[0] != B:
        raise ValueError("block_table rows must equal len(seq_lens)")
    for n, t in (("k_new", k_new), ("v_new", v_new)):
        if t is not None and tuple(t.shape) != (B, H_kv, D):
            raise ValueError(f"{n} must be [B, H_kv, D]")
    if hh_score is not None and tuple(hh_score.shape) != (NB * P, H_kv):
        raise ValueError("hh_score must be [num_blocks * page_size, H_kv]")
    _rc("pagestats_update", lib.pagestats_update(
        _ptr(kv_cache), NB, P, H_kv, D, _ptr(k_min), _ptr(k_max), _ptr(k_mean),
        _ptr(block_table), block_table.shape[1], _ptr(seq_lens), B, _ptr(k_new),
        _ptr(v_new), _ptr(hh_score), _stream(stream)))


def _shape(name, t, shape):
    """t (if given) must have exactly `shape`."""
    if t is not None and tuple(t.shape) != tuple(int(x) for x in shape):
        raise ValueError(f"{name} must have shape {tuple(int(x) for x in shape)}, "
                         f"got {tuple(t.shape)}")


def _batch(B, block_table, seq_lens):
    """seq_lens is [B] and block_table (if given) has B rows."""
    if seq_lens.shape[0] != B:
        raise ValueError(f"seq_lens must be [B] = [{B}], got {tuple(seq_lens.shape)}")
    if block_table is not None and block_table.shape[0] != B:
        raise ValueError(f"block_table must have B = {B} rows, got {tuple(block_table.shape)}")


def _stats(k_min, k_max, k_mean, D, dev, NB=None):
    """The three page statistics share [num_blocks, H_kv, D]; returns (NB, H_kv)."""
    _check("k_min", k_min, torch.bfloat16, 3, dev)
    _check("k_max", k_max, torch.bfloat16, 3, dev)
    _check("k_mean", k_mean, torch.float32, 3, dev)
    nb, H_kv, d = k_min.shape
    if d != D:
        raise ValueError(f"page statistics have head dim {d}, the query {D}")
    if NB is not None and nb != NB:
        raise ValueError(f"page statistics cover {nb} blocks, the cache {NB}")
    _shape("k_max", k_max, (nb, H_kv, D))
    _shape("k_mean", k_mean, (nb, H_kv, D))
    return nb, H_kv


def _selection(sel_idx, sel_cnt, sel_blk, B, H_sel, dev, k_cap=None):
    """sel_idx [B, H_sel, k_cap], sel_cnt [B, H_sel], sel_blk like sel_idx."""
    _check("sel_idx", sel_idx, torch.int32, 3, dev)
    _check("sel_cnt", sel_cnt, torch.int32, 2, dev)
    _check("sel_blk", sel_blk, torch.int32, 3, dev)
    if sel_idx is not None:
        if tuple(sel_idx.shape[:2]) != (B, H_sel):
            raise ValueError(f"sel_idx must be [B, H_sel, k_cap] = [{B}, {H_sel}, k_cap], "
                             f"got {tuple(sel_idx.shape)}")
        if k_cap is not None and sel_idx.shape[2] != k_cap:
            raise ValueError(f"sel_idx must have k_cap = {k_cap} columns")
    _shape("sel_cnt", sel_cnt, (B, H_sel))
    if sel_blk is not None:
        if sel_idx is None:
            raise ValueError("sel_blk needs sel_idx")
        _shape("sel_blk", sel_blk, sel_idx.shape)


def _cache(kv_cache, D, dev):
    """kv_cache bf16 [2, num_blocks, P, H_kv, D]; returns (NB, P, H_kv)."""
    _check("kv_cache", kv_cache, torch.bfloat16, 5, dev)
    two, NB, P, H_kv, D2 = kv_cache.shape
    if two != 2:
        raise ValueError("kv_cache must be [2, num_blocks, page_size, H_kv, D]")
    if D2 != D:
        raise ValueError("q and kv_cache head dims differ")
    return NB, P, H_kv


def _score_args(q, k_min, k_max, k_mean, block_table, seq_lens, scores, H_out):
    _check("q", q, torch.float32, 3)
    dev = q.device
    B, H_q, D = q.shape
    _, H_kv = _stats(k_min, k_max, k_mean, D, dev)
    _check("block_table", block_table, torch.int32, 2, dev)
    _check("seq_lens", seq_lens, torch.int32, 1, dev)
    _batch(B, block_table, seq_lens)
    _check("scores", scores, torch.float32, 3, dev)
    if tuple(scores.shape[:2]) != (B, H_out(H_q, H_kv)):
        raise ValueError(f"scores must be [{B}, {H_out(H_q, H_kv)}, score_ld], "
                         f"got {tuple(scores.shape)}")
    return B, H_q, H_kv, D


def _alibi_arg(alibi, H_q, dev):
    if alibi is None:
        return None
    _check("alibi", alibi, torch.float32, 1, dev)
    if alibi.shape[0] != H_q:
        raise ValueError("ALiBi slopes must be [H_q]")
    return alibi


def page_score(q, k_min, k_max, k_mean, block_table, seq_lens, page_size,
               w_avg, w_peak, scores, stream=None):
    """scores[b, i, p] ([B, H_q, score_ld]) for p < N_b from the page statistics."""
    lib = load_library()
    B, H_q, H_kv, D = _score_args(q, k_min, k_max, k_mean, block_table, seq_lens,
                                  scores, lambda hq, hkv: hq)
    _rc("page_score", lib.page_score(
        _ptr(q), B, H_q, H_kv, D, _ptr(k_min), _ptr(k_max), _ptr(k_mean),
        _ptr(block_table), block_table.shape[1], _ptr(seq_lens), int(page_size),
        float(w_avg), float(w_peak), _ptr(scores), scores.shape[2], _stream(stream)))


def page_score_ex(q, k_min, k_max, k_mean, block_table, seq_lens, page_size,
                  w_avg, w_peak, scores, alibi=None, stream=None):
    """page_score with ALiBi heads: alibi ([H_q], optional) = ALiBi slopes
    divided by the softmax scale."""
    lib = load_library()
    B, H_q, H_kv, D = _score_args(q, k_min, k_max, k_mean, block_table, seq_lens,
                                  scores, lambda hq, hkv: hq)
    alibi = _alibi_arg(alibi, H_q, q.device)
    _rc("page_score_ex", lib.page_score_ex(
        _ptr(q), B, H_q, H_kv, D, _ptr(k_min), _ptr(k_max), _ptr(k_mean),
        _ptr(block_table), block_table.shape[1], _ptr(seq_lens), int(page_size),
        float(w_avg), float(w_peak), _ptr(scores), scores.shape[2], _ptr(alibi),
        _stream(stream)))


def page_score_group(q, k_min, k_max, k_mean, block_table, seq_lens, page_size,
                     w_avg, w_peak, scores, alibi=None, stream=None):
    """scores[b, h, p] ([B, H_kv, score_ld]): the mean of the kv head's query
    group's page scores, for one selection per kv head."""
    lib = load_library()
    B, H_q, H_kv, D = _score_args(q, k_min, k_max, k_mean, block_table, seq_lens,
                                  scores, lambda hq, hkv: hkv)
    alibi = _alibi_arg(alibi, H_q, q.device)
    _rc("page_score_group", lib.page_score_group(
        _ptr(q), B, H_q, H_kv, D, _ptr(k_min), _ptr(k_max), _ptr(k_mean),
        _ptr(block_table), block_table.shape[1], _ptr(seq_lens), int(page_size),
        float(w_avg), float(w_peak), _ptr(scores), scores.shape[2], _ptr(alibi),
        _stream(stream)))


def _topk_args(scores, seq_lens, sel_idx, sel_cnt):
    _check("scores", scores, torch.float32, 3)
    dev = scores.device
    B, H_sel, ld = scores.shape
    _check("seq_lens", seq_lens, torch.int32, 1, dev)
    _batch(B, None, seq_lens)
    if sel_idx is None or sel_cnt is None:
        raise ValueError("sel_idx and sel_cnt are required")
    _selection(sel_idx, sel_cnt, None, B, H_sel, dev)
    return dev, B, H_sel, ld


def page_topk(scores, seq_lens, page_size, topk_pages, sel_idx, sel_cnt,
              topk_frac=0.0, reserved_bos=0, reserved_eos=1, stream=None):
    """Top-k rows of scores [B, H_sel, score_ld] into sel_idx [B, H_sel, k_cap]
    and sel_cnt [B, H_sel]."""
    lib = load_library()
    _, B, H_sel, ld = _topk_args(scores, seq_lens, sel_idx, sel_cnt)
    _rc("page_topk", lib.page_topk(
        _ptr(scores), ld, B, H_sel, _ptr(seq_lens), int(page_size), int(topk_pages),
        float(topk_frac), int(reserved_bos), int(reserved_eos), _ptr(sel_idx),
        _ptr(sel_cnt), sel_idx.shape[2], _stream(stream)))


def page_topk_blk(scores, seq_lens, page_size, topk_pages, sel_idx, sel_cnt,
                  block_table, sel_blk, topk_frac=0.0, reserved_bos=0, reserved_eos=1,
                  stream=None):
    """page_topk that also writes the selected pages' physical blocks
    (sel_blk, like sel_idx; None = page_topk's result only)."""
    lib = load_library()
    dev, B, H_sel, ld = _topk_args(scores, seq_lens, sel_idx, sel_cnt)
    _check("block_table", block_table, torch.int32, 2, dev)
    _batch(B, block_table, seq_lens)
    _selection(sel_idx, sel_cnt, sel_blk, B, H_sel, dev)
    _rc("page_topk_blk", lib.page_topk_blk(
        _ptr(scores), ld, B, H_sel, _ptr(seq_lens), int(page_size), int(topk_pages),
        float(topk_frac), int(reserved_bos), int(reserved_eos), _ptr(sel_idx),
        _ptr(sel_cnt), sel_idx.shape[2], _ptr(block_table), block_table.shape[1],
        _ptr(sel_blk), _stream(stream)))


def _decode_args(q, kv_cache, block_table, seq_lens, sel_idx, sel_cnt, sel_blk,
                 H_sel=None):
    _check("q", q, torch.float32, 3)
    dev = q.device
    B, H_q, D = q.shape
    NB, P, H_kv = _cache(kv_cache, D, dev)
    _check("block_table", block_table, torch.int32, 2, dev)
    _check("seq_lens", seq_lens, torch.int32, 1, dev)
    _batch(B, block_table, seq_lens)
    if sel_idx is None or sel_cnt is None:
        raise ValueError("sel_idx and sel_cnt are required")
    _check("sel_idx", sel_idx, torch.int32, 3, dev)
    if H_sel is None:
        H_sel = sel_idx.shape[1]
    if H_sel not in (H_q, H_kv):
        raise ValueError(f"the selection must have H_q = {H_q} or H_kv = {H_kv} rows "
                         f"per request, got {H_sel}")
    _selection(sel_idx, sel_cnt, sel_blk, B, H_sel, dev)
    return dev, B, H_q, D, NB, P, H_kv, H_sel


def _partials(o_part, lse_part, B, H_q, D, dev, num_splits=None):
    _check("o_part", o_part, torch.float32, 4, dev)
    _check("lse_part", lse_part, torch.float32, 3, dev)
    ns = o_part.shape[2] if num_splits is None else int(num_splits)
    _shape("o_part", o_part, (B, H_q, ns, D))
    _shape("lse_part", lse_part, (B, H_q, ns))
    return ns


def _outputs(out, lse_out, B, H_q, D, dev, required=True):
    if required and out is None:
        raise ValueError("out is required")
    _check("out", out, torch.float32, 3, dev)
    _check("lse_out", lse_out, torch.float32, 2, dev)
    _shape("out", out, (B, H_q, D))
    _shape("lse_out", lse_out, (B, H_q))


def sparse_paged_decode(q, kv_cache, block_table, seq_lens, sel_idx, sel_cnt,
                        scale, o_part, lse_part, stream=None):
    """Split-K partials over the selected pages.  H_sel = sel_idx.shape[1];
    num_splits = o_part.shape[2]."""
    lib = load_library()
    dev, B, H_q, D, NB, P, H_kv, H_sel = _decode_args(q, kv_cache, block_table, seq_lens,
                                                      sel_idx, sel_cnt, None)
    ns = _partials(o_part, lse_part, B, H_q, D, dev)
    _rc("sparse_paged_decode", lib.sparse_paged_decode(
        _ptr(q), B, H_q, H_kv, D, _ptr(kv_cache), NB, P, _ptr(block_table),
        block_table.shape[1], _ptr(seq_lens), _ptr(sel_idx), _ptr(sel_cnt),
        sel_idx.shape[2], H_sel, float(scale), ns, _ptr(o_part), _ptr(lse_part),
        _stream(stream)))


def sparse_paged_decode_ex(q, kv_cache, block_table, seq_lens, sel_idx, sel_cnt,
                           scale, o_part, lse_part, sel_blk=None, alibi_slopes=None,
                           stream=None):
    """sparse_paged_decode with page_topk_blk's block ids (sel_blk) and ALiBi
    slopes ([H_q], logit units); both optional."""
    lib = load_library()
    dev, B, H_q, D, NB, P, H_kv, H_sel = _decode_args(q, kv_cache, block_table, seq_lens,
                                                      sel_idx, sel_cnt, sel_blk)
    ns = _partials(o_part, lse_part, B, H_q, D, dev)
    alibi_slopes = _alibi_arg(alibi_slopes, H_q, dev)
    _rc("sparse_paged_decode_ex", lib.sparse_paged_decode_ex(
        _ptr(q), B, H_q, H_kv, D, _ptr(kv_cache), NB, P, _ptr(block_table),
        block_table.shape[1], _ptr(seq_lens), _ptr(sel_idx), _ptr(sel_cnt),
        _ptr(sel_blk), sel_idx.shape[2], H_sel, float(scale), ns, _ptr(o_part),
        _ptr(lse_part), _ptr(alibi_slopes), _stream(stream)))


def sparse_paged_decode_merged(q, kv_cache, block_table, seq_lens, sel_idx, sel_cnt,
                               scale, num_splits, out, lse_out=None, o_part=None,
                               lse_part=None, sel_blk=None, alibi_slopes=None,
                               stream=None):
    """Decode with one selection per query head and the split merge in the same
    launch: out [B, H_q, D] (and lse_out [B, H_q]); num_splits <= 8."""
    lib = load_library()
    dev, B, H_q, D, NB, P, H_kv, _ = _decode_args(q, kv_cache, block_table, seq_lens,
                                                  sel_idx, sel_cnt, sel_blk, H_sel=q.shape[1])
    _outputs(out, lse_out, B, H_q, D, dev)
    if (o_part is None) != (lse_part is None):
        raise ValueError("o_part and lse_part go together")
    if o_part is not None:
        _partials(o_part, lse_part, B, H_q, D, dev, num_splits)
    alibi_slopes = _alibi_arg(alibi_slopes, H_q, dev)
    _rc("sparse_paged_decode_merged", lib.sparse_paged_decode_merged(
        _ptr(q), B, H_q, H_kv, D, _ptr(kv_cache), NB, P, _ptr(block_table),
        block_table.shape[1], _ptr(seq_lens), _ptr(sel_idx), _ptr(sel_cnt),
        _ptr(sel_blk), sel_idx.shape[2], float(scale), int(num_splits), _ptr(o_part),
        _ptr(lse_part), _ptr(alibi_slopes), _ptr(out), _ptr(lse_out), _stream(stream)))


def entmax_scratch_floats(B, H_q, k_cap, page_size):
    """Floats of scratch entmax15_paged_decode needs."""
    n = load_library().entmax_scratch_floats(int(B), int(H_q), int(k_cap), int(page_size))
    if n < 0:
        raise ValueError("bad arguments to entmax_scratch_floats")
    return int(n)


def entmax15_paged_decode(q, kv_cache, block_table, seq_lens, sel_idx, sel_cnt, scale,
                          o_part, lse_part, scratch, sel_blk=None, alibi_slopes=None,
                          stream=None):
    """1.5-entmax attention over the selected pages as split partials
    (o_part [B, H_q, splits, D], lse_part = ln of each split's mass), to be
    combined by lse_merge.  alibi_slopes ([H_q], logit units) adds
    slope * (pos - (S - 1)) to each logit."""
    lib = load_library()
    dev, B, H_q, D, NB, P, H_kv, H_sel = _decode_args(q, kv_cache, block_table, seq_lens,
                                                      sel_idx, sel_cnt, sel_blk)
    ns = _partials(o_part, lse_part, B, H_q, D, dev)
    if scratch is None:
        raise ValueError("scratch is required")
    _check("scratch", scratch, torch.float32, 1, dev)
    alibi_slopes = _alibi_arg(alibi_slopes, H_q, dev)
    _rc("entmax15_paged_decode", lib.entmax15_paged_decode(
        _ptr(q), B, H_q, H_kv, D, _ptr(kv_cache), NB, P, _ptr(block_table),
        block_table.shape[1], _ptr(seq_lens), _ptr(sel_idx), _ptr(sel_cnt), _ptr(sel_blk),
        sel_idx.shape[2], H_sel, float(scale), ns, _ptr(alibi_slopes), _ptr(o_part),
        _ptr(lse_part), _ptr(scratch), scratch.numel(), _stream(stream)))


def entmax15_paged_decode_merged(q, kv_cache, block_table, seq_lens, sel_idx, sel_cnt,
                                 scale, out, lse_out=None, tau_out=None, scratch=None,
                                 sel_blk=None, alibi_slopes=None, stream=None):
    """1.5-entmax attention over the selected pages in one launch: out
    [B, H_q, D] = sum p v / sum p; lse_out, tau_out [B, H_q] optional; scratch
    (fp32, B * H_q * k_cap * P floats) only when k_cap * P > 8192."""
    lib = load_library()
    dev, B, H_q, D, NB, P, H_kv, H_sel = _decode_args(q, kv_cache, block_table, seq_lens,
                                                      sel_idx, sel_cnt, sel_blk)
    _outputs(out, lse_out, B, H_q, D, dev)
    _check("tau_out", tau_out, torch.float32, 2, dev)
    _shape("tau_out", tau_out, (B, H_q))
    _check("scratch", scratch, torch.float32, 1, dev)
    alibi_slopes = _alibi_arg(alibi_slopes, H_q, dev)
    _rc("entmax15_paged_decode_merged", lib.entmax15_paged_decode_merged(
        _ptr(q), B, H_q, H_kv, D, _ptr(kv_cache), NB, P, _ptr(block_table),
        block_table.shape[1], _ptr(seq_lens), _ptr(sel_idx), _ptr(sel_cnt), _ptr(sel_blk),
        sel_idx.shape[2], H_sel, float(scale), _ptr(alibi_slopes), _ptr(out),
        _ptr(lse_out), _ptr(tau_out), _ptr(scratch),
        0 if scratch is None else scratch.numel(), _stream(stream)))


def page_var_update(kv_cache, k_mean, k_var, block_table, seq_lens, tail_only=False,
                    stream=None):
    """Per-page key variance around k_mean ([num_blocks, H_kv, D] fp32), for
    every page (rebuild) or only the page holding each request's last token."""
    lib = load_library()
    _check("kv_cache", kv_cache, torch.bfloat16, 5)
    dev = kv_cache.device
    _, NB, P, H_kv, D = kv_cache.shape
    for n, t in (("k_mean", k_mean), ("k_var", k_var)):
        _check(n, t, torch.float32, 3, dev)
        if t is not None and tuple(t.shape) != (NB, H_kv, D):
            raise ValueError(f"{n} must be [num_blocks, H_kv, D]")
    _check("block_table", block_table, torch.int32, 2, dev)
    _check("seq_lens", seq_lens, torch.int32, 1, dev)
    B = seq_lens.shape[0]
    if block_table.shape[0] != B:
        raise ValueError("block_table rows must equal len(seq_lens)")
    _rc("page_var_update", lib.page_var_update(
        _ptr(kv_cache), NB, P, H_kv, D, _ptr(k_mean), _ptr(k_var), _ptr(block_table),
        block_table.shape[1], _ptr(seq_lens), B, 1 if tail_only else 0, _stream(stream)))


def gauss_moments(q, k_mean, k_var, block_table, seq_lens, page_size, scale, mu, var,
                  alibi_slopes=None, stream=None):
    """mu, var [B, H_q, ld] of each page's logits (Gaussian page model);
    alibi_slopes [H_q] in logit units."""
    lib = load_library()
    _check("q", q, torch.float32, 3)
    dev = q.device
    B, H_q, D = q.shape
    _check("k_mean", k_mean, torch.float32, 3, dev)
    _check("k_var", k_var, torch.float32, 3, dev)
    NB, H_kv, d = k_mean.shape
    if d != D:
        raise ValueError("k_mean and q head dims differ")
    _shape("k_var", k_var, (NB, H_kv, D))
    if H_q % H_kv:
        raise ValueError("H_q must be a multiple of H_kv")
    _check("block_table", block_table, torch.int32, 2, dev)
    _check("seq_lens", seq_lens, torch.int32, 1, dev)
    _batch(B, block_table, seq_lens)
    _check("mu", mu, torch.float32, 3, dev)
    _check("var", var, torch.float32, 3, dev)
    if mu is None or var is None:
        raise ValueError("mu and var are required")
    if tuple(mu.shape[:2]) != (B, H_q) or mu.shape != var.shape:
        raise ValueError("mu and var must be [B, H_q, ld]")
    alibi_slopes = _alibi_arg(alibi_slopes, H_q, dev)
    _rc("gauss_moments", lib.gauss_moments(
        _ptr(q), B, H_q, H_kv, D, _ptr(k_mean), _ptr(k_var), _ptr(block_table),
        block_table.shape[1], _ptr(seq_lens), int(page_size), float(scale),
        _ptr(alibi_slopes), _ptr(mu), _ptr(var), mu.shape[2], _stream(stream)))


def gauss_select(mu, var, seq_lens, page_size, block_table, mixture, k_cap, est, sel_idx,
                 sel_cnt, tau=None, sel_blk=None, reserved_bos=0, reserved_eos=1,
                 stream=None):
    """tau-hat and the adaptive page selection of every (request, query head):
    est [B, H_q, ld] receives the estimated page maxima, sel_idx
    [B, H_q, k_cap] / sel_cnt [B, H_q] the selection (as page_topk's)."""
    lib = load_library()
    _check("mu", mu, torch.float32, 3)
    dev = mu.device
    B, H_q, ld = mu.shape
    _check("var", var, torch.float32, 3, dev)
    _check("est", est, torch.float32, 3, dev)
    _check("seq_lens", seq_lens, torch.int32, 1, dev)
    _check("block_table", block_table, torch.int32, 2, dev)
    _batch(B, block_table, seq_lens)
    _check("tau", tau, torch.float32, 2, dev)
    if var is None or est is None or var.shape != mu.shape or est.shape != mu.shape:
        raise ValueError("mu, var and est must share the shape [B, H_q, ld]")
    if sel_idx is None or sel_cnt is None:
        raise ValueError("sel_idx and sel_cnt are required")
    _selection(sel_idx, sel_cnt, sel_blk, B, H_q, dev, int(k_cap))
    _shape("tau", tau, (B, H_q))
    _rc("gauss_select", lib.gauss_select(
        _ptr(mu), _ptr(var), ld, B, H_q, _ptr(seq_lens), int(page_size), _ptr(block_table),
        block_table.shape[1], 1 if mixture else 0, int(reserved_bos), int(reserved_eos),
        int(k_cap), _ptr(tau), _ptr(est), _ptr(sel_idx), _ptr(sel_cnt), _ptr(sel_blk),
        _stream(stream)))


def _optional_selection(sel_idx, sel_cnt, sel_blk, B, H_q, k_cap, dev):
    if (sel_idx is None) != (sel_cnt is None):
        raise ValueError("sel_idx and sel_cnt go together")
    if sel_blk is not None and sel_idx is None:
        raise ValueError("sel_blk needs sel_idx")
    _selection(sel_idx, sel_cnt, sel_blk, B, H_q, dev, int(k_cap))


def sparse_select_decode(scores, q, kv_cache, block_table, seq_lens, topk_pages, k_cap,
                         scale, num_splits, out, lse_out=None, topk_frac=0.0,
                         reserved_bos=0, reserved_eos=1, sel_idx=None, sel_cnt=None,
                         sel_blk=None, alibi_slopes=None, stream=None):
    """page_topk + sparse_paged_decode_merged in one launch (one selection per
    query head, score_ld <= 4096, num_splits <= 8); optionally writes the
    selection like page_topk_blk."""
    lib = load_library()
    _check("q", q, torch.float32, 3)
    dev = q.device
    B, H_q, D = q.shape
    _check("scores", scores, torch.float32, 3, dev)
    NB, P, H_kv = _cache(kv_cache, D, dev)
    if scores is None or tuple(scores.shape[:2]) != (B, H_q):
        raise ValueError("scores must be [B, H_q, score_ld]")
    _check("block_table", block_table, torch.int32, 2, dev)
    _check("seq_lens", seq_lens, torch.int32, 1, dev)
    _batch(B, block_table, seq_lens)
    _outputs(out, lse_out, B, H_q, D, dev)
    _optional_selection(sel_idx, sel_cnt, sel_blk, B, H_q, k_cap, dev)
    alibi_slopes = _alibi_arg(alibi_slopes, H_q, dev)
    _rc("sparse_select_decode", lib.sparse_select_decode(
        _ptr(scores), scores.shape[2], int(topk_pages), float(topk_frac), int(reserved_bos),
        int(reserved_eos), _ptr(q), B, H_q, H_kv, D, _ptr(kv_cache), NB, P,
        _ptr(block_table), block_table.shape[1], _ptr(seq_lens), int(k_cap), float(scale),
        int(num_splits), _ptr(alibi_slopes), _ptr(out), _ptr(lse_out), _ptr(sel_idx),
        _ptr(sel_cnt), _ptr(sel_blk), _stream(stream)))


def sparse_select_decode_group(scores, q, kv_cache, block_table, seq_lens, topk_pages,
                               k_cap, scale, o_part, lse_part, topk_frac=0.0, reserved_bos=0,
                               reserved_eos=1, sel_idx=None, sel_cnt=None, sel_blk=None,
                               alibi_slopes=None, stream=None):
    """page_topk + sparse_paged_decode in one launch for one selection per kv
    head (scores [B, H_kv, score_ld], score_ld <= 8192): the split partials
    o_part [B, H_q, splits, D] / lse_part [B, H_q, splits] (num_splits =
    o_part.shape[2]); optionally writes the selection like page_topk_blk."""
    lib = load_library()
    _check("q", q, torch.float32, 3)
    dev = q.device
    B, H_q, D = q.shape
    _check("scores", scores, torch.float32, 3, dev)
    NB, P, H_kv = _cache(kv_cache, D, dev)
    if scores is None or tuple(scores.shape[:2]) != (B, H_kv):
        raise ValueError("scores must be [B, H_kv, score_ld]")
    _check("block_table", block_table, torch.int32, 2, dev)
    _check("seq_lens", seq_lens, torch.int32, 1, dev)
    _batch(B, block_table, seq_lens)
    if o_part is None or lse_part is None:
        raise ValueError("o_part and lse_part are required")
    ns = _partials(o_part, lse_part, B, H_q, D, dev)
    _optional_selection(sel_idx, sel_cnt, sel_blk, B, H_kv, k_cap, dev)
    alibi_slopes = _alibi_arg(alibi_slopes, H_q, dev)
    _rc("sparse_select_decode_group", lib.sparse_select_decode_group(
        _ptr(scores), scores.shape[2], int(topk_pages), float(topk_frac), int(reserved_bos),
        int(reserved_eos), _ptr(q), B, H_q, H_kv, D, _ptr(kv_cache), NB, P,
        _ptr(block_table), block_table.shape[1], _ptr(seq_lens), int(k_cap), float(scale),
        ns, _ptr(alibi_slopes), _ptr(o_part), _ptr(lse_part), _ptr(sel_idx), _ptr(sel_cnt),
        _ptr(sel_blk), _stream(stream)))


def sparse_select_decode_split(scores, q, kv_cache, block_table, seq_lens, topk_pages,
                               k_cap, scale, o_part, lse_part, topk_frac=0.0, reserved_bos=0,
                               reserved_eos=1, sel_idx=None, sel_cnt=None, sel_blk=None,
                               alibi_slopes=None, stream=None):
    """page_topk + sparse_paged_decode in one launch for one selection per
    query head (scores [B, H_q, score_ld], score_ld <= 8192) at any split
    count: the split partials o_part [B, H_q, splits, D] / lse_part
    [B, H_q, splits] (num_splits = o_part.shape[2]) for lse_merge;
    optionally writes the selection like page_topk_blk."""
    lib = load_library()
    _check("q", q, torch.float32, 3)
    dev = q.device
    B, H_q, D = q.shape
    _check("scores", scores, torch.float32, 3, dev)
    NB, P, H_kv = _cache(kv_cache, D, dev)
    if scores is None or tuple(scores.shape[:2]) != (B, H_q):
        raise ValueError("scores must be [B, H_q, score_ld]")
    _check("block_table", block_table, torch.int32, 2, dev)
    _check("seq_lens", seq_lens, torch.int32, 1, dev)
    _batch(B, block_table, seq_lens)
    if o_part is None or lse_part is None:
        raise ValueError("o_part and lse_part are required")
    ns = _partials(o_part, lse_part, B, H_q, D, dev)
    _optional_selection(sel_idx, sel_cnt, sel_blk, B, H_q, k_cap, dev)
    alibi_slopes = _alibi_arg(alibi_slopes, H_q, dev)
    _rc("sparse_select_decode_split", lib.sparse_select_decode_split(
        _ptr(scores), scores.shape[2], int(topk_pages), float(topk_frac), int(reserved_bos),
        int(reserved_eos), _ptr(q), B, H_q, H_kv, D, _ptr(kv_cache), NB, P,
        _ptr(block_table), block_table.shape[1], _ptr(seq_lens), int(k_cap), float(scale),
        ns, _ptr(alibi_slopes), _ptr(o_part), _ptr(lse_part), _ptr(sel_idx), _ptr(sel_cnt),
        _ptr(sel_blk), _stream(stream)))


def sparse_select_decode_split_blocks_count(num_splits, page_size) -> int:
    """Partials per query head that sparse_select_decode_split_blocks writes."""
    n = load_library().sparse_select_decode_split_blocks_count(int(num_splits), int(page_size))
    if n < 0:
        raise ValueError(f"no block count for num_splits={num_splits}, page_size={page_size}")
    return n


def sparse_select_decode_split_blocks(scores, q, kv_cache, block_table, seq_lens, topk_pages,
                                      k_cap, scale, num_splits, o_part, lse_part,
                                      topk_frac=0.0, reserved_bos=0, reserved_eos=1,
                                      sel_idx=None, sel_cnt=None, sel_blk=None,
                                      alibi_slopes=None, stream=None):
    """sparse_select_decode_split whose blocks merge their splits: o_part
    [B, H_q, nb, D] / lse_part [B, H_q, nb] receive one partial per block,
    nb = sparse_select_decode_split_blocks_count(num_splits, page_size), for
    lse_merge."""
    lib = load_library()
    _check("q", q, torch.float32, 3)
    dev = q.device
    B, H_q, D = q.shape
    _check("scores", scores, torch.float32, 3, dev)
    NB, P, H_kv = _cache(kv_cache, D, dev)
    if scores is None or tuple(scores.shape[:2]) != (B, H_q):
        raise ValueError("scores must be [B, H_q, score_ld]")
    _check("block_table", block_table, torch.int32, 2, dev)
    _check("seq_lens", seq_lens, torch.int32, 1, dev)
    _batch(B, block_table, seq_lens)
    if o_part is None or lse_part is None:
        raise ValueError("o_part and lse_part are required")
    nb = sparse_select_decode_split_blocks_count(num_splits, P)
    _partials(o_part, lse_part, B, H_q, D, dev, num_splits=nb)
    _optional_selection(sel_idx, sel_cnt, sel_blk, B, H_q, k_cap, dev)
    alibi_slopes = _alibi_arg(alibi_slopes, H_q, dev)
    _rc("sparse_select_decode_split_blocks", lib.sparse_select_decode_split_blocks(
        _ptr(scores), scores.shape[2], int(topk_pages), float(topk_frac), int(reserved_bos),
        int(reserved_eos), _ptr(q), B, H_q, H_kv, D, _ptr(kv_cache), NB, P,
        _ptr(block_table), block_table.shape[1], _ptr(seq_lens), int(k_cap), float(scale),
        int(num_splits), _ptr(alibi_slopes), _ptr(o_part), _ptr(lse_part), _ptr(sel_idx),
        _ptr(sel_cnt), _ptr(sel_blk), _stream(stream)))


def sparse_page_decode(q, kv_cache, k_min, k_max, k_mean, block_table, seq_lens, w_avg,
                       w_peak, topk_pages, k_cap, scale, num_splits, out, lse_out=None,
                       topk_frac=0.0, reserved_bos=0, reserved_eos=1, scores=None,
                       sel_idx=None, sel_cnt=None, sel_blk=None, alibi_slopes=None,
                       stream=None):
    """The page-level step in one launch (score, select, decode, merge; one
    selection per query head, bt_ld <= 4096, num_splits <= 8)."""
    lib = load_library()
    _check("q", q, torch.float32, 3)
    dev = q.device
    B, H_q, D = q.shape
    NB, P, H_kv = _cache(kv_cache, D, dev)
    _stats(k_min, k_max, k_mean, D, dev, NB)
    if k_min.shape[1] != H_kv:
        raise ValueError("page statistics and kv_cache kv-head counts differ")
    _check("block_table", block_table, torch.int32, 2, dev)
    _check("seq_lens", seq_lens, torch.int32, 1, dev)
    _batch(B, block_table, seq_lens)
    _outputs(out, lse_out, B, H_q, D, dev)
    bt_ld = block_table.shape[1]
    _check("scores", scores, torch.float32, 3, dev)
    _shape("scores", scores, (B, H_q, bt_ld))
    _optional_selection(sel_idx, sel_cnt, sel_blk, B, H_q, k_cap, dev)
    alibi_slopes = _alibi_arg(alibi_slopes, H_q, dev)
    _rc("sparse_page_decode", lib.sparse_page_decode(
        _ptr(q), B, H_q, H_kv, D, _ptr(kv_cache), NB, P, _ptr(k_min), _ptr(k_max),
        _ptr(k_mean), _ptr(block_table), bt_ld, _ptr(seq_lens), float(w_avg), float(w_peak),
        int(topk_pages), float(topk_frac), int(reserved_bos), int(reserved_eos), int(k_cap),
        float(scale), int(num_splits), _ptr(alibi_slopes), _ptr(out), _ptr(lse_out),
        _ptr(scores), _ptr(sel_idx), _ptr(sel_cnt), _ptr(sel_blk), _stream(stream)))


def lse_merge(o_part, lse_part, out, lse_out=None, stream=None):
    """Merge [..., splits, D] partials into out [..., D] (and lse_out [...])."""
    lib = load_library()
    _check("o_part", o_part, torch.float32)
    dev = o_part.device
    _check("lse_part", lse_part, torch.float32, None, dev)
    _check("out", out, torch.float32, None, dev)
    _check("lse_out", lse_out, torch.float32, None, dev)
    if o_part.dim() < 2 or lse_part is None or out is None:
        raise ValueError("o_part [..., splits, D], lse_part and out are required")
    lead = tuple(o_part.shape[:-2])
    ns, D = o_part.shape[-2], o_part.shape[-1]
    _shape("lse_part", lse_part, lead + (ns,))
    _shape("out", out, lead + (D,))
    _shape("lse_out", lse_out, lead)
    rows = o_part.numel() // (ns * D) if o_part.numel() else 0
    _rc("lse_merge", lib.lse_merge(_ptr(o_part), _ptr(lse_part), rows, ns, D,
                                   _ptr(out), _ptr(lse_out), _stream(stream)))


def h2o_scratch_floats(B, H_kv, max_tokens) -> int:
    return int(load_library().h2o_scratch_floats(int(B), int(H_kv), int(max_tokens)))


def h2o_heads_scratch_floats(B, H_q, max_tokens) -> int:
    return int(load_library().h2o_heads_scratch_floats(int(B), int(H_q), int(max_tokens)))


def _h2o(name, q, kv_cache, block_table, seq_lens, hh_score, scores, scratch, scale,
         decay, reserved_bos, reserved_eos, stream):
    lib = load_library()
    _check("q", q, torch.float32, 3)
    dev = q.device
    B, H_q, D = q.shape
    NB, P, H_kv = _cache(kv_cache, D, dev)
    _check("block_table", block_table, torch.int32, 2, dev)
    _check("seq_lens", seq_lens, torch.int32, 1, dev)
    _batch(B, block_table, seq_lens)
    for n, t in (("hh_score", hh_score), ("scores", scores), ("scratch", scratch)):
        if t is None:
            raise ValueError(f"{n} is required")
    _check("hh_score", hh_score, torch.bfloat16, 2, dev)
    _check("scores", scores, torch.float32, 3, dev)
    _check("scratch", scratch, torch.float32, 1, dev)
    _shape("hh_score", hh_score, (NB * P, H_kv))
    if tuple(scores.shape[:2]) != (B, H_kv):
        raise ValueError("scores must be [B, H_kv, score_ld]")
    _rc(name, getattr(lib, name)(
        _ptr(q), B, H_q, H_kv, D, _ptr(kv_cache), NB, P, _ptr(block_table),
        block_table.shape[1], _ptr(seq_lens), int(reserved_bos), int(reserved_eos),
        float(scale), float(decay), _ptr(hh_score), _ptr(scores), scores.shape[2],
        _ptr(scratch), scratch.numel(), _stream(stream)))


def h2o_select_decode_scratch_floats(B, H_q, H_kv, max_tokens, per_head=False) -> int:
    return int(load_library().h2o_select_decode_scratch_floats(
        int(B), int(H_q), int(H_kv), int(max_tokens), 1 if per_head else 0))


def h2o_select_decode(q, kv_cache, block_table, seq_lens, hh_score, scratch, scale,
                      topk_pages, k_cap, o_part, lse_part, decay=0.984375, reserved_bos=0,
                      reserved_eos=1, per_head=False, scores=None, topk_frac=0.0,
                      sel_idx=None, sel_cnt=None, sel_blk=None, k_new=None, v_new=None,
                      stream=None):
    """Token-level accumulate + per-kv-head selection + decode in two launches:
    hh_score updated in place, split partials o_part [B, H_q, splits, D] /
    lse_part [B, H_q, splits] (num_splits = o_part.shape[2]) for lse_merge;
    scores [B, H_kv, score_ld] and the selection are optional copies.  With
    k_new / v_new [B, H_kv, D] bf16 the step's append (cache rows and hh slot
    of token S - 1) is done in the first launch."""
    lib = load_library()
    _check("q", q, torch.float32, 3)
    dev = q.device
    B, H_q, D = q.shape
    NB, P, H_kv = _cache(kv_cache, D, dev)
    _check("block_table", block_table, torch.int32, 2, dev)
    _check("seq_lens", seq_lens, torch.int32, 1, dev)
    _batch(B, block_table, seq_lens)
    for n, t in (("hh_score", hh_score), ("scratch", scratch), ("o_part", o_part),
                 ("lse_part", lse_part)):
        if t is None:
            raise ValueError(f"{n} is required")
    _check("hh_score", hh_score, torch.bfloat16, 2, dev)
    _shape("hh_score", hh_score, (NB * P, H_kv))
    _check("scratch", scratch, torch.float32, 1, dev)
    ns = _partials(o_part, lse_part, B, H_q, D, dev)
    _check("scores", scores, torch.float32, 3, dev)
    if scores is not None and tuple(scores.shape[:2]) != (B, H_kv):
        raise ValueError("scores must be [B, H_kv, score_ld]")
    _optional_selection(sel_idx, sel_cnt, sel_blk, B, H_kv, k_cap, dev)
    if (k_new is None) != (v_new is None):
        raise ValueError("k_new and v_new must be given together")
    for n, t in (("k_new", k_new), ("v_new", v_new)):
        _check(n, t, torch.bfloat16, 3, dev)
        if t is not None:
            _shape(n, t, (B, H_kv, D))
    _rc("h2o_select_decode", lib.h2o_select_decode(
        _ptr(q), B, H_q, H_kv, D, _ptr(kv_cache), NB, P, _ptr(block_table),
        block_table.shape[1], _ptr(seq_lens), int(reserved_bos), int(reserved_eos),
        float(scale), float(decay), 1 if per_head else 0, _ptr(hh_score), _ptr(scores),
        0 if scores is None else scores.shape[2], int(topk_pages), float(topk_frac),
        int(k_cap), ns, _ptr(o_part), _ptr(lse_part), _ptr(sel_idx), _ptr(sel_cnt),
        _ptr(sel_blk), _ptr(k_new), _ptr(v_new), _ptr(scratch), scratch.numel(),
        _stream(stream)))


def h2o_accumulate(q, kv_cache, block_table, seq_lens, hh_score, scores, scratch,
                   scale, decay=0.984375, reserved_bos=0, reserved_eos=1,
                   stream=None):
    """Token-level H2O step (page_size 1), group-mean query: updates hh_score in
    place and writes the new values as scores [B, H_kv, score_ld]."""
    _h2o("h2o_accumulate", q, kv_cache, block_table, seq_lens, hh_score, scores,
         scratch, scale, decay, reserved_bos, reserved_eos, stream)


def h2o_accumulate_heads(q, kv_cache, block_table, seq_lens, hh_score, scores, scratch,
                         scale, decay=0.984375, reserved_bos=0, reserved_eos=1,
                         stream=None):
    """The same step with every query head's own softmax, averaged over its
    group; scratch of h2o_heads_scratch_floats(B, H_q, bt_ld) floats."""
    _h2o("h2o_accumulate_heads", q, kv_cache, block_table, seq_lens, hh_score, scores,
         scratch, scale, decay, reserved_bos, reserved_eos, stream)


def h2o_accumulate_noalloc(q, kv_cache, block_table, seq_lens, hh_score, scores, scale,
                           decay=0.984375, reserved_bos=0, reserved_eos=1, stream=None):
    """h2o_accumulate with the library's fixed scratch buffer: no device memory
    is allocated by the call (nor by this wrapper).  Needs
    h2o_scratch_floats(B, H_kv, bt_ld) <= NOALLOC_SCRATCH_FLOATS; calls that
    overlap on one GPU share that buffer and race."""
    lib = load_library()
    _check("q", q, torch.float32, 3)
    dev = q.device
    B, H_q, D = q.shape
    NB, P, H_kv = _cache(kv_cache, D, dev)
    _check("block_table", block_table, torch.int32, 2, dev)
    _check("seq_lens", seq_lens, torch.int32, 1, dev)
    _batch(B, block_table, seq_lens)
    for n, t in (("hh_score", hh_score), ("scores", scores)):
        if t is None:
            raise ValueError(f"{n} is required")
    _check("hh_score", hh_score, torch.bfloat16, 2, dev)
    _check("scores", scores, torch.float32, 3, dev)
    _shape("hh_score", hh_score, (NB * P, H_kv))
    if tuple(scores.shape[:2]) != (B, H_kv):
        raise ValueError("scores must be [B, H_kv, score_ld]")
    _rc("h2o_accumulate_noalloc", lib.h2o_accumulate_noalloc(
        _ptr(q), B, H_q, H_kv, D, _ptr(kv_cache), NB, P, _ptr(block_table),
        block_table.shape[1], _ptr(seq_lens), int(reserved_bos), int(reserved_eos),
        float(scale), float(decay), _ptr(hh_score), _ptr(scores), scores.shape[2],
        _stream(stream)))


# ------------------------------------------------------ bandwidth references

def skv_ref_stream_read(buf, sink, nbytes=None, stream=None):
    """Read nbytes (default: all) of the device tensor buf once, streaming
    (skv_reference.h); sink is a uint32-sized device buffer of >= 1024 words."""
    lib = load_library()
    if not isinstance(buf, torch.Tensor) or not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous GPU tensor")
    _check("sink", sink, torch.int32, 1, buf.device)
    if sink.numel() < 1024:
        raise ValueError("sink must hold 1024 words")
    n = buf.numel() * buf.element_size() if nbytes is None else int(nbytes)
    if n > buf.numel() * buf.element_size():
        raise ValueError("nbytes exceeds the buffer")
    _rc("skv_ref_stream_read", lib.skv_ref_stream_read(_ptr(buf), n, _ptr(sink),
                                                       _stream(stream)))


def skv_ref_gather_read(kv_cache, items, sink, stream=None):
    """Read the K and V rows of the page-heads items [n, 3] = (block, kv head,
    valid rows) of kv_cache (skv_reference.h); sink >= 256 words."""
    lib = load_library()
    _check("kv_cache", kv_cache, torch.bfloat16, 5)
    dev = kv_cache.device
    _, NB, P, H_kv, D = kv_cache.shape
    _check("items", items, torch.int32, 2, dev)
    if items.shape[1] != 3:
        raise ValueError("items must be [n, 3]")
    _check("sink", sink, torch.int32, 1, dev)
    if sink.numel() < 256:
        raise ValueError("sink must hold 256 words")
    _rc("skv_ref_gather_read", lib.skv_ref_gather_read(
        _ptr(kv_cache), NB, P, H_kv, D, _ptr(items), items.shape[0], _ptr(sink),
        _stream(stream)))
