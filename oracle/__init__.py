"""Float64 CPU oracle for page-scored sparse decode attention.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only callers.  The product library never imports,
links or runs anything here, and nothing here imports the product package.

The arithmetic lives in ``sparsekv_oracle.c`` (plain C, float64).  This module
compiles it with gcc (``build()``) and wraps each function for numpy arrays.
Every function is pinned by the ``not gpu`` tests against closed forms,
invariants, brute force or values printed on the pages.  One rule is a
reading the pages do not fix: ``gauss_select``'s estimated maximum
(mu + sigma * sqrt(2 ln n)); its tests pin the code to that reading, and
against the pages it is parity unpinned.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sparsekv_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build() -> str:
    """Compile the oracle into ``oracle/liboracle.so`` (always recompiles)."""
    tmp = _LIB_PATH + ".tmp"
    subprocess.check_call(
        ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-Wall", "-Wextra",
         "-fno-fast-math", _SRC, "-o", tmp, "-lm"])
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or (
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    i32, i64, f64 = ctypes.c_int, ctypes.c_int64, ctypes.c_double
    lib.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_double.restype = f64
    lib.oracle_double_to_bf16.argtypes = [f64]
    lib.oracle_double_to_bf16.restype = ctypes.c_uint16
    lib.oracle_page_stats.argtypes = [P, i64, i32, i32, i32, P, i64, P, i32, P, P, P]
    lib.oracle_page_score.argtypes = [P, i32, i32, i32, i32, P, P, P, P, i64, P,
                                      i32, f64, f64, P, i64]
    lib.oracle_page_score_group.argtypes = [P, i32, i32, i32, i32, P, P, P, P, i64, P,
                                      i32, f64, f64, P, i64]
    lib.oracle_page_score_alibi.argtypes = [P, i32, i32, i32, i32, P, P, P, P, i64, P,
                                            i32, f64, f64, P, i32, P, i64]
    lib.oracle_budget.argtypes = [i32, i32, f64]
    lib.oracle_budget.restype = i32
    lib.oracle_select.argtypes = [P, i32, i32, f64, i32, i32, P]
    lib.oracle_select.restype = i32
    lib.oracle_attend.argtypes = [P, i32, P, i64, i32, i32, i32, P, i32, P, i32,
                                  f64, P, P]
    lib.oracle_attend_alibi.argtypes = [P, i32, P, i64, i32, i32, i32, P, i32, P, i32,
                                        f64, f64, P, P]
    lib.oracle_lse_merge.argtypes = [P, P, i32, i32, P, P]
    lib.oracle_page_var.argtypes = [P, i64, i32, i32, i32, P, i64, P, i32, P]
    lib.oracle_gauss_moments.argtypes = [P, i32, i32, i32, i32, P, P, P, i64, P, i32, f64,
                                         P, P, P, i64]
    lib.oracle_gauss_tau.argtypes = [P, P, P, i32, i32]
    lib.oracle_gauss_tau.restype = f64
    lib.oracle_gauss_select.argtypes = [P, P, P, i32, f64, i32, i32, i32, P]
    lib.oracle_gauss_select.restype = i32
    lib.oracle_entmax15_tau.argtypes = [P, i32]
    lib.oracle_entmax15_tau.restype = f64
    lib.oracle_attend_entmax15.argtypes = [P, i32, P, i64, i32, i32, i32, P, i32, P, i32,
                                           f64, P, P]
    lib.oracle_attend_entmax15_alibi.argtypes = [P, i32, P, i64, i32, i32, i32, P, i32, P,
                                                 i32, f64, f64, P, P]
    lib.oracle_append.argtypes = [P, i64, i32, i32, i32, P, i64, P, i32, P, P, P]
    lib.oracle_h2o_recurrence.argtypes = [P, P, i32, f64]
    lib.oracle_h2o_step.argtypes = [P, i32, i32, i32, i32, P, i64, P, i64, P,
                                    i32, i32, f64, f64, P, P, i64]
    lib.oracle_h2o_step_heads.argtypes = lib.oracle_h2o_step.argtypes
    lib.oracle_decode_step.argtypes = [P, i32, i32, i32, i32, P, i64, i32, P, i64,
                                       P, P, P, P, f64, f64, i32, f64, i32, i32,
                                       f64, P, i64, P, P, i32, P, P]
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    """Contiguous array of the given dtype (copies only when needed)."""
    return np.ascontiguousarray(a, dtype=dtype)


# --------------------------------------------------------------- bf16

def bf16_to_double(bits) -> np.ndarray:
    """Exact decode of bf16 bit patterns (uint16) to float64."""
    lib = _load()
    b = np.asarray(bits, dtype=np.uint16)
    out = np.array([lib.oracle_bf16_to_double(int(x)) for x in b.ravel()])
    return out.reshape(b.shape)


def bf16_decode(bits) -> np.ndarray:
    """Vectorised exact decode (same definition: the bits are the top half of
    an IEEE binary32)."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def double_to_bf16(x) -> np.ndarray:
    """Round-to-nearest-even of float64 values to bf16 bit patterns."""
    lib = _load()
    a = np.asarray(x, dtype=np.float64)
    out = np.array([lib.oracle_double_to_bf16(float(v)) for v in a.ravel()],
                   dtype=np.uint16)
    return out.reshape(a.shape)


# ------------------------------------------------------ the method

def page_stats(kv_cache, block_table, seq_lens, page_size):
    """k_min, k_max, k_mean (float64, [num_blocks, H_kv, D]) of every page of
    every request; unreferenced blocks are NaN."""
    lib = _load()
    kv = _c(kv_cache, np.uint16)
    _, NB, P, H_kv, D = kv.shape
    assert P == page_size
    bt = _c(block_table, np.int32)
    sl = _c(seq_lens, np.int32)
    out = [np.full((NB, H_kv, D), np.nan) for _ in range(3)]
    lib.oracle_page_stats(_ptr(kv), NB, P, H_kv, D, _ptr(bt), bt.shape[1],
                          _ptr(sl), sl.shape[0], *[_ptr(o) for o in out])
    return tuple(out)


def page_score(q, kmin, kmax, kmean, block_table, seq_lens, page_size,
               w_avg, w_peak, ld=None):
    """Page scores [B, H_q, ld] (float64, NaN beyond each row's N_b)."""
    lib = _load()
    qd = _c(q, np.float64)
    B, H_q, D = qd.shape
    mn, mx, me = (_c(a, np.float64) for a in (kmin, kmax, kmean))
    H_kv = mn.shape[1]
    bt = _c(block_table, np.int32)
    sl = _c(seq_lens, np.int32)
    if ld is None:
        ld = bt.shape[1]
    s = np.full((B, H_q, ld), np.nan)
    lib.oracle_page_score(_ptr(qd), B, H_q, H_kv, D, _ptr(mn), _ptr(mx), _ptr(me),
                          _ptr(bt), bt.shape[1], _ptr(sl), page_size,
                          float(w_avg), float(w_peak), _ptr(s), ld)
    return s


def page_score_group(q, kmin, kmax, kmean, block_table, seq_lens, page_size,
                     w_avg, w_peak, ld=None):
    """Group-shared page scores [B, H_kv, ld]: the mean over each kv head's
    query group of the per-head scores (float64, NaN beyond N_b)."""
    lib = _load()
    qd = _c(q, np.float64)
    B, H_q, D = qd.shape
    mn, mx, me = (_c(a, np.float64) for a in (kmin, kmax, kmean))
    H_kv = mn.shape[1]
    bt = _c(block_table, np.int32)
    sl = _c(seq_lens, np.int32)
    if ld is None:
        ld = bt.shape[1]
    s = np.full((B, H_kv, ld), np.nan)
    lib.oracle_page_score_group(_ptr(qd), B, H_q, H_kv, D, _ptr(mn), _ptr(mx),
                                _ptr(me), _ptr(bt), bt.shape[1], _ptr(sl), page_size,
                                float(w_avg), float(w_peak), _ptr(s), ld)
    return s


def budget(N, topk_pages, topk_frac=0.0) -> int:
    return int(_load().oracle_budget(int(N), int(topk_pages), float(topk_frac)))


def select(scores_row, topk_pages, topk_frac=0.0, bos=0, eos=1) -> np.ndarray:
    """Ascending selected indices of one row of N scores."""
    lib = _load()
    s = _c(scores_row, np.float64)
    N = s.shape[0]
    out = np.full(max(N, 1), -1, dtype=np.int32)
    n = lib.oracle_select(_ptr(s), N, int(topk_pages), float(topk_frac),
                          int(bos), int(eos), _ptr(out))
    return out[:n].copy()


def attend(q_row, kv_cache, kv_head, bt_row, seq_len, pages, scale):
    """(o [D], lse) of one query row over the tokens of the given pages."""
    lib = _load()
    qd = _c(q_row, np.float64)
    kv = _c(kv_cache, np.uint16)
    _, NB, P, H_kv, D = kv.shape
    bt = _c(bt_row, np.int32)
    pg = _c(pages, np.int32)
    o = np.zeros(D)
    lse = np.zeros(1)
    lib.oracle_attend(_ptr(qd), D, _ptr(kv), NB, P, H_kv, int(kv_head), _ptr(bt),
                      int(seq_len), _ptr(pg), pg.shape[0], float(scale),
                      _ptr(o), _ptr(lse))
    return o, float(lse[0])


def attend_alibi(q_row, kv_cache, kv_head, bt_row, seq_len, pages, scale, slope):
    """attend() with the ALiBi bias slope * (t - (seq_len - 1)) on each logit."""
    lib = _load()
    qd = _c(q_row, np.float64)
    kv = _c(kv_cache, np.uint16)
    _, NB, P, H_kv, D = kv.shape
    bt = _c(bt_row, np.int32)
    pg = _c(pages, np.int32)
    o = np.zeros(D)
    lse = np.zeros(1)
    lib.oracle_attend_alibi(_ptr(qd), D, _ptr(kv), NB, P, H_kv, int(kv_head), _ptr(bt),
                            int(seq_len), _ptr(pg), pg.shape[0], float(scale),
                            float(slope), _ptr(o), _ptr(lse))
    return o, float(lse[0])


def page_score_alibi(q, kmin, kmax, kmean, block_table, seq_lens, page_size,
                     w_avg, w_peak, alibi, aggregate=False, ld=None):
    """ALiBi-aware page scores: [B, H_q, ld], or [B, H_kv, ld] group means when
    aggregate; alibi [H_q] in score units (slope / softmax scale)."""
    lib = _load()
    qd = _c(q, np.float64)
    B, H_q, D = qd.shape
    mn, mx, me = (_c(a, np.float64) for a in (kmin, kmax, kmean))
    H_kv = mn.shape[1]
    bt = _c(block_table, np.int32)
    sl = _c(seq_lens, np.int32)
    al = _c(alibi, np.float64)
    if ld is None:
        ld = bt.shape[1]
    s = np.full((B, H_kv if aggregate else H_q, ld), np.nan)
    lib.oracle_page_score_alibi(_ptr(qd), B, H_q, H_kv, D, _ptr(mn), _ptr(mx), _ptr(me),
                                _ptr(bt), bt.shape[1], _ptr(sl), page_size, float(w_avg),
                                float(w_peak), _ptr(al), int(bool(aggregate)), _ptr(s), ld)
    return s


def entmax15_tau(z):
    """tau of 1.5-entmax over the logits z (bisection in float64)."""
    zz = _c(z, np.float64)
    return float(_load().oracle_entmax15_tau(_ptr(zz), zz.shape[0]))


def attend_entmax15(q_row, kv_cache, kv_head, bt_row, seq_len, pages, scale, slope=None):
    """(o [D], tau) of 1.5-entmax attention of one query row over the tokens
    of the given pages; slope (logit units) adds the ALiBi bias
    slope * (pos - (S - 1))."""
    lib = _load()
    qd = _c(q_row, np.float64)
    kv = _c(kv_cache, np.uint16)
    _, NB, P, H_kv, D = kv.shape
    bt = _c(bt_row, np.int32)
    pg = _c(pages, np.int32)
    o = np.zeros(D)
    tau = np.zeros(1)
    if slope is None:
        lib.oracle_attend_entmax15(_ptr(qd), D, _ptr(kv), NB, P, H_kv, int(kv_head),
                                   _ptr(bt), int(seq_len), _ptr(pg), pg.shape[0],
                                   float(scale), _ptr(o), _ptr(tau))
    else:
        lib.oracle_attend_entmax15_alibi(_ptr(qd), D, _ptr(kv), NB, P, H_kv, int(kv_head),
                                         _ptr(bt), int(seq_len), _ptr(pg), pg.shape[0],
                                         float(scale), float(slope), _ptr(o), _ptr(tau))
    return o, float(tau[0])


def page_var(kv_cache, block_table, seq_lens, page_size):
    """Population variance per (block, kv head, d) over each page's valid rows
    (float64 [num_blocks, H_kv, D]; unused blocks stay NaN)."""
    lib = _load()
    kv = _c(kv_cache, np.uint16)
    _, NB, P, H_kv, D = kv.shape
    bt = _c(block_table, np.int32)
    sl = _c(seq_lens, np.int32)
    out = np.full((NB, H_kv, D), np.nan)
    lib.oracle_page_var(_ptr(kv), NB, P, H_kv, D, _ptr(bt), bt.shape[1], _ptr(sl),
                        sl.shape[0], _ptr(out))
    return out


def gauss_moments(q, kmean, kvar, block_table, seq_lens, page_size, scale, alibi=None,
                  ld=None):
    """(mu, var) [B, H_q, ld] of each page's logits z = scale q.k."""
    lib = _load()
    qd = _c(q, np.float64)
    B, H_q, D = qd.shape
    me, va = _c(kmean, np.float64), _c(kvar, np.float64)
    H_kv = me.shape[1]
    bt = _c(block_table, np.int32)
    sl = _c(seq_lens, np.int32)
    if ld is None:
        ld = bt.shape[1]
    mu = np.full((B, H_q, ld), np.nan)
    var = np.full((B, H_q, ld), np.nan)
    al = None if alibi is None else _c(alibi, np.float64)
    lib.oracle_gauss_moments(_ptr(qd), B, H_q, H_kv, D, _ptr(me), _ptr(va), _ptr(bt),
                             bt.shape[1], _ptr(sl), page_size, float(scale),
                             None if al is None else _ptr(al), _ptr(mu), _ptr(var), ld)
    return mu, var


def gauss_tau(mu, var, n, mixture):
    """tau-hat of one row from its pages' (mu, var) and valid-row counts n."""
    m, v = _c(mu, np.float64), _c(var, np.float64)
    nn = _c(n, np.int32)
    return float(_load().oracle_gauss_tau(_ptr(m), _ptr(v), _ptr(nn), m.shape[0],
                                          int(bool(mixture))))


def gauss_select(mu, var, n, tau, bos, eos, k_cap):
    """Ascending pages of one row selected against tau-hat."""
    m, v = _c(mu, np.float64), _c(var, np.float64)
    nn = _c(n, np.int32)
    N = m.shape[0]
    out = np.full(max(N, 1), -1, dtype=np.int32)
    c = _load().oracle_gauss_select(_ptr(m), _ptr(v), _ptr(nn), N, float(tau), int(bos),
                                    int(eos), int(k_cap), _ptr(out))
    return out[:c].copy()


def lse_merge(o_parts, lses):
    """N-way LSE merge of partials [n, D] -> (out [D], lse)."""
    lib = _load()
    o = _c(o_parts, np.float64)
    l = _c(lses, np.float64)
    n, D = o.shape
    out = np.zeros(D)
    lse = np.zeros(1)
    lib.oracle_lse_merge(_ptr(o), _ptr(l), n, D, _ptr(out), _ptr(lse))
    return out, float(lse[0])


def append(kv_cache, block_table, seq_lens, k_new, v_new, hh=None):
    """In-place append of k_new / v_new ([B, H_kv, D] bf16 bits) at token
    S_b - 1, zeroing hh ([num_blocks*P, H_kv] bf16 bits) at the written slot."""
    lib = _load()
    assert kv_cache.flags.c_contiguous and kv_cache.dtype == np.uint16
    _, NB, P, H_kv, D = kv_cache.shape
    bt = _c(block_table, np.int32)
    sl = _c(seq_lens, np.int32)
    kn = _c(k_new, np.uint16)
    vn = _c(v_new, np.uint16)
    if hh is not None:
        assert hh.flags.c_contiguous and hh.dtype == np.uint16
    lib.oracle_append(_ptr(kv_cache), NB, P, H_kv, D, _ptr(bt), bt.shape[1],
                      _ptr(sl), sl.shape[0], _ptr(kn), _ptr(vn), _ptr(hh))


def h2o_recurrence(p, hh, decay):
    """In-place accumulator step: hh <- bf16(bf16(p) + bf16(decay) * hh)."""
    lib = _load()
    pd = _c(p, np.float64)
    assert hh.flags.c_contiguous and hh.dtype == np.uint16
    assert hh.size == pd.size
    lib.oracle_h2o_recurrence(_ptr(pd), _ptr(hh), pd.size, float(decay))


def h2o_step(q, kv_cache, block_table, seq_lens, hh, bos, eos, scale, decay,
             ld=None, per_head=False):
    """Token-level H2O step (page_size 1).  Updates hh ([num_blocks, H_kv] bf16
    bits) in place and returns scores [B, H_kv, ld] (float64, NaN beyond S_b).
    per_head=False: softmax of the group-mean query; True: every query head's
    own softmax, averaged over the group."""
    lib = _load()
    qd = _c(q, np.float64)
    B, H_q, D = qd.shape
    kv = _c(kv_cache, np.uint16)
    _, NB, P, H_kv, _ = kv.shape
    assert P == 1
    bt = _c(block_table, np.int32)
    sl = _c(seq_lens, np.int32)
    assert hh.flags.c_contiguous and hh.dtype == np.uint16
    if ld is None:
        ld = bt.shape[1]
    s = np.full((B, H_kv, ld), np.nan)
    fn = lib.oracle_h2o_step_heads if per_head else lib.oracle_h2o_step
    fn(_ptr(qd), B, H_q, H_kv, D, _ptr(kv), NB, _ptr(bt), bt.shape[1], _ptr(sl),
       int(bos), int(eos), float(scale), float(decay), _ptr(hh), _ptr(s), ld)
    return s


def decode_step(q, kv_cache, block_table, seq_lens, stats, w_avg, w_peak,
                topk_pages, topk_frac, bos, eos, scale, k_cap):
    """Whole page-level step: returns (scores, sel_idx, sel_cnt, out, lse)."""
    lib = _load()
    qd = _c(q, np.float64)
    B, H_q, D = qd.shape
    kv = _c(kv_cache, np.uint16)
    _, NB, P, H_kv, _ = kv.shape
    bt = _c(block_table, np.int32)
    sl = _c(seq_lens, np.int32)
    mn, mx, me = (_c(a, np.float64) for a in stats)
    ld = bt.shape[1]
    scores = np.full((B, H_q, ld), np.nan)
    sel = np.full((B, H_q, k_cap), -1, dtype=np.int32)
    cnt = np.zeros((B, H_q), dtype=np.int32)
    out = np.zeros((B, H_q, D))
    lse = np.zeros((B, H_q))
    lib.oracle_decode_step(_ptr(qd), B, H_q, H_kv, D, _ptr(kv), NB, P, _ptr(bt),
                           ld, _ptr(sl), _ptr(mn), _ptr(mx), _ptr(me),
                           float(w_avg), float(w_peak), int(topk_pages),
                           float(topk_frac), int(bos), int(eos), float(scale),
                           _ptr(scores), ld, _ptr(sel), _ptr(cnt), k_cap,
                           _ptr(out), _ptr(lse))
    return scores, sel, cnt, out, lse
